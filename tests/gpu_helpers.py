"""Helpers shared by the GPU tests: moving seeded inputs to the device and
running the block through the C ABI."""
from __future__ import annotations

import sys

import numpy as np

from oracle import relative_error as rel_err  # noqa: F401  (the pinned parity metric)

TOL = {"bf16": 1e-2, "f32": 1e-4}  # max|y_gpu - y_ref| / max|y_ref|


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(arr: np.ndarray, dtype: str):
    import torch

    if dtype == "bf16":
        a = np.ascontiguousarray(arr)
        assert a.dtype == np.uint16
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def from_dev(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def scale_q_rows(inp, k: int):
    """Multiplies the Q rows of W_in by 2^-k in place (exact in bf16 and fp32, so the device and
    the oracle still see identical values).  Keeps attention scores O(1) for very wide models,
    where N(0, 0.02^2) weights give scores whose spread grows with sqrt(d)."""
    from workload import round_to_bf16

    A = inp.cfg.A
    w = inp.w_in.copy()
    w[:A] *= np.float32(2.0 ** -k)
    if inp.bits is not None:
        vals, bits = round_to_bf16(w)
        assert np.array_equal(vals, w)
        inp.bits["w_in"] = bits
    inp.w_in = w
    return inp


def upload(inp):
    cfg = inp.cfg
    arrs = inp.device_arrays()
    return {k: to_dev(v, cfg.dtype) for k, v in arrs.items()}


def run_block(cfg, dev, handle=None, want_parts=False):
    """Forward on the GPU; returns y (float64 numpy [B, S, d]) and optionally u, qkv, ag."""
    import torch

    import transformer_block_fwd_amd as tb

    own = handle is None
    h = tb.pblock_create(cfg) if own else handle
    try:
        out = torch.empty_like(dev["x"])
        tb.pblock_forward(h, dev["x"], (dev["gamma"], dev["beta"], dev["w_in"], dev["w_out"]), cfg, out)
        parts = None
        if want_parts:
            tdt = dev["x"].dtype
            M = cfg.B * cfg.S
            u = torch.empty((M, cfg.d), dtype=tdt, device="cuda")
            qkv = torch.empty((M, 3 * cfg.A), dtype=tdt, device="cuda")
            ag = torch.empty((M, cfg.k_out), dtype=tdt, device="cuda")
            tb.pblock_copy_intermediates(h, u, qkv, ag)
            parts = dict(u=from_dev(u), qkv=from_dev(qkv), ag=from_dev(ag))
        torch.cuda.synchronize()
        y = from_dev(out).reshape(cfg.B, cfg.S, cfg.d)
    finally:
        if own:
            tb.pblock_destroy(h)
    return (y, parts) if want_parts else y




_ORACLE_Y: dict = {}  # full oracle outputs, by (config, seed), shared by the tests of one process


def oracle_y_cached(inp, seed: int):
    """The oracle's full block forward on ``inp`` (made from ``inp.cfg`` with ``seed``), computed
    once per process: several full-size tests compare against the same workload."""
    import oracle

    c = inp.cfg
    key = (c, seed)
    if key not in _ORACLE_Y:
        _ORACLE_Y.clear()  # one full-size reference at a time (hundreds of MB each)
        _ORACLE_Y[key] = oracle.block_forward(inp.x, inp.gamma, inp.beta, inp.w_in, inp.w_out, c.H, c.hd, c.W,
                                              eps=c.ln_eps, add_residual=bool(c.add_residual))
    return _ORACLE_Y[key]
