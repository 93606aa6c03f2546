"""GPU parity of the serial (pre-LN) layer built from the same kernels, through
the C ABI, against the fp64 oracle's serial_block_forward."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, from_dev, log, rel_err, to_dev, upload
from workload import CONFIGS, BlockConfig, make_inputs, make_ln2

pytestmark = pytest.mark.gpu

SERIAL_SMALL = [
    # name, B, S, d, H, hd, ffn, W, dtype
    ("serial_bf16_ragged", 2, 200, 256, 2, 128, 320, 37, "bf16"),
    ("serial_bf16_hd64", 1, 333, 192, 3, 64, 128, 100, "bf16"),
    ("serial_bf16_w1", 1, 130, 128, 2, 64, 64, 1, "bf16"),
    ("serial_bf16_multi_tile", 1, 700, 512, 4, 128, 768, 300, "bf16"),
    ("serial_bf16_big_ntail", 3, 1100, 1024, 8, 128, 2112, 200, "bf16"),
    ("serial_f32_ragged", 2, 77, 128, 2, 64, 192, 9, "f32"),
    ("serial_f32_w_ge_s", 1, 150, 256, 2, 128, 128, 1000, "f32"),
]


def run_serial(cfg, dev, ln2_dev, handle=None):
    import torch

    import transformer_block_fwd_amd as tb

    own = handle is None
    h = tb.pblock_create(cfg) if own else handle
    try:
        out = torch.empty_like(dev["x"])
        tb.pblock_forward_serial(h, dev["x"], (dev["gamma"], dev["beta"], dev["w_in"], dev["w_out"]),
                                 (ln2_dev["gamma2"], ln2_dev["beta2"]), cfg, out)
        torch.cuda.synchronize()
        return from_dev(out).reshape(cfg.B, cfg.S, cfg.d)
    finally:
        if own:
            tb.pblock_destroy(h)


def upload_ln2(cfg, ln2):
    return {"gamma2": to_dev(ln2["gamma2_dev"], cfg.dtype), "beta2": to_dev(ln2["beta2_dev"], cfg.dtype)}


@pytest.mark.parametrize("case", SERIAL_SMALL, ids=[c[0] for c in SERIAL_SMALL])
def test_serial_small_full(case):
    name, B, S, d, H, hd, ffn, W, dtype = case
    cfg = BlockConfig(name, B=B, S=S, d=d, H=H, hd=hd, ffn=ffn, W=W, dtype=dtype)
    log(f"[case] serial {cfg}")
    inp = make_inputs(cfg, seed=8, affine=True)
    ln2 = make_ln2(cfg, seed=8, affine=True)
    y = run_serial(cfg, upload(inp), upload_ln2(cfg, ln2))
    ref = oracle.serial_block_forward(inp.x, inp.gamma, inp.beta, ln2["gamma2"], ln2["beta2"], inp.w_in, inp.w_out,
                                      cfg.H, cfg.hd, cfg.W, eps=cfg.ln_eps)
    err = rel_err(y, ref)
    log(f"[parity] {name}: rel err {err:.3e} (tol {TOL[dtype]})")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("name", ["small", "shard175b"])
def test_serial_full_size(name):
    """Full-size shapes (the 175B shard shape with the residual stream on): every output
    against the oracle's serial layer."""
    import torch

    cfg = CONFIGS[name].replace(add_residual=1)
    log(f"[case] serial {cfg}")
    inp = make_inputs(cfg, seed=0)
    ln2 = make_ln2(cfg, seed=0, affine=True)
    dev = upload(inp)
    y = run_serial(cfg, dev, upload_ln2(cfg, ln2))
    del dev
    torch.cuda.empty_cache()
    assert np.isfinite(y).all()
    ref = oracle.serial_block_forward(inp.x, inp.gamma, inp.beta, ln2["gamma2"], ln2["beta2"], inp.w_in, inp.w_out,
                                      cfg.H, cfg.hd, cfg.W, eps=cfg.ln_eps)
    err = rel_err(y, ref)
    log(f"[parity] serial {name}: all {y.size} outputs, rel err {err:.3e} (tol {TOL['bf16']})")
    assert err <= TOL["bf16"]


def test_serial_matches_parallel_with_one_sublayer_off():
    """W_2 = 0: the serial layer is x + attention branch, as is the parallel block with
    FC1 rows zero (GPU against GPU; the GEMM split differs, so to tolerance)."""
    from gpu_helpers import run_block

    cfg = BlockConfig("one_sublayer", B=2, S=300, d=256, H=2, hd=128, ffn=384, W=64, dtype="bf16")
    inp = make_inputs(cfg, seed=9, affine=True)
    dev = upload(inp)
    A = cfg.A
    ln1 = {"gamma2": dev["gamma"], "beta2": dev["beta"]}
    w_out_attn = dev["w_out"].clone()
    w_out_attn[:, A:] = 0
    y_serial = run_serial(cfg, dict(dev, w_out=w_out_attn), ln1)
    w_in_attn = dev["w_in"].clone()
    w_in_attn[3 * A:] = 0
    y_par = run_block(cfg, dict(dev, w_in=w_in_attn))
    err = rel_err(y_serial, y_par)
    log(f"[parity] serial vs parallel, MLP off: {err:.3e}")
    assert err <= TOL["bf16"]


def test_serial_rejects_partial_and_leaves_out_untouched():
    """add_residual = 0 is refused before any launch; out keeps its contents."""
    import torch

    import transformer_block_fwd_amd as tb
    from transformer_block_fwd_amd import _abi

    cfg = BlockConfig("rej", B=1, S=64, d=128, H=1, hd=64, ffn=64, W=8, dtype="bf16", add_residual=0)
    inp = make_inputs(cfg, seed=1)
    dev = upload(inp)
    ln2 = upload_ln2(cfg, make_ln2(cfg))
    h = tb.pblock_create(cfg)
    try:
        out = torch.full_like(dev["x"], 3.0)
        c = tb.as_cfg(cfg)
        w = _abi.PblockWeights(dev["gamma"].data_ptr(), dev["beta"].data_ptr(), dev["w_in"].data_ptr(),
                               dev["w_out"].data_ptr())
        st = _abi.lib().pblock_forward_serial(ctypes.c_void_p(h), ctypes.c_void_p(dev["x"].data_ptr()),
                                              ctypes.byref(w), ctypes.c_void_p(ln2["gamma2"].data_ptr()),
                                              ctypes.c_void_p(ln2["beta2"].data_ptr()), ctypes.byref(c),
                                              ctypes.c_void_p(out.data_ptr()), None)
        assert st == _abi.PBLOCK_ERR_ARG
        st = _abi.lib().pblock_forward_serial(ctypes.c_void_p(h), ctypes.c_void_p(dev["x"].data_ptr()),
                                              ctypes.byref(w), None, ctypes.c_void_p(ln2["beta2"].data_ptr()),
                                              ctypes.byref(c), ctypes.c_void_p(out.data_ptr()), None)
        assert st == _abi.PBLOCK_ERR_NULL
        torch.cuda.synchronize()
        assert bool((out.float() == 3.0).all())
    finally:
        tb.pblock_destroy(h)


def test_serial_timing_categories():
    """The timing API attributes the serial form's seven launches to the four categories."""
    import torch

    import transformer_block_fwd_amd as tb

    cfg = BlockConfig("timing", B=1, S=256, d=256, H=2, hd=128, ffn=256, W=32, dtype="bf16")
    inp = make_inputs(cfg, seed=2)
    dev = upload(inp)
    ln2 = upload_ln2(cfg, make_ln2(cfg))
    h = tb.pblock_create(cfg)
    try:
        tb.pblock_set_timing(h, True)
        for _ in range(3):
            run_serial(cfg, dev, ln2, handle=h)
        ms, n = tb.pblock_kernel_times(h)
        assert n == 3
        assert all(v > 0 for v in ms.values()), ms
        torch.cuda.synchronize()
    finally:
        tb.pblock_destroy(h)


def test_mfma_loop_runs():
    """The measurement aid's register-only MFMA loops (both forms, even and odd iteration counts) complete
    and write finite sums."""
    import torch

    import transformer_block_fwd_amd as tb

    for form in ("16x16x32", "32x32x16"):
        for iters in (10, 11):
            sink = torch.full((8 * 256,), float("nan"), dtype=torch.float32, device="cuda")
            tb.pblock_mfma_loop(8, iters, sink, form=form)
            torch.cuda.synchronize()
            assert bool(torch.isfinite(sink).all()), (form, iters)
