"""GPU parity of the backward pass (pblock_forward_train + pblock_backward) through the C ABI,
against the fp64 oracle's block_backward: dx, dgamma, dbeta, dW_in, dW_out."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, from_dev, log, rel_err, run_block, scale_q_rows, to_dev, upload
from workload import CONFIGS, BlockConfig, make_dy, make_inputs

pytestmark = pytest.mark.gpu

GRAD_KEYS = ("dx", "dgamma", "dbeta", "dw_in", "dw_out")

SHAPES = [
    # name, B, S, d, H, hd, ffn, W, add_residual
    ("bwd_ragged", 2, 200, 256, 2, 128, 320, 37, 1),
    ("bwd_hd64", 1, 333, 192, 3, 64, 128, 100, 1),
    ("bwd_multi_tile", 1, 700, 512, 4, 128, 768, 300, 0),
    ("bwd_w1", 1, 130, 128, 2, 64, 64, 1, 1),
    ("bwd_w_ge_s", 2, 150, 256, 2, 128, 192, 1000, 1),
    ("bwd_one_token", 1, 1, 128, 1, 64, 64, 4, 1),
    ("bwd_big_ntail", 3, 1100, 1024, 8, 128, 2112, 200, 1),
    # B*S a multiple of 256: dy is read in place as the GEMMs' row operand (no staging copy);
    # d = 192 also has the K-major dy reads clamp at the last 8 columns
    ("bwd_whole_tiles", 2, 256, 256, 2, 128, 320, 64, 1),
    ("bwd_whole_tiles_d192", 1, 768, 192, 3, 64, 128, 100, 0),
    # the two weight-gradient GEMMs in one launch: dW_out 11 x 13 = 143 tiles (an odd count, so
    # the second GEMM's workgroups start mid-XCD) and dW_in 15 x 11 = 165, each a partial wave
    ("bwd_paired_wgrad", 1, 2048, 2816, 2, 128, 3072, 256, 0),
    # d = 16384, the largest the backward accepts (Q rows of W_in scaled by 2^-3, see below)
    ("bwd_max_d", 1, 130, 16384, 2, 64, 128, 40, 1),
]
# For very wide models N(0, 0.02^2) weights give attention scores whose spread grows with
# sqrt(d) (~6.5 at d = 16384); these shapes scale the Q rows of W_in by an exact power of two
# so that the scores stay O(1), like the other small shapes.
Q_SCALE = {"bwd_max_d": 3}


def run_train(cfg, dev, dy_dev, handle=None):
    """forward_train then backward on the GPU; returns y and the gradients as float64 numpy."""
    import torch

    import transformer_block_fwd_amd as tb

    own = handle is None
    h = tb.pblock_create(cfg) if own else handle
    try:
        ws = torch.empty(tb.pblock_train_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
        out = torch.empty_like(dev["x"])
        weights = (dev["gamma"], dev["beta"], dev["w_in"], dev["w_out"])
        tb.pblock_forward_train(h, dev["x"], weights, cfg, out, ws)
        grads = {"dx": torch.empty_like(dev["x"]), "dln_gamma": torch.empty_like(dev["gamma"]),
                 "dln_beta": torch.empty_like(dev["beta"]), "dw_in": torch.empty_like(dev["w_in"]),
                 "dw_out": torch.empty_like(dev["w_out"])}
        tb.pblock_backward(h, dev["x"], weights, cfg, dy_dev, grads, ws)
        torch.cuda.synchronize()
        res = {"y": from_dev(out).reshape(cfg.B, cfg.S, cfg.d), "dx": from_dev(grads["dx"]).reshape(cfg.B, cfg.S, cfg.d),
               "dgamma": from_dev(grads["dln_gamma"]), "dbeta": from_dev(grads["dln_beta"]),
               "dw_in": from_dev(grads["dw_in"]).reshape(cfg.n_in, cfg.d),
               "dw_out": from_dev(grads["dw_out"]).reshape(cfg.d, cfg.k_out)}
        return res
    finally:
        if own:
            tb.pblock_destroy(h)


def check_grads(name, got, ref, tol):
    worst = 0.0
    for k in GRAD_KEYS:
        err = rel_err(got[k], ref[k])
        log(f"[parity] {name} {k}: rel err {err:.3e}")
        worst = max(worst, err)
    assert worst <= tol, f"{name}: worst gradient error {worst:.3e} > {tol}"


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_backward_small_full(shape):
    name, B, S, d, H, hd, ffn, W, res = shape
    cfg = BlockConfig(name, B=B, S=S, d=d, H=H, hd=hd, ffn=ffn, W=W, dtype="bf16", add_residual=res)
    log(f"[case] backward {cfg}")
    inp = make_inputs(cfg, seed=31, affine=True)
    if name in Q_SCALE:
        scale_q_rows(inp, Q_SCALE[name])
    dyd = make_dy(cfg, seed=31)
    dev = upload(inp)
    got = run_train(cfg, dev, to_dev(dyd["dy_dev"], "bf16"))
    ref = oracle.block_backward(inp.x, inp.gamma, inp.beta, inp.w_in, inp.w_out, dyd["dy"], cfg.H, cfg.hd, cfg.W,
                                eps=cfg.ln_eps, add_residual=bool(res))
    check_grads(name, got, ref, TOL["bf16"])
    # the training forward is the plain forward
    y0 = run_block(cfg, dev)
    assert np.array_equal(got["y"], y0)


# At the 175B shard shape the attention scores have a standard deviation of ~4.9 (max ~29), so
# the bf16 storage of u and of q, k, v (2^-9 relative each) already moves the exact attention
# output by 1.64e-2 of its maximum: the fp64 oracle fed the bf16-rounded u, q, k, v lands there
# (tests/test_precision_floor.py computes it on the CPU).  Every gradient inherits that floor through the stored attention
# output (dW_out), D = dO.O and dS, so the bar for this shape is 2e-2; the small shapes, whose
# scores are O(0.1), keep the 1e-2 of the forward.
TOL_BWD_SHARD = 2e-2


def test_backward_shard175b_full():
    """The 175B shard shape (no residual): every gradient element against the oracle."""
    import torch

    cfg = CONFIGS["shard175b"]
    log(f"[case] backward {cfg}")
    inp = make_inputs(cfg, seed=0)
    dyd = make_dy(cfg, seed=0)
    dev = upload(inp)
    got = run_train(cfg, dev, to_dev(dyd["dy_dev"], "bf16"))
    del dev
    torch.cuda.empty_cache()
    ref = oracle.block_backward(inp.x, inp.gamma, inp.beta, inp.w_in, inp.w_out, dyd["dy"], cfg.H, cfg.hd, cfg.W,
                                eps=cfg.ln_eps, add_residual=bool(cfg.add_residual))
    check_grads("shard175b", got, ref, TOL_BWD_SHARD)


def test_window_at_int32_max_is_full_causal():
    """W = 2^31 - 1, the largest window the cfg can hold, is full causal attention: the forward
    and every gradient are bit-identical to W = S (the window sums never overflow)."""
    cfg = BlockConfig("w_max", B=2, S=300, d=256, H=2, hd=128, ffn=256, W=300, dtype="bf16")
    inp = make_inputs(cfg, seed=33, affine=True)
    dyd = make_dy(cfg, seed=33)
    dev = upload(inp)
    dy = to_dev(dyd["dy_dev"], "bf16")
    got_s = run_train(cfg, dev, dy)
    got_max = run_train(cfg.replace(W=2 ** 31 - 1), dev, dy)
    for k in ("y",) + GRAD_KEYS:
        assert np.array_equal(got_s[k], got_max[k]), k
    ref = oracle.block_backward(inp.x, inp.gamma, inp.beta, inp.w_in, inp.w_out, dyd["dy"], cfg.H, cfg.hd, cfg.S,
                                eps=cfg.ln_eps, add_residual=True)
    check_grads("w_max", got_max, ref, TOL["bf16"])


def test_backward_rejections():
    import torch

    import transformer_block_fwd_amd as tb
    from transformer_block_fwd_amd import _abi

    cfg = BlockConfig("rej", B=1, S=64, d=128, H=1, hd=64, ffn=64, W=8, dtype="bf16")
    inp = make_inputs(cfg, seed=1)
    dev = upload(inp)
    dy = to_dev(make_dy(cfg, seed=1)["dy_dev"], "bf16")
    h = tb.pblock_create(cfg)
    try:
        need = tb.pblock_train_workspace_bytes(cfg)
        ws = torch.empty(need + 512, dtype=torch.uint8, device="cuda")
        c = tb.as_cfg(cfg)
        w = _abi.PblockWeights(dev["gamma"].data_ptr(), dev["beta"].data_ptr(), dev["w_in"].data_ptr(),
                               dev["w_out"].data_ptr())
        grads = {k: torch.full_like(v, 7.0) for k, v in
                 (("dx", dev["x"]), ("dln_gamma", dev["gamma"]), ("dln_beta", dev["beta"]), ("dw_in", dev["w_in"]),
                  ("dw_out", dev["w_out"]))}
        g = _abi.PblockGrads(*(grads[k].data_ptr() for k in ("dx", "dln_gamma", "dln_beta", "dw_in", "dw_out")))
        f = _abi.lib().pblock_backward

        def call(ws_ptr, nbytes, gg=g, cc=c):
            return f(ctypes.c_void_p(h), ctypes.c_void_p(dev["x"].data_ptr()), ctypes.byref(w), ctypes.byref(cc),
                     ctypes.c_void_p(dy.data_ptr()), None if gg is None else ctypes.byref(gg), ctypes.c_void_p(ws_ptr),
                     nbytes, None)

        assert call(ws.data_ptr(), need - 256) == _abi.PBLOCK_ERR_ARG
        assert call(ws.data_ptr() + 16, need) == _abi.PBLOCK_ERR_ALIGN
        assert call(0, need) == _abi.PBLOCK_ERR_NULL
        assert call(ws.data_ptr(), need, gg=None) == _abi.PBLOCK_ERR_NULL
        g_alias = _abi.PblockGrads(g.dx, g.dln_gamma, g.dln_gamma, g.dw_in, g.dw_out)
        assert call(ws.data_ptr(), need, gg=g_alias) == _abi.PBLOCK_ERR_ALIAS
        g_ws = _abi.PblockGrads(ws.data_ptr() + 1024, g.dln_gamma, g.dln_beta, g.dw_in, g.dw_out)
        assert call(ws.data_ptr(), need, gg=g_ws) == _abi.PBLOCK_ERR_ALIAS
        # dy inside the workspace (dy may be read in place while the scratch is written)
        assert f(ctypes.c_void_p(h), ctypes.c_void_p(dev["x"].data_ptr()), ctypes.byref(w), ctypes.byref(c),
                 ctypes.c_void_p(ws.data_ptr() + 4096), ctypes.byref(g), ctypes.c_void_p(ws.data_ptr()), need,
                 None) == _abi.PBLOCK_ERR_ALIAS
        c32 = tb.as_cfg(cfg.replace(dtype="f32"))
        assert _abi.lib().pblock_train_workspace_bytes(ctypes.byref(c32)) == _abi.PBLOCK_ERR_DTYPE
        torch.cuda.synchronize()
        for k, v in grads.items():
            assert bool((v.float() == 7.0).all()), k
    finally:
        tb.pblock_destroy(h)


def test_backward_timing_categories():
    import torch

    import transformer_block_fwd_amd as tb

    cfg = BlockConfig("btiming", B=1, S=256, d=256, H=2, hd=128, ffn=256, W=32, dtype="bf16")
    inp = make_inputs(cfg, seed=2)
    dev = upload(inp)
    dy = to_dev(make_dy(cfg, seed=2)["dy_dev"], "bf16")
    h = tb.pblock_create(cfg)
    try:
        tb.pblock_set_timing(h, True)
        for _ in range(2):
            run_train(cfg, dev, dy, handle=h)
        ms, n = tb.pblock_kernel_times(h, backward=True)
        assert n == 4  # two forward_train and two backward calls
        # B*S = 256 fills whole GEMM tiles: dy is read in place and the staging step is empty
        assert all(v > 0 for k, v in ms.items() if k != "bwd_prep"), ms
        assert ms["bwd_prep"] >= 0, ms
        torch.cuda.synchronize()
    finally:
        tb.pblock_destroy(h)
