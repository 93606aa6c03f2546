"""GPU parity of the variant switches (tanh GeLU, linear biases, rotary embedding of q and
k, a second LayerNorm for the MLP branch) through the C ABI, against the fp64 oracle's
block_forward_variant."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, from_dev, log, rel_err, run_block, to_dev, upload
from workload import CONFIGS, BlockConfig, make_inputs, make_ln2, make_variant_params

pytestmark = pytest.mark.gpu

SHAPES = [
    # name, B, S, d, H, hd, ffn, W, dtype
    ("v_bf16_ragged", 2, 200, 256, 2, 128, 320, 37, "bf16"),
    ("v_bf16_hd64", 1, 333, 192, 3, 64, 128, 100, "bf16"),
    ("v_bf16_multi_tile", 1, 700, 512, 4, 128, 768, 300, "bf16"),
    ("v_f32", 2, 77, 128, 2, 64, 192, 9, "f32"),
]
KNOBS = {
    "tanh": dict(gelu_tanh=True),
    "bias": dict(bias=True),
    "rope": dict(rope=True, rope_base=10000.0),
    "two_ln": dict(two_ln=True),
    "all": dict(gelu_tanh=True, bias=True, rope=True, rope_base=500.0, two_ln=True),
}


def upload_extra(cfg, vp, ln2):
    return {"b_in": to_dev(vp["b_in_dev"], cfg.dtype), "b_out": to_dev(vp["b_out_dev"], cfg.dtype),
            "ln2_gamma": to_dev(ln2["gamma2_dev"], cfg.dtype), "ln2_beta": to_dev(ln2["beta2_dev"], cfg.dtype)}


def run_variant(cfg, dev, extra, knobs, handle=None):
    import torch

    import transformer_block_fwd_amd as tb

    own = handle is None
    h = tb.pblock_create(cfg) if own else handle
    try:
        out = torch.empty_like(dev["x"])
        ex = {}
        if knobs.get("bias"):
            ex.update(b_in=extra["b_in"], b_out=extra["b_out"])
        if knobs.get("two_ln"):
            ex.update(ln2_gamma=extra["ln2_gamma"], ln2_beta=extra["ln2_beta"])
        var = tb.make_variant(gelu_tanh=knobs.get("gelu_tanh", False), rope=knobs.get("rope", False),
                              rope_base=knobs.get("rope_base", 10000.0), two_ln=knobs.get("two_ln", False))
        tb.pblock_forward_variant(h, dev["x"], (dev["gamma"], dev["beta"], dev["w_in"], dev["w_out"]), ex, cfg, var,
                                  out)
        torch.cuda.synchronize()
        return from_dev(out).reshape(cfg.B, cfg.S, cfg.d)
    finally:
        if own:
            tb.pblock_destroy(h)


def oracle_kwargs(knobs, vp, ln2):
    kw = dict(gelu_form="tanh" if knobs.get("gelu_tanh") else "erf",
              rope_base=knobs.get("rope_base") if knobs.get("rope") else None)
    if knobs.get("bias"):
        kw.update(b_in=vp["b_in"], b_out=vp["b_out"])
    if knobs.get("two_ln"):
        kw.update(gamma2=ln2["gamma2"], beta2=ln2["beta2"])
    return kw


@pytest.mark.parametrize("knob", sorted(KNOBS))
@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_variant_small_full(shape, knob):
    name, B, S, d, H, hd, ffn, W, dtype = shape
    cfg = BlockConfig(name, B=B, S=S, d=d, H=H, hd=hd, ffn=ffn, W=W, dtype=dtype)
    knobs = KNOBS[knob]
    log(f"[case] variant {knob} {cfg}")
    inp = make_inputs(cfg, seed=21, affine=True)
    vp = make_variant_params(cfg, seed=21)
    ln2 = make_ln2(cfg, seed=21, affine=True)
    y = run_variant(cfg, upload(inp), upload_extra(cfg, vp, ln2), knobs)
    ref = oracle.block_forward_variant(inp.x, inp.gamma, inp.beta, inp.w_in, inp.w_out, cfg.H, cfg.hd, cfg.W,
                                       eps=cfg.ln_eps, **oracle_kwargs(knobs, vp, ln2))
    err = rel_err(y, ref)
    log(f"[parity] {name} {knob}: rel err {err:.3e} (tol {TOL[dtype]})")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("name", ["small", "shard175b"])
def test_variant_full_size(name):
    """Every switch on at full size (with the residual): every output against the oracle's
    variant block."""
    import torch

    cfg = CONFIGS[name].replace(add_residual=1)
    knobs = KNOBS["all"]
    log(f"[case] variant all {cfg}")
    inp = make_inputs(cfg, seed=0)
    vp = make_variant_params(cfg, seed=0)
    ln2 = make_ln2(cfg, seed=0, affine=True)
    dev = upload(inp)
    y = run_variant(cfg, dev, upload_extra(cfg, vp, ln2), knobs)
    del dev
    torch.cuda.empty_cache()
    assert np.isfinite(y).all()
    ref = oracle.block_forward_variant(inp.x, inp.gamma, inp.beta, inp.w_in, inp.w_out, cfg.H, cfg.hd, cfg.W,
                                       eps=cfg.ln_eps, **oracle_kwargs(knobs, vp, ln2))
    err = rel_err(y, ref)
    log(f"[parity] variant {name}: all {y.size} outputs, rel err {err:.3e} (tol {TOL['bf16']})")
    assert err <= TOL["bf16"]


def test_all_off_equals_forward_bitwise():
    """With every switch off the variant entry runs pblock_forward's launches: same bits."""
    cfg = BlockConfig("off", B=2, S=300, d=256, H=2, hd=128, ffn=384, W=64, dtype="bf16")
    inp = make_inputs(cfg, seed=22, affine=True)
    dev = upload(inp)
    y0 = run_block(cfg, dev)
    y1 = run_variant(cfg, dev, None, {})
    assert np.array_equal(y0, y1)


def test_rope_base_change_rebuilds_table():
    """Two bases on one handle, alternating: each result matches the oracle for its base."""
    import transformer_block_fwd_amd as tb

    cfg = BlockConfig("rope2", B=1, S=257, d=256, H=2, hd=64, ffn=128, W=100, dtype="bf16")
    inp = make_inputs(cfg, seed=23, affine=True)
    dev = upload(inp)
    h = tb.pblock_create(cfg)
    try:
        for base in (10000.0, 37.0, 10000.0):
            y = run_variant(cfg, dev, None, dict(rope=True, rope_base=base), handle=h)
            ref = oracle.block_forward_variant(inp.x, inp.gamma, inp.beta, inp.w_in, inp.w_out, cfg.H, cfg.hd,
                                               cfg.W, eps=cfg.ln_eps, rope_base=base)
            err = rel_err(y, ref)
            log(f"[parity] rope base {base}: {err:.3e}")
            assert err <= TOL["bf16"]
    finally:
        tb.pblock_destroy(h)


def test_rope_on_a_second_stream():
    """Rotary calls on one handle from two streams in turn (each synchronised before the next):
    the table is rebuilt on the second stream, and both results equal the oracle's and each other."""
    import torch

    import transformer_block_fwd_amd as tb

    cfg = BlockConfig("rope_streams", B=1, S=193, d=256, H=2, hd=64, ffn=128, W=64, dtype="bf16")
    inp = make_inputs(cfg, seed=29, affine=True)
    dev = upload(inp)
    ref = oracle.block_forward_variant(inp.x, inp.gamma, inp.beta, inp.w_in, inp.w_out, cfg.H, cfg.hd, cfg.W,
                                       eps=cfg.ln_eps, rope_base=10000.0)
    h = tb.pblock_create(cfg)
    s2 = torch.cuda.Stream()
    try:
        y1 = run_variant(cfg, dev, None, dict(rope=True, rope_base=10000.0), handle=h)
        with torch.cuda.stream(s2):
            y2 = run_variant(cfg, dev, None, dict(rope=True, rope_base=10000.0), handle=h)
        y3 = run_variant(cfg, dev, None, dict(rope=True, rope_base=10000.0), handle=h)
        for y in (y1, y2, y3):
            assert rel_err(y, ref) <= TOL["bf16"]
        assert np.array_equal(y1, y2) and np.array_equal(y1, y3)
    finally:
        tb.pblock_destroy(h)


def test_variant_rejections_leave_out_untouched():
    import torch

    import transformer_block_fwd_amd as tb
    from transformer_block_fwd_amd import _abi

    cfg = BlockConfig("rej", B=1, S=64, d=128, H=1, hd=64, ffn=64, W=8, dtype="bf16")
    inp = make_inputs(cfg, seed=1)
    dev = upload(inp)
    vp = make_variant_params(cfg, seed=1)
    ex = upload_extra(cfg, vp, make_ln2(cfg))
    h = tb.pblock_create(cfg)
    try:
        out = torch.full_like(dev["x"], 3.0)
        c = tb.as_cfg(cfg)
        w = _abi.PblockWeights(dev["gamma"].data_ptr(), dev["beta"].data_ptr(), dev["w_in"].data_ptr(),
                               dev["w_out"].data_ptr())
        f = _abi.lib().pblock_forward_variant

        def call(var, vw):
            return f(ctypes.c_void_p(h), ctypes.c_void_p(dev["x"].data_ptr()), ctypes.byref(w),
                     None if vw is None else ctypes.byref(vw), ctypes.byref(c),
                     None if var is None else ctypes.byref(var), ctypes.c_void_p(out.data_ptr()), None)

        good_vw = _abi.PblockVariantWeights(ex["b_in"].data_ptr(), ex["b_out"].data_ptr(),
                                            ex["ln2_gamma"].data_ptr(), ex["ln2_beta"].data_ptr())
        assert call(None, good_vw) == _abi.PBLOCK_ERR_NULL
        assert call(_abi.PblockVariant(2, 0, 10000.0, 0), good_vw) == _abi.PBLOCK_ERR_ARG
        assert call(_abi.PblockVariant(0, 1, 0.0, 0), good_vw) == _abi.PBLOCK_ERR_ARG
        assert call(_abi.PblockVariant(0, 1, float("inf"), 0), good_vw) == _abi.PBLOCK_ERR_ARG
        assert call(_abi.PblockVariant(0, 0, 1.0, 1), None) == _abi.PBLOCK_ERR_NULL
        assert call(_abi.PblockVariant(0, 0, 1.0, 1),
                    _abi.PblockVariantWeights(0, 0, ex["ln2_gamma"].data_ptr(), 0)) == _abi.PBLOCK_ERR_NULL
        bad_align = _abi.PblockVariantWeights(ex["b_in"].data_ptr() + 2, 0, 0, 0)
        assert call(_abi.PblockVariant(0, 0, 1.0, 0), bad_align) == _abi.PBLOCK_ERR_ALIGN
        alias = _abi.PblockVariantWeights(0, out.data_ptr() + 64, 0, 0)
        assert call(_abi.PblockVariant(0, 0, 1.0, 0), alias) == _abi.PBLOCK_ERR_ALIAS
        torch.cuda.synchronize()
        assert bool((out.float() == 3.0).all())
        # a NULL variant-weights block is fine when nothing needs it
        assert call(_abi.PblockVariant(1, 1, 10000.0, 0), None) == _abi.PBLOCK_OK
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out.float()).all())
    finally:
        tb.pblock_destroy(h)


def test_variant_timing_categories():
    """The two-LayerNorm form's launches land in the four timing categories."""
    import torch

    import transformer_block_fwd_amd as tb

    cfg = BlockConfig("vtiming", B=1, S=256, d=256, H=2, hd=128, ffn=256, W=32, dtype="bf16")
    inp = make_inputs(cfg, seed=2)
    dev = upload(inp)
    ex = upload_extra(cfg, make_variant_params(cfg), make_ln2(cfg))
    h = tb.pblock_create(cfg)
    try:
        tb.pblock_set_timing(h, True)
        for _ in range(3):
            run_variant(cfg, dev, ex, KNOBS["all"], handle=h)
        ms, n = tb.pblock_kernel_times(h)
        assert n == 3
        assert all(v > 0 for v in ms.values()), ms
        torch.cuda.synchronize()
    finally:
        tb.pblock_destroy(h)
