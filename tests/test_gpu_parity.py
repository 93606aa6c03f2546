"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar: max|y_gpu - y_ref| / max|y_ref| <= 1e-2 for bf16 and <= 1e-4 for fp32,
elementwise over every output, for the small shapes and for the full-size
workloads in the launch configuration the benchmark times (only the 2^24-token
limit case compares row blocks the oracle computes one by one).  Invariants that hold at any size are
checked bit-for-bit where the arithmetic makes them exact.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, from_dev, log, oracle_y_cached, rel_err, run_block, scale_q_rows, to_dev, upload
from workload import CONFIGS, BlockConfig, make_inputs

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import transformer_block_fwd_amd as tb  # noqa: E402


def oracle_y(inp):
    c = inp.cfg
    return oracle.block_forward(inp.x, inp.gamma, inp.beta, inp.w_in, inp.w_out, c.H, c.hd, c.W,
                                eps=c.ln_eps, add_residual=bool(c.add_residual))


SMALL = [
    # name, B, S, d, H, hd, ffn, W, dtype, affine, add_residual
    ("bf16_ragged", 2, 200, 256, 2, 128, 320, 37, "bf16", True, 1),
    ("bf16_hd64", 1, 333, 192, 3, 64, 128, 100, "bf16", True, 1),
    ("bf16_w1", 1, 130, 128, 2, 64, 64, 1, "bf16", False, 1),
    ("bf16_w2", 2, 97, 128, 1, 128, 64, 2, "bf16", True, 1),
    ("bf16_w_ge_s_partial", 3, 129, 256, 2, 128, 256, 1000, "bf16", True, 0),
    ("bf16_one_token", 1, 1, 64, 1, 64, 64, 4, "bf16", True, 1),
    ("bf16_window_edges", 1, 515, 256, 2, 128, 128, 64, "bf16", True, 1),
    ("bf16_window_65", 1, 300, 256, 2, 128, 128, 65, "bf16", True, 1),
    ("bf16_multi_tile", 1, 700, 512, 4, 128, 768, 300, "bf16", True, 1),
    ("bf16_big_ragged_m", 4, 1000, 2048, 16, 128, 8192, 256, "bf16", False, 1),
    ("bf16_big_ntail", 3, 1100, 1024, 8, 128, 2112, 200, "bf16", True, 1),
    ("f32_ragged", 2, 77, 128, 2, 64, 192, 9, "f32", True, 1),
    ("f32_hd128", 1, 150, 256, 2, 128, 128, 64, "f32", True, 0),
    ("f32_w1", 1, 40, 64, 1, 64, 64, 1, "f32", True, 1),
]


def small_cfg(name, B, S, d, H, hd, ffn, W, dtype, affine, add_res):
    return BlockConfig(name, B=B, S=S, d=d, H=H, hd=hd, ffn=ffn, W=W, dtype=dtype, add_residual=add_res), affine


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_shapes_full(case):
    cfg, affine = small_cfg(*case)
    log(f"[case] {cfg}")
    inp = make_inputs(cfg, seed=3, affine=affine)
    y = run_block(cfg, upload(inp))
    err = rel_err(y, oracle_y(inp))
    log(f"[parity] {cfg.name}: rel err {err:.3e} (tol {TOL[cfg.dtype]})")
    assert err <= TOL[cfg.dtype]


@pytest.mark.parametrize("case", [SMALL[0], SMALL[1], SMALL[11], SMALL[12]], ids=lambda c: c[0])
def test_stage_parity(case):
    """LayerNorm output, Q|K|V, and [attention | GeLU] each against the oracle's."""
    cfg, affine = small_cfg(*case)
    log(f"[case] stages {cfg}")
    inp = make_inputs(cfg, seed=4, affine=affine)
    y, parts = run_block(cfg, upload(inp), want_parts=True)
    y_ref, ref = oracle.block_forward(inp.x, inp.gamma, inp.beta, inp.w_in, inp.w_out, cfg.H, cfg.hd, cfg.W,
                                      eps=cfg.ln_eps, add_residual=bool(cfg.add_residual), return_parts=True)
    tol = TOL[cfg.dtype]
    M = cfg.M
    for name in ("u", "qkv", "ag"):
        err = rel_err(parts[name], ref[name].reshape(M, -1))
        log(f"[parity] {cfg.name} stage {name}: {err:.3e}")
        assert err <= tol, name
    assert rel_err(y, y_ref) <= tol


def test_tiny_config_fp32():
    cfg = CONFIGS["tiny"]
    log(f"[case] {cfg}")
    inp = make_inputs(cfg, seed=0)
    y = run_block(cfg, upload(inp))
    err = rel_err(y, oracle_y(inp))
    log(f"[parity] tiny: all {y.size} outputs, rel err {err:.3e} (tol {TOL['f32']})")
    assert err <= TOL["f32"]


def test_small_config_full():
    cfg = CONFIGS["small"]
    log(f"[case] {cfg}")
    inp = make_inputs(cfg, seed=0)
    y = run_block(cfg, upload(inp))
    err = rel_err(y, oracle_y(inp))
    log(f"[parity] small: all {y.size} outputs, rel err {err:.3e} (tol {TOL['bf16']})")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("name", ["shard175b", "long", "fullcausal"])
def test_large_config_full(name):
    """Full-size workloads in the launch configuration the benchmark times: every output
    element against the oracle's full forward."""
    cfg = CONFIGS[name]
    log(f"[case] {cfg}")
    inp = make_inputs(cfg, seed=0)
    dev = upload(inp)
    y = run_block(cfg, dev)
    del dev
    torch.cuda.empty_cache()
    assert np.isfinite(y).all()
    err = rel_err(y, oracle_y_cached(inp, 0))
    log(f"[parity] {name}: all {y.size} outputs, rel err {err:.3e} (tol {TOL['bf16']})")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_largest_model_dim(dtype):
    """d = 32768, the largest the library accepts: the widest LayerNorm rows (16 or 32 vectors per
    thread, one row per workgroup), K = 32768 in the input GEMM and N = 32768 in the output GEMM;
    every output against the oracle, with a ragged token count.  The Q rows of W_in are scaled by
    2^-3 (exactly): with N(0, 0.02^2) weights the scores at this width would have a spread of ~13,
    where the bf16 storage of q and k alone moves the softmax by more than the tolerance."""
    cfg = BlockConfig("max_d_" + dtype, B=1, S=130, d=32768, H=2, hd=64, ffn=128, W=40, dtype=dtype)
    log(f"[case] {cfg}")
    inp = scale_q_rows(make_inputs(cfg, seed=21, affine=True), 3)
    y = run_block(cfg, upload(inp))
    err = rel_err(y, oracle_y(inp))
    log(f"[parity] {cfg.name}: rel err {err:.3e} (tol {TOL[dtype]})")
    assert err <= TOL[dtype]


def test_largest_token_count_sampled():
    """B*S = 2^24 tokens, the largest the library accepts (16 sequences of 2^20): element offsets
    into QKV pass 2^31, so every index on the path must be 64-bit.  Row blocks at the start and
    end of the first and last sequences against the oracle, computed one by one."""
    cfg = BlockConfig("max_tokens", B=16, S=1 << 20, d=64, H=1, hd=64, ffn=64, W=64, dtype="bf16")
    log(f"[case] {cfg}")
    inp = make_inputs(cfg, seed=22, affine=True)
    dev = upload(inp)
    h = tb.pblock_create(cfg)
    try:
        out = torch.empty_like(dev["x"])
        tb.pblock_forward(h, dev["x"], (dev["gamma"], dev["beta"], dev["w_in"], dev["w_out"]), cfg, out)
        torch.cuda.synchronize()
        S = cfg.S
        blocks = [(0, 0, 32), (0, S - 32, S), (15, 0, 32), (15, S // 2, S // 2 + 32), (15, S - 32, S)]
        got = np.concatenate([from_dev(out[b, i0:i1]) for b, i0, i1 in blocks])
    finally:
        tb.pblock_destroy(h)
        del dev
        torch.cuda.empty_cache()
    refs = oracle.block_forward_rows(inp.x, inp.gamma, inp.beta, inp.w_in, inp.w_out, cfg.H, cfg.hd, cfg.W, blocks,
                                     eps=cfg.ln_eps, add_residual=True)
    err = rel_err(got, np.concatenate(refs))
    log(f"[parity] max_tokens: {len(blocks)} row blocks, rel err {err:.3e}")
    assert err <= TOL["bf16"]


def test_branch_sum_on_gpu():
    """Branch sum (the full block without residual) == attention branch alone
    (FC1 rows zero, GeLU(0) = 0) + MLP branch alone (V rows zero).  All three
    are emitted without the residual so each is rounded to bf16 at the scale
    of the branches, not at the scale of x."""
    cfg = BlockConfig("branches", B=2, S=160, d=256, H=2, hd=128, ffn=384, W=40, dtype="bf16")
    inp = make_inputs(cfg, seed=5, affine=True)
    dev = upload(inp)
    A = cfg.A
    part = cfg.replace(add_residual=0)
    y_full = run_block(part, dev)
    y_res = run_block(cfg, dev)
    w_attn = dev["w_in"].clone()
    w_attn[3 * A:] = 0
    w_mlp = dev["w_in"].clone()
    w_mlp[2 * A:3 * A] = 0
    y_attn = run_block(part, {**dev, "w_in": w_attn})
    y_mlp = run_block(part, {**dev, "w_in": w_mlp})
    err = rel_err(y_attn + y_mlp, y_full)
    log(f"[parity] branch sum: {err:.3e}")
    assert err <= TOL["bf16"]
    # and the residual variant is the partial plus x, to bf16 rounding of the sum
    assert np.abs(y_res - (y_full + inp.x)).max() <= 2 ** -7 * np.abs(y_res).max()
    assert np.abs(y_attn).max() > 1e-3 and np.abs(y_mlp).max() > 1e-3


@pytest.mark.parametrize("R", [2, 4])
def test_tensor_parallel_partials_on_gpu(R):
    """R shards (heads and FFN columns split) emitting partials: sum + x == unsharded y."""
    cfg = BlockConfig("tp", B=1, S=256, d=512, H=4, hd=128, ffn=1024, W=64, dtype="bf16")
    inp = make_inputs(cfg, seed=6)
    A = cfg.A
    y_full = oracle_y(inp)
    hs, fs = cfg.H // R, cfg.ffn // R
    total = np.zeros_like(y_full)
    for r in range(R):
        rows = [inp.bits["w_in"][p * A + r * hs * cfg.hd: p * A + (r + 1) * hs * cfg.hd] for p in range(3)]
        rows.append(inp.bits["w_in"][3 * A + r * fs: 3 * A + (r + 1) * fs])
        wi = np.concatenate(rows, axis=0)
        wo = np.concatenate([inp.bits["w_out"][:, r * hs * cfg.hd:(r + 1) * hs * cfg.hd],
                             inp.bits["w_out"][:, A + r * fs:A + (r + 1) * fs]], axis=1)
        sc = cfg.replace(H=hs, ffn=fs, add_residual=0)
        dev = {"x": to_dev(inp.bits["x"], "bf16"), "gamma": to_dev(inp.bits["gamma"], "bf16"),
               "beta": to_dev(inp.bits["beta"], "bf16"), "w_in": to_dev(wi, "bf16"), "w_out": to_dev(wo, "bf16")}
        total += run_block(sc, dev)
    err = rel_err(total + inp.x, y_full)
    log(f"[parity] tp R={R}: {err:.3e}")
    assert err <= TOL["bf16"]


def test_window_locality_bitwise():
    """Changing tokens outside query i's window leaves y_i bit-identical; other
    batches are untouched."""
    cfg = BlockConfig("loc", B=2, S=300, d=256, H=2, hd=128, ffn=256, W=50, dtype="bf16")
    inp = make_inputs(cfg, seed=7)
    dev = upload(inp)
    y0 = run_block(cfg, dev)
    i = 200
    x2 = dev["x"].clone()
    x2[0, i - cfg.W] = torch.randn(cfg.d, device="cuda").to(torch.bfloat16)
    x2[0, i + 1] = torch.randn(cfg.d, device="cuda").to(torch.bfloat16)
    y1 = run_block(cfg, {**dev, "x": x2})
    assert np.array_equal(y1[0, i], y0[0, i])
    assert np.array_equal(y1[1], y0[1])
    assert np.abs(y1[0, i + 1] - y0[0, i + 1]).max() > 0
    x3 = dev["x"].clone()
    x3[0, i - cfg.W + 1] = torch.randn(cfg.d, device="cuda").to(torch.bfloat16)
    y2 = run_block(cfg, {**dev, "x": x3})
    assert np.abs(y2[0, i] - y0[0, i]).max() > 0


def test_w1_attention_is_value_copy():
    """W = 1: the attention output equals the value projection bit for bit."""
    cfg = BlockConfig("w1", B=2, S=100, d=128, H=2, hd=128, ffn=128, W=1, dtype="bf16")
    inp = make_inputs(cfg, seed=8, affine=True)
    _, parts = run_block(cfg, upload(inp), want_parts=True)
    A = cfg.A
    assert np.array_equal(parts["ag"][:, :A], parts["qkv"][:, 2 * A:3 * A])


def test_window_covering_sequence_is_causal_bitwise():
    """W = S and W = 3S run the same band path and give identical outputs."""
    cfg = BlockConfig("ws", B=2, S=320, d=256, H=2, hd=128, ffn=256, W=320, dtype="bf16")
    inp = make_inputs(cfg, seed=9)
    dev = upload(inp)
    ya = run_block(cfg, dev)
    yb = run_block(cfg.replace(W=3 * cfg.S), dev)
    assert np.array_equal(ya, yb)
    assert rel_err(ya, oracle_y(inp)) <= TOL["bf16"]


ATTN_CASES = [(1, 1), (2, 1), (64, 64), (65, 64), (127, 63), (128, 129), (300, 1), (300, 2), (300, 63), (300, 64),
              (300, 65), (513, 128), (513, 300), (700, 700), (1000, 1)]


@pytest.mark.parametrize("hd", [64, 128])
def test_attention_entry_point(hd):
    """pblock_swa_attention against the oracle's band attention over many (S, W)."""
    rng = np.random.Generator(np.random.PCG64(10))
    H, B = 2, 2
    A = H * hd
    for S, W in ATTN_CASES:
        qkv = (rng.standard_normal((B * S, 3 * A), dtype=np.float32) * 1.5).astype(np.float32)
        qkv_t = torch.from_numpy(qkv).cuda().to(torch.bfloat16)
        o = torch.zeros((B * S, A), dtype=torch.bfloat16, device="cuda")
        tb.pblock_swa_attention(qkv_t, 3 * A, o, A, B, S, H, hd, W, "bf16")
        torch.cuda.synchronize()
        qv = from_dev(qkv_t).reshape(B, S, 3, H, hd)
        ref = np.stack([oracle.swa_attention(qv[b, :, 0], qv[b, :, 1], qv[b, :, 2], W) for b in range(B)])
        err = rel_err(from_dev(o).reshape(B, S, H, hd), ref)
        log(f"[parity] attention hd={hd} S={S} W={W}: {err:.3e}")
        assert err <= TOL["bf16"], (S, W)


@pytest.mark.parametrize("hd", [64, 128])
@pytest.mark.parametrize("H", [2, 512], ids=["few_heads", "many_heads"])
def test_attention_head_counts(H, hd):
    """Few and many heads (a launch under one workgroup per CU, and one of several waves of
    them) against the oracle; ragged S, a window that is not a multiple of the key tile."""
    rng = np.random.Generator(np.random.PCG64(12))
    B, S, W = 1, 300, 65
    A = H * hd
    qkv = (rng.standard_normal((B * S, 3 * A), dtype=np.float32) * 1.5).astype(np.float32)
    qkv_t = torch.from_numpy(qkv).cuda().to(torch.bfloat16)
    o = torch.zeros((B * S, A), dtype=torch.bfloat16, device="cuda")
    tb.pblock_swa_attention(qkv_t, 3 * A, o, A, B, S, H, hd, W, "bf16")
    torch.cuda.synchronize()
    qv = from_dev(qkv_t).reshape(S, 3, H, hd)
    ref = oracle.swa_attention(qv[:, 0], qv[:, 1], qv[:, 2], W)
    err = rel_err(from_dev(o).reshape(S, H, hd), ref)
    log(f"[parity] attention H={H} hd={hd}: {err:.3e}")
    assert err <= TOL["bf16"]


def test_attention_entry_fp32():
    rng = np.random.Generator(np.random.PCG64(11))
    B, S, H, hd, W = 1, 200, 2, 64, 33
    A = H * hd
    qkv = rng.standard_normal((B * S, 3 * A)).astype(np.float32)
    qkv_t = torch.from_numpy(qkv).cuda()
    o = torch.zeros((B * S, A), dtype=torch.float32, device="cuda")
    tb.pblock_swa_attention(qkv_t, 3 * A, o, A, B, S, H, hd, W, "f32")
    torch.cuda.synchronize()
    qv = qkv.astype(np.float64).reshape(B, S, 3, H, hd)
    ref = oracle.swa_attention(qv[0, :, 0], qv[0, :, 1], qv[0, :, 2], W)
    assert rel_err(from_dev(o).reshape(S, H, hd), ref) <= TOL["f32"]


def test_deterministic_and_reusable_handle():
    """Same inputs -> bit-identical outputs; a handle serves a smaller B*S."""
    cfg = BlockConfig("det", B=4, S=128, d=256, H=2, hd=128, ffn=256, W=32, dtype="bf16")
    inp = make_inputs(cfg, seed=12)
    dev = upload(inp)
    h = tb.pblock_create(cfg)
    try:
        y1 = run_block(cfg, dev, handle=h)
        y2 = run_block(cfg, dev, handle=h)
        assert np.array_equal(y1, y2)
        small = cfg.replace(B=2)
        dev2 = {**dev, "x": dev["x"][:2].contiguous()}
        y3 = run_block(small, dev2, handle=h)
        assert np.array_equal(y3, y1[:2])
        with pytest.raises(tb.PblockError) as ei:
            run_block(cfg.replace(B=5), {**dev, "x": torch.cat([dev["x"], dev["x"][:1]])}, handle=h)
        assert ei.value.code == tb._abi.PBLOCK_ERR_CFG_MISMATCH
    finally:
        tb.pblock_destroy(h)


def test_split_k_tails_on_a_reused_handle():
    """The output GEMM runs entirely as split-K tail tiles at this shape (8 x 4 = 32 tiles on 256
    compute units: 8 k-chunks each, no whole wave first), through the handle's partial-tile
    scratch: 20 forwards on one handle, every one bit-identical to the first, the first within
    tolerance of the oracle."""
    cfg = BlockConfig("tails", B=2, S=1024, d=1024, H=8, hd=128, ffn=2304, W=128, dtype="bf16")
    inp = make_inputs(cfg, seed=15, affine=True)
    dev = upload(inp)
    h = tb.pblock_create(cfg)
    try:
        out = torch.empty_like(dev["x"])
        w = (dev["gamma"], dev["beta"], dev["w_in"], dev["w_out"])
        tb.pblock_forward(h, dev["x"], w, cfg, out)
        first = out.clone()
        for _ in range(19):
            tb.pblock_forward(h, dev["x"], w, cfg, out)
            assert bool(torch.equal(out, first))
        torch.cuda.synchronize()
    finally:
        tb.pblock_destroy(h)
    ref = oracle.block_forward(inp.x, inp.gamma, inp.beta, inp.w_in, inp.w_out, cfg.H, cfg.hd, cfg.W,
                               eps=cfg.ln_eps, add_residual=True)
    err = rel_err(from_dev(first).reshape(cfg.B, cfg.S, cfg.d), ref)
    log(f"[parity] split-K tails, reused handle: {err:.3e}")
    assert err <= TOL["bf16"]


# Shapes whose GEMMs would end in a partial wave of 256 x 256 tiles, on 256 compute units:
#   "in_split4": GEMM-in 8 x 39 = 312 tiles = one wave + 56 tiles in 4 k-chunks; GEMM-out 8
#     tiles in 32 k-chunks.
#   "in_split3_out_wide": GEMM-in 16 x 21 = 336 tiles = one wave + 80 tiles in 3 k-chunks (the
#     175B-shard GEMM-in's split); GEMM-out 16 x 24 = 384 tiles of 256 x 256, run as one wave of
#     16 x 16 tiles of 256 x 384 (k = 4288, an odd number of 64-deep slabs).
#   "in_tail_holds_qkv": GEMM-in 8 x 37 = 296 tiles = one wave + 40 tiles in 4 k-chunks, the
#     first of them Q, K, V columns (3A = 9216 > 8192): their reduce must run before attention
#     (in the first two cases the tail is FC1 columns only and its reduce runs inside the
#     attention launch).
#   "out_wide_odd_k": GEMM-out 4096 x 6144 with k = 320, an odd number of 64-deep slabs, in
#     256 x 384 tiles.
#   "out_192": GEMM-out 16 x 36 = 576 tiles of 256 x 256; 256 x 384 tiles would be 384 (a wave
#     and a half), 256 x 192 tiles are 768 = three whole waves: those.
#   "out_half_height": GEMM-out 16 x 23 = 368 tiles = one wave + 112, which neither 384- nor
#     192-wide tiles turn into whole waves: the 112 run as 224 tiles of 128 x 256.
#   "out_wide_odd_k_partial", "out_192_partial": the same GEMM-out shapes as "out_wide_odd_k" and
#     "out_192" without the residual (the tensor-parallel partial), so the output GEMM takes its
#     direct (lane-swap, no LDS) epilogue form in 384- and 192-wide tiles.  Without the residual
#     the outputs are smaller: bf16 storage of the intermediates and of y alone puts y 8.79e-3
#     and 6.28e-3 of its max from the exact oracle there (computed on the CPU as in
#     test_precision_floor.py), and the GPU's errors sit at those floors.
# A ninth field, when present, is add_residual (default 1).
SPLIT_TAILS = [
    ("in_split4", 1, 2048, 256, 2, 128, 9216, 128),
    ("in_split3_out_wide", 2, 2048, 6144, 4, 128, 3776, 256),
    ("in_tail_holds_qkv", 1, 2048, 256, 24, 128, 256, 128),
    ("out_wide_odd_k", 2, 2048, 6144, 1, 128, 192, 64),
    ("out_192", 2, 2048, 9216, 2, 128, 256, 128),
    ("out_half_height", 2, 2048, 5888, 2, 128, 256, 128),
    ("out_wide_odd_k_partial", 2, 2048, 6144, 1, 128, 192, 64, 0),
    ("out_192_partial", 2, 2048, 9216, 2, 128, 256, 128, 0),
]


@pytest.mark.parametrize("case", SPLIT_TAILS, ids=[c[0] for c in SPLIT_TAILS])
def test_split_k_tails_after_whole_waves(case):
    """Every output of a forward whose GEMMs would leave a partial wave of 256 x 256 tiles (a
    split-K tail summed in chunk order by the reduce kernel, 384- or 192-wide tiles in whole
    waves, or half-height tiles) against the oracle, and three forwards on one handle
    bit-identical."""
    name, B, S, d, H, hd, ffn, W = case[:8]
    add_residual = case[8] if len(case) > 8 else 1
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the tile counts above assume 256 compute units")
    cfg = BlockConfig(name, B=B, S=S, d=d, H=H, hd=hd, ffn=ffn, W=W, dtype="bf16", add_residual=add_residual)
    inp = make_inputs(cfg, seed=31, affine=True)
    dev = upload(inp)
    h = tb.pblock_create(cfg)
    try:
        y = run_block(cfg, dev, handle=h)
        for _ in range(2):
            assert np.array_equal(run_block(cfg, dev, handle=h), y)
    finally:
        tb.pblock_destroy(h)
    err = rel_err(y.reshape(B, S, d), oracle_y(inp))
    log(f"[parity] split-K tail {name}: {err:.3e}")
    assert err <= TOL["bf16"]


def test_errors_leave_output_untouched():
    """Rejected calls (through the raw C ABI, past the binding's own checks)
    enqueue nothing: the output keeps its sentinel."""
    import ctypes

    cfg = BlockConfig("err", B=1, S=64, d=128, H=1, hd=64, ffn=64, W=8, dtype="bf16")
    inp = make_inputs(cfg, seed=13)
    dev = upload(inp)
    lib = tb._abi.lib()
    h = tb.pblock_create(cfg)
    try:
        out = torch.full_like(dev["x"], 7.0)
        w = tb.PblockWeights(dev["gamma"].data_ptr(), dev["beta"].data_ptr(), dev["w_in"].data_ptr(),
                             dev["w_out"].data_ptr())
        stream = torch.cuda.current_stream().cuda_stream

        def call(c, x_ptr, out_ptr, weights=w):
            return lib.pblock_forward(ctypes.c_void_p(h), x_ptr, ctypes.byref(weights), ctypes.byref(tb.as_cfg(c)),
                                      out_ptr, stream)

        x_ptr, o_ptr = dev["x"].data_ptr(), out.data_ptr()
        assert call(cfg.replace(d=192), x_ptr, o_ptr) == tb._abi.PBLOCK_ERR_CFG_MISMATCH
        assert call(cfg.replace(S=65), x_ptr, o_ptr) == tb._abi.PBLOCK_ERR_CFG_MISMATCH
        assert call(cfg.replace(hd=96), x_ptr, o_ptr) == tb._abi.PBLOCK_ERR_SHAPE
        assert call(cfg, x_ptr, x_ptr) == tb._abi.PBLOCK_ERR_ALIAS
        assert call(cfg, x_ptr + 2, o_ptr) == tb._abi.PBLOCK_ERR_ALIGN
        assert call(cfg, 0, o_ptr) == tb._abi.PBLOCK_ERR_NULL
        bad_w = tb.PblockWeights(w.ln_gamma, w.ln_beta, 0, w.w_out)
        assert call(cfg, x_ptr, o_ptr, bad_w) == tb._abi.PBLOCK_ERR_NULL
        torch.cuda.synchronize()
        assert bool((out == 7.0).all())
    finally:
        tb.pblock_destroy(h)


def test_kernel_timing_api():
    cfg = BlockConfig("timing", B=1, S=512, d=512, H=4, hd=128, ffn=1024, W=128, dtype="bf16")
    inp = make_inputs(cfg, seed=14)
    dev = upload(inp)
    h = tb.pblock_create(cfg)
    try:
        tb.pblock_set_timing(h, True)
        for _ in range(3):
            run_block(cfg, dev, handle=h)
        ms, n = tb.pblock_kernel_times(h)
        assert n == 3
        assert all(v > 0 for v in ms.values()), ms
    finally:
        tb.pblock_destroy(h)
