"""GPU checks of the position-chunked forward (the compute side of the
tensor/sequence-parallel overlap): parity with the oracle for several chunk
counts, agreement with the unchunked forward, per-chunk completion events in
order, and per-chunk input waits that gate reads of x."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, from_dev, log, oracle_y_cached, rel_err, run_block, upload
from workload import CONFIGS, BlockConfig, make_inputs

pytestmark = pytest.mark.gpu

CHUNK_CASES = [
    # name, B, S, d, H, hd, ffn, W, dtype, n_chunks
    ("chunk_bf16_8", 1, 1024, 512, 4, 128, 768, 200, "bf16", 8),
    ("chunk_bf16_ragged", 2, 333, 256, 2, 128, 320, 37, "bf16", 5),
    ("chunk_bf16_window_spans_chunks", 1, 700, 256, 2, 64, 256, 300, "bf16", 7),
    ("chunk_bf16_one", 1, 300, 256, 2, 128, 128, 65, "bf16", 1),
    ("chunk_bf16_per_position", 1, 40, 128, 1, 64, 64, 9, "bf16", 40),
    ("chunk_f32", 2, 150, 128, 2, 64, 192, 20, "f32", 4),
]


def run_chunked(cfg, dev, n_chunks, ready=None, done=None, stream=None):
    import torch

    import transformer_block_fwd_amd as tb

    h = tb.pblock_create(cfg)
    try:
        out = torch.empty_like(dev["x"])
        tb.pblock_forward_chunked(h, dev["x"], (dev["gamma"], dev["beta"], dev["w_in"], dev["w_out"]), cfg, out,
                                  n_chunks, ready, done, stream)
        torch.cuda.synchronize()
        return from_dev(out).reshape(cfg.B, cfg.S, cfg.d)
    finally:
        tb.pblock_destroy(h)


@pytest.mark.parametrize("per_chunk_input", [False, True], ids=["whole_input", "per_chunk_input"])
@pytest.mark.parametrize("case", CHUNK_CASES, ids=[c[0] for c in CHUNK_CASES])
def test_chunked_matches_oracle(case, per_chunk_input):
    """Without input events only the output GEMM is cut into chunks; an input-event array (here
    all NULL) makes every step run chunk by chunk.  Both match the oracle and the whole forward."""
    name, B, S, d, H, hd, ffn, W, dtype, n = case
    cfg = BlockConfig(name, B=B, S=S, d=d, H=H, hd=hd, ffn=ffn, W=W, dtype=dtype)
    log(f"[case] chunked x{n} per_chunk_input={per_chunk_input} {cfg}")
    inp = make_inputs(cfg, seed=12, affine=True)
    dev = upload(inp)
    y = run_chunked(cfg, dev, n, ready=[None] * n if per_chunk_input else None)
    ref = oracle.block_forward(inp.x, inp.gamma, inp.beta, inp.w_in, inp.w_out, cfg.H, cfg.hd, cfg.W,
                               eps=cfg.ln_eps, add_residual=True)
    err = rel_err(y, ref)
    log(f"[parity] {name}: rel err {err:.3e}")
    assert err <= TOL[dtype]
    y_whole = run_block(cfg, dev)
    err2 = rel_err(y, y_whole)
    log(f"[parity] {name}: chunked vs whole {err2:.3e}")
    assert err2 <= TOL[dtype]


@pytest.mark.parametrize("per_chunk_input", [False, True], ids=["whole_input", "per_chunk_input"])
@pytest.mark.parametrize("n_chunks", [4, 8])
def test_chunked_shard175b_full(n_chunks, per_chunk_input):
    """The 175B shard workload in the chunked launch configurations the benchmark times (4 and 8
    chunks, with and without per-chunk input): every output against the oracle, chunk boundaries
    (where a chunk's windows reach back into the one before) included."""
    import torch

    cfg = CONFIGS["shard175b"]
    log(f"[case] shard175b chunked x{n_chunks} per_chunk_input={per_chunk_input}")
    inp = make_inputs(cfg, seed=0)
    dev = upload(inp)
    y = run_chunked(cfg, dev, n_chunks, ready=[None] * n_chunks if per_chunk_input else None)
    del dev
    torch.cuda.empty_cache()
    assert np.isfinite(y).all()
    err = rel_err(y, oracle_y_cached(inp, 0))
    log(f"[parity] shard175b chunked x{n_chunks} per_chunk_input={per_chunk_input}: all {y.size} outputs, "
        f"rel err {err:.3e} (tol {TOL['bf16']})")
    assert err <= TOL["bf16"]


def test_chunked_ignores_stale_workspace():
    """A per-chunk forward on a handle whose workspace holds NaN from an earlier bad batch
    (a forward on an all-NaN x): each chunk's attention reads only key rows its own or
    earlier chunks projected, so the output is finite and equals the whole forward's to
    tolerance.  Chunk boundaries at multiples of 100 positions fall inside 64-key tiles."""
    import torch

    import transformer_block_fwd_amd as tb

    cfg = BlockConfig("stale", B=2, S=700, d=256, H=2, hd=128, ffn=256, W=100, dtype="bf16")
    n = 7
    inp = make_inputs(cfg, seed=16, affine=True)
    dev = upload(inp)
    y_whole = run_block(cfg, dev)
    w = (dev["gamma"], dev["beta"], dev["w_in"], dev["w_out"])
    h = tb.pblock_create(cfg)
    try:
        out = torch.empty_like(dev["x"])
        tb.pblock_forward(h, torch.full_like(dev["x"], float("nan")), w, cfg, out)
        torch.cuda.synchronize()
        assert bool(torch.isnan(out.float()).all())  # the workspace now holds NaN everywhere
        tb.pblock_forward_chunked(h, dev["x"], w, cfg, out, n, [None] * n, None)
        torch.cuda.synchronize()
        y = from_dev(out).reshape(cfg.B, cfg.S, cfg.d)
    finally:
        tb.pblock_destroy(h)
    assert np.isfinite(y).all()
    err = rel_err(y, y_whole)
    log(f"[parity] chunked over a NaN workspace vs whole: {err:.3e}")
    assert err <= TOL["bf16"]
    ref = oracle.block_forward(inp.x, inp.gamma, inp.beta, inp.w_in, inp.w_out, cfg.H, cfg.hd, cfg.W,
                               eps=cfg.ln_eps, add_residual=True)
    assert rel_err(y, ref) <= TOL["bf16"]


def test_done_events_in_order():
    """Every chunk's completion event fires, in chunk order."""
    import torch

    cfg = BlockConfig("events", B=1, S=2048, d=1024, H=8, hd=128, ffn=2048, W=256, dtype="bf16")
    inp = make_inputs(cfg, seed=13)
    dev = upload(inp)
    n = 8
    start = torch.cuda.Event(enable_timing=True)
    done = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    start.record()
    y = run_chunked(cfg, dev, n, done=done)
    assert np.isfinite(y).all()
    t = [start.elapsed_time(e) for e in done]
    log(f"[events] chunk completion ms: {[round(v, 3) for v in t]}")
    assert all(b >= a for a, b in zip(t, t[1:]))
    assert t[0] > 0


def test_ready_events_gate_reads_of_x():
    """x arrives chunk by chunk on a second stream (copies from a staging buffer, each
    followed by that chunk's ready event); the chunked forward waits per chunk, so the
    result equals the forward on the staged x, not on the zeros x held before."""
    import torch

    cfg = BlockConfig("ready", B=1, S=1536, d=512, H=4, hd=128, ffn=1024, W=128, dtype="bf16")
    n = 6
    inp = make_inputs(cfg, seed=14, affine=True)
    dev = upload(inp)
    staged = dev["x"].clone()
    dev["x"].zero_()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    ready = [torch.cuda.Event() for _ in range(n)]
    rows = cfg.S // n
    x2 = dev["x"].view(cfg.S, cfg.d)
    s2 = staged.view(cfg.S, cfg.d)
    with torch.cuda.stream(side):
        torch.cuda._sleep(2_000_000)  # the copies start well after the forward is enqueued
        for k in range(n):
            x2[k * rows:(k + 1) * rows].copy_(s2[k * rows:(k + 1) * rows])
            ready[k].record(side)
    y = run_chunked(cfg, dev, n, ready=ready, stream=torch.cuda.current_stream())
    ref = oracle.block_forward(inp.x, inp.gamma, inp.beta, inp.w_in, inp.w_out, cfg.H, cfg.hd, cfg.W,
                               eps=cfg.ln_eps, add_residual=True)
    err = rel_err(y, ref)
    log(f"[parity] ready-gated chunks: rel err {err:.3e}")
    assert err <= TOL["bf16"]


def test_chunk_count_rejected():
    import torch

    import transformer_block_fwd_amd as tb

    cfg = BlockConfig("rej", B=1, S=16, d=128, H=1, hd=64, ffn=64, W=4, dtype="bf16")
    inp = make_inputs(cfg, seed=1)
    dev = upload(inp)
    h = tb.pblock_create(cfg)
    try:
        out = torch.full_like(dev["x"], 5.0)
        for bad in (0, 17):
            with pytest.raises(tb.PblockError):
                tb.pblock_forward_chunked(h, dev["x"], (dev["gamma"], dev["beta"], dev["w_in"], dev["w_out"]), cfg,
                                          out, bad)
        torch.cuda.synchronize()
        assert bool((out.float() == 5.0).all())
    finally:
        tb.pblock_destroy(h)
