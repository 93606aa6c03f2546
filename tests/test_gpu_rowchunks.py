"""GPU checks of the row-chunk publication (pblock_forward_rowchunks) and its consumer
(pblock_pack_chunks): the output against the oracle and the whole forward, the flags, and a
consumer on another stream that copies each chunk as soon as it is published, while the output
GEMM still runs -- every piece it copied must hold the final rows."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, from_dev, log, oracle_y_cached, rel_err, run_block, upload
from workload import CONFIGS, BlockConfig, make_inputs

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import transformer_block_fwd_amd as tb  # noqa: E402

NO_STAMP = np.uint64(0xFFFFFFFFFFFFFFFF)

CASES = [
    # name, B, S, d, H, hd, ffn, W, n_chunks
    ("rc_one_seq_4", 1, 1024, 512, 4, 128, 768, 200, 4),
    ("rc_ragged_5", 2, 333, 256, 2, 128, 320, 37, 5),             # chunk and sequence ends inside tiles
    ("rc_aligned_seqs_8", 3, 512, 256, 2, 64, 256, 100, 8),       # S % 256 == 0: position-major tile order
    ("rc_one_chunk", 1, 300, 256, 2, 128, 128, 65, 1),
    ("rc_64_chunks", 1, 700, 256, 2, 64, 256, 50, 64),
    ("rc_short_seqs", 8, 40, 128, 1, 64, 64, 9, 40),              # many sequences in one tile
    ("rc_big_ntail_6", 3, 1100, 1024, 8, 128, 2112, 200, 6),      # whole waves plus a half-height tail
]


def weights(dev):
    return (dev["gamma"], dev["beta"], dev["w_in"], dev["w_out"])


def pieces(y, B, S, n):
    """Piece k of the send layout: chunk k's rows of y [B, S, d], sequence by sequence."""
    out = []
    for k in range(n):
        p0, p1 = k * S // n, (k + 1) * S // n
        out.append(y[:, p0:p1].reshape(-1, y.shape[-1]))
    return np.concatenate(out)


def run_rowchunks(cfg, dev, n, epoch, h=None, flags=None, stream=None):
    own = h is None
    h = tb.pblock_create(cfg) if own else h
    try:
        if flags is None:
            flags = torch.zeros(n, dtype=torch.int32, device="cuda")
        out = torch.empty_like(dev["x"])
        tb.pblock_forward_rowchunks(h, dev["x"], weights(dev), cfg, out, n, flags, epoch, stream)
        torch.cuda.synchronize()
        return from_dev(out).reshape(cfg.B, cfg.S, cfg.d), flags.cpu().numpy().astype(np.int64)
    finally:
        if own:
            tb.pblock_destroy(h)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_rowchunks_matches_oracle_and_forward(case):
    name, B, S, d, H, hd, ffn, W, n = case
    cfg = BlockConfig(name, B=B, S=S, d=d, H=H, hd=hd, ffn=ffn, W=W, dtype="bf16")
    log(f"[case] rowchunks x{n} {cfg}")
    inp = make_inputs(cfg, seed=17, affine=True)
    dev = upload(inp)
    h = tb.pblock_create(cfg)
    try:
        y, flags = run_rowchunks(cfg, dev, n, 7, h=h)
        assert (flags == 7).all(), flags
        # a second call on the same handle (counters reset by each chunk's last tile), new epoch
        y2, flags2 = run_rowchunks(cfg, dev, n, 8, h=h)
        assert (flags2 == 8).all(), flags2
        assert np.array_equal(y, y2)
    finally:
        tb.pblock_destroy(h)
    ref = oracle.block_forward(inp.x, inp.gamma, inp.beta, inp.w_in, inp.w_out, cfg.H, cfg.hd, cfg.W,
                               eps=cfg.ln_eps, add_residual=True)
    err = rel_err(y, ref)
    log(f"[parity] {name}: rel err {err:.3e}")
    assert err <= TOL["bf16"]
    assert rel_err(y, run_block(cfg, dev)) <= TOL["bf16"]


@pytest.mark.parametrize("n_chunks", [4, 8])
def test_rowchunks_shard175b_full(n_chunks):
    """The 175B shard workload (partial output, no residual): every output against the oracle."""
    cfg = CONFIGS["shard175b"]
    log(f"[case] shard175b rowchunks x{n_chunks}")
    inp = make_inputs(cfg, seed=0)
    dev = upload(inp)
    y, flags = run_rowchunks(cfg, dev, n_chunks, 3)
    del dev
    torch.cuda.empty_cache()
    assert (flags == 3).all()
    err = rel_err(y, oracle_y_cached(inp, 0))
    log(f"[parity] shard175b rowchunks x{n_chunks}: all {y.size} outputs, rel err {err:.3e} (tol {TOL['bf16']})")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("n_chunks", [4, 8])
def test_pack_consumes_chunks_while_the_gemm_runs(n_chunks):
    """The consumer waits on another stream, enqueued first; the producer publishes chunk by
    chunk.  Each piece the consumer copied at its chunk's publication equals the final rows (a
    flag set before its rows were complete would leave stale or partial rows in the piece: send
    starts as NaN) and the oracle's; the first chunks are published well before the last (their
    rows are done after the first wave of output tiles, the last chunk's after the remainder)."""
    cfg = CONFIGS["shard175b"]
    log(f"[case] shard175b pack x{n_chunks}")
    inp = make_inputs(cfg, seed=0)
    dev = upload(inp)
    h = tb.pblock_create(cfg)
    try:
        out = torch.empty_like(dev["x"])
        send = torch.full_like(dev["x"], float("nan"))
        flags = torch.zeros(n_chunks, dtype=torch.int32, device="cuda")
        stamps = torch.zeros(n_chunks, dtype=torch.int64, device="cuda")
        from transformer_block_fwd_amd.streams import cu_masked_stream, destroy_stream

        prod = torch.cuda.Stream()
        # the consumer on a hardware queue of its own (two pool streams may share one and then run
        # one after the other), on the device's last 32 compute units
        n_cus = torch.cuda.get_device_properties(0).multi_processor_count
        cons_handle = cu_masked_stream(n_cus - 32, 32, n_cus)
        torch.cuda.synchronize()
        for epoch in (1, 2):  # twice: the second consumer must not take the first call's flags
            out.fill_(float("nan"))
            send.fill_(float("nan"))
            torch.cuda.synchronize()
            tb.pblock_pack_chunks(out, cfg, n_chunks, flags, epoch, send, stamps, cons_handle)
            with torch.cuda.stream(prod):
                tb.pblock_forward_rowchunks(h, dev["x"], weights(dev), cfg, out, n_chunks, flags, epoch, prod)
            torch.cuda.synchronize()
            st = stamps.cpu().numpy().astype(np.uint64)
            assert (st != NO_STAMP).all(), st
            y = from_dev(out).reshape(cfg.B, cfg.S, cfg.d)
            got = from_dev(send)
            assert np.array_equal(got.reshape(-1, cfg.d), pieces(y, cfg.B, cfg.S, n_chunks))
            rel = (st.astype(np.int64) - int(st.min())) * 10  # ns (100 MHz clock)
            log(f"[pack] epoch {epoch}: chunk publication times after the first (us): "
                f"{[round(v / 1000, 1) for v in rel]}")
            first, last = rel[: n_chunks // 4 or 1].max(), rel[-1]
            assert last - first > 20_000, rel  # the last chunk at least 20 us after the first ones
    finally:
        torch.cuda.synchronize()
        tb.pblock_destroy(h)
        destroy_stream(cons_handle)
    del dev
    torch.cuda.empty_cache()
    err = rel_err(got.reshape(-1, cfg.d), pieces(oracle_y_cached(inp, 0), cfg.B, cfg.S, n_chunks))
    log(f"[parity] shard175b packed pieces x{n_chunks}: rel err {err:.3e}")
    assert err <= TOL["bf16"]


def test_pack_wait_is_bounded():
    """Flags that never reach the epoch: every wait ends after its bound, the stamps say so and
    send is not written."""
    cfg = BlockConfig("pack_timeout", B=1, S=256, d=128, H=1, hd=64, ffn=64, W=16, dtype="bf16")
    n = 4
    out = torch.zeros((cfg.B, cfg.S, cfg.d), dtype=torch.bfloat16, device="cuda")
    send = torch.full_like(out, 5.0)
    flags = torch.zeros(n, dtype=torch.int32, device="cuda")
    stamps = torch.zeros(n, dtype=torch.int64, device="cuda")
    tb.pblock_pack_chunks(out, cfg, n, flags, 9, send, stamps)
    torch.cuda.synchronize()
    assert (stamps.cpu().numpy().astype(np.uint64) == NO_STAMP).all()
    assert bool((send == 5.0).all())


def test_rowchunks_rejections():
    import ctypes

    cfg = BlockConfig("rc_rej", B=1, S=64, d=128, H=1, hd=64, ffn=64, W=8, dtype="bf16")
    inp = make_inputs(cfg, seed=2)
    dev = upload(inp)
    lib = tb._abi.lib()
    h = tb.pblock_create(cfg)
    try:
        out = torch.full_like(dev["x"], 4.0)
        flags = torch.zeros(65, dtype=torch.int32, device="cuda")
        w = tb.PblockWeights(*[t.data_ptr() for t in weights(dev)])
        stream = torch.cuda.current_stream().cuda_stream

        def call(c, n, fl, epoch, o=out.data_ptr()):
            return lib.pblock_forward_rowchunks(ctypes.c_void_p(h), dev["x"].data_ptr(), ctypes.byref(w),
                                                ctypes.byref(tb.as_cfg(c)), o, n, fl, epoch, stream)

        E = tb._abi
        assert call(cfg, 0, flags.data_ptr(), 1) == E.PBLOCK_ERR_ARG
        assert call(cfg, 65, flags.data_ptr(), 1) == E.PBLOCK_ERR_ARG
        assert call(cfg.replace(S=32, B=2), 33, flags.data_ptr(), 1) == E.PBLOCK_ERR_ARG  # n > S
        assert call(cfg, 4, 0, 1) == E.PBLOCK_ERR_NULL
        assert call(cfg, 4, flags.data_ptr() + 2, 1) == E.PBLOCK_ERR_ALIGN
        assert call(cfg, 4, flags.data_ptr(), 0) == E.PBLOCK_ERR_ARG
        assert call(cfg, 4, out.data_ptr(), 1) == E.PBLOCK_ERR_ALIAS
        torch.cuda.synchronize()
        assert bool((out == 4.0).all())
        assert bool((flags == 0).all())
    finally:
        tb.pblock_destroy(h)
    f32 = cfg.replace(dtype="f32", name="rc_f32")
    h = tb.pblock_create(f32)
    try:
        x = torch.zeros((1, 64, 128), device="cuda")
        g = torch.ones(128, device="cuda")
        wi = torch.zeros((f32.n_in, 128), device="cuda")
        wo = torch.zeros((128, f32.k_out), device="cuda")
        with pytest.raises(tb.PblockError) as ei:
            tb.pblock_forward_rowchunks(h, x, (g, g, wi, wo), f32, torch.empty_like(x), 4,
                                        torch.zeros(4, dtype=torch.int32, device="cuda"), 1)
        assert ei.value.code == tb._abi.PBLOCK_ERR_DTYPE
    finally:
        tb.pblock_destroy(h)
