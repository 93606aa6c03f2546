"""GPU: the block captured in a HIP graph (torch.cuda.CUDAGraph on ROCm) replays to the eager
result, bit for bit, replay after replay.

pblock_forward only enqueues kernels on the caller's stream (no allocation, no host
synchronisation, no memset), so a caller can capture it once and replay it; the training pair
adds a device-to-device copy and fill kernels, which capture too.  Every kernel here is
deterministic (fixed summation orders, no atomics), so a replay must equal the eager call
exactly.  Eager calls on the same handle run between the replays, and every replay is checked,
not only the first.
"""
import pytest

from gpu_helpers import log, to_dev, upload
from workload import BlockConfig, make_dy, make_inputs

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import transformer_block_fwd_amd as tb  # noqa: E402

REPLAYS = 4

FORWARD_CASES = [
    # few tiles: every GEMM tile goes through the split-K tail and its reduce launch
    BlockConfig("graph_bf16", B=2, S=300, d=512, H=4, hd=128, ffn=768, W=100, dtype="bf16"),
    BlockConfig("graph_bf16_partial", B=1, S=200, d=256, H=2, hd=64, ffn=320, W=37, dtype="bf16",
                add_residual=0),
    BlockConfig("graph_f32", B=1, S=150, d=256, H=2, hd=64, ffn=256, W=33, dtype="f32"),
]


def capture(fn):
    """Runs fn once on a side stream (warm-up), then captures it into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("cfg", FORWARD_CASES, ids=[c.name for c in FORWARD_CASES])
def test_forward_graph_replays_match_eager(cfg):
    log(f"[graph] forward {cfg.name}")
    dev = upload(make_inputs(cfg, seed=21, affine=True))
    weights = (dev["gamma"], dev["beta"], dev["w_in"], dev["w_out"])
    h = tb.pblock_create(cfg)
    g = None
    try:
        ref = torch.empty_like(dev["x"])
        tb.pblock_forward(h, dev["x"], weights, cfg, ref)
        torch.cuda.synchronize()
        out = torch.empty_like(dev["x"])
        g = capture(lambda: tb.pblock_forward(h, dev["x"], weights, cfg, out))
        for r in range(REPLAYS):
            out.zero_()
            other = torch.empty_like(dev["x"])
            tb.pblock_forward(h, dev["x"], weights, cfg, other)  # eager, same handle and workspace
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref), f"{cfg.name}: replay {r} differs from the eager forward"
            assert torch.equal(other, ref), f"{cfg.name}: eager forward {r} after a replay differs"
        log(f"[graph] {cfg.name}: {REPLAYS} replays equal to the eager forward, bit for bit")
    finally:
        torch.cuda.synchronize()
        del g
        tb.pblock_destroy(h)


TRAIN_CASES = [
    # B*S = 600: dy is staged into whole 256-row tiles (a copy node); 512: dy is read in place
    BlockConfig("graph_train_staged", B=2, S=300, d=256, H=2, hd=128, ffn=320, W=64, dtype="bf16"),
    BlockConfig("graph_train_inplace", B=2, S=256, d=256, H=2, hd=64, ffn=256, W=48, dtype="bf16",
                add_residual=0),
]


@pytest.mark.parametrize("cfg", TRAIN_CASES, ids=[c.name for c in TRAIN_CASES])
def test_training_step_graph_replays_match_eager(cfg):
    log(f"[graph] training step {cfg.name}")
    dev = upload(make_inputs(cfg, seed=22, affine=True))
    dy = to_dev(make_dy(cfg, seed=22)["dy_dev"], "bf16")
    weights = (dev["gamma"], dev["beta"], dev["w_in"], dev["w_out"])
    h = tb.pblock_create(cfg)
    g = None
    try:
        ws = torch.empty(tb.pblock_train_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")

        def new_grads():
            return {"dx": torch.empty_like(dev["x"]), "dln_gamma": torch.empty_like(dev["gamma"]),
                    "dln_beta": torch.empty_like(dev["beta"]), "dw_in": torch.empty_like(dev["w_in"]),
                    "dw_out": torch.empty_like(dev["w_out"])}

        def step(out, grads):
            tb.pblock_forward_train(h, dev["x"], weights, cfg, out, ws)
            tb.pblock_backward(h, dev["x"], weights, cfg, dy, grads, ws)

        ref_y, ref_g = torch.empty_like(dev["x"]), new_grads()
        step(ref_y, ref_g)
        torch.cuda.synchronize()
        y, grads = torch.empty_like(dev["x"]), new_grads()
        g = capture(lambda: step(y, grads))
        for r in range(REPLAYS):
            y.zero_()
            for t in grads.values():
                t.zero_()
            step(torch.empty_like(dev["x"]), new_grads())  # eager, same handle and workspace
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y, ref_y), f"{cfg.name}: replay {r}: y differs"
            for k, t in grads.items():
                assert torch.equal(t, ref_g[k]), f"{cfg.name}: replay {r}: {k} differs"
        log(f"[graph] {cfg.name}: {REPLAYS} replays of forward_train + backward equal to eager, bit for bit")
    finally:
        torch.cuda.synchronize()
        del g
        tb.pblock_destroy(h)
