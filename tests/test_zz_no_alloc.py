"""The no-allocation forward (pblock_forward_static) against pblock_forward, through the raw
C ABI: two calls in a row on one GPU, the second with a smaller input, each equal to the
handle's forward bit for bit (same kernels, same launches) and within the parity bar of the
oracle; a cfg beyond the static workspace is rejected before any launch."""
import ctypes

import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, from_dev, log, rel_err, run_block, upload
from workload import CONFIGS, BlockConfig, make_inputs

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import transformer_block_fwd_amd as tb  # noqa: E402


def _static_forward(cfg, dev, out):
    lib = tb._abi.lib()
    w = tb.PblockWeights(dev["gamma"].data_ptr(), dev["beta"].data_ptr(), dev["w_in"].data_ptr(),
                         dev["w_out"].data_ptr())
    stream = torch.cuda.current_stream().cuda_stream
    return lib.pblock_forward_static(dev["x"].data_ptr(), ctypes.byref(w), ctypes.byref(tb.as_cfg(cfg)),
                                     out.data_ptr(), stream)


@pytest.mark.parametrize("first,second", [
    (BlockConfig("static_big", B=2, S=1000, d=1024, H=8, hd=128, ffn=2304, W=200, dtype="bf16"),
     BlockConfig("static_small", B=1, S=333, d=1024, H=8, hd=128, ffn=2304, W=37, dtype="bf16")),
    (CONFIGS["shard175b"], BlockConfig("static_f32", B=1, S=200, d=256, H=2, hd=64, ffn=256, W=40, dtype="f32")),
], ids=["bf16_then_smaller", "shard175b_then_f32"])
def test_static_forward_matches_handle_forward(first, second):
    for cfg, seed in ((first, 41), (second, 42)):
        log(f"[case] static forward {cfg}")
        inp = make_inputs(cfg, seed=seed, affine=True)
        dev = upload(inp)
        out = torch.full_like(dev["x"], float("nan"))
        assert _static_forward(cfg, dev, out) == tb._abi.PBLOCK_OK, tb._abi.last_error()
        torch.cuda.synchronize()
        y_static = from_dev(out).reshape(cfg.B, cfg.S, cfg.d)
        y_handle = run_block(cfg, dev)
        assert np.isfinite(y_static).all()
        assert np.array_equal(y_static, y_handle)
        err = rel_err(y_static, y_handle)
        assert err <= TOL[cfg.dtype]
        if cfg.M <= 4096:
            ref = oracle.block_forward(inp.x, inp.gamma, inp.beta, inp.w_in, inp.w_out, cfg.H, cfg.hd, cfg.W,
                                       eps=cfg.ln_eps, add_residual=bool(cfg.add_residual))
            err_o = rel_err(y_static, ref)
            log(f"[parity] static forward {cfg.name}: vs oracle {err_o:.3e}, vs handle forward bitwise equal")
            assert err_o <= TOL[cfg.dtype]
        del dev
        torch.cuda.empty_cache()


def test_static_forward_rejects_oversized_cfg():
    """The long workload needs more than the 256 MiB static workspace: rejected, nothing launched."""
    cfg = CONFIGS["long"].replace(S=4096)  # 4096 tokens of the long shape: about 390 MB
    need = tb.pblock_workspace_bytes(cfg)
    assert need > 256 << 20
    x = torch.zeros((cfg.B, cfg.S, cfg.d), dtype=torch.bfloat16, device="cuda")
    g = torch.ones(cfg.d, dtype=torch.bfloat16, device="cuda")
    b = torch.zeros(cfg.d, dtype=torch.bfloat16, device="cuda")
    wi = torch.zeros((cfg.n_in, cfg.d), dtype=torch.bfloat16, device="cuda")
    wo = torch.zeros((cfg.d, cfg.k_out), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(x, 3.0)
    rc = _static_forward(cfg, {"x": x, "gamma": g, "beta": b, "w_in": wi, "w_out": wo}, out)
    assert rc == tb._abi.PBLOCK_ERR_SHAPE
    assert "static" in tb._abi.last_error()
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
