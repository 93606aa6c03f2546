"""The precision floor behind the backward pass's tolerance at the 175B shard shape (CPU only).

At that shape (d = 12288, N(0, 0.02^2) weights) the attention scores q.k/sqrt(hd) have a
standard deviation of about 5, so storing u = LN(x) and q, k, v in bf16 (unit roundoff 2^-9,
reading c-9 of the precision choices) moves the exact attention output by more than the 1e-2
bar itself.  The fp64 oracle fed bf16-rounded u, q, k, v is compared here with the exact fp64
oracle: the gap must exceed 1e-2 (so no bf16 implementation can meet 1e-2 on quantities that
carry the attention output, as the backward's gradients do through the stored output, D = dO.O
and dS) and stay below 2e-2 (the bar the GPU backward is held to at this shape).  The forward's
y still meets 1e-2 there because the attention branch is a small part of y.
"""
import numpy as np

import oracle
from workload import CONFIGS, make_inputs, round_to_bf16

BWD_SHARD_TOL = 2e-2  # the backward bar at the 175B shard shape (tests/test_gpu_backward.py)


def _bf16(a):
    vals, _ = round_to_bf16(np.asarray(a, np.float32))
    return vals.astype(np.float64)


def _attention(qkv, cfg):
    S, H, hd, A = cfg.S, cfg.H, cfg.hd, cfg.A
    q = qkv[:, :A].reshape(S, H, hd)
    k = qkv[:, A:2 * A].reshape(S, H, hd)
    v = qkv[:, 2 * A:3 * A].reshape(S, H, hd)
    return oracle.swa_attention(q, k, v, cfg.W), q, k


def test_bf16_storage_floor_at_shard_shape():
    cfg = CONFIGS["shard175b"]
    inp = make_inputs(cfg, seed=0)
    A = cfg.A
    x = inp.x[0].astype(np.float64)
    w_qkv = inp.w_in[:3 * A].astype(np.float64)
    u = oracle.layer_norm(x, inp.gamma, inp.beta, cfg.ln_eps)
    o_exact, q, k = _attention(u @ w_qkv.T, cfg)
    # the same steps with u and then q, k, v stored in bf16, all arithmetic still fp64
    o_bf16, _, _ = _attention(_bf16(_bf16(u) @ w_qkv.T), cfg)
    err = oracle.relative_error(o_bf16, o_exact)
    scores = np.einsum("shd,shd->sh", q[1:], k[:-1]) / np.sqrt(cfg.hd)  # neighbouring pairs
    print(f"[floor] shard175b attention output: bf16 storage moves it by {err:.3e} of its max; "
          f"score std {scores.std():.2f}")
    assert scores.std() > 3.0
    assert 1e-2 < err < BWD_SHARD_TOL


def test_bf16_storage_floor_small_shape():
    """At the small workload's shape (d = 2048) the scores stay O(1) and the same storage
    rounding stays well inside 1e-2: the floor is a property of the 175B shard's width."""
    cfg = CONFIGS["small"].replace(B=1, S=512)
    inp = make_inputs(cfg, seed=0)
    A = cfg.A
    x = inp.x[0].astype(np.float64)
    w_qkv = inp.w_in[:3 * A].astype(np.float64)
    u = oracle.layer_norm(x, inp.gamma, inp.beta, cfg.ln_eps)
    o_exact, _, _ = _attention(u @ w_qkv.T, cfg)
    o_bf16, _, _ = _attention(_bf16(_bf16(u) @ w_qkv.T), cfg)
    err = oracle.relative_error(o_bf16, o_exact)
    print(f"[floor] small attention output: {err:.3e}")
    assert err < 1e-2


def _forward_bf16_storage(inp, cfg):
    """The oracle's steps with u, q|k|v, [attention | GeLU] and y rounded to bf16 where the
    library stores them (reading c-9); every product and sum still in fp64."""
    A, B, S = cfg.A, cfg.B, cfg.S
    x = inp.x.astype(np.float64)
    u = _bf16(oracle.layer_norm(x, inp.gamma, inp.beta, cfg.ln_eps))
    z = u @ inp.w_in.astype(np.float64).T
    qkv = _bf16(z[..., :3 * A])
    o = np.empty((B, S, cfg.H, cfg.hd))
    for b in range(B):
        o[b], _, _ = _attention(qkv[b], cfg)
    ag = _bf16(np.concatenate([o.reshape(B, S, A), oracle.gelu(z[..., 3 * A:])], axis=-1))
    y = ag @ inp.w_out.astype(np.float64).T
    return _bf16(y + x if cfg.add_residual else y)


def test_forward_storage_floor_at_shard_shape():
    """The forward at the 175B shard shape: bf16 storage alone puts y 8.3e-3 (of max|y|) from the
    exact oracle, so the 1e-2 bar leaves a margin of about a sixth there for the kernels' own
    fp32 accumulation-order differences; at the small workload the floor is 3.2e-3."""
    for name, lo, hi in (("shard175b", 7e-3, 9e-3), ("small", 2e-3, 4.5e-3)):
        cfg = CONFIGS[name]
        inp = make_inputs(cfg, seed=0)
        y_ref = oracle.block_forward(inp.x, inp.gamma, inp.beta, inp.w_in, inp.w_out, cfg.H, cfg.hd, cfg.W,
                                     eps=cfg.ln_eps, add_residual=bool(cfg.add_residual))
        err = oracle.relative_error(_forward_bf16_storage(inp, cfg), y_ref)
        print(f"[floor] {name} forward: bf16 storage of the intermediates and y moves y by {err:.4e} of its max")
        assert lo < err < hi
