"""Checks that pin the oracle to facts outside itself.

Each ``pin_*`` function takes an oracle module (``oracle.block`` or a copy of
it with a planted mistake) and raises AssertionError when the oracle disagrees
with brute force, a closed form, an invariant or a library routine.  The
reference values come from, in turn:
  * pure-Python loops over single query/key pairs (brute force);
  * torch CPU float64 library routines (layer_norm, gelu, scaled-dot-product
    attention with an explicit band mask or is_causal);
  * closed forms: W = 1 (each token sees only itself), W = 2 (a two-key softmax
    is a logistic function), uniform attention when Q is zero, LayerNorm of
    zero-mean unit-variance sign patterns, the normal CDF at 1;
  * invariants: branch-sum identity, tensor-parallel decomposition, locality of
    the window, batch independence;
  * for the variant switches: torch's linear-with-bias and tanh gelu, the rotary
    embedding as complex multiplication (RoFormer's complex form), rotations of
    basis vectors worked out by hand, and RoPE's dependence on relative position
    only;
  * for the backward pass: torch autograd in float64, central finite
    differences of the (separately pinned) forward, LayerNorm's shift and scale
    invariance, and the exactly zero q/k gradients at W = 1.
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F

PHI_1 = 0.8413447460685429  # standard normal CDF at 1 (textbook table value)


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _rand_block(seed, B, S, d, H, hd, ffn, affine=True):
    rng = _rng(seed)
    x = rng.standard_normal((B, S, d)) * 1.3 + 0.4
    w_in = rng.standard_normal((3 * H * hd + ffn, d)) * (1.0 / math.sqrt(d))
    w_out = rng.standard_normal((d, H * hd + ffn)) * (1.0 / math.sqrt(H * hd + ffn))
    if affine:
        gamma = 1.0 + 0.3 * rng.standard_normal(d)
        beta = 0.2 * rng.standard_normal(d)
    else:
        gamma, beta = np.ones(d), np.zeros(d)
    return x, gamma, beta, w_in, w_out


def _torch_band_attention(q, k, v, W):
    """q, k, v: [S, H, hd] numpy fp64 -> torch SDPA with a boolean band mask."""
    S = q.shape[0]
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    mask = (j <= i) & (j > i - W)
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))[None] for a in (q, k, v))
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    return o[0].numpy().transpose(1, 0, 2)


def _torch_block(x, gamma, beta, w_in, w_out, H, hd, W, eps, add_residual=True):
    """The block assembled from torch float64 library routines."""
    tx = torch.from_numpy(x)
    A = H * hd
    u = F.layer_norm(tx, (x.shape[-1],), torch.from_numpy(gamma), torch.from_numpy(beta), eps)
    z = u @ torch.from_numpy(w_in).T
    B, S, _ = x.shape
    q = z[..., :A].reshape(B, S, H, hd).transpose(1, 2)
    k = z[..., A:2 * A].reshape(B, S, H, hd).transpose(1, 2)
    v = z[..., 2 * A:3 * A].reshape(B, S, H, hd).transpose(1, 2)
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    mask = (j <= i) & (j > i - W)
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask).transpose(1, 2).reshape(B, S, A)
    wo = torch.from_numpy(w_out)
    y = o @ wo[:, :A].T + F.gelu(z[..., 3 * A:], approximate="none") @ wo[:, A:].T
    if add_residual:
        y = y + tx
    return y.numpy()


def _torch_serial_block(x, g1, b1, g2, b2, w_in, w_out, H, hd, W, eps):
    """The serial pre-LN layer assembled from torch float64 library routines."""
    tx = torch.from_numpy(x)
    A = H * hd
    B, S, d = x.shape
    wi = torch.from_numpy(w_in)
    wo = torch.from_numpy(w_out)
    u1 = F.layer_norm(tx, (d,), torch.from_numpy(g1), torch.from_numpy(b1), eps)
    qkv = F.linear(u1, wi[:3 * A])
    q, k, v = (qkv[..., c * A:(c + 1) * A].reshape(B, S, H, hd).transpose(1, 2) for c in range(3))
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=(j <= i) & (j > i - W)).transpose(1, 2).reshape(B, S, A)
    h = tx + F.linear(o, wo[:, :A])
    u2 = F.layer_norm(h, (d,), torch.from_numpy(g2), torch.from_numpy(b2), eps)
    return (h + F.linear(F.gelu(F.linear(u2, wi[3 * A:]), approximate="none"), wo[:, A:])).numpy()


def _torch_rope(t, base):
    """[B, S, H, hd] -> rotated, as RoFormer's complex form: the pair (t_2i, t_2i+1) is the
    complex number t_2i + i t_2i+1, multiplied by e^(i p theta_i), theta_i = base^(-2i/hd)."""
    B, S, H, hd = t.shape
    theta = torch.pow(torch.tensor(float(base), dtype=torch.float64), -torch.arange(0, hd, 2, dtype=torch.float64) / hd)
    ang = torch.arange(S, dtype=torch.float64)[:, None] * theta[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)  # [S, hd/2]
    tc = torch.view_as_complex(t.reshape(B, S, H, hd // 2, 2).contiguous())
    return torch.view_as_real(tc * rot[None, :, None, :]).reshape(B, S, H, hd)


def _torch_variant_block(x, g, b, wi, wo, H, hd, W, eps, add_residual=True, gelu_form="erf", b_in=None, b_out=None,
                         rope_base=None, g2=None, b2=None):
    """The variant block from torch float64 library routines (layer_norm, linear with bias,
    gelu in either form, band-masked scaled-dot-product attention), RoPE as complex products."""
    tx = torch.from_numpy(x)
    B, S, d = x.shape
    A = H * hd
    t = torch.from_numpy
    ua = F.layer_norm(tx, (d,), t(g), t(b), eps)
    um = ua if g2 is None else F.layer_norm(tx, (d,), t(g2), t(b2), eps)
    wi_t = t(wi)
    bi = None if b_in is None else t(b_in)
    z = F.linear(ua, wi_t[:3 * A], None if bi is None else bi[:3 * A])
    f = F.linear(um, wi_t[3 * A:], None if bi is None else bi[3 * A:])
    q, k, v = (z[..., c * A:(c + 1) * A].reshape(B, S, H, hd) for c in range(3))
    if rope_base is not None:
        q, k = _torch_rope(q, rope_base), _torch_rope(k, rope_base)
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    o = F.scaled_dot_product_attention(q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2),
                                       attn_mask=(j <= i) & (j > i - W)).transpose(1, 2).reshape(B, S, A)
    act = F.gelu(f, approximate="none" if gelu_form == "erf" else "tanh")
    y = F.linear(torch.cat([o, act], dim=-1), t(wo), None if b_out is None else t(b_out))
    if add_residual:
        y = y + tx
    return y.numpy()


def _variant_params(seed, d, n_in, two_ln=True):
    rng = _rng(seed)
    b_in = 0.3 * rng.standard_normal(n_in)
    b_out = 0.3 * rng.standard_normal(d)
    g2 = 1.0 + 0.3 * rng.standard_normal(d) if two_ln else None
    b2 = 0.2 * rng.standard_normal(d) if two_ln else None
    return b_in, b_out, g2, b2


# ----------------------------------------------------------------------------- attention


def pin_attention_brute_force(ob):
    """Blocked band attention == per-pair Python loops, for odd S and several W."""
    rng = _rng(11)
    for S, H, hd in ((1, 1, 4), (37, 2, 8), (133, 1, 4)):
        q = rng.standard_normal((S, H, hd))
        k = rng.standard_normal((S, H, hd))
        v = rng.standard_normal((S, H, hd))
        for W in sorted({1, 2, 7, max(1, S - 1), S, 2 * S}):
            got = ob.swa_attention(q, k, v, W, slab=16)
            for h in range(H):
                for i in range(S):
                    keys = [j for j in range(S) if j <= i and i - j < W]
                    s = [sum(q[i, h, t] * k[j, h, t] for t in range(hd)) / math.sqrt(hd) for j in keys]
                    mx = max(s)
                    e = [math.exp(a - mx) for a in s]
                    den = sum(e)
                    for t in range(hd):
                        ref = sum(e[n] * v[keys[n], h, t] for n in range(len(keys))) / den
                        assert abs(got[i, h, t] - ref) <= 1e-12 * (1 + abs(ref)), (S, W, h, i, t)


def pin_attention_vs_torch_band(ob):
    """Band attention == torch SDPA with an explicit boolean band mask."""
    rng = _rng(12)
    for S, W in ((300, 1), (300, 37), (300, 128), (257, 256), (129, 500)):
        q, k, v = (rng.standard_normal((S, 3, 16)) for _ in range(3))
        got = ob.swa_attention(q, k, v, W)
        ref = _torch_band_attention(q, k, v, W)
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def pin_attention_full_causal(ob):
    """W >= S is plain causal attention (torch SDPA is_causal=True)."""
    rng = _rng(13)
    S = 211
    q, k, v = (rng.standard_normal((S, 2, 16)) for _ in range(3))
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))[None] for a in (q, k, v))
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True)[0].numpy().transpose(1, 0, 2)
    for W in (S, S + 1, 4 * S):
        np.testing.assert_allclose(ob.swa_attention(q, k, v, W), ref, rtol=1e-11, atol=1e-12)


def pin_attention_w1_is_identity(ob):
    """W = 1: each query sees only its own key, so the output is its own value."""
    rng = _rng(14)
    q, k, v = (rng.standard_normal((77, 3, 8)) * 5 for _ in range(3))
    np.testing.assert_allclose(ob.swa_attention(q, k, v, 1), v, rtol=0, atol=1e-13)


def pin_attention_two_keys(ob):
    """W = 2: o_i = s(delta) v_i + (1 - s(delta)) v_{i-1}, s = logistic,
    delta = (q_i.k_i - q_i.k_{i-1}) / sqrt(hd); o_0 = v_0."""
    rng = _rng(15)
    S, H, hd = 50, 2, 8
    q, k, v = (rng.standard_normal((S, H, hd)) for _ in range(3))
    got = ob.swa_attention(q, k, v, 2, slab=7)
    for h in range(H):
        np.testing.assert_allclose(got[0, h], v[0, h], atol=1e-14)
        for i in range(1, S):
            delta = (q[i, h] @ k[i, h] - q[i, h] @ k[i - 1, h]) / math.sqrt(hd)
            w = 1.0 / (1.0 + math.exp(-delta))
            np.testing.assert_allclose(got[i, h], w * v[i, h] + (1 - w) * v[i - 1, h], rtol=1e-12, atol=1e-13)


def pin_attention_offset_keys(ob):
    """Queries given at an offset with only their needed keys == the full call."""
    rng = _rng(16)
    S, W = 200, 33
    q, k, v = (rng.standard_normal((S, 2, 8)) for _ in range(3))
    full = ob.swa_attention(q, k, v, W)
    i0, i1 = 120, 170
    j0 = i0 - W + 1
    part = ob.swa_attention(q[i0:i1], k[j0:i1], v[j0:i1], W, q_pos0=i0, k_pos0=j0)
    np.testing.assert_allclose(part, full[i0:i1], rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------------------- LN, GeLU


def pin_layer_norm(ob):
    """LayerNorm == torch layer_norm; gamma=1, beta=0 rows have mean 0 and
    variance var/(var+eps)."""
    rng = _rng(21)
    x = rng.standard_normal((5, 7, 96)) * 3 + 2
    g = 1 + 0.5 * rng.standard_normal(96)
    b = 0.3 * rng.standard_normal(96)
    for eps in (1e-5, 0.1):
        ref = F.layer_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), torch.from_numpy(b), eps).numpy()
        np.testing.assert_allclose(ob.layer_norm(x, g, b, eps), ref, rtol=1e-12, atol=1e-12)
    eps = 0.5
    u = ob.layer_norm(x, np.ones(96), np.zeros(96), eps)
    var = x.var(axis=-1)
    np.testing.assert_allclose(u.mean(axis=-1), 0, atol=1e-12)
    np.testing.assert_allclose(u.var(axis=-1), var / (var + eps), rtol=1e-12)


def pin_gelu(ob):
    """GeLU == torch exact gelu and x*Phi(x) via math.erf; odd-part identity;
    GeLU(0) = 0; GeLU(1) = Phi(1)."""
    z = np.linspace(-9, 9, 2001)
    ref = F.gelu(torch.from_numpy(z), approximate="none").numpy()
    got = ob.gelu(z)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)
    loop = np.array([t * 0.5 * (1 + math.erf(t / math.sqrt(2))) for t in z])
    np.testing.assert_allclose(got, loop, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(ob.gelu(-z), got - z, rtol=1e-12, atol=1e-12)
    assert ob.gelu(np.array([0.0]))[0] == 0.0
    assert abs(ob.gelu(np.array([1.0]))[0] - PHI_1) < 1e-15
    # the tanh approximation differs visibly at z ~ 2.7: the exact form is the one computed
    tanh_form = 0.5 * 2.7 * (1 + math.tanh(math.sqrt(2 / math.pi) * (2.7 + 0.044715 * 2.7 ** 3)))
    assert abs(ob.gelu(np.array([2.7]))[0] - tanh_form) > 1e-4


# ----------------------------------------------------------------------------- whole block


def pin_block_vs_torch(ob):
    """Whole block == the same block assembled from torch fp64 library routines,
    with odd shapes, several windows, random gamma/beta."""
    for seed, (B, S, d, H, hd, ffn), W in ((31, (2, 45, 24, 3, 8, 40), 9),
                                           (32, (1, 70, 32, 2, 16, 48), 70),
                                           (33, (3, 17, 16, 1, 8, 8), 1)):
        x, g, b, wi, wo = _rand_block(seed, B, S, d, H, hd, ffn)
        for add_res in (True, False):
            got = ob.block_forward(x, g, b, wi, wo, H, hd, W, eps=1e-5, add_residual=add_res)
            ref = _torch_block(x, g, b, wi, wo, H, hd, W, 1e-5, add_res)
            np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-11)


def pin_block_w1_closed_form(ob):
    """W = 1: the attention branch is the linear map (u W_v^T) W_o^T."""
    B, S, d, H, hd, ffn = 2, 19, 24, 3, 4, 20
    x, g, b, wi, wo = _rand_block(41, B, S, d, H, hd, ffn)
    A = H * hd
    u = F.layer_norm(torch.from_numpy(x), (d,), torch.from_numpy(g), torch.from_numpy(b), 1e-5).numpy()
    ref = x + (u @ wi[2 * A:3 * A].T) @ wo[:, :A].T \
        + F.gelu(torch.from_numpy(u @ wi[3 * A:].T)).numpy() @ wo[:, A:].T
    got = ob.block_forward(x, g, b, wi, wo, H, hd, 1)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def pin_block_branch_sum(ob):
    """Parallel block == sum of its separately computed branches: the attention
    branch alone (FC1 rows zero, so GeLU(0) = 0) plus the MLP branch alone
    (V rows zero, so attention outputs 0)."""
    B, S, d, H, hd, ffn, W = 2, 40, 32, 2, 8, 48, 11
    x, g, b, wi, wo = _rand_block(51, B, S, d, H, hd, ffn)
    A = H * hd
    full = ob.block_forward(x, g, b, wi, wo, H, hd, W)
    wi_attn = wi.copy()
    wi_attn[3 * A:] = 0
    wi_mlp = wi.copy()
    wi_mlp[2 * A:3 * A] = 0
    y_attn = ob.block_forward(x, g, b, wi_attn, wo, H, hd, W, add_residual=False)
    y_mlp = ob.block_forward(x, g, b, wi_mlp, wo, H, hd, W, add_residual=False)
    np.testing.assert_allclose(full - x, y_attn + y_mlp, rtol=1e-11, atol=1e-12)
    assert np.abs(y_attn).max() > 1e-3 and np.abs(y_mlp).max() > 1e-3


def pin_block_tensor_parallel(ob):
    """Split heads and FFN columns over R shards; the shards' partials plus x
    reproduce the unsharded block (the reduce-scatter's sum)."""
    B, S, d, H, hd, ffn, W = 1, 33, 16, 4, 4, 32, 6
    x, g, b, wi, wo = _rand_block(61, B, S, d, H, hd, ffn)
    A = H * hd
    full = ob.block_forward(x, g, b, wi, wo, H, hd, W)
    for R in (2, 4):
        hs, fs = H // R, ffn // R
        total = np.zeros_like(full)
        for r in range(R):
            rows = []
            for part in range(3):  # Q, K, V slices of this shard's heads
                rows.append(wi[part * A + r * hs * hd: part * A + (r + 1) * hs * hd])
            rows.append(wi[3 * A + r * fs: 3 * A + (r + 1) * fs])
            wi_r = np.concatenate(rows, axis=0)
            wo_r = np.concatenate([wo[:, r * hs * hd:(r + 1) * hs * hd], wo[:, A + r * fs:A + (r + 1) * fs]], axis=1)
            total += ob.block_forward(x, g, b, wi_r, wo_r, hs, hd, W, add_residual=False)
        np.testing.assert_allclose(total + x, full, rtol=1e-11, atol=1e-12)


def pin_block_locality(ob):
    """Perturbing tokens outside query i's window leaves y_i bit-identical;
    perturbing inside changes it; batches are independent."""
    B, S, d, H, hd, ffn, W = 2, 40, 16, 2, 8, 16, 5
    x, g, b, wi, wo = _rand_block(71, B, S, d, H, hd, ffn)
    y = ob.block_forward(x, g, b, wi, wo, H, hd, W)
    bump = 3.0 * _rng(72).standard_normal(d)  # not a constant: LayerNorm removes constant shifts
    i = 25
    for j in (i - W, i + 1, 0, S - 1):
        xp = x.copy()
        xp[0, j] += bump
        yp = ob.block_forward(xp, g, b, wi, wo, H, hd, W)
        assert np.array_equal(yp[0, i], y[0, i]), j
        assert np.array_equal(yp[1], y[1])
    for j in (i - W + 1, i - 1):
        xp = x.copy()
        xp[0, j] += bump
        yp = ob.block_forward(xp, g, b, wi, wo, H, hd, W)
        assert np.abs(yp[0, i] - y[0, i]).max() > 1e-6, j


def pin_block_uniform_closed_form(ob):
    """Hand-derived block.  Rows of x are m + s*p with p a zero-mean, unit-
    variance sign pattern, so with eps = 0 LayerNorm returns gamma*p + beta.
    With W_q = 0 every score is 0 and attention is the plain mean of V over the
    window; W_v = I and W_fc1 = I, W_out = [I | I] give
        y_i = x_i + mean_{j in window(i)} u_j + GeLU(u_i),
    and GeLU(+1) = Phi(1), GeLU(-1) = Phi(1) - 1."""
    d = hd = ffn = 4
    H = 1
    pats = np.array([[1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1], [-1, 1, 1, -1], [-1, -1, 1, 1]], float)
    S = len(pats)
    m = np.array([0.5, -2.0, 3.0, 0.0, 1.25])
    s = np.array([2.0, 0.5, 1.0, 3.0, 0.25])
    x = (m[:, None] + s[:, None] * pats)[None]
    eye = np.eye(4)
    w_in = np.concatenate([np.zeros((4, 4)), 0.7 * eye[::-1], eye, eye], axis=0)  # Q=0, K arbitrary, V=I, FC1=I
    w_out = np.concatenate([eye, eye], axis=1)
    g1 = {1.0: PHI_1, -1.0: PHI_1 - 1.0}
    for W in (1, 2, 3, 5):
        y = ob.block_forward(x, np.ones(d), np.zeros(d), w_in, w_out, H, hd, W, eps=0.0)
        for i in range(S):
            lo = max(0, i - W + 1)
            mean_u = pats[lo:i + 1].mean(axis=0)
            ref = x[0, i] + mean_u + np.array([g1[v] for v in pats[i]])
            np.testing.assert_allclose(y[0, i], ref, rtol=0, atol=1e-13)


def pin_rows_match_full(ob):
    """Row-sampled forward == full forward on the same rows."""
    B, S, d, H, hd, ffn, W = 2, 90, 16, 2, 8, 24, 13
    x, g, b, wi, wo = _rand_block(81, B, S, d, H, hd, ffn)
    full = ob.block_forward(x, g, b, wi, wo, H, hd, W)
    blocks = [(0, 0, 7), (1, 5, 30), (1, 60, 90), (0, 12, 13)]
    for (bb, i0, i1), y in zip(blocks, ob.block_forward_rows(x, g, b, wi, wo, H, hd, W, blocks)):
        np.testing.assert_allclose(y, full[bb, i0:i1], rtol=1e-12, atol=1e-13)


def pin_serial_vs_torch(ob):
    """Serial pre-LN layer == the same layer assembled from torch fp64 library routines
    (odd shapes, several windows, distinct random LN1 and LN2 parameters)."""
    for seed, (B, S, d, H, hd, ffn), W in ((61, (2, 45, 24, 3, 8, 40), 9),
                                           (62, (1, 70, 32, 2, 16, 48), 70),
                                           (63, (3, 17, 16, 1, 8, 8), 1)):
        x, g1, b1, wi, wo = _rand_block(seed, B, S, d, H, hd, ffn)
        rng = _rng(seed + 100)
        g2 = 1.0 + 0.3 * rng.standard_normal(d)
        b2 = 0.2 * rng.standard_normal(d)
        got = ob.serial_block_forward(x, g1, b1, g2, b2, wi, wo, H, hd, W)
        ref = _torch_serial_block(x, g1, b1, g2, b2, wi, wo, H, hd, W, 1e-5)
        np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-11)


def pin_serial_single_sublayer(ob):
    """With one sub-layer switched off the serial and parallel forms coincide: W_2 = 0
    leaves h = x + attention branch (the parallel block with FC1 rows zero); W_o = 0
    leaves h = x and y = x + MLP(LN2 x) (the parallel block with V rows zero, LN2 = LN1).
    With both on, they differ (LN2 sees h, not x)."""
    B, S, d, H, hd, ffn, W = 2, 40, 32, 2, 8, 48, 11
    x, g, b, wi, wo = _rand_block(71, B, S, d, H, hd, ffn)
    A = H * hd
    wo_attn = wo.copy()
    wo_attn[:, A:] = 0
    wi_attn = wi.copy()
    wi_attn[3 * A:] = 0
    np.testing.assert_allclose(ob.serial_block_forward(x, g, b, g, b, wi, wo_attn, H, hd, W),
                               ob.block_forward(x, g, b, wi_attn, wo, H, hd, W), rtol=1e-11, atol=1e-12)
    wo_mlp = wo.copy()
    wo_mlp[:, :A] = 0
    wi_mlp = wi.copy()
    wi_mlp[2 * A:3 * A] = 0
    np.testing.assert_allclose(ob.serial_block_forward(x, g, b, g, b, wi, wo_mlp, H, hd, W),
                               ob.block_forward(x, g, b, wi_mlp, wo, H, hd, W), rtol=1e-11, atol=1e-12)
    both = ob.serial_block_forward(x, g, b, g, b, wi, wo, H, hd, W)
    assert np.abs(both - ob.block_forward(x, g, b, wi, wo, H, hd, W)).max() > 1e-3


def pin_serial_rows_match_full(ob):
    """serial_block_forward_rows == slices of serial_block_forward."""
    B, S, d, H, hd, ffn, W = 2, 90, 24, 3, 8, 40, 13
    x, g1, b1, wi, wo = _rand_block(81, B, S, d, H, hd, ffn)
    g2, b2 = g1[::-1].copy(), b1[::-1].copy()
    full = ob.serial_block_forward(x, g1, b1, g2, b2, wi, wo, H, hd, W)
    blocks = [(0, 0, 5), (1, 7, 30), (0, 60, 90), (1, 89, 90)]
    for (b, i0, i1), y in zip(blocks, ob.serial_block_forward_rows(x, g1, b1, g2, b2, wi, wo, H, hd, W, blocks)):
        np.testing.assert_allclose(y, full[b, i0:i1], rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- variant switches


def pin_gelu_tanh(ob):
    """tanh GeLU == torch's tanh-approximate gelu and a math.tanh loop; it stays within
    1e-3 of the exact form and differs from it by more than 1e-4 somewhere."""
    z = np.linspace(-9, 9, 2001)
    got = ob.gelu_tanh(z)
    np.testing.assert_allclose(got, F.gelu(torch.from_numpy(z), approximate="tanh").numpy(), rtol=1e-13,
                               atol=1e-15)
    loop = np.array([0.5 * t * (1 + math.tanh(math.sqrt(2 / math.pi) * (t + 0.044715 * t ** 3))) for t in z])
    np.testing.assert_allclose(got, loop, rtol=1e-13, atol=1e-15)
    gap = np.abs(got - ob.gelu(z)).max()
    assert 1e-4 < gap < 1e-3, gap


def pin_rope_hand_values(ob):
    """Rotations of basis vectors worked out by hand: hd = 4, base 10000, so the two pair
    frequencies are 1 and 10000^(-1/2) = 0.01; e0 at position p goes to (cos p, sin p, 0, 0),
    e3 to (0, 0, -sin 0.01p, cos 0.01p); position 0 is the identity."""
    pos = np.array([0, 1, 3, 1000])
    for p_idx, p in enumerate(pos):
        e0 = np.zeros((len(pos), 1, 4))
        e0[:, 0, 0] = 1.0
        e3 = np.zeros((len(pos), 1, 4))
        e3[:, 0, 3] = 1.0
        r0 = ob.rope(e0, pos, 10000.0)[p_idx, 0]
        r3 = ob.rope(e3, pos, 10000.0)[p_idx, 0]
        np.testing.assert_allclose(r0, [math.cos(p), math.sin(p), 0, 0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(r3, [0, 0, -math.sin(0.01 * p), math.cos(0.01 * p)], rtol=0, atol=1e-12)


def pin_rope_relative_position(ob):
    """RoPE scores depend on relative position only: q at p and k at p' score the same as
    at p + c and p' + c; it is a rotation (norms kept); and a block whose windows never
    reach a prepended prefix gives the same rows as without the prefix."""
    rng = _rng(91)
    q = rng.standard_normal((1, 3, 16))
    k = rng.standard_normal((1, 3, 16))
    for p, pp in ((5, 2), (40, 40), (7, 100)):
        base = np.einsum("hd,hd->h", ob.rope(q, [p], 500.0)[0], ob.rope(k, [pp], 500.0)[0])
        for c in (1, 13, 999):
            sh = np.einsum("hd,hd->h", ob.rope(q, [p + c], 500.0)[0], ob.rope(k, [pp + c], 500.0)[0])
            np.testing.assert_allclose(sh, base, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(ob.rope(q, [17], 500.0), axis=-1), np.linalg.norm(q, axis=-1),
                               rtol=1e-13)
    B, S, d, H, hd, ffn, W, P = 1, 30, 16, 2, 8, 24, 5, 11
    x, g, b, wi, wo = _rand_block(92, B, S + P, d, H, hd, ffn)
    long = ob.block_forward_variant(x, g, b, wi, wo, H, hd, W, rope_base=100.0)
    short = ob.block_forward_variant(x[:, P:], g, b, wi, wo, H, hd, W, rope_base=100.0)
    np.testing.assert_allclose(long[:, P + W - 1:], short[:, W - 1:], rtol=1e-11, atol=1e-12)
    assert np.abs(long[:, P:P + W - 1] - short[:, :W - 1]).max() > 1e-6


def pin_variant_vs_torch(ob):
    """Each switch alone and all together == the torch-assembled block (odd shapes, several W)."""
    cases = [
        (101, (2, 45, 24, 3, 8, 40), 9, dict(gelu_form="tanh")),
        (102, (1, 70, 32, 2, 16, 48), 70, dict(bias=True)),
        (103, (2, 33, 16, 2, 8, 24), 6, dict(rope_base=10000.0)),
        (104, (1, 50, 24, 1, 16, 40), 17, dict(two_ln=True)),
        (105, (3, 21, 16, 2, 8, 16), 4, dict(gelu_form="tanh", bias=True, rope_base=50.0, two_ln=True)),
    ]
    for seed, (B, S, d, H, hd, ffn), W, kw in cases:
        x, g, b, wi, wo = _rand_block(seed, B, S, d, H, hd, ffn)
        b_in, b_out, g2, b2 = _variant_params(seed + 1, d, wi.shape[0])
        args = dict(gelu_form=kw.get("gelu_form", "erf"), rope_base=kw.get("rope_base"))
        if kw.get("bias"):
            args.update(b_in=b_in, b_out=b_out)
        for add_res in (True, False):
            got = ob.block_forward_variant(x, g, b, wi, wo, H, hd, W, add_residual=add_res, **args,
                                           gamma2=g2 if kw.get("two_ln") else None,
                                           beta2=b2 if kw.get("two_ln") else None)
            ref = _torch_variant_block(x, g, b, wi, wo, H, hd, W, 1e-5, add_res, **args,
                                       g2=g2 if kw.get("two_ln") else None, b2=b2 if kw.get("two_ln") else None)
            np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-11)


def pin_variant_reductions(ob):
    """With every switch off the variant block is block_forward; the second LayerNorm with
    the first one's parameters changes nothing; at W = 1 RoPE changes nothing (a token
    attending only to itself gets its own v, which is not rotated), and the attention branch
    is (u W_v^T + b_v) W_o^T."""
    B, S, d, H, hd, ffn, W = 2, 27, 16, 2, 8, 24, 7
    x, g, b, wi, wo = _rand_block(111, B, S, d, H, hd, ffn)
    b_in, b_out, _, _ = _variant_params(112, d, wi.shape[0], two_ln=False)
    np.testing.assert_allclose(ob.block_forward_variant(x, g, b, wi, wo, H, hd, W),
                               ob.block_forward(x, g, b, wi, wo, H, hd, W), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(ob.block_forward_variant(x, g, b, wi, wo, H, hd, W, gamma2=g, beta2=b),
                               ob.block_forward(x, g, b, wi, wo, H, hd, W), rtol=1e-13, atol=1e-14)
    A = H * hd
    r1 = ob.block_forward_variant(x, g, b, wi, wo, H, hd, 1, b_in=b_in, b_out=b_out, rope_base=10.0)
    u = F.layer_norm(torch.from_numpy(x), (d,), torch.from_numpy(g), torch.from_numpy(b), 1e-5).numpy()
    ref = x + (u @ wi[2 * A:3 * A].T + b_in[2 * A:3 * A]) @ wo[:, :A].T \
        + F.gelu(torch.from_numpy(u @ wi[3 * A:].T + b_in[3 * A:])).numpy() @ wo[:, A:].T + b_out
    np.testing.assert_allclose(r1, ref, rtol=1e-11, atol=1e-12)


def pin_variant_rows_match_full(ob):
    """block_forward_variant_rows == slices of block_forward_variant, every switch on."""
    B, S, d, H, hd, ffn, W = 2, 90, 16, 2, 8, 24, 13
    x, g, b, wi, wo = _rand_block(121, B, S, d, H, hd, ffn)
    b_in, b_out, g2, b2 = _variant_params(122, d, wi.shape[0])
    kw = dict(gelu_form="tanh", b_in=b_in, b_out=b_out, rope_base=1000.0, gamma2=g2, beta2=b2)
    full = ob.block_forward_variant(x, g, b, wi, wo, H, hd, W, **kw)
    blocks = [(0, 0, 7), (1, 5, 30), (1, 60, 90), (0, 12, 13)]
    for (bb, i0, i1), y in zip(blocks, ob.block_forward_variant_rows(x, g, b, wi, wo, H, hd, W, blocks, **kw)):
        np.testing.assert_allclose(y, full[bb, i0:i1], rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------- backward pass


def _torch_block_grads(x, g, b, wi, wo, H, hd, W, eps, dy, add_residual=True):
    """Gradients of sum(dy * block(x)) by torch autograd through float64 library routines."""
    t = {k: torch.from_numpy(np.array(v)).requires_grad_(True) for k, v in
         dict(x=x, gamma=g, beta=b, w_in=wi, w_out=wo).items()}
    B, S, d = x.shape
    A = H * hd
    u = F.layer_norm(t["x"], (d,), t["gamma"], t["beta"], eps)
    z = u @ t["w_in"].T
    q, k, v = (z[..., c * A:(c + 1) * A].reshape(B, S, H, hd).transpose(1, 2) for c in range(3))
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=(j <= i) & (j > i - W)).transpose(1, 2).reshape(B, S, A)
    y = torch.cat([o, F.gelu(z[..., 3 * A:], approximate="none")], dim=-1) @ t["w_out"].T
    if add_residual:
        y = y + t["x"]
    (y * torch.from_numpy(dy)).sum().backward()
    return dict(dx=t["x"].grad.numpy(), dgamma=t["gamma"].grad.numpy(), dbeta=t["beta"].grad.numpy(),
                dw_in=t["w_in"].grad.numpy(), dw_out=t["w_out"].grad.numpy())


def pin_gelu_grad(ob):
    """GeLU derivative == torch autograd of the exact gelu and central differences of x*Phi(x)."""
    z = np.linspace(-8, 8, 1601)
    tz = torch.from_numpy(z).requires_grad_(True)
    F.gelu(tz, approximate="none").sum().backward()
    np.testing.assert_allclose(ob.gelu_grad(z), tz.grad.numpy(), rtol=1e-12, atol=1e-14)
    h = 1e-5
    fd = np.array([((t + h) * 0.5 * (1 + math.erf((t + h) / math.sqrt(2)))
                    - (t - h) * 0.5 * (1 + math.erf((t - h) / math.sqrt(2)))) / (2 * h) for t in z])
    np.testing.assert_allclose(ob.gelu_grad(z), fd, rtol=0, atol=1e-8)


def pin_layer_norm_backward(ob):
    """LayerNorm backward == torch autograd; dx of the normalisation is orthogonal to the
    all-ones vector (shift invariance) and, with eps = 0, to xhat (scale invariance), row
    by row."""
    rng = _rng(131)
    x = rng.standard_normal((3, 5, 24)) * 2.0 + 1.0
    g = 1.0 + 0.3 * rng.standard_normal(24)
    b = 0.2 * rng.standard_normal(24)
    du = rng.standard_normal((3, 5, 24))
    tx, tg, tb = (torch.from_numpy(a.copy()).requires_grad_(True) for a in (x, g, b))
    (F.layer_norm(tx, (24,), tg, tb, 1e-5) * torch.from_numpy(du)).sum().backward()
    dx, dg, db = ob.layer_norm_backward(x, g, du, 1e-5)
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dg, tg.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(db, tb.grad.numpy(), rtol=1e-11, atol=1e-12)
    # shift invariance holds for any eps; scale invariance only without eps
    np.testing.assert_allclose(dx.sum(-1), 0.0, atol=1e-11)
    dx0, _, _ = ob.layer_norm_backward(x, g, du, 0.0)
    xhat = (x - x.mean(-1, keepdims=True)) / np.sqrt(x.var(-1, keepdims=True))
    np.testing.assert_allclose(dx0.sum(-1), 0.0, atol=1e-11)
    np.testing.assert_allclose((dx0 * xhat).sum(-1), 0.0, atol=1e-11)


def pin_attention_backward(ob):
    """Band attention backward == torch autograd through band-masked SDPA (odd S, several
    W); at W = 1 dq = dk = 0 and dv = do exactly."""
    rng = _rng(141)
    for S, H, hd, W in ((37, 2, 8, 5), (70, 1, 16, 70), (133, 2, 4, 17)):
        q, k, v, do = (rng.standard_normal((S, H, hd)) for _ in range(4))
        tq, tk, tv = (torch.from_numpy(a.transpose(1, 0, 2).copy()).requires_grad_(True) for a in (q, k, v))
        i = torch.arange(S)[:, None]
        j = torch.arange(S)[None, :]
        o = F.scaled_dot_product_attention(tq[None], tk[None], tv[None], attn_mask=(j <= i) & (j > i - W))[0]
        (o * torch.from_numpy(do.transpose(1, 0, 2).copy())).sum().backward()
        dq, dk, dv = ob.swa_attention_backward(q, k, v, do, W)
        for got, ref in ((dq, tq), (dk, tk), (dv, tv)):
            np.testing.assert_allclose(got, ref.grad.numpy().transpose(1, 0, 2), rtol=1e-10, atol=1e-11)
    q, k, v, do = (rng.standard_normal((20, 2, 8)) for _ in range(4))
    dq, dk, dv = ob.swa_attention_backward(q, k, v, do, 1)
    assert np.abs(dq).max() == 0.0 and np.abs(dk).max() == 0.0
    np.testing.assert_allclose(dv, do, rtol=0, atol=1e-15)


def pin_block_backward_vs_autograd(ob):
    """Whole-block gradients == torch autograd (odd shapes, several W, with and without the
    residual, random gamma/beta)."""
    for seed, (B, S, d, H, hd, ffn), W in ((151, (2, 45, 24, 3, 8, 40), 9),
                                           (152, (1, 70, 32, 2, 16, 48), 70),
                                           (153, (3, 17, 16, 1, 8, 8), 1)):
        x, g, b, wi, wo = _rand_block(seed, B, S, d, H, hd, ffn)
        dy = _rng(seed + 7).standard_normal(x.shape)
        for add_res in (True, False):
            got = ob.block_backward(x, g, b, wi, wo, dy, H, hd, W, eps=1e-5, add_residual=add_res)
            ref = _torch_block_grads(x, g, b, wi, wo, H, hd, W, 1e-5, dy, add_res)
            for key in ref:
                np.testing.assert_allclose(got[key], ref[key], rtol=1e-9, atol=1e-10, err_msg=key)


def pin_block_backward_finite_differences(ob):
    """<gradient, direction> == central difference of sum(dy * block_forward) along random
    directions of each input and parameter (the forward is pinned on its own)."""
    B, S, d, H, hd, ffn, W = 1, 19, 16, 2, 4, 24, 6
    x, g, b, wi, wo = _rand_block(161, B, S, d, H, hd, ffn)
    rng = _rng(162)
    dy = rng.standard_normal(x.shape)
    grads = ob.block_backward(x, g, b, wi, wo, dy, H, hd, W)
    params = dict(x=x, gamma=g, beta=b, w_in=wi, w_out=wo)
    names = dict(x="dx", gamma="dgamma", beta="dbeta", w_in="dw_in", w_out="dw_out")

    def loss(p):
        return float((dy * ob.block_forward(p["x"], p["gamma"], p["beta"], p["w_in"], p["w_out"], H, hd, W)).sum())

    eps = 1e-6
    for name, val in params.items():
        for _ in range(2):
            direction = rng.standard_normal(val.shape)
            plus = dict(params, **{name: val + eps * direction})
            minus = dict(params, **{name: val - eps * direction})
            fd = (loss(plus) - loss(minus)) / (2 * eps)
            an = float((grads[names[name]] * direction).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def pin_block_backward_w1(ob):
    """At W = 1 every token attends to itself only, so the loss does not depend on q or k:
    the W_in rows of Q and K get exactly zero gradient, those of V and FC1 do not."""
    B, S, d, H, hd, ffn = 2, 13, 16, 2, 8, 24
    x, g, b, wi, wo = _rand_block(171, B, S, d, H, hd, ffn)
    dy = _rng(172).standard_normal(x.shape)
    dw_in = ob.block_backward(x, g, b, wi, wo, dy, H, hd, 1)["dw_in"]
    A = H * hd
    assert np.abs(dw_in[:2 * A]).max() == 0.0
    assert np.abs(dw_in[2 * A:3 * A]).min() > 0.0 and np.abs(dw_in[3 * A:]).max() > 1e-3


def pin_relative_error(ob):
    """The parity metric max|y_test - y_ref| / max|y_ref|, on hand-worked values: the
    denominator is the reference's largest magnitude (not the tested array's), the numerator
    the largest elementwise difference (not a mean, not a per-element ratio); swapping the
    arguments changes the value; an all-zero reference gives the absolute error."""
    ref = np.array([[1.0, 2.0], [3.0, -4.0]])
    test = np.array([[1.0, 2.0], [3.0, -4.4]])
    # max |diff| = 0.4 at the reference's largest element, max |ref| = 4
    assert abs(ob.relative_error(test, ref) - 0.1) < 1e-15
    # a difference away from the largest element: 0.25 / 4
    test2 = np.array([[1.25, 2.0], [3.0, -4.0]])
    assert abs(ob.relative_error(test2, ref) - 0.0625) < 1e-15
    # swapped arguments: max |diff| = 4, divided by max |ref| = 2 or by max |test| = 6
    a, b = np.array([1.0, 6.0]), np.array([1.0, 2.0])
    assert abs(ob.relative_error(a, b) - 2.0) < 1e-15
    assert abs(ob.relative_error(b, a) - 4.0 / 6.0) < 1e-15
    # all-zero reference: the absolute error
    assert ob.relative_error(np.array([0.5, -0.75]), np.zeros(2)) == 0.75
    assert ob.relative_error(np.zeros(3), np.zeros(3)) == 0.0
    # equal arrays, any shape: 0; scaling both by c > 0 leaves the value unchanged
    rng = _rng(40)
    x = rng.standard_normal((3, 5, 7))
    y = x + 1e-3 * rng.standard_normal(x.shape)
    assert ob.relative_error(x, x) == 0.0
    r = ob.relative_error(y, x)
    assert abs(ob.relative_error(8.0 * y, 8.0 * x) - r) < 1e-15
    # brute force over the elements in plain Python
    num = max(abs(float(p) - float(q)) for p, q in zip(y.ravel(), x.ravel()))
    den = max(abs(float(q)) for q in x.ravel())
    assert abs(r - num / den) < 1e-15


ALL_PINS = [
    pin_relative_error,
    pin_attention_brute_force,
    pin_attention_vs_torch_band,
    pin_attention_full_causal,
    pin_attention_w1_is_identity,
    pin_attention_two_keys,
    pin_attention_offset_keys,
    pin_layer_norm,
    pin_gelu,
    pin_block_vs_torch,
    pin_block_w1_closed_form,
    pin_block_branch_sum,
    pin_block_tensor_parallel,
    pin_block_locality,
    pin_block_uniform_closed_form,
    pin_rows_match_full,
    pin_serial_vs_torch,
    pin_serial_single_sublayer,
    pin_serial_rows_match_full,
    pin_gelu_tanh,
    pin_rope_hand_values,
    pin_rope_relative_position,
    pin_variant_vs_torch,
    pin_variant_reductions,
    pin_variant_rows_match_full,
    pin_gelu_grad,
    pin_layer_norm_backward,
    pin_attention_backward,
    pin_block_backward_vs_autograd,
    pin_block_backward_finite_differences,
    pin_block_backward_w1,
]
