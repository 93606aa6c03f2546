"""Oracle: a plain fp64 CPU forward of the parallel transformer block with
sliding-window causal attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The library's product path never
calls it, and it shares no code with the HIP path: the only thing both sides
use is the seeded input generator in ``workload``.

What it computes, and where the pages define it (MegaScale guided reading on
the ai-training-network-primer site):
  * section 2 "Changing the model to help the system": the parallel block feeds
    the attention and feed-forward sub-layers from the same input and sums their
    outputs; sliding-window attention lets each token attend only to a fixed
    window of nearby tokens;
  * section 3 "Overlap in all three dimensions" (tensor and sequence
    parallelism): a layer-norm precedes the parallel linear layers, and with
    tensor parallelism each GPU holds a slice of heads and FFN columns whose
    partial outputs are summed by a reduce-scatter;
  * section 4 "Operators, data pipeline, and starting up": attention is exact
    (FlashAttention-2), LayerNorm and GeLU are the named operators.

Readings where the pages are silent (each listed with its reason in the design
notes): one LayerNorm output feeds both branches; biased variance, eps = 1e-5,
affine gamma/beta; exact erf GeLU; window = keys j in [i-W+1, i], W keys
including the query itself, never crossing a sequence; scale 1/sqrt(hd); no
positional encoding, no biases, no dropout; the residual x is added unless the
caller asks for the tensor-parallel partial.

Every array is promoted to float64 on entry; nothing is rounded in between.
Matrix products use numpy's ``@`` (a library routine) and the error function
comes from scipy.  Attention is evaluated per slab of queries against only the
keys that can fall in their windows, with an explicit band mask, so its cost
grows with S*W rather than S^2.

The serial (pre-LayerNorm) layer the parallel block replaces is here too, for
the comparison of the two forms (section 2 contrasts them; section 8's ablation
prices the parallel form); "standard layer" is read as the pre-LN layout.  So
are the alternatives to the silent choices above, as explicit switches of
block_forward_variant: the tanh GeLU, linear biases, rotary position embedding
of q and k (RoFormer), and a second LayerNorm for the MLP branch.  And so is
the backward pass of the block (section 3: what is done in the forward pass is
done in the backward pass too): block_backward, the chain rule through every
step, with the softmax Jacobian written out.

Pins (all in the CPU test-suite): dense brute-force band attention, W >= S vs
torch's causal attention, W = 1 closed form, 2-key closed form, the branch-sum
identity, LayerNorm and GeLU against torch and math.erf, tensor-parallel
decomposition, locality, and hand-derived closed-form blocks; the serial layer
against torch library routines and, with one sub-layer switched off, against
the parallel block; the variant switches against torch library routines
(layer_norm, linear with bias, tanh gelu) with the rotation done as complex
multiplication, RoPE's dependence on relative position only, hand-computed
rotations, and reduction to block_forward with every switch off; the backward
pass against torch autograd in float64, central finite differences, the zero
gradient of q and k at W = 1, LayerNorm's shift and scale invariance, and the
GeLU derivative against torch.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf


def layer_norm(x, gamma, beta, eps: float):
    """LayerNorm over the last axis: (x - mean) / sqrt(biased var + eps) * gamma + beta."""
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * np.asarray(gamma, np.float64) + np.asarray(beta, np.float64)


def gelu(z):
    """Exact GeLU: z * Phi(z) = z/2 * (1 + erf(z / sqrt(2)))."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def window_lo(i: int, W: int) -> int:
    """First key position query i may attend to (inclusive); the last is i."""
    return max(0, i - W + 1)


def swa_attention(q, k, v, W: int, q_pos0: int = 0, k_pos0: int = 0, slab: int = 128):
    """Sliding-window causal softmax attention for one sequence.

    q: [Sq, H, hd] holding positions q_pos0 .. q_pos0+Sq-1.
    k, v: [Sk, H, hd] holding positions k_pos0 .. k_pos0+Sk-1; they must cover
    every key the queries' windows reach.
    Query at position i attends to keys j with i-W+1 <= j <= i; scores are
    q_i . k_j / sqrt(hd) and the weights are their softmax over the window.
    Returns [Sq, H, hd].
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Sq, H, hd = q.shape
    out = np.zeros_like(q)
    scale = 1.0 / math.sqrt(hd)
    for s0 in range(0, Sq, slab):
        s1 = min(Sq, s0 + slab)
        i0, i1 = q_pos0 + s0, q_pos0 + s1 - 1  # absolute query positions in the slab
        j0 = window_lo(i0, W)
        j1 = i1
        if j0 < k_pos0 or j1 >= k_pos0 + k.shape[0]:
            raise ValueError("keys do not cover the queries' windows")
        kk = k[j0 - k_pos0:j1 - k_pos0 + 1]  # [L, H, hd]
        vv = v[j0 - k_pos0:j1 - k_pos0 + 1]
        qi = np.arange(i0, i1 + 1)[:, None]
        kj = np.arange(j0, j1 + 1)[None, :]
        allowed = (kj <= qi) & (kj >= qi - W + 1)  # [slab, L]
        qs = q[s0:s1].transpose(1, 0, 2)  # [H, slab, hd]
        scores = (qs @ kk.transpose(1, 2, 0)) * scale  # [H, slab, L]
        scores = np.where(allowed[None], scores, -np.inf)
        m = scores.max(axis=-1, keepdims=True)
        p = np.exp(scores - m)
        p /= p.sum(axis=-1, keepdims=True)
        out[s0:s1] = (p @ vv.transpose(1, 0, 2)).transpose(1, 0, 2)
    return out


def split_projection(z, H: int, hd: int):
    """Split u @ W_in^T into Q, K, V (each [..., H, hd]) and the FC1 pre-activation."""
    A = H * hd
    lead = z.shape[:-1]
    q = z[..., 0:A].reshape(*lead, H, hd)
    k = z[..., A:2 * A].reshape(*lead, H, hd)
    v = z[..., 2 * A:3 * A].reshape(*lead, H, hd)
    f = z[..., 3 * A:]
    return q, k, v, f


def block_forward(x, gamma, beta, w_in, w_out, H: int, hd: int, W: int,
                  eps: float = 1e-5, add_residual: bool = True, return_parts: bool = False):
    """y = [x +] ( Attn_SWA(LN x) || GeLU(LN x W_fc1^T) ) W_out^T for x [B, S, d].

    The attention heads and the GeLU activations sit side by side and go
    through one output projection, which is the sum of the attention
    out-projection and FC2 (W_out's columns are [heads ; FC2]).
    """
    x = np.asarray(x, np.float64)
    w_in = np.asarray(w_in, np.float64)
    w_out = np.asarray(w_out, np.float64)
    B, S, d = x.shape
    A = H * hd
    u = layer_norm(x, gamma, beta, eps)
    z = u @ w_in.T
    q, k, v, f = split_projection(z, H, hd)
    o = np.empty((B, S, H, hd))
    for b in range(B):
        o[b] = swa_attention(q[b], k[b], v[b], W)
    g = gelu(f)
    ag = np.concatenate([o.reshape(B, S, A), g], axis=-1)
    y = ag @ w_out.T
    if add_residual:
        y = y + x
    if return_parts:
        return y, dict(u=u, qkv=z[..., :3 * A], ag=ag)
    return y


def block_forward_rows(x, gamma, beta, w_in, w_out, H: int, hd: int, W: int, row_blocks,
                       eps: float = 1e-5, add_residual: bool = True):
    """Output rows y[b, i0:i1] for each (b, i0, i1) in ``row_blocks``.

    Only the LayerNorm rows, projections and keys those queries need are
    formed (keys i0-W+1 .. i1-1), so full-size workloads can be checked on
    samples.  Returns a list of [i1-i0, d] arrays.
    """
    w_in = np.asarray(w_in, np.float64)
    w_out = np.asarray(w_out, np.float64)
    A = H * hd
    outs = []
    for b, i0, i1 in row_blocks:
        j0 = window_lo(i0, W)
        xs = np.asarray(x[b, j0:i1], np.float64)
        u = layer_norm(xs, gamma, beta, eps)
        z_kv = u @ w_in[A:3 * A].T
        k = z_kv[:, :A].reshape(-1, H, hd)
        v = z_kv[:, A:].reshape(-1, H, hd)
        uq = u[i0 - j0:]
        q = (uq @ w_in[:A].T).reshape(-1, H, hd)
        f = uq @ w_in[3 * A:].T
        o = swa_attention(q, k, v, W, q_pos0=i0, k_pos0=j0)
        ag = np.concatenate([o.reshape(-1, A), gelu(f)], axis=-1)
        y = ag @ w_out.T
        if add_residual:
            y = y + xs[i0 - j0:]
        outs.append(y)
    return outs


def serial_block_forward(x, gamma, beta, gamma2, beta2, w_in, w_out, H: int, hd: int, W: int,
                         eps: float = 1e-5):
    """The standard (serial) layer the parallel block replaces, in pre-LayerNorm form
    (MegaScale guided reading, section 2: the usual layer is sequential, its
    feed-forward part taking the attention part's result as input):

        h = x + Attn_SWA(LN1 x) W_o^T
        y = h + GeLU(LN2(h) W_1^T) W_2^T

    with the same packed matrices as block_forward: W_in rows [Q; K; V; W_1], W_out
    columns [W_o ; W_2].  LN1 = (gamma, beta), LN2 = (gamma2, beta2).
    """
    x = np.asarray(x, np.float64)
    w_in = np.asarray(w_in, np.float64)
    w_out = np.asarray(w_out, np.float64)
    B, S, d = x.shape
    A = H * hd
    u1 = layer_norm(x, gamma, beta, eps)
    q, k, v, _ = split_projection(u1 @ w_in[:3 * A].T, H, hd)
    o = np.empty((B, S, H, hd))
    for b in range(B):
        o[b] = swa_attention(q[b], k[b], v[b], W)
    h = x + o.reshape(B, S, A) @ w_out[:, :A].T
    u2 = layer_norm(h, gamma2, beta2, eps)
    return h + gelu(u2 @ w_in[3 * A:].T) @ w_out[:, A:].T


def serial_block_forward_rows(x, gamma, beta, gamma2, beta2, w_in, w_out, H: int, hd: int, W: int,
                              row_blocks, eps: float = 1e-5):
    """Output rows y[b, i0:i1] of serial_block_forward for each (b, i0, i1) in
    ``row_blocks``, forming only the keys those queries reach.  Returns a list of
    [i1-i0, d] arrays."""
    w_in = np.asarray(w_in, np.float64)
    w_out = np.asarray(w_out, np.float64)
    A = H * hd
    outs = []
    for b, i0, i1 in row_blocks:
        j0 = window_lo(i0, W)
        xs = np.asarray(x[b, j0:i1], np.float64)
        u1 = layer_norm(xs, gamma, beta, eps)
        z_kv = u1 @ w_in[A:3 * A].T
        k = z_kv[:, :A].reshape(-1, H, hd)
        v = z_kv[:, A:].reshape(-1, H, hd)
        q = (u1[i0 - j0:] @ w_in[:A].T).reshape(-1, H, hd)
        o = swa_attention(q, k, v, W, q_pos0=i0, k_pos0=j0)
        h = xs[i0 - j0:] + o.reshape(-1, A) @ w_out[:, :A].T
        u2 = layer_norm(h, gamma2, beta2, eps)
        outs.append(h + gelu(u2 @ w_in[3 * A:].T) @ w_out[:, A:].T)
    return outs


# ----------------------------------------------------------------------------- backward pass
# The pages' context is training (section 3 carries the forward's scheme over to the backward): the
# gradients of the block's loss with respect to its input and parameters, given the gradient
# dy of its output, by the chain rule through each step of block_forward.


def gelu_grad(z):
    """d/dz of the exact GeLU z * Phi(z): Phi(z) + z * phi(z), phi the standard normal density."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * (1.0 + erf(z / math.sqrt(2.0))) + z * np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def swa_attention_backward(q, k, v, do, W: int, slab: int = 128):
    """Gradients of swa_attention(q, k, v, W) for one sequence given the output gradient do.

    With s_ij = q_i.k_j / sqrt(hd) on the band and p_i = softmax(s_i): dp_ij = do_i.v_j,
    ds_ij = p_ij (dp_ij - sum_l p_il dp_il) (the softmax Jacobian), dq_i = sum_j ds_ij k_j /
    sqrt(hd), dk_j = sum_i ds_ij q_i / sqrt(hd), dv_j = sum_i p_ij do_i.  Returns dq, dk, dv,
    each [S, H, hd]; slabs of queries meet only the keys their windows reach.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    S, H, hd = q.shape
    scale = 1.0 / math.sqrt(hd)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for s0 in range(0, S, slab):
        s1 = min(S, s0 + slab)
        j0 = window_lo(s0, W)
        j1 = s1 - 1
        qi = np.arange(s0, s1)[:, None]
        kj = np.arange(j0, j1 + 1)[None, :]
        allowed = (kj <= qi) & (kj >= qi - W + 1)
        qs = q[s0:s1].transpose(1, 0, 2)  # [H, n, hd]
        kk = k[j0:j1 + 1].transpose(1, 0, 2)  # [H, L, hd]
        vv = v[j0:j1 + 1].transpose(1, 0, 2)
        dos = do[s0:s1].transpose(1, 0, 2)
        scores = np.where(allowed[None], (qs @ kk.transpose(0, 2, 1)) * scale, -np.inf)
        p = np.exp(scores - scores.max(axis=-1, keepdims=True))
        p /= p.sum(axis=-1, keepdims=True)  # [H, n, L], zero outside the band
        dp = dos @ vv.transpose(0, 2, 1)
        ds = p * (dp - (p * dp).sum(axis=-1, keepdims=True))
        dq[s0:s1] += (ds @ kk).transpose(1, 0, 2) * scale
        dk[j0:j1 + 1] += (ds.transpose(0, 2, 1) @ qs).transpose(1, 0, 2) * scale
        dv[j0:j1 + 1] += (p.transpose(0, 2, 1) @ dos).transpose(1, 0, 2)
    return dq, dk, dv


def layer_norm_backward(x, gamma, du, eps: float):
    """Gradients of u = (x - mu) / sigma * gamma + beta (sigma = sqrt(biased var + eps)) over
    the last axis: dx = (g - mean(g) - xhat * mean(g * xhat)) / sigma with g = du * gamma,
    dgamma = sum(du * xhat), dbeta = sum(du) over all rows."""
    x = np.asarray(x, np.float64)
    du = np.asarray(du, np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    sigma = np.sqrt(((x - mu) ** 2).mean(axis=-1, keepdims=True) + eps)
    xhat = (x - mu) / sigma
    g = du * np.asarray(gamma, np.float64)
    dx = (g - g.mean(axis=-1, keepdims=True) - xhat * (g * xhat).mean(axis=-1, keepdims=True)) / sigma
    lead = tuple(range(du.ndim - 1))
    return dx, (du * xhat).sum(axis=lead), du.sum(axis=lead)


def block_backward(x, gamma, beta, w_in, w_out, dy, H: int, hd: int, W: int, eps: float = 1e-5,
                   add_residual: bool = True):
    """Gradients of block_forward with respect to x, gamma, beta, W_in and W_out given dy
    [B, S, d].  Returns a dict with dx [B, S, d], dgamma [d], dbeta [d], dw_in
    [3A + ffn, d], dw_out [d, A + ffn]."""
    x = np.asarray(x, np.float64)
    w_in = np.asarray(w_in, np.float64)
    w_out = np.asarray(w_out, np.float64)
    dy = np.asarray(dy, np.float64)
    B, S, d = x.shape
    A = H * hd
    # forward, keeping what the chain rule needs
    u = layer_norm(x, gamma, beta, eps)
    z = u @ w_in.T
    q, k, v, f = split_projection(z, H, hd)
    o = np.empty((B, S, H, hd))
    for b in range(B):
        o[b] = swa_attention(q[b], k[b], v[b], W)
    ag = np.concatenate([o.reshape(B, S, A), gelu(f)], axis=-1)
    # y = ag W_out^T (+ x)
    dw_out = dy.reshape(-1, d).T @ ag.reshape(-1, ag.shape[-1])
    dag = dy @ w_out
    do = dag[..., :A].reshape(B, S, H, hd)
    df = dag[..., A:] * gelu_grad(f)
    dz = np.empty_like(z)
    for b in range(B):
        dq, dk, dv = swa_attention_backward(q[b], k[b], v[b], do[b], W)
        dz[b, :, 0:A] = dq.reshape(S, A)
        dz[b, :, A:2 * A] = dk.reshape(S, A)
        dz[b, :, 2 * A:3 * A] = dv.reshape(S, A)
    dz[..., 3 * A:] = df
    dw_in = dz.reshape(-1, z.shape[-1]).T @ u.reshape(-1, d)
    du = dz @ w_in
    dx, dgamma, dbeta = layer_norm_backward(x, gamma, du, eps)
    if add_residual:
        dx = dx + dy
    return dict(dx=dx, dgamma=dgamma, dbeta=dbeta, dw_in=dw_in, dw_out=dw_out)


# ----------------------------------------------------------------------------- variant knobs
# The pages leave several choices open (no positional encoding, bias or GeLU form is named,
# and "the same input" could be one LayerNorm or one per branch).  The functions below add
# each alternative as an explicit switch; with every switch off they reduce to
# block_forward.


def gelu_tanh(z):
    """GeLU's tanh approximation (Hendrycks and Gimpel, "Gaussian Error Linear Units",
    section 2): z/2 * (1 + tanh(sqrt(2/pi) * (z + 0.044715 z^3)))."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def rope(t, positions, base: float):
    """Rotary position embedding (RoFormer, Su et al., section 3): in every head vector of
    hd features, the pair (t[2i], t[2i+1]) at position p is rotated by the angle
    p * base^(-2i/hd), i = 0 .. hd/2 - 1.

    t: [n, H, hd] for the positions in ``positions`` (length n).  Returns a new array.
    """
    t = np.asarray(t, np.float64)
    hd = t.shape[-1]
    theta = float(base) ** (-2.0 * np.arange(hd // 2) / hd)  # [hd/2]
    ang = np.asarray(positions, np.float64)[:, None] * theta[None, :]  # [n, hd/2]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    even, odd = t[..., 0::2], t[..., 1::2]
    out = np.empty_like(t)
    out[..., 0::2] = even * c - odd * s
    out[..., 1::2] = even * s + odd * c
    return out


def _variant_rows(xs, pos0, q_from, gamma, beta, w_in, w_out, H, hd, W, eps, add_residual, gelu_form, b_in,
                  b_out, rope_base, gamma2, beta2):
    """Output rows q_from.. of one sequence slice xs (positions pos0 .. pos0+len-1), whose
    first rows supply the keys the later queries reach."""
    A = H * hd
    u_attn = layer_norm(xs, gamma, beta, eps)
    u_mlp = u_attn if gamma2 is None else layer_norm(xs, gamma2, beta2, eps)
    z = u_attn @ w_in[:3 * A].T
    f = u_mlp[q_from:] @ w_in[3 * A:].T
    if b_in is not None:
        z = z + b_in[:3 * A]
        f = f + b_in[3 * A:]
    q, k, v, _ = split_projection(z, H, hd)
    if rope_base is not None:
        pos = pos0 + np.arange(xs.shape[0])
        q = rope(q, pos, rope_base)
        k = rope(k, pos, rope_base)
    o = swa_attention(q[q_from:], k, v, W, q_pos0=pos0 + q_from, k_pos0=pos0)
    act = gelu(f) if gelu_form == "erf" else gelu_tanh(f)
    y = np.concatenate([o.reshape(-1, A), act], axis=-1) @ w_out.T
    if b_out is not None:
        y = y + b_out
    if add_residual:
        y = y + xs[q_from:]
    return y


def _check_gelu_form(gelu_form):
    if gelu_form not in ("erf", "tanh"):
        raise ValueError("gelu_form must be 'erf' or 'tanh'")


def block_forward_variant(x, gamma, beta, w_in, w_out, H: int, hd: int, W: int, eps: float = 1e-5,
                          add_residual: bool = True, gelu_form: str = "erf", b_in=None, b_out=None,
                          rope_base=None, gamma2=None, beta2=None):
    """The parallel block with the open choices as switches:

        ua = LN(x; gamma, beta);  um = ua, or LN(x; gamma2, beta2) with a second LayerNorm
        [q | k | v] = ua W_qkv^T (+ b_in[:3A]);  f = um W_1^T (+ b_in[3A:])
        q, k rotated by their position (rope_base given), positions 0 .. S-1 per sequence
        y = [Attn_SWA(q, k, v) | act(f)] W_out^T (+ b_out) (+ x),  act = exact or tanh GeLU.
    """
    _check_gelu_form(gelu_form)
    x = np.asarray(x, np.float64)
    w_in = np.asarray(w_in, np.float64)
    w_out = np.asarray(w_out, np.float64)
    b_in = None if b_in is None else np.asarray(b_in, np.float64)
    b_out = None if b_out is None else np.asarray(b_out, np.float64)
    B, S, d = x.shape
    y = np.empty((B, S, d))
    for b in range(B):
        y[b] = _variant_rows(x[b], 0, 0, gamma, beta, w_in, w_out, H, hd, W, eps, add_residual, gelu_form, b_in,
                             b_out, rope_base, gamma2, beta2)
    return y


def block_forward_variant_rows(x, gamma, beta, w_in, w_out, H: int, hd: int, W: int, row_blocks,
                               eps: float = 1e-5, add_residual: bool = True, gelu_form: str = "erf", b_in=None,
                               b_out=None, rope_base=None, gamma2=None, beta2=None):
    """Output rows y[b, i0:i1] of block_forward_variant for each (b, i0, i1) in
    ``row_blocks``, forming only the keys those queries reach (positions i0-W+1 ..)."""
    _check_gelu_form(gelu_form)
    w_in = np.asarray(w_in, np.float64)
    w_out = np.asarray(w_out, np.float64)
    b_in = None if b_in is None else np.asarray(b_in, np.float64)
    b_out = None if b_out is None else np.asarray(b_out, np.float64)
    outs = []
    for b, i0, i1 in row_blocks:
        j0 = window_lo(i0, W)
        xs = np.asarray(x[b, j0:i1], np.float64)
        outs.append(_variant_rows(xs, j0, i0 - j0, gamma, beta, w_in, w_out, H, hd, W, eps, add_residual,
                                  gelu_form, b_in, b_out, rope_base, gamma2, beta2))
    return outs


def relative_error(y_test, y_ref) -> float:
    """max |y_test - y_ref| / max |y_ref| (the parity metric)."""
    y_test = np.asarray(y_test, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    denom = np.abs(y_ref).max()
    return float(np.abs(y_test - y_ref).max() / denom) if denom > 0 else float(np.abs(y_test).max())
