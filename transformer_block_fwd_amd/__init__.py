"""Python binding of the pblock C ABI (include/pblock.h).

Forward pass of one parallel transformer block with sliding-window causal
attention on an MI355X (gfx950):

    y = [x +] Attn_SWA(LN(x)) + MLP(LN(x))

Every step runs in the HIP library; this module only marshals arguments
(torch tensors -> device pointers, the current torch stream -> hipStream_t)
and turns error codes into exceptions.  Function names mirror the C ABI.
"""
from __future__ import annotations

import ctypes

from . import _abi
from ._abi import (  # noqa: F401
    PBLOCK_BF16,
    PBLOCK_F32,
    PblockCfg,
    PblockError,
    PblockGrads,
    PblockVariant,
    PblockVariantWeights,
    PblockWeights,
)

__all__ = [
    "PBLOCK_BF16", "PBLOCK_F32", "PblockCfg", "PblockError", "PblockWeights", "ParallelBlock", "make_cfg",
    "pblock_validate_cfg", "pblock_workspace_bytes", "pblock_flops", "pblock_create", "pblock_forward",
    "pblock_destroy", "pblock_intermediates", "pblock_copy_intermediates", "pblock_set_timing",
    "pblock_kernel_times", "pblock_swa_attention", "pblock_strerror", "pblock_last_error", "KERNEL_NAMES",
    "PblockVariant", "PblockVariantWeights", "make_variant", "pblock_forward_variant",
    "PblockGrads", "pblock_train_workspace_bytes", "pblock_forward_train", "pblock_backward",
    "pblock_forward_serial", "pblock_forward_chunked", "pblock_mfma_loop", "as_cfg", "BACKWARD_KERNEL_NAMES",
    "pblock_activation", "ACTIVATION_FORMS", "pblock_forward_static", "pblock_forward_rowchunks",
    "pblock_pack_chunks", "MFMA_FORMS",
]

KERNEL_NAMES = ("layernorm", "gemm_in", "attention", "gemm_out")
BACKWARD_KERNEL_NAMES = ("bwd_prep", "bwd_gemm_dgrad", "bwd_attention", "bwd_gemm_wgrad", "bwd_layernorm")

_DTYPES = {"bf16": PBLOCK_BF16, "f32": PBLOCK_F32, PBLOCK_BF16: PBLOCK_BF16, PBLOCK_F32: PBLOCK_F32}


def make_cfg(B, S, d, H, hd, ffn, W, dtype="bf16", add_residual=1, ln_eps=1e-5) -> PblockCfg:
    return PblockCfg(int(B), int(S), int(d), int(H), int(hd), int(ffn), int(W), _DTYPES[dtype],
                     int(add_residual), float(ln_eps))


def as_cfg(cfg) -> PblockCfg:
    """A PblockCfg, or any object with B, S, d, H, hd, ffn, W, dtype (and
    optionally add_residual, ln_eps) attributes."""
    if isinstance(cfg, PblockCfg):
        return cfg
    return make_cfg(cfg.B, cfg.S, cfg.d, cfg.H, cfg.hd, cfg.ffn, cfg.W, cfg.dtype,
                    getattr(cfg, "add_residual", 1), getattr(cfg, "ln_eps", 1e-5))


def _ptr(t) -> int:
    """Device pointer of a torch tensor (must be contiguous and on a GPU) or an int."""
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _check_tensor(t, name, dtype_code, numel):
    if t is None or isinstance(t, int):
        return
    import torch

    want = torch.bfloat16 if dtype_code == PBLOCK_BF16 else torch.float32
    if t.dtype != want:
        raise TypeError(f"{name} must be {want}, got {t.dtype}")
    if t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")


def _stream(stream) -> int:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def pblock_strerror(code: int) -> str:
    return _abi.lib().pblock_strerror(int(code)).decode()


def pblock_last_error() -> str:
    return _abi.last_error()


def pblock_validate_cfg(cfg) -> int:
    c = as_cfg(cfg)
    return _abi.lib().pblock_validate_cfg(ctypes.byref(c))


def pblock_workspace_bytes(cfg) -> int:
    c = as_cfg(cfg)
    v = _abi.lib().pblock_workspace_bytes(ctypes.byref(c))
    _abi.check(v if v < 0 else 0, "pblock_workspace_bytes")
    return v


def pblock_flops(cfg) -> float:
    c = as_cfg(cfg)
    return _abi.lib().pblock_flops(ctypes.byref(c))


def pblock_create(cfg) -> int:
    c = as_cfg(cfg)
    h = ctypes.c_void_p()
    _abi.check(_abi.lib().pblock_create(ctypes.byref(c), ctypes.byref(h)), "pblock_create")
    return h.value


def pblock_destroy(handle: int) -> None:
    _abi.check(_abi.lib().pblock_destroy(ctypes.c_void_p(handle)), "pblock_destroy")


def pblock_forward(handle: int, x, weights, cfg, out, stream=None) -> None:
    """weights = (ln_gamma, ln_beta, w_in, w_out); all tensors contiguous on the GPU."""
    c = as_cfg(cfg)
    gamma, beta, w_in, w_out = weights
    M, A = c.B * c.S, c.H * c.hd
    for t, name, n in ((x, "x", M * c.d), (out, "out", M * c.d), (gamma, "ln_gamma", c.d), (beta, "ln_beta", c.d),
                       (w_in, "w_in", (3 * A + c.ffn) * c.d), (w_out, "w_out", c.d * (A + c.ffn))):
        _check_tensor(t, name, c.dtype, n)
    w = PblockWeights(_ptr(gamma), _ptr(beta), _ptr(w_in), _ptr(w_out))
    _abi.check(_abi.lib().pblock_forward(ctypes.c_void_p(handle), _ptr(x), ctypes.byref(w), ctypes.byref(c),
                                         _ptr(out), _stream(stream)), "pblock_forward")


def pblock_forward_static(x, weights, cfg, out, stream=None) -> None:
    """pblock_forward with the library's static device workspace: no handle, no allocation."""
    c = as_cfg(cfg)
    gamma, beta, w_in, w_out = weights
    M, A = c.B * c.S, c.H * c.hd
    for t, name, n in ((x, "x", M * c.d), (out, "out", M * c.d), (gamma, "ln_gamma", c.d), (beta, "ln_beta", c.d),
                       (w_in, "w_in", (3 * A + c.ffn) * c.d), (w_out, "w_out", c.d * (A + c.ffn))):
        _check_tensor(t, name, c.dtype, n)
    w = PblockWeights(_ptr(gamma), _ptr(beta), _ptr(w_in), _ptr(w_out))
    _abi.check(_abi.lib().pblock_forward_static(_ptr(x), ctypes.byref(w), ctypes.byref(c), _ptr(out), _stream(stream)),
               "pblock_forward_static")


def pblock_forward_serial(handle: int, x, weights, ln2, cfg, out, stream=None) -> None:
    """The serial (pre-LN) layer from the same kernels: weights = (ln_gamma, ln_beta, w_in, w_out) as for
    pblock_forward, ln2 = (ln2_gamma, ln2_beta)."""
    c = as_cfg(cfg)
    gamma, beta, w_in, w_out = weights
    gamma2, beta2 = ln2
    M, A = c.B * c.S, c.H * c.hd
    for t, name, n in ((x, "x", M * c.d), (out, "out", M * c.d), (gamma, "ln_gamma", c.d), (beta, "ln_beta", c.d),
                       (gamma2, "ln2_gamma", c.d), (beta2, "ln2_beta", c.d),
                       (w_in, "w_in", (3 * A + c.ffn) * c.d), (w_out, "w_out", c.d * (A + c.ffn))):
        _check_tensor(t, name, c.dtype, n)
    w = PblockWeights(_ptr(gamma), _ptr(beta), _ptr(w_in), _ptr(w_out))
    _abi.check(_abi.lib().pblock_forward_serial(ctypes.c_void_p(handle), _ptr(x), ctypes.byref(w), _ptr(gamma2),
                                                _ptr(beta2), ctypes.byref(c), _ptr(out), _stream(stream)),
               "pblock_forward_serial")


def make_variant(gelu_tanh=False, rope=False, rope_base=10000.0, two_ln=False) -> PblockVariant:
    return PblockVariant(int(bool(gelu_tanh)), int(bool(rope)), float(rope_base), int(bool(two_ln)))


def pblock_forward_variant(handle: int, x, weights, extra, cfg, variant, out, stream=None) -> None:
    """The parallel block with the variant switches: weights = (ln_gamma, ln_beta, w_in, w_out),
    extra = dict with any of b_in [3A+ffn], b_out [d], ln2_gamma [d], ln2_beta [d] (or None),
    variant = a PblockVariant (see make_variant)."""
    c = as_cfg(cfg)
    gamma, beta, w_in, w_out = weights
    extra = extra or {}
    M, A = c.B * c.S, c.H * c.hd
    for t, name, n in ((x, "x", M * c.d), (out, "out", M * c.d), (gamma, "ln_gamma", c.d), (beta, "ln_beta", c.d),
                       (w_in, "w_in", (3 * A + c.ffn) * c.d), (w_out, "w_out", c.d * (A + c.ffn)),
                       (extra.get("b_in"), "b_in", 3 * A + c.ffn), (extra.get("b_out"), "b_out", c.d),
                       (extra.get("ln2_gamma"), "ln2_gamma", c.d), (extra.get("ln2_beta"), "ln2_beta", c.d)):
        _check_tensor(t, name, c.dtype, n)
    if not isinstance(variant, PblockVariant):
        raise TypeError("variant must be a PblockVariant (make_variant)")
    w = PblockWeights(_ptr(gamma), _ptr(beta), _ptr(w_in), _ptr(w_out))
    vw = PblockVariantWeights(_ptr(extra.get("b_in")), _ptr(extra.get("b_out")), _ptr(extra.get("ln2_gamma")),
                              _ptr(extra.get("ln2_beta")))
    _abi.check(_abi.lib().pblock_forward_variant(ctypes.c_void_p(handle), _ptr(x), ctypes.byref(w), ctypes.byref(vw),
                                                 ctypes.byref(c), ctypes.byref(variant), _ptr(out), _stream(stream)),
               "pblock_forward_variant")


def pblock_train_workspace_bytes(cfg) -> int:
    c = as_cfg(cfg)
    v = _abi.lib().pblock_train_workspace_bytes(ctypes.byref(c))
    _abi.check(v if v < 0 else 0, "pblock_train_workspace_bytes")
    return v


def _check_weights(c, x, weights, extra=()):
    gamma, beta, w_in, w_out = weights
    M, A = c.B * c.S, c.H * c.hd
    for t, name, n in ((x, "x", M * c.d), (gamma, "ln_gamma", c.d), (beta, "ln_beta", c.d),
                       (w_in, "w_in", (3 * A + c.ffn) * c.d), (w_out, "w_out", c.d * (A + c.ffn))) + tuple(extra):
        _check_tensor(t, name, c.dtype, n)
    return PblockWeights(_ptr(gamma), _ptr(beta), _ptr(w_in), _ptr(w_out))


def pblock_forward_train(handle: int, x, weights, cfg, out, ws, stream=None) -> None:
    """pblock_forward plus the activations the backward needs, saved in ws (a device tensor of at
    least pblock_train_workspace_bytes(cfg) bytes, 256-byte aligned)."""
    c = as_cfg(cfg)
    w = _check_weights(c, x, weights, ((out, "out", c.B * c.S * c.d),))
    nbytes = ws.numel() * ws.element_size()
    _abi.check(_abi.lib().pblock_forward_train(ctypes.c_void_p(handle), _ptr(x), ctypes.byref(w), ctypes.byref(c),
                                               _ptr(out), _ptr(ws), nbytes, _stream(stream)),
               "pblock_forward_train")


def pblock_backward(handle: int, x, weights, cfg, dy, grads, ws, stream=None) -> None:
    """Gradients for dy of the forward saved in ws: grads = dict(dx, dln_gamma, dln_beta, dw_in, dw_out)
    of device tensors shaped like x, ln_gamma, ln_beta, w_in, w_out."""
    c = as_cfg(cfg)
    M, A = c.B * c.S, c.H * c.hd
    w = _check_weights(c, x, weights, (
        (dy, "dy", M * c.d), (grads["dx"], "dx", M * c.d), (grads["dln_gamma"], "dln_gamma", c.d),
        (grads["dln_beta"], "dln_beta", c.d), (grads["dw_in"], "dw_in", (3 * A + c.ffn) * c.d),
        (grads["dw_out"], "dw_out", c.d * (A + c.ffn))))
    g = PblockGrads(_ptr(grads["dx"]), _ptr(grads["dln_gamma"]), _ptr(grads["dln_beta"]), _ptr(grads["dw_in"]),
                    _ptr(grads["dw_out"]))
    nbytes = ws.numel() * ws.element_size()
    _abi.check(_abi.lib().pblock_backward(ctypes.c_void_p(handle), _ptr(x), ctypes.byref(w), ctypes.byref(c),
                                          _ptr(dy), ctypes.byref(g), _ptr(ws), nbytes, _stream(stream)),
               "pblock_backward")


def _event_array(events, n, stream):
    """ctypes array of hipEvent_t handles for torch.cuda.Event objects (None entries stay NULL)."""
    if events is None:
        return None
    if len(events) != n:
        raise ValueError(f"expected {n} events, got {len(events)}")
    arr = (ctypes.c_void_p * n)()
    for i, e in enumerate(events):
        if e is None:
            continue
        if not e.cuda_event:  # torch creates the underlying event at its first record
            e.record()
        arr[i] = e.cuda_event
    return arr


def pblock_forward_chunked(handle: int, x, weights, cfg, out, n_chunks: int, ready_events=None, done_events=None,
                           stream=None) -> None:
    """The block in n_chunks position chunks; ready_events / done_events: lists of torch.cuda.Event (or None)
    waited on before / recorded after each chunk."""
    c = as_cfg(cfg)
    gamma, beta, w_in, w_out = weights
    M, A = c.B * c.S, c.H * c.hd
    for t, name, n in ((x, "x", M * c.d), (out, "out", M * c.d), (gamma, "ln_gamma", c.d), (beta, "ln_beta", c.d),
                       (w_in, "w_in", (3 * A + c.ffn) * c.d), (w_out, "w_out", c.d * (A + c.ffn))):
        _check_tensor(t, name, c.dtype, n)
    w = PblockWeights(_ptr(gamma), _ptr(beta), _ptr(w_in), _ptr(w_out))
    ready = _event_array(ready_events, n_chunks, stream)
    done = _event_array(done_events, n_chunks, stream)
    _abi.check(_abi.lib().pblock_forward_chunked(ctypes.c_void_p(handle), _ptr(x), ctypes.byref(w), ctypes.byref(c),
                                                 _ptr(out), int(n_chunks), ready, done, _stream(stream)),
               "pblock_forward_chunked")


def pblock_forward_rowchunks(handle: int, x, weights, cfg, out, n_chunks: int, flags, epoch: int,
                             stream=None) -> None:
    """The forward with its output published chunk by chunk: flags (int32/uint32 GPU tensor of
    n_chunks) gets epoch at chunk k's entry once its rows of out are final."""
    c = as_cfg(cfg)
    gamma, beta, w_in, w_out = weights
    M, A = c.B * c.S, c.H * c.hd
    for t, name, n in ((x, "x", M * c.d), (out, "out", M * c.d), (gamma, "ln_gamma", c.d), (beta, "ln_beta", c.d),
                       (w_in, "w_in", (3 * A + c.ffn) * c.d), (w_out, "w_out", c.d * (A + c.ffn))):
        _check_tensor(t, name, c.dtype, n)
    _check_words(flags, "flags", 4, n_chunks)
    w = PblockWeights(_ptr(gamma), _ptr(beta), _ptr(w_in), _ptr(w_out))
    _abi.check(_abi.lib().pblock_forward_rowchunks(ctypes.c_void_p(handle), _ptr(x), ctypes.byref(w), ctypes.byref(c),
                                                   _ptr(out), int(n_chunks), _ptr(flags), int(epoch),
                                                   _stream(stream)), "pblock_forward_rowchunks")


def pblock_pack_chunks(out, cfg, n_chunks: int, flags, epoch: int, send, stamps, stream=None) -> None:
    """Copies each published chunk of out into its piece of send (see the header); stamps is an
    int64/uint64 GPU tensor of n_chunks receiving the device clock at each publication."""
    c = as_cfg(cfg)
    n = c.B * c.S * c.d
    for t, name in ((out, "out"), (send, "send")):
        _check_tensor(t, name, c.dtype, n)
    _check_words(flags, "flags", 4, n_chunks)
    _check_words(stamps, "stamps", 8, n_chunks)
    _abi.check(_abi.lib().pblock_pack_chunks(_ptr(out), ctypes.byref(c), int(n_chunks), _ptr(flags), int(epoch),
                                             _ptr(send), _ptr(stamps), _stream(stream)), "pblock_pack_chunks")


def _check_words(t, name, itemsize, n):
    if not t.is_cuda or not t.is_contiguous() or t.dtype.itemsize != itemsize or t.numel() < n:
        raise ValueError(f"{name} must be a contiguous GPU tensor of {itemsize}-byte words with >= {n} elements")


MFMA_FORMS = {"16x16x32": _abi.PBLOCK_MFMA_16X16X32, "32x32x16": _abi.PBLOCK_MFMA_32X32X16}


def pblock_mfma_loop(workgroups: int, iterations: int, sink, stream=None, form: str = "16x16x32") -> None:
    """Measurement aid: register-only bf16 MFMA loop, workgroups * 4 * iterations * 16 * 32768 FLOP, of
    the GEMMs' 16x16x32 instruction or of the 32x32x16 one (form); sink is a float32 GPU tensor of at
    least workgroups * 256 elements."""
    if sink.dtype.itemsize != 4 or sink.numel() < workgroups * 256 or not sink.is_cuda:
        raise ValueError("sink must be a float32 GPU tensor of at least workgroups * 256 elements")
    if form not in MFMA_FORMS:
        raise ValueError(f"form must be one of {sorted(MFMA_FORMS)}")
    _abi.check(_abi.lib().pblock_mfma_loop(int(workgroups), int(iterations), MFMA_FORMS[form], _ptr(sink),
                                           _stream(stream)),
               "pblock_mfma_loop")


def pblock_intermediates(handle: int) -> tuple[int, int, int]:
    u, qkv, ag = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
    _abi.check(_abi.lib().pblock_intermediates(ctypes.c_void_p(handle), ctypes.byref(u), ctypes.byref(qkv),
                                               ctypes.byref(ag)), "pblock_intermediates")
    return u.value, qkv.value, ag.value


def pblock_copy_intermediates(handle: int, u=None, qkv=None, ag=None, stream=None) -> None:
    _abi.check(_abi.lib().pblock_copy_intermediates(ctypes.c_void_p(handle), _ptr(u), _ptr(qkv), _ptr(ag),
                                                    _stream(stream)), "pblock_copy_intermediates")


def pblock_set_timing(handle: int, enable: bool) -> None:
    _abi.check(_abi.lib().pblock_set_timing(ctypes.c_void_p(handle), int(bool(enable))), "pblock_set_timing")


def pblock_kernel_times(handle: int, backward: bool = False) -> tuple[dict, int]:
    """Summed milliseconds per kernel category since timing was enabled, and the number of
    timed calls; the backward categories too with ``backward``."""
    names = KERNEL_NAMES + (BACKWARD_KERNEL_NAMES if backward else ())
    ms = (ctypes.c_float * len(names))()
    n = ctypes.c_int()
    _abi.check(_abi.lib().pblock_kernel_times(ctypes.c_void_p(handle), ms, len(names), ctypes.byref(n)),
               "pblock_kernel_times")
    return dict(zip(names, [float(v) for v in ms])), n.value


ACTIVATION_FORMS = {"gelu_erf_f32": _abi.PBLOCK_ACT_GELU_ERF_F32, "gelu_erf_bf16": _abi.PBLOCK_ACT_GELU_ERF_BF16,
                    "gelu_tanh": _abi.PBLOCK_ACT_GELU_TANH, "gelu_erf_grad": _abi.PBLOCK_ACT_GELU_ERF_GRAD}


def pblock_activation(z, out, form: str, stream=None) -> None:
    """The device GeLU form ``form`` (a key of ACTIVATION_FORMS) of each float32 value of z into out."""
    n = z.numel()
    for t, name in ((z, "z"), (out, "out")):
        if t.dtype.itemsize != 4 or not t.is_floating_point() or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 GPU tensor")
    if out.numel() != n:
        raise ValueError("z and out must have the same number of elements")
    _abi.check(_abi.lib().pblock_activation(_ptr(z), _ptr(out), int(n), ACTIVATION_FORMS[form], _stream(stream)),
               "pblock_activation")


def pblock_swa_attention(qkv, ld_qkv, o, ld_o, B, S, H, hd, W, dtype="bf16", stream=None) -> None:
    _abi.check(_abi.lib().pblock_swa_attention(_ptr(qkv), int(ld_qkv), _ptr(o), int(ld_o), int(B), int(S), int(H),
                                               int(hd), int(W), _DTYPES[dtype], _stream(stream)),
               "pblock_swa_attention")


class ParallelBlock:
    """Owns a pblock handle (and so its workspace) for one block shape."""

    def __init__(self, cfg):
        self.cfg = as_cfg(cfg)
        self.handle = pblock_create(self.cfg)

    def forward(self, x, gamma, beta, w_in, w_out, out=None, cfg=None, stream=None):
        import torch

        c = as_cfg(cfg) if cfg is not None else self.cfg
        if out is None:
            out = torch.empty_like(x)
        pblock_forward(self.handle, x, (gamma, beta, w_in, w_out), c, out, stream)
        return out

    def close(self):
        if self.handle:
            pblock_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass
