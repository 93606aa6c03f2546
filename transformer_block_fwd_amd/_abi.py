"""ctypes declarations of include/pblock.h and loading of libpblock.so.

There is no fallback: if the HIP library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpblock.so")

PBLOCK_OK = 0
STATUS_NAMES = {
    0: "PBLOCK_OK",
    -1: "PBLOCK_ERR_NULL",
    -2: "PBLOCK_ERR_SHAPE",
    -3: "PBLOCK_ERR_DTYPE",
    -4: "PBLOCK_ERR_ALIGN",
    -5: "PBLOCK_ERR_ALIAS",
    -6: "PBLOCK_ERR_CFG_MISMATCH",
    -7: "PBLOCK_ERR_DEVICE",
    -8: "PBLOCK_ERR_NOMEM",
    -9: "PBLOCK_ERR_HIP",
    -10: "PBLOCK_ERR_ARG",
}
globals().update({name: code for code, name in STATUS_NAMES.items()})

PBLOCK_F32 = 0
PBLOCK_BF16 = 1

# device GeLU forms of pblock_activation
PBLOCK_ACT_GELU_ERF_F32 = 0
PBLOCK_ACT_GELU_ERF_BF16 = 1
PBLOCK_ACT_GELU_TANH = 2
PBLOCK_ACT_GELU_ERF_GRAD = 3
PBLOCK_MFMA_16X16X32 = 0
PBLOCK_MFMA_32X32X16 = 1


class PblockCfg(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32),
        ("S", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("hd", ctypes.c_int32),
        ("ffn", ctypes.c_int32),
        ("W", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("add_residual", ctypes.c_int32),
        ("ln_eps", ctypes.c_float),
    ]


class PblockWeights(ctypes.Structure):
    _fields_ = [
        ("ln_gamma", ctypes.c_void_p),
        ("ln_beta", ctypes.c_void_p),
        ("w_in", ctypes.c_void_p),
        ("w_out", ctypes.c_void_p),
    ]


class PblockVariant(ctypes.Structure):
    _fields_ = [
        ("gelu_tanh", ctypes.c_int32),
        ("rope", ctypes.c_int32),
        ("rope_base", ctypes.c_float),
        ("two_ln", ctypes.c_int32),
    ]


class PblockVariantWeights(ctypes.Structure):
    _fields_ = [
        ("b_in", ctypes.c_void_p),
        ("b_out", ctypes.c_void_p),
        ("ln2_gamma", ctypes.c_void_p),
        ("ln2_beta", ctypes.c_void_p),
    ]


class PblockGrads(ctypes.Structure):
    _fields_ = [
        ("dx", ctypes.c_void_p),
        ("dln_gamma", ctypes.c_void_p),
        ("dln_beta", ctypes.c_void_p),
        ("dw_in", ctypes.c_void_p),
        ("dw_out", ctypes.c_void_p),
    ]


class PblockError(RuntimeError):
    def __init__(self, code: int, where: str, detail: str = ""):
        self.code = code
        name = STATUS_NAMES.get(code, str(code))
        super().__init__(f"{where}: {name}" + (f" ({detail})" if detail else ""))


_c = ctypes
_SIGNATURES = {
    "pblock_validate_cfg": (_c.c_int, [_c.POINTER(PblockCfg)]),
    "pblock_workspace_bytes": (_c.c_int64, [_c.POINTER(PblockCfg)]),
    "pblock_flops": (_c.c_double, [_c.POINTER(PblockCfg)]),
    "pblock_create": (_c.c_int, [_c.POINTER(PblockCfg), _c.POINTER(_c.c_void_p)]),
    "pblock_forward": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.POINTER(PblockWeights), _c.POINTER(PblockCfg),
                                  _c.c_void_p, _c.c_void_p]),
    "pblock_destroy": (_c.c_int, [_c.c_void_p]),
    "pblock_strerror": (_c.c_char_p, [_c.c_int]),
    "pblock_last_error": (_c.c_char_p, []),
    "pblock_intermediates": (_c.c_int, [_c.c_void_p, _c.POINTER(_c.c_void_p), _c.POINTER(_c.c_void_p),
                                        _c.POINTER(_c.c_void_p)]),
    "pblock_copy_intermediates": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p]),
    "pblock_set_timing": (_c.c_int, [_c.c_void_p, _c.c_int]),
    "pblock_kernel_times": (_c.c_int, [_c.c_void_p, _c.POINTER(_c.c_float), _c.c_int, _c.POINTER(_c.c_int)]),
    "pblock_swa_attention": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_void_p, _c.c_int64, _c.c_int32, _c.c_int32,
                                        _c.c_int32, _c.c_int32, _c.c_int32, _c.c_int32, _c.c_void_p]),
    "pblock_forward_serial": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.POINTER(PblockWeights), _c.c_void_p,
                                         _c.c_void_p, _c.POINTER(PblockCfg), _c.c_void_p, _c.c_void_p]),
    "pblock_mfma_loop": (_c.c_int, [_c.c_int32, _c.c_int32, _c.c_int32, _c.c_void_p, _c.c_void_p]),
    "pblock_forward_variant": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.POINTER(PblockWeights),
                                          _c.POINTER(PblockVariantWeights), _c.POINTER(PblockCfg),
                                          _c.POINTER(PblockVariant), _c.c_void_p, _c.c_void_p]),
    "pblock_train_workspace_bytes": (_c.c_int64, [_c.POINTER(PblockCfg)]),
    "pblock_forward_train": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.POINTER(PblockWeights), _c.POINTER(PblockCfg),
                                        _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_void_p]),
    "pblock_backward": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.POINTER(PblockWeights), _c.POINTER(PblockCfg),
                                   _c.c_void_p, _c.POINTER(PblockGrads), _c.c_void_p, _c.c_int64, _c.c_void_p]),
    "pblock_forward_static": (_c.c_int, [_c.c_void_p, _c.POINTER(PblockWeights), _c.POINTER(PblockCfg), _c.c_void_p,
                                         _c.c_void_p]),
    "pblock_forward_rowchunks": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.POINTER(PblockWeights),
                                            _c.POINTER(PblockCfg), _c.c_void_p, _c.c_int32, _c.c_void_p,
                                            _c.c_uint32, _c.c_void_p]),
    "pblock_pack_chunks": (_c.c_int, [_c.c_void_p, _c.POINTER(PblockCfg), _c.c_int32, _c.c_void_p, _c.c_uint32,
                                      _c.c_void_p, _c.c_void_p, _c.c_void_p]),
    "pblock_activation": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int32, _c.c_void_p]),
    "pblock_forward_chunked": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.POINTER(PblockWeights), _c.POINTER(PblockCfg),
                                          _c.c_void_p, _c.c_int32, _c.POINTER(_c.c_void_p),
                                          _c.POINTER(_c.c_void_p), _c.c_void_p]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"pblock HIP library not found at {LIB_PATH}; build it with "
                "`python -m transformer_block_fwd_amd.build` (there is no CPU fallback)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def last_error() -> str:
    return lib().pblock_last_error().decode(errors="replace")


def check(code: int, where: str) -> None:
    if code != PBLOCK_OK:
        raise PblockError(code, where, last_error())
