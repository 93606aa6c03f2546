"""HIP streams for running a consumer of the row-chunk publication (pblock_pack_chunks) next to
the block's kernels.

A stream created with a compute-unit mask gets a hardware queue of its own (the mask is a
property of the queue), so its kernels run concurrently with the producer's instead of waiting
behind them in a shared queue; the mask also keeps the consumer's workgroups on a few compute
units.  Plumbing only (ctypes on the HIP runtime that torch has loaded); the library itself
never creates streams.
"""
from __future__ import annotations

import ctypes

_hip = None


def _runtime() -> ctypes.CDLL:
    global _hip
    if _hip is None:
        lib = ctypes.CDLL("libamdhip64.so")
        lib.hipExtStreamCreateWithCUMask.restype = ctypes.c_int
        lib.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint32,
                                                     ctypes.POINTER(ctypes.c_uint32)]
        lib.hipStreamDestroy.restype = ctypes.c_int
        lib.hipStreamDestroy.argtypes = [ctypes.c_void_p]
        _hip = lib
    return _hip


def cu_masked_stream(first_cu: int, count: int, n_cus: int) -> int:
    """A new stream (hipStream_t as an int) whose kernels run only on compute units
    [first_cu, first_cu + count) of the current device's n_cus; destroy it with destroy_stream."""
    if not (0 <= first_cu and count >= 1 and first_cu + count <= n_cus):
        raise ValueError("compute-unit range outside the device")
    words = (n_cus + 31) // 32
    mask = (ctypes.c_uint32 * words)()
    for cu in range(first_cu, first_cu + count):
        mask[cu // 32] |= 1 << (cu % 32)
    s = ctypes.c_void_p()
    err = _runtime().hipExtStreamCreateWithCUMask(ctypes.byref(s), words, mask)
    if err != 0:
        raise RuntimeError(f"hipExtStreamCreateWithCUMask failed ({err})")
    return int(s.value)


def destroy_stream(stream: int) -> None:
    err = _runtime().hipStreamDestroy(ctypes.c_void_p(stream))
    if err != 0:
        raise RuntimeError(f"hipStreamDestroy failed ({err})")
