"""Oracle package: plain fp64 CPU reference of the parallel block.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.
"""
from .block import (  # noqa: F401
    block_backward,
    block_forward,
    block_forward_rows,
    block_forward_variant,
    block_forward_variant_rows,
    gelu,
    gelu_grad,
    gelu_tanh,
    layer_norm,
    layer_norm_backward,
    relative_error,
    rope,
    serial_block_forward,
    serial_block_forward_rows,
    split_projection,
    swa_attention,
    swa_attention_backward,
    window_lo,
)
