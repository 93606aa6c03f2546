"""Seeded synthetic inputs for the parallel transformer block.

This module is shared by the oracle side and the HIP side, and on purpose holds
none of the block's arithmetic: only the workload shapes, the seeded random
draws, the packing of weights into the order the library reads them, and the
rounding of the drawn fp32 values to bf16 storage.

Shapes follow the MegaScale guided reading (ai-training-network-primer page,
"Results": the 175B model with hidden size 12,288 and tensor parallelism 8),
plus smaller and longer blocks that exercise the sliding window.

Recipe (every config):
  * generator ``numpy.random.Generator(PCG64(seed))``, default seed 0;
  * draw order: x ~ N(0, 1) of shape [B, S, d]; then W_in ~ N(0, 0.02^2) of
    shape [3*H*hd + ffn, d]; then W_out ~ N(0, 0.02^2) of shape [d, H*hd + ffn];
  * LayerNorm gamma = 1, beta = 0, unless ``affine=True``, which then draws
    gamma ~ N(1, 0.1^2) and beta ~ N(0, 0.1^2) (both [d]) after W_out;
  * bf16 configs round every drawn fp32 value to bf16 with round-to-nearest-even;
    the fp32 config keeps the fp32 draws.

Weight packing: W_in rows are [Q heads (head-major) ; K heads ; V heads ; FC1],
each head's rows contiguous, and W_out columns are [attention heads
(head-major) ; FC2].  Both are K-contiguous (row-major [out, in]).
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class BlockConfig:
    """Shape of one parallel block.

    W is the number of keys each query sees, itself included; W >= S is full
    causal attention.  ``add_residual`` = 0 asks for the branch sum only (the
    tensor-parallel shard's partial, which the residual joins after the
    reduce-scatter).
    """

    name: str
    B: int
    S: int
    d: int
    H: int
    hd: int
    ffn: int
    W: int
    dtype: str  # "f32" or "bf16"
    add_residual: int = 1
    ln_eps: float = 1e-5

    @property
    def M(self) -> int:
        return self.B * self.S

    @property
    def A(self) -> int:
        return self.H * self.hd

    @property
    def n_in(self) -> int:
        return 3 * self.A + self.ffn

    @property
    def k_out(self) -> int:
        return self.A + self.ffn

    def replace(self, **kw) -> "BlockConfig":
        return dataclasses.replace(self, **kw)

    def keys_per_head(self) -> int:
        """Number of (query, key) pairs inside the causal window, per (b, h)."""
        S, W = self.S, self.W
        w = min(W, S)
        return S * w - w * (w - 1) // 2

    def flops(self) -> float:
        """Algorithmic FLOPs of one forward: the two GEMMs plus QK^T and PV
        over the keys inside the window (masked-out work is not counted)."""
        gemm = 2.0 * self.M * self.d * self.n_in + 2.0 * self.M * self.k_out * self.d
        attn = 4.0 * self.B * self.H * self.hd * self.keys_per_head()
        return gemm + attn

    def gemm1_flops(self) -> float:
        return 2.0 * self.M * self.d * self.n_in

    def gemm2_flops(self) -> float:
        return 2.0 * self.M * self.k_out * self.d

    def attn_flops(self) -> float:
        return 4.0 * self.B * self.H * self.hd * self.keys_per_head()


CONFIGS: dict[str, BlockConfig] = {
    # tiny fp32 block: the debug path
    "tiny": BlockConfig("tiny", B=1, S=128, d=256, H=4, hd=64, ffn=1024, W=32, dtype="f32"),
    # small bf16 block
    "small": BlockConfig("small", B=4, S=1024, d=2048, H=16, hd=128, ffn=8192, W=256, dtype="bf16"),
    # one 1/8 tensor-parallel shard of the 175B layer: emits the pre-reduce-scatter partial
    "shard175b": BlockConfig("shard175b", B=1, S=2048, d=12288, H=12, hd=128, ffn=6144, W=512,
                             dtype="bf16", add_residual=0),
    # long sequence with a 1024-key window
    "long": BlockConfig("long", B=1, S=8192, d=4096, H=32, hd=128, ffn=16384, W=1024, dtype="bf16"),
    # window covering the whole sequence: full causal attention through the band path
    "fullcausal": BlockConfig("fullcausal", B=2, S=4096, d=4096, H=32, hd=128, ffn=16384, W=4096,
                              dtype="bf16"),
}
CONFIG_ORDER = ["tiny", "small", "shard175b", "long", "fullcausal"]


def round_to_bf16(a: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Round fp32 values to bf16 (round to nearest, ties to even).

    Returns (values as float32, raw bf16 bits as uint16).  Inputs are finite.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    hi = (rounded >> np.uint32(16)).astype(np.uint16)
    return rounded.view(np.float32), hi


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class BlockInputs:
    """Host arrays of one workload.

    ``x``, ``gamma``, ``beta``, ``w_in``, ``w_out`` hold float32 values that are
    exactly what the device receives (bf16-representable for bf16 configs).
    ``bits`` holds the raw uint16 bf16 storage for bf16 configs (else None).
    """

    cfg: BlockConfig
    x: np.ndarray
    gamma: np.ndarray
    beta: np.ndarray
    w_in: np.ndarray
    w_out: np.ndarray
    bits: dict | None

    def device_arrays(self) -> dict[str, np.ndarray]:
        """Arrays in the storage type the library reads (uint16 bf16 bits or float32)."""
        if self.cfg.dtype == "bf16":
            return dict(self.bits)
        return dict(x=self.x, gamma=self.gamma, beta=self.beta, w_in=self.w_in, w_out=self.w_out)


def make_inputs(cfg: BlockConfig, seed: int = 0, affine: bool = False) -> BlockInputs:
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((cfg.B, cfg.S, cfg.d), dtype=np.float32)
    w_in = rng.standard_normal((cfg.n_in, cfg.d), dtype=np.float32)
    w_in *= np.float32(0.02)
    w_out = rng.standard_normal((cfg.d, cfg.k_out), dtype=np.float32)
    w_out *= np.float32(0.02)
    if affine:
        gamma = (1.0 + 0.1 * rng.standard_normal(cfg.d, dtype=np.float32)).astype(np.float32)
        beta = (0.1 * rng.standard_normal(cfg.d, dtype=np.float32)).astype(np.float32)
    else:
        gamma = np.ones(cfg.d, dtype=np.float32)
        beta = np.zeros(cfg.d, dtype=np.float32)
    bits = None
    if cfg.dtype == "bf16":
        bits = {}
        out = {}
        for name, arr in (("x", x), ("gamma", gamma), ("beta", beta), ("w_in", w_in), ("w_out", w_out)):
            vals, b = round_to_bf16(arr)
            out[name] = vals
            bits[name] = b
        x, gamma, beta, w_in, w_out = out["x"], out["gamma"], out["beta"], out["w_in"], out["w_out"]
    elif cfg.dtype != "f32":
        raise ValueError(f"unknown dtype {cfg.dtype}")
    return BlockInputs(cfg, x, gamma, beta, w_in, w_out, bits)


def make_ln2(cfg: BlockConfig, seed: int = 0, affine: bool = False) -> dict[str, np.ndarray]:
    """Second LayerNorm's parameters for the serial form of the layer, drawn like the first
    (gamma = 1, beta = 0, or N(1, 0.1^2) / N(0, 0.1^2) with ``affine``) from their own stream.

    Returns float32 values exactly as the device receives them under "gamma2"/"beta2" and
    the storage arrays the library reads under "gamma2_dev"/"beta2_dev"."""
    rng = np.random.Generator(np.random.PCG64([seed, 2]))
    if affine:
        gamma = (1.0 + 0.1 * rng.standard_normal(cfg.d, dtype=np.float32)).astype(np.float32)
        beta = (0.1 * rng.standard_normal(cfg.d, dtype=np.float32)).astype(np.float32)
    else:
        gamma = np.ones(cfg.d, dtype=np.float32)
        beta = np.zeros(cfg.d, dtype=np.float32)
    if cfg.dtype == "bf16":
        (g, gb), (b, bb) = round_to_bf16(gamma), round_to_bf16(beta)
        return dict(gamma2=g, beta2=b, gamma2_dev=gb, beta2_dev=bb)
    return dict(gamma2=gamma, beta2=beta, gamma2_dev=gamma, beta2_dev=beta)


def make_variant_params(cfg: BlockConfig, seed: int = 0) -> dict[str, np.ndarray]:
    """Biases of the two projections for the variant block, b_in [3A + ffn] and b_out [d],
    each N(0, 0.1^2) from their own stream; float32 values as the device receives them under
    "b_in"/"b_out" and the storage arrays under "b_in_dev"/"b_out_dev"."""
    rng = np.random.Generator(np.random.PCG64([seed, 3]))
    b_in = (0.1 * rng.standard_normal(cfg.n_in, dtype=np.float32)).astype(np.float32)
    b_out = (0.1 * rng.standard_normal(cfg.d, dtype=np.float32)).astype(np.float32)
    if cfg.dtype == "bf16":
        (bi, bid), (bo, bod) = round_to_bf16(b_in), round_to_bf16(b_out)
        return dict(b_in=bi, b_out=bo, b_in_dev=bid, b_out_dev=bod)
    return dict(b_in=b_in, b_out=b_out, b_in_dev=b_in, b_out_dev=b_out)


def make_dy(cfg: BlockConfig, seed: int = 0) -> dict[str, np.ndarray]:
    """Output gradient dy [B, S, d] ~ N(0, 1) for the backward pass, from its own stream;
    float32 values as the device receives them under "dy" and the storage array under "dy_dev"."""
    rng = np.random.Generator(np.random.PCG64([seed, 4]))
    dy = rng.standard_normal((cfg.B, cfg.S, cfg.d), dtype=np.float32)
    if cfg.dtype == "bf16":
        v, bits = round_to_bf16(dy)
        return dict(dy=v, dy_dev=bits)
    return dict(dy=dy, dy_dev=dy)


def sample_row_blocks(cfg: BlockConfig, block: int = 32, seed: int = 1) -> list[tuple[int, int, int]]:
    """Query row blocks (b, i0, i1) for sampled checks at full size.

    Covers the sequence start (partial windows), the first full window, a
    random interior block and the sequence end, for the first and last batch.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    S, W = cfg.S, cfg.W
    blk = min(block, S)
    starts = {0, max(0, min(S - blk, W - blk // 2)), S - blk}
    if S > blk:
        starts.add(int(rng.integers(0, S - blk + 1)))
    batches = sorted({0, cfg.B - 1})
    return [(b, s, s + blk) for b in batches for s in sorted(starts)]
