// bf16 GEMM on gfx950 matrix cores: C[m, n] = sum_k X[m, k] * Wt[n, k].
//
// Both operands are K-contiguous (activations [M, K] and nn.Linear-style
// weights [N, K]), which is exactly what the 32x32x16 bf16 MFMA wants: every
// lane feeds 8 consecutive k of one row from a single 16-byte LDS read.
//
// Tiling: a workgroup of WM x WN wavefronts owns a BM x BN output tile; each
// wavefront owns (BM/WM) x (BN/WN) as a grid of 32x32 MFMA tiles held in fp32
// accumulators.  The k loop walks 64-wide slabs through two LDS stages: the
// next slab is fetched from global memory into registers while the current
// one feeds the MFMAs, then written to the other stage, so there is one
// barrier per slab.  LDS rows are 128 bytes; the 16-byte chunk index is XORed
// with (row & 7) so both the row-wise stores and the fragment reads (8 lanes
// on 8 different rows, same logical chunk) hit distinct banks.
//
// The weight fragment is the MFMA's first operand and the activation fragment
// its second, so each lane ends up with 4 consecutive output columns of one
// output row per accumulator group: the epilogue writes 8-byte runs.
//
// Workgroups are remapped so that each of the 8 XCDs (workgroup id mod 8
// selects the XCD) owns a contiguous run of tiles that sweeps M fastest: the
// tiles sharing a weight stripe sit on the same XCD and share its L2.
//
// Epilogues:
//   kEpiSplitGelu: columns < nsplit are stored as bf16 to out0 (the Q|K|V
//     projections); columns >= nsplit get the exact GeLU and go to out1 at
//     column off1 + (n - nsplit) (the FC1 activations next to the attention
//     output, so the second GEMM reads one K-contiguous operand).
//   kEpiResidual: optional residual x added in fp32, one rounding to bf16.
#pragma once

#include "common.hpp"

namespace pblk {

struct GemmArgs {
  const uint16_t* a;  // activations [M, K], row stride lda
  int64_t lda;
  const uint16_t* b;  // weights [N, K], row stride ldb
  int64_t ldb;
  int M, N, K;
  uint16_t* out0;
  int64_t ld0;
  uint16_t* out1;
  int64_t ld1;
  int64_t off1;
  int nsplit;
  const uint16_t* resid;  // kEpiResidual: [M, N] with row stride ldr, or nullptr
  int64_t ldr;
};

__device__ __forceinline__ int xcd_remap(int bid, int G) {
  const int xcd = bid & 7, idx = bid >> 3;
  const int per = G >> 3, rem = G & 7;
  return (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(WM* WN * 64, 1) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int NT = WM * WN * 64;
  constexpr int BK = 64;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int RPP = NT / 8;  // rows covered per pass of 16-byte chunk loads
  constexpr int A_LD = BM / RPP, B_LD = BN / RPP;
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(BM % RPP == 0 && BN % RPP == 0, "tile rows must be a multiple of the load pass");
  constexpr int STAGE = (BM + BN) * BK;  // elements per LDS stage
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = (g.N + BN - 1) / BN;
  const int L = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  const int m0 = (L % tiles_m) * BM;
  const int n0 = (L / tiles_m) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 31, lg = lane >> 5;

  // global -> register staging
  const int cchunk = tid & 7, crow = tid >> 3;
  const uint16_t* a_src[A_LD];
  const uint16_t* b_src[B_LD];
#pragma unroll
  for (int p = 0; p < A_LD; ++p) {
    const int r = min(m0 + crow + p * RPP, g.M - 1);
    a_src[p] = g.a + int64_t(r) * g.lda + cchunk * 8;
  }
#pragma unroll
  for (int p = 0; p < B_LD; ++p) {
    const int r = min(n0 + crow + p * RPP, g.N - 1);
    b_src[p] = g.b + int64_t(r) * g.ldb + cchunk * 8;
  }
  u32x4 ra[A_LD], rb[B_LD];
  auto load_global = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int p = 0; p < A_LD; ++p) ra[p] = *reinterpret_cast<const u32x4*>(a_src[p] + k0);
#pragma unroll
    for (int p = 0; p < B_LD; ++p) rb[p] = *reinterpret_cast<const u32x4*>(b_src[p] + k0);
  };
  auto store_lds = [&](int stage) {
    uint16_t* sa = smem + stage * STAGE;
    uint16_t* sb = sa + BM * BK;
#pragma unroll
    for (int p = 0; p < A_LD; ++p) {
      const int r = crow + p * RPP;
      *reinterpret_cast<u32x4*>(sa + r * BK + ((cchunk ^ (r & 7)) << 3)) = ra[p];
    }
#pragma unroll
    for (int p = 0; p < B_LD; ++p) {
      const int r = crow + p * RPP;
      *reinterpret_cast<u32x4*>(sb + r * BK + ((cchunk ^ (r & 7)) << 3)) = rb[p];
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = g.K / BK;
  load_global(0);
  store_lds(0);
  __syncthreads();

  const int a_row0 = wm * TM + lr;
  const int b_row0 = wn * TN + lr;
  const int swz = lr & 7;

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_global(kt + 1);
    const uint16_t* sa = smem + cur * STAGE;
    const uint16_t* sb = sa + BM * BK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int ch = ((kk * 2 + lg) ^ swz) << 3;
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const bf16x8*>(sa + (a_row0 + i * 32) * BK + ch);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(sb + (b_row0 + j * 32) * BK + ch);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) store_lds(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds C[m][n .. n+3] for m = ... + lr, n = ... + 8*r4 + 4*lg
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * TM + i * 32 + lr;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int n = n0 + wn * TN + j * 32 + r4 * 8 + lg * 4;
        if (n >= g.N) continue;
        float v0 = acc[i][j][r4 * 4 + 0], v1 = acc[i][j][r4 * 4 + 1];
        float v2 = acc[i][j][r4 * 4 + 2], v3 = acc[i][j][r4 * 4 + 3];
        uint16_t* dst;
        if constexpr (EPI == kEpiSplitGelu) {
          if (n < g.nsplit) {
            dst = g.out0 + int64_t(m) * g.ld0 + n;
          } else {
            v0 = gelu_erf(v0); v1 = gelu_erf(v1); v2 = gelu_erf(v2); v3 = gelu_erf(v3);
            dst = g.out1 + int64_t(m) * g.ld1 + g.off1 + (n - g.nsplit);
          }
        } else {
          if (g.resid != nullptr) {
            const u32x2 xr = *reinterpret_cast<const u32x2*>(g.resid + int64_t(m) * g.ldr + n);
            v0 += __uint_as_float(xr.x << 16); v1 += __uint_as_float(xr.x & 0xFFFF0000u);
            v2 += __uint_as_float(xr.y << 16); v3 += __uint_as_float(xr.y & 0xFFFF0000u);
          }
          dst = g.out0 + int64_t(m) * g.ld0 + n;
        }
        u32x2 o;
        o.x = pack_bf16x2(v0, v1);
        o.y = pack_bf16x2(v2, v3);
        *reinterpret_cast<u32x2*>(dst) = o;
      }
    }
  }
}

}  // namespace pblk
