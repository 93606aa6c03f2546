// bf16 GEMM on gfx950 matrix cores: C[m, n] = sum_k X[m, k] * Wt[n, k].
//
// Both operands are K-contiguous (activations [M, K] and nn.Linear-style
// weights [N, K]), which is what the 32x32x16 bf16 MFMA wants: every lane
// feeds 8 consecutive k of one row from a single 16-byte LDS read.
//
// Tile: 256 x 256 outputs per workgroup of 8 wavefronts (2 per SIMD), laid
// out 2 (M) x 4 (N); each wavefront owns 128 x 64 as 4 x 2 MFMA tiles of
// 32 x 32 with fp32 accumulators.  The k loop walks 64-wide slabs through two
// LDS stages (2 x 64 KiB).  Global data moves straight into LDS with
// buffer_load_dwordx4 ... lds (no staging registers): each instruction fills
// 1 KiB = 8 rows of 128 bytes.  The 16-byte chunk index inside a row is XORed
// with (row & 7) on the source side, so the fragment reads (8 lanes on 8 rows,
// same logical chunk) hit distinct LDS banks.  Rows past M or N fall outside
// the buffer descriptor's range and read as zero.
//
// Schedule: persistent stream-K.  The (tile, k-slab) iteration space is cut
// into one equal contiguous share per workgroup (one workgroup per CU), so
// every CU does the same number of MFMAs whatever the tile count -- no
// partial last wave.  A tile whose k range is split between workgroups is
// finished by the last contributor to arrive (per-tile atomic counter, no
// waiting): contributors store fp32 partials, and the finisher sums all of
// them in contributor order (bitwise deterministic), applies the epilogue
// and resets the counter for the next launch.  Workgroup ids are remapped so
// that each XCD (id mod 8) owns a contiguous run of iterations: tiles that
// share a weight stripe (M sweeps fastest) sit on the same XCD's L2.
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

constexpr int kGemmBM = 256, kGemmBN = 256, kGemmBK = 64;
constexpr int kGemmThreads = 512;

struct StreamK {
  float* partials;  // [2 * G][kGemmBM * kGemmBN] fp32 (slot, then float4 row, then thread)
  int* counters;    // [tiles], zero between launches
  int tiles_m;
  int KT;           // k slabs per tile
  int64_t iters;    // tiles * KT
  int G;            // persistent workgroups (== gridDim.x)
};

// Iteration-space share of (virtual) workgroup g: [sk_start(g), sk_start(g + 1)).
__device__ __forceinline__ int64_t sk_start(int g, int64_t iters, int G) { return (int64_t(g) * iters) / G; }

__device__ __forceinline__ int xcd_remap(int bid, int G) {
  const int xcd = bid & 7, idx = bid >> 3;
  const int per = G >> 3, rem = G & 7;
  return (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

#define PBLK_LDS __attribute__((address_space(3)))

template <int EPI>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_bf16_sk_kernel(GemmArgs g, StreamK sk) {
  constexpr int BM = kGemmBM, BN = kGemmBN, BK = kGemmBK;
  constexpr int WN = 4;
  constexpr int TM = 128, TN = 64;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int STAGE = (BM + BN) * BK;  // elements per LDS stage
  __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * STAGE];
  __shared__ int s_old;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 31, lg = lane >> 5;
  const int G = sk.G;
  const int vg = xcd_remap(blockIdx.x, G);

  // DMA lane geometry: lane l of a 1 KiB block fills LDS row l/8 of the block,
  // physical chunk l%8, which holds logical chunk (l%8) ^ (l/8) of that row.
  const int dma_row = lane >> 3;
  const int dma_chunk = (lane & 7) ^ (lane >> 3);

  const int a_row0 = wm * TM + lr;
  const int b_row0 = wn * TN + lr;
  const int swz = lr & 7;

  int64_t it = sk_start(vg, sk.iters, G);
  const int64_t it_end = sk_start(vg + 1, sk.iters, G);

  while (it < it_end) {
    const int t = int(it / sk.KT);
    const int kb = int(it - int64_t(t) * sk.KT);
    const int ke = int(min<int64_t>(sk.KT, kb + (it_end - it)));
    const int m0 = (t % sk.tiles_m) * BM;
    const int n0 = (t / sk.tiles_m) * BN;

    // buffer descriptors anchored at the tile's first row; rows past the end read as zero
    const uint16_t* a_base = g.a + int64_t(m0) * g.lda;
    const uint16_t* b_base = g.b + int64_t(n0) * g.ldb;
    const int64_t a_bytes = int64_t(g.M - m0) * g.lda * 2, b_bytes = int64_t(g.N - n0) * g.ldb * 2;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a_base), 0, int(min<int64_t>(a_bytes, 0x7FFFFFFF)), 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(b_base), 0, int(min<int64_t>(b_bytes, 0x7FFFFFFF)), 0x00020000);
    // wave w fills blocks 4w .. 4w+3 of each operand: tile rows 32w + 8i + l/8
    const uint32_t a_voff = uint32_t((int64_t(wave * 32 + dma_row) * g.lda + dma_chunk * 8) * 2);
    const uint32_t b_voff = uint32_t((int64_t(wave * 32 + dma_row) * g.ldb + dma_chunk * 8) * 2);
    const uint32_t a_step = uint32_t(8 * g.lda * 2), b_step = uint32_t(8 * g.ldb * 2);

    auto issue = [&](int kt, int stage) {
      const uint32_t koff = uint32_t(kt * BK * 2);
      uint16_t* sa = smem + stage * STAGE + wave * 4 * 512;
      uint16_t* sb = smem + stage * STAGE + BM * BK + wave * 4 * 512;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (PBLK_LDS void*)(sa + i * 512), 16, a_voff + i * a_step, koff,
                                                 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (PBLK_LDS void*)(sb + i * 512), 16, b_voff + i * b_step, koff,
                                                 0, 0);
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    issue(kb, 0);
    __syncthreads();
    for (int kt = kb; kt < ke; ++kt) {
      const int cur = (kt - kb) & 1;
      if (kt + 1 < ke) issue(kt + 1, cur ^ 1);
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
      __syncthreads();
    }

    bool finish = (kb == 0 && ke == sk.KT);
    if (!finish) {
      // contributors of tile t: the workgroups whose shares intersect [t*KT, (t+1)*KT)
      const int64_t t0 = int64_t(t) * sk.KT, t1 = t0 + sk.KT;
      int g_lo = int((t0 * G) / sk.iters);
      while (g_lo > 0 && sk_start(g_lo, sk.iters, G) > t0) --g_lo;
      while (sk_start(g_lo + 1, sk.iters, G) <= t0) ++g_lo;
      int g_hi = int(((t1 - 1) * G) / sk.iters);
      while (g_hi > 0 && sk_start(g_hi, sk.iters, G) > t1 - 1) --g_hi;
      while (g_hi + 1 < G && sk_start(g_hi + 1, sk.iters, G) <= t1 - 1) ++g_hi;
      const int n_contrib = g_hi - g_lo + 1;
      // A workgroup keeps the partial of the tile its share starts in (its first
      // segment) in slot 0 and that of the tile its share ends in in slot 1.  Every
      // contributor after g_lo starts inside t; g_lo starts inside t only if its
      // share begins exactly at t0.
      const int lo_slot = 2 * g_lo + (sk_start(g_lo, sk.iters, G) == t0 ? 0 : 1);
      const int my_slot = (vg == g_lo) ? lo_slot : 2 * vg;
      constexpr int TILE4 = BM * BN / 4;
      f32x4* mine = reinterpret_cast<f32x4*>(sk.partials) + int64_t(my_slot) * TILE4;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r4 = (i * FN + j) * 4 + q;
            const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            mine[r4 * kGemmThreads + tid] = v;
          }
      __threadfence();
      __syncthreads();
      if (tid == 0) s_old = atomicAdd(sk.counters + t, 1);
      __syncthreads();
      finish = (s_old == n_contrib - 1);
      if (finish) {
        __threadfence();
        // sum every contributor's partial (own included) in contributor order:
        // the result does not depend on which workgroup arrived last
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
        for (int c = g_lo; c <= g_hi; ++c) {
          const f32x4* p = reinterpret_cast<const f32x4*>(sk.partials) + int64_t(c == g_lo ? lo_slot : 2 * c) * TILE4;
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const f32x4 v = p[((i * FN + j) * 4 + q) * kGemmThreads + tid];
                acc[i][j][4 * q] += v[0];
                acc[i][j][4 * q + 1] += v[1];
                acc[i][j][4 * q + 2] += v[2];
                acc[i][j][4 * q + 3] += v[3];
              }
        }
        if (tid == 0) sk.counters[t] = 0;
      }
    }

    if (finish) {
      // lane holds C[m][n .. n+3] for m = ... + lr, n = ... + 8*r4 + 4*lg
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
    it += (ke - kb);
  }
}

}  // namespace pblk
