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
// global_load_lds_dwordx4 (no staging registers): each instruction fills
// 1 KiB = 8 rows of 128 bytes.  The 16-byte chunk index inside a row is XORed
// with (row & 7) on the source side, so the fragment reads (8 lanes on 8 rows,
// same logical chunk) hit distinct LDS banks.  Rows past M or N are clamped to
// the last valid row (their results are never stored).
//
// Schedule: data-parallel waves plus a split-K tail.  With G workgroups
// resident at once (one per CU), the first floor(T / G) * G tiles run whole,
// one workgroup each, in k-lockstep.  The remaining T mod G tiles would fill
// only part of a last wave, so each is cut into `split` k-chunks (split =
// G / tail) and the chunks run together as one more wave: every CU gets
// nearly the same number of MFMAs whatever the tile count.  A chunk stores
// its fp32 partial; the last chunk to arrive (per-tile atomic counter, no
// waiting) sums all of them in chunk order (bitwise deterministic), applies
// the epilogue and resets the counter for the next launch.
//
// L2 locality: workgroup ids are remapped so each XCD (id mod 8) owns a
// contiguous run of work units, and units are ordered in groups of 8 M-tiles
// (M fastest): the 32 workgroups an XCD runs at once cover an 8 (M) x 4 (N)
// block of tiles at the same k, so they share activation and weight slabs in
// that XCD's L2.
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

// Work decomposition of one GEMM launch (grid = dp_units + tail * split).
struct GemmSched {
  float* partials;  // [tail * split][kGemmBM * kGemmBN] fp32 (chunk slot, then float4 row, then thread)
  int* counters;    // [tail], zero between launches
  int tiles_m, tiles_n;
  int KT;           // k slabs per tile
  int dp_units;     // tiles computed whole (a multiple of the resident workgroup count)
  int tail;         // tiles computed in k-chunks
  int split;        // k-chunks per tail tile
};

constexpr int kGroupM = 8;

// Contiguous-per-XCD renumbering of workgroup ids 0 .. n-1 (id mod 8 picks the XCD).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int xcd = bid & 7, idx = bid >> 3;
  const int per = n >> 3, rem = n & 7;
  return (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

// Tile coordinates of linear tile index L: groups of kGroupM M-tiles, M fastest.
__device__ __forceinline__ void tile_coords(int L, int tiles_m, int tiles_n, int* tm, int* tn) {
  const int group = kGroupM * tiles_n;
  const int first_m = (L / group) * kGroupM;
  const int gsz = min(tiles_m - first_m, kGroupM);
  const int r = L % group;
  *tm = first_m + r % gsz;
  *tn = r / gsz;
}

#define PBLK_LDS __attribute__((address_space(3)))

template <int EPI>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_bf16_kernel(GemmArgs g, GemmSched sk) {
  constexpr int BM = kGemmBM, BN = kGemmBN, BK = kGemmBK;
  constexpr int WN = 4;
  constexpr int TM = 128, TN = 64;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int STAGE = (BM + BN) * BK;  // elements per LDS stage
  // two LDS stages as two distinct arrays: the compiler can then tell that the
  // DMA filling one stage never aliases the fragment reads of the other, and
  // does not wait for the prefetch before reading the current slab
  __shared__ __attribute__((aligned(1024))) uint16_t smem0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t smem1[STAGE];
  __shared__ int s_old;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 31, lg = lane >> 5;
  // DMA lane geometry: lane l of a 1 KiB block fills LDS row l/8 of the block,
  // physical chunk l%8, which holds logical chunk (l%8) ^ (l/8) of that row.
  const int dma_row = lane >> 3;
  const int dma_chunk = (lane & 7) ^ (lane >> 3);

  const int a_row0 = wm * TM + lr;
  const int b_row0 = wn * TN + lr;
  const int swz = lr & 7;

  // this workgroup's unit: a whole tile, or k-chunk `chunk` of tail tile `tl`
  int L, kb, ke, tl = -1, chunk = 0;
  if (int(blockIdx.x) < sk.dp_units) {
    L = xcd_remap(blockIdx.x, sk.dp_units);
    kb = 0;
    ke = sk.KT;
  } else {
    const int nu = sk.tail * sk.split;
    const int u = xcd_remap(blockIdx.x - sk.dp_units, nu);
    chunk = u / sk.tail;
    tl = u % sk.tail;
    L = sk.dp_units + tl;
    kb = int((int64_t(chunk) * sk.KT) / sk.split);
    ke = int((int64_t(chunk + 1) * sk.KT) / sk.split);
  }
  int tm, tn;
  tile_coords(L, sk.tiles_m, sk.tiles_n, &tm, &tn);
  {
    const int m0 = tm * BM;
    const int n0 = tn * BN;

    // per-lane source pointers (rows clamped to the last valid row)
    const uint16_t* a_src[4];
    const uint16_t* b_src[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = min(m0 + wave * 32 + 8 * i + dma_row, g.M - 1);
      const int rb = min(n0 + wave * 32 + 8 * i + dma_row, g.N - 1);
      a_src[i] = g.a + int64_t(ra) * g.lda + dma_chunk * 8;
      b_src[i] = g.b + int64_t(rb) * g.ldb + dma_chunk * 8;
    }

    auto issue = [&](int kt, uint16_t* stage) {
      const int koff = kt * BK;
      uint16_t* sa = stage + wave * 4 * 512;
      uint16_t* sb = stage + BM * BK + wave * 4 * 512;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds(a_src[i] + koff, (PBLK_LDS void*)(sa + i * 512), 16, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds(b_src[i] + koff, (PBLK_LDS void*)(sb + i * 512), 16, 0, 0);
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    auto compute = [&](const uint16_t* stage) {
      const uint16_t* sa = stage;
      const uint16_t* sb = stage + BM * BK;
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
        // keep the next step's fragment loads from being hoisted here (register pressure)
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // Slab kb lands in stage 0.  Each pass of the loop handles two slabs, the
    // first read from stage 0 while the next slab streams into stage 1, the
    // second the other way round; an odd last slab is read from stage 0.
    issue(kb, smem0);
    __syncthreads();
    int kt = kb;
    for (; kt + 1 < ke; kt += 2) {
      issue(kt + 1, smem1);
      compute(smem0);
      __syncthreads();
      if (kt + 2 < ke) issue(kt + 2, smem0);
      compute(smem1);
      __syncthreads();
    }
    if (kt < ke) {
      compute(smem0);
      __syncthreads();
    }

    bool finish = (tl < 0);
    if (!finish) {
      constexpr int TILE4 = BM * BN / 4;
      f32x4* mine = reinterpret_cast<f32x4*>(sk.partials) + int64_t(tl * sk.split + chunk) * TILE4;
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
      if (tid == 0) s_old = atomicAdd(sk.counters + tl, 1);
      __syncthreads();
      finish = (s_old == sk.split - 1);
      if (finish) {
        __threadfence();
        // sum every chunk's partial (own included) in chunk order: the result does
        // not depend on which chunk arrived last
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
        for (int c = 0; c < sk.split; ++c) {
          const f32x4* p = reinterpret_cast<const f32x4*>(sk.partials) + int64_t(tl * sk.split + c) * TILE4;
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
        if (tid == 0) sk.counters[tl] = 0;
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
  }
}

}  // namespace pblk
