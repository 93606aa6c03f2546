// bf16 GEMM on gfx950 matrix cores: C[m, n] = sum_k X[m, k] * Wt[n, k].
//
// Both operands are K-contiguous (activations [M, K] and nn.Linear-style
// weights [N, K]), which is what the 32x32x16 bf16 MFMA wants: every lane
// feeds 8 consecutive k of one row from a single 16-byte LDS read.
//
// Tile: 256 x 256 outputs per workgroup of 8 wavefronts (2 per SIMD), laid
// out 2 (M) x 4 (N); each wavefront owns 128 x 64 as 4 x 2 MFMA tiles of
// 32 x 32 with fp32 accumulators.
//
// Pipeline: the k loop walks 32-wide slabs through four LDS stages (4 x 32 KiB,
// each a separately named array so the compiler can see that filling one
// stage never aliases reading another).  Global data moves straight into LDS
// with global_load_lds_dwordx4 (no staging registers), three slabs ahead of
// the MFMAs; each step waits only until this wave's copies of the current
// slab have landed (s_waitcnt vmcnt with the two later slabs still in flight),
// then one barrier publishes the slab and frees the stage read one step
// earlier for the next prefetch.  Each copy instruction fills 1 KiB = 16 rows
// of 64 bytes; the 16-byte chunk index inside a row is XORed with
// ((row >> 1) & 3) on the source side and undone on the fragment reads.
// Rows past M or N are clamped to the last valid row (never stored).
//
// Schedule: data-parallel waves plus a split-K tail.  With G workgroups
// resident at once (one per CU), the first floor(T / G) * G tiles run whole,
// one workgroup each, in k-lockstep.  The remaining T mod G tiles would fill
// only part of a last wave, so each is cut into `split` k-chunks
// (split = G / tail) that run together as one more wave.  A chunk stores its
// fp32 partial tile; a second small kernel sums the chunks of each tail tile
// in chunk order (bitwise deterministic, no atomics, no cross-workgroup
// fences) and applies the epilogue.
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
  const uint16_t* a;
  int64_t lda;
  const uint16_t* b;
  int64_t ldb;
  int M, N, K;
  uint16_t* out0;
  int64_t ld0;
  uint16_t* out1;
  int64_t ld1;
  int64_t off1;
  int nsplit;
  const uint16_t* resid;
  int64_t ldr;
};

constexpr int kGemmBM = 256, kGemmBN = 256, kGemmBK = 32, kGemmThreads = 512, kGemmStages = 4;
constexpr int kGemmStage = (kGemmBM + kGemmBN) * kGemmBK;  // elements per LDS stage (32 KiB)

// Work decomposition of one GEMM launch (grid = dp_units + tail * split).
struct GemmSched {
  float* partials;  // [tail * split][kGemmBM * kGemmBN] fp32 (chunk slot, then float4 row, then thread)
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

// s_waitcnt vmcnt(N) lgkmcnt(0), expcnt untouched (gfx9 encoding of the immediate)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}
// Workgroup barrier that no memory access may be moved across (the waits are explicit).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int EPI>
__device__ __forceinline__ void store_outputs(const GemmArgs& g, int m, int n, float v0, float v1, float v2, float v3) {
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

template <int EPI>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_bf16_kernel(GemmArgs g, GemmSched sk) {
  constexpr int BM = kGemmBM, BN = kGemmBN, BK = kGemmBK, NT = kGemmThreads, NSTAGE = kGemmStages;
  constexpr int STAGE = kGemmStage;
  constexpr int WN = 4, TM = 128, TN = 64, FM = 4, FN = 2;
  __shared__ __attribute__((aligned(1024))) uint16_t st0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t st1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t st2[STAGE];
  __shared__ __attribute__((aligned(1024))) uint16_t st3[STAGE];
  auto stage_ptr = [&](int s) -> uint16_t* { return s == 0 ? st0 : s == 1 ? st1 : s == 2 ? st2 : st3; };

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 31, lg = lane >> 5;
  // DMA: lane l of a 1 KiB block fills row l/4 (of 16), physical chunk l%4 = logical chunk ^ ((row>>1)&3)
  const int dma_row = lane >> 2;
  const int dma_chunk = (lane & 3) ^ ((lane >> 3) & 3);
  const int a_row0 = wm * TM + lr;
  const int b_row0 = wn * TN + lr;
  const int swz = (lr >> 1) & 3;

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
  const int m0 = tm * BM, n0 = tn * BN;

  const uint16_t* a_src[2];
  const uint16_t* b_src[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ra = min(m0 + wave * 32 + 16 * i + dma_row, g.M - 1);
    const int rb = min(n0 + wave * 32 + 16 * i + dma_row, g.N - 1);
    a_src[i] = g.a + int64_t(ra) * g.lda + dma_chunk * 8;
    b_src[i] = g.b + int64_t(rb) * g.ldb + dma_chunk * 8;
  }
  auto issue = [&](int kt, uint16_t* stage) {
    const int koff = kt * BK;
    uint16_t* sa = stage + wave * 2 * 512;
    uint16_t* sb = stage + BM * BK + wave * 2 * 512;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_global_load_lds(a_src[i] + koff, (PBLK_LDS void*)(sa + i * 512), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
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
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(sa + (a_row0 + i * 32) * BK + ch);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(sb + (b_row0 + j * 32) * BK + ch);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
  };

  // prologue: slabs kb .. kb+NSTAGE-2 into stages 0 .. NSTAGE-2, issued unconditionally
  // (a segment shorter than that reloads its last slab) so the wait counts below are exact
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s) issue(min(kb + s, ke - 1), stage_ptr(s));

  // steady state: every step has NSTAGE-2 later slabs in flight and prefetches one more
  int kt = kb;
  for (; kt + 2 * NSTAGE - 1 <= ke; kt += NSTAGE) {
#pragma unroll
    for (int q = 0; q < NSTAGE; ++q) {
      wait_vm_lgkm0<4 * (NSTAGE - 2)>();
      lds_barrier();
      issue(kt + q + NSTAGE - 1, stage_ptr((q + NSTAGE - 1) % NSTAGE));
      compute(stage_ptr(q));
    }
  }
  // the last (fewer than 2*NSTAGE-1) slabs: drain with full waits
#pragma unroll
  for (int q = 0; q < 2 * NSTAGE - 1; ++q) {
    const int j = kt + q;
    if (j < ke) {
      wait_vm_lgkm0<0>();
      lds_barrier();
      if (j + NSTAGE - 1 < ke) issue(j + NSTAGE - 1, stage_ptr((q + NSTAGE - 1) % NSTAGE));
      compute(stage_ptr(q % NSTAGE));
    }
  }

  if (tl >= 0) {
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
          mine[r4 * NT + tid] = v;
        }
    return;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * TM + i * 32 + lr;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int n = n0 + wn * TN + j * 32 + r4 * 8 + lg * 4;
        if (n >= g.N) continue;
        store_outputs<EPI>(g, m, n, acc[i][j][r4 * 4], acc[i][j][r4 * 4 + 1], acc[i][j][r4 * 4 + 2],
                           acc[i][j][r4 * 4 + 3]);
      }
  }
}

// Sums the k-chunk partials of each tail tile in chunk order and applies the epilogue.
// grid = tail * 4 workgroups of 128 threads; workgroup (tile, quarter) handles the
// main kernel's threads [128*quarter, 128*quarter + 128) of that tile.
template <int EPI>
__global__ __launch_bounds__(128) void gemm_bf16_tail_reduce_kernel(GemmArgs g, GemmSched sk) {
  constexpr int BM = kGemmBM, BN = kGemmBN, NT = kGemmThreads;
  constexpr int WN = 4, TM = 128, TN = 64, FM = 4, FN = 2;
  const int tl = blockIdx.x >> 2;
  const int tid = (blockIdx.x & 3) * 128 + threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 31, lg = lane >> 5;
  int tm, tn;
  tile_coords(sk.dp_units + tl, sk.tiles_m, sk.tiles_n, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;
  constexpr int TILE4 = BM * BN / 4;
  const f32x4* base = reinterpret_cast<const f32x4*>(sk.partials) + int64_t(tl * sk.split) * TILE4;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * TM + i * 32 + lr;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r4 = (i * FN + j) * 4 + q;
        f32x4 s = base[r4 * NT + tid];
        for (int c = 1; c < sk.split; ++c) s += base[int64_t(c) * TILE4 + r4 * NT + tid];
        const int n = n0 + wn * TN + j * 32 + q * 8 + lg * 4;
        if (m < g.M && n < g.N) store_outputs<EPI>(g, m, n, s[0], s[1], s[2], s[3]);
      }
  }
}

}  // namespace pblk
