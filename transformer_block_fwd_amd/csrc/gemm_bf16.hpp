// bf16 GEMM on gfx950 matrix cores: C[m, n] = sum_k X[m, k] * Wt[n, k].
//
// Both operands are K-contiguous (activations [M, K] and nn.Linear-style
// weights [N, K]), which is what the 16x16x32 bf16 MFMA wants: every lane
// feeds 8 consecutive k of one row from a single 16-byte LDS read.
//
// Tile: 256 x 256 outputs per workgroup of 4 wavefronts (one per SIMD), laid
// out 2 (M) x 2 (N); each wavefront owns 128 x 128 as 8 x 8 MFMA tiles of
// 16 x 16 whose fp32 accumulators (256 per lane) live in the AGPR file.  The
// 16x16x32 form sustains more throughput on this chip than 32x32x16 at the same
// operand traffic (it moves fewer accumulator bits per flop).
//
// Pipeline: the k loop walks 64-wide slabs through two LDS stages (each an A
// and a B array of 32 KiB, separately named so the compiler can see that
// filling one never aliases reading another).  Global data moves straight
// into LDS with global_load_lds_dwordx4; one instruction fills 1 KiB = 8 rows
// of 128 bytes, the 16-byte chunk index inside a row XORed with
// ((row >> 1) & 7) on the source side and undone on the fragment reads (the 16
// rows one read pass touches then hit 16 distinct bank groups).  A slab is two
// 32-deep k-steps of 64 MFMAs per wavefront, run as four phases of 32:
//   phase 1 (k-step 0, rows 0..3): the fragments of k-step 1 are read behind
//     its MFMAs, so the whole stage is consumed early; a barrier then frees it;
//   phases 2..4: the 16 copies of slab t+2 into the freed stage, spread evenly
//     over their 96 MFMAs (a CU's load path takes about 64 bytes per clock: bursts
//     of copies stall the MFMAs queued behind them);
//   before phase 4: wait for this wave's copies of slab t+1, barrier; phase 4
//     also reads k-step 0 of slab t+1 behind its MFMAs.
// The interleave is written out in program order (see the phase lambda).
//
// Operand bounds: A rows are read up to the end of the last 256-row tile (the
// caller allocates A in whole 256-row tiles; rows past M are never stored); B
// has N % 8 == 0 rows and an 8-row block past N is clamped as a whole to the
// last block.  K % 64 == 0.
//
// Schedule: data-parallel waves plus a split-K tail.  With G workgroups
// resident at once (one per CU), the first floor(T / G) * G tiles run whole,
// one workgroup each, in k-lockstep.  The remaining T mod G tiles would fill
// only part of a last wave, so each is cut into `split` k-chunks
// (split = G / tail) that run together as one more wave.  A chunk stores its
// fp32 partial tile (row-major, written through the same LDS staging as the
// epilogue); a second small kernel sums the chunks of each tail tile in chunk
// order with coalesced reads (bitwise deterministic, no atomics, no
// cross-workgroup fences) and applies the epilogue.
//
// When whole waves come first and the remainder would be cut in two k-chunks (between a
// third and a half of a wave of tiles), it runs instead as twice as many 128 x 256
// half-height tiles in a second launch of the BM = 128 form: one wave, every tile whole,
// no partials.  Before either: when 256 x 192 tiles (the BN = 192 form, each wavefront
// 128 x 96 as 8 x 6 MFMA tiles) fill whole waves where 256 x 256 tiles leave a partial one,
// the GEMM runs as those, every tile whole (the 175B shard's output GEMM: 8 x 64 = 512 tiles,
// two waves, against 384 = 1.5 waves of 256 x 256).
//
// L2 locality: workgroup ids are remapped so each XCD (id mod 8) owns a
// contiguous run of work units, and units are ordered in groups of 8 M-tiles
// (M fastest): the 32 workgroups an XCD runs at once cover an 8 (M) x 4 (N)
// block of tiles at the same k, so they share activation and weight slabs in
// that XCD's L2.
//
// Epilogue, two forms chosen by the host (template parameter DIRECT):
//   direct, for launches with no bias, rotary step, tanh GeLU or residual (the plain and the
//     training forward, every gradient GEMM: weights, fp32 output, GeLU backward) and their
//     split-K partials: one v_permlane16_swap per accumulator register pairs up two 16-column
//     MFMA blocks so that every lane holds 8 consecutive columns of one row, stored with one
//     16-byte write (no LDS, no barriers);
//   staged, for the rest: the accumulators go out through LDS in four rounds of 64 rows
//     (fp32, chunk-permuted), so every global store is a full 16-byte piece of a row and a
//     wavefront writes whole 512-byte rows.
//   kEpiSplitGelu: columns < nsplit are stored as bf16 to out0 (the Q|K|V
//     projections); columns >= nsplit get the exact GeLU and go to out1 at
//     column off1 + (n - nsplit) (the FC1 activations next to the attention
//     output, so the second GEMM reads one K-contiguous operand).
//   kEpiResidual: optional residual x added in fp32, one rounding to bf16 (without it, a
//     plain bf16 store).
//   kEpiGeluBwd: columns < nsplit stored as bf16 to out0; columns >= nsplit multiplied by
//     GeLU'(F) (F read from pre) and stored to out1 at column off1 + (n - nsplit).
//   kEpiF32: fp32 store to out_f32 (row stride ld0).
// Optional variant steps, in fp32 before the rounding: a bias per column (first), the
// rotary embedding of the q and k columns, the tanh form of GeLU.
// nsplit, the strides and off1 are multiples of 8.
#pragma once

#include "backward.hpp"
#include "common.hpp"
#include "rope.hpp"

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
  // Variant switches of the epilogue (all off when zero / null):
  const uint16_t* bias;  // [N] added to every row before anything else
  const float* rope;     // (cos, sin) per (position, pair): rotary embedding of columns n < rope_n
  int rope_n;            // columns [0, rope_n) are q and k heads of width hd
  int seq;               // rows are sequences of seq positions (position = m % seq)
  int hd;
  int gelu_tanh;         // 1: tanh-form GeLU on the FC1 columns
  // Backward-pass use: the FC1 pre-activation F [M, N - nsplit] (row stride ld_pre), stored by
  // kEpiSplitGelu when non-null and read by kEpiGeluBwd; fp32 output of kEpiF32.
  uint16_t* pre;
  int64_t ld_pre;
  float* out_f32;
};

constexpr int kGemmBM = 256, kGemmBN = 256, kGemmBK = 64, kGemmThreads = 256;
constexpr int kGemmHalf = 256 * kGemmBK;  // elements of one operand tile of a stage (32 KiB)

// Work decomposition of one GEMM launch (grid = dp_units + tail * split).
struct GemmSched {
  float* partials;  // [tail * split][kGemmBM][kGemmBN] fp32, row-major partial tile per (tail tile, chunk)
  int tiles_m, tiles_n;
  int KT;           // k slabs per tile
  int dp_units;     // tiles computed whole (whole waves, or all tiles when a split would be 1)
  int tail;         // tiles computed in k-chunks
  int split;        // k-chunks per tail tile
  int unit_base;    // half-height launch: unit u is half u % 2 of 256-row tile unit_base + u / 2
  int wave_units;   // publishing launches: workgroups resident at once (one wave)
};

constexpr int kGroupM = 8;

// Publication of finished row chunks by the output GEMM (position-chunked forward).  Chunk k
// holds positions [floor(k S / n), floor((k+1) S / n)) of every sequence; a row r is position
// r % S of sequence r / S.  Tiles run in publication order (rows of earlier chunks first);
// every tile that finishes adds one to the counter of each chunk its rows touch, and the tile
// that brings counter k to need[k] (the number of tiles touching chunk k in this launch pair)
// resets the counter and sets flags[k] = epoch with release semantics at device scope.
constexpr int kMaxChunks = 64;
struct RowPublish {
  uint32_t* counters;  // [n] zero between calls (the last tile of a chunk resets its counter)
  uint32_t* flags;     // [n] caller's flags
  uint32_t epoch;
  int n;               // chunks, 1 .. kMaxChunks
  int S;               // positions per sequence
  int B;               // sequences: M-tiles run position-major over them when S % 256 == 0
  int group_m;         // M-tiles per group of the publication order (M fastest inside a group)
  uint32_t need[kMaxChunks];
};

// Chunk of position p (0 <= p < S) among n chunks: the k with floor(k S / n) <= p < floor((k+1) S / n).
__host__ __device__ __forceinline__ int chunk_of(int p, int S, int n) {
  return int((int64_t(p + 1) * n - 1) / S);
}
// Bit k set iff some row in [r0, r1) lies in chunk k.
__host__ __device__ __forceinline__ uint64_t chunk_mask(int r0, int r1, int S, int n) {
  uint64_t mask = 0;
  for (int r = r0; r < r1;) {
    const int b = r / S;
    const int end = min((b + 1) * S, r1);
    const int ka = chunk_of(r - b * S, S, n), kb = chunk_of(end - 1 - b * S, S, n);
    const uint64_t upto = kb >= 63 ? ~uint64_t(0) : ((uint64_t(1) << (kb + 1)) - 1);
    mask |= upto & ~((uint64_t(1) << ka) - 1);
    r = end;
  }
  return mask;
}
// 256-row tile coordinates of tile index L in publication order: groups of group_m M-tiles
// (in position-major order over the sequences when whole tiles hold one sequence each), M
// fastest inside a group.
__host__ __device__ __forceinline__ void tile_coords_pub(int L, int tiles_m, int tiles_n, const RowPublish& pub,
                                                         int* tm, int* tn) {
  const int gm = pub.group_m;
  const int group = gm * tiles_n;
  const int first = (L / group) * gm;
  const int gsz = min(tiles_m - first, gm);
  const int r = L % group;
  const int im = first + r % gsz;
  *tn = r / gsz;
  if (pub.B > 1 && pub.S % 256 == 0) {
    const int per_seq = pub.S / 256;
    *tm = (im % pub.B) * per_seq + im / pub.B;
  } else {
    *tm = im;
  }
}

// Contiguous-per-XCD renumbering of workgroup ids 0 .. n-1 (id mod 8 picks the XCD).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int xcd = bid & 7, idx = bid >> 3;
  const int per = n >> 3, rem = n & 7;
  return (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}
// Tile coordinates of linear tile index L: groups of kGroupM M-tiles, M fastest.
__host__ __device__ __forceinline__ void tile_coords(int L, int tiles_m, int tiles_n, int* tm, int* tn) {
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
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Workgroup barrier that no memory access may be moved across (the waits are explicit).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Epilogue of 8 consecutive columns n .. n+7 of row m, one 16-byte store.  Already loaded, when
// not null: xres, the residual's 8 values (kEpiResidual); bpre, the bias of the 8 columns.
template <int EPI>
__device__ __forceinline__ void store_chunk8(const GemmArgs& g, int m, int n, f32x4 lo, f32x4 hi,
                                             const u32x4* xres = nullptr, const u32x4* bpre = nullptr) {
  float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  uint16_t* dst;
  if (g.bias != nullptr) {
    const u32x4 br = bpre != nullptr ? *bpre : *reinterpret_cast<const u32x4*>(g.bias + n);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] += __uint_as_float(br[e] << 16);
      v[2 * e + 1] += __uint_as_float(br[e] & 0xFFFF0000u);
    }
  }
  if constexpr (EPI == kEpiSplitGelu) {
    if (n < g.nsplit) {
      if (n < g.rope_n) rope_rotate8(v, g.rope, m % g.seq, n & (g.hd - 1), g.hd);
      dst = g.out0 + int64_t(m) * g.ld0 + n;
    } else {
      if (g.pre != nullptr) {
        const u32x4 pw = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                          pack_bf16x2(v[6], v[7])};
        *reinterpret_cast<u32x4*>(g.pre + int64_t(m) * g.ld_pre + (n - g.nsplit)) = pw;
      }
      if (g.gelu_tanh) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = gelu_tanh(v[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = gelu_erf_bf16out(v[e]);
      }
      dst = g.out1 + int64_t(m) * g.ld1 + g.off1 + (n - g.nsplit);
    }
  } else if constexpr (EPI == kEpiGeluBwd) {
    if (n < g.nsplit) {
      dst = g.out0 + int64_t(m) * g.ld0 + n;
    } else {
      const u32x4 fr = *reinterpret_cast<const u32x4*>(g.pre + int64_t(m) * g.ld_pre + (n - g.nsplit));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] *= gelu_erf_grad(__uint_as_float(fr[e] << 16));
        v[2 * e + 1] *= gelu_erf_grad(__uint_as_float(fr[e] & 0xFFFF0000u));
      }
      dst = g.out1 + int64_t(m) * g.ld1 + g.off1 + (n - g.nsplit);
    }
  } else if constexpr (EPI == kEpiF32) {
    f32x4* o = reinterpret_cast<f32x4*>(g.out_f32 + int64_t(m) * g.ld0 + n);
    o[0] = f32x4{v[0], v[1], v[2], v[3]};
    o[1] = f32x4{v[4], v[5], v[6], v[7]};
    return;
  } else {
    if (g.resid != nullptr) {
      const u32x4 xr = xres != nullptr ? *xres : *reinterpret_cast<const u32x4*>(g.resid + int64_t(m) * g.ldr + n);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] += __uint_as_float(xr[e] << 16);
        v[2 * e + 1] += __uint_as_float(xr[e] & 0xFFFF0000u);
      }
    }
    dst = g.out0 + int64_t(m) * g.ld0 + n;
  }
  const u32x4 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
  *reinterpret_cast<u32x4*>(dst) = o;
}

// Epilogue of a 256-column tile through LDS, BM/64 rounds: in round i every wave stages its
// rows wm*BM/2 + i*32 + 0..31 as fp32 (stage pair i&1 of the LDS arrays, the wm half in its own
// array, 16-byte chunks XOR-permuted by row), then all threads store 64 full rows: bf16 outputs
// with 16-byte writes, or, for a split-K chunk, its fp32 partial tile (row-major BM x 256) with
// 32-byte writes.  Lane l of MFMA tile (i, j) holds row 16 i + l % 16 and columns
// 16 j + 4 (l / 16) + 0..3; the caller has made sure no wave still reads the LDS arrays.
//
// The store loop stays rolled: unrolled, its copies of every variant's branches made the
// epilogue longer than the instruction cache, and it ran at the speed of instruction fetch.
// The residual form is the exception: its loads are all issued at the start, each thread's 8
// rows per round for every round, so that their latency is paid once per tile (one load in
// flight at a time costs a memory latency per row), and its store loop is unrolled so that
// they stay in registers.
template <int EPI, int BM, int MI, int NJ, int BN = kGemmBN>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& g, f32x4 (&acc)[MI][NJ], uint16_t* a0, uint16_t* b0,
                                              uint16_t* a1, uint16_t* b1, float* part, int m0, int n0, int wm,
                                              int wn) {
  constexpr int R = BM / 64;
  constexpr bool kRes = EPI == kEpiResidual;
  static_assert(BN == 2 * 16 * NJ && BN <= 256, "two wavefronts of NJ 16-column blocks across the tile");
  const int tid = threadIdx.x, lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int c0 = (tid & 31) * 2, nl = (tid & 31) * 8;
  const bool col_ok = nl < BN;  // a 192-column tile leaves the last 8 threads of each row idle
  // every row a thread stores has the same 8 columns: their bias is loaded once
  u32x4 bias8 = {0u, 0u, 0u, 0u};
  if (g.bias != nullptr && part == nullptr && col_ok && n0 + nl < g.N) bias8 = *reinterpret_cast<const u32x4*>(g.bias + n0 + nl);
  u32x4 xr[kRes ? R : 1][8];
  if constexpr (kRes) {
    if (part == nullptr && g.resid != nullptr) {
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          const int r = p * 8 + (tid >> 5);
          const int ml = (r >> 5) * (BM / 2) + i * 32 + (r & 31);
          if (col_ok && m0 + ml < g.M && n0 + nl < g.N)
            xr[i][p] = *reinterpret_cast<const u32x4*>(g.resid + int64_t(m0 + ml) * g.ldr + (n0 + nl));
        }
    }
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    float* mine = reinterpret_cast<float*>((i & 1) ? (wm ? b1 : a1) : (wm ? b0 : a0));
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int row = 16 * h + lr, c = wn * (BN / 8) + 4 * j + lq;  // c: 16-byte chunk of the row
        *reinterpret_cast<f32x4*>(mine + row * 256 + ((c ^ lr) << 2)) = acc[2 * i + h][j];
      }
    lds_barrier();
#pragma unroll(kRes ? 8 : 1)
    for (int p = 0; p < 8; ++p) {
      const int r = p * 8 + (tid >> 5);
      const int half = r >> 5, lrow = r & 31;
      // a select between the LDS arrays themselves (through a pointer array the compiler loses
      // the address space and reads LDS with flat loads)
      const float* src = reinterpret_cast<const float*>((i & 1) ? (half ? b1 : a1) : (half ? b0 : a0));
      const f32x4 lo = *reinterpret_cast<const f32x4*>(src + lrow * 256 + ((c0 ^ (lrow & 15)) << 2));
      const f32x4 hi = *reinterpret_cast<const f32x4*>(src + lrow * 256 + (((c0 + 1) ^ (lrow & 15)) << 2));
      const int ml = half * (BM / 2) + i * 32 + lrow;
      if (!col_ok) {
      } else if (part != nullptr) {
        f32x4* dst = reinterpret_cast<f32x4*>(part + ml * BN + nl);
        dst[0] = lo;
        dst[1] = hi;
      } else if (m0 + ml < g.M && n0 + nl < g.N) {
        if constexpr (kRes) store_chunk8<EPI>(g, m0 + ml, n0 + nl, lo, hi, g.resid != nullptr ? &xr[i][p] : nullptr, &bias8);
        else store_chunk8<EPI>(g, m0 + ml, n0 + nl, lo, hi, nullptr, &bias8);
      }
    }
  }
}

// Whether a launch takes a GEMM's direct (lane-swap, no LDS) epilogue form: the plain forms, with
// no bias, rotary step, tanh GeLU or residual (the saved pre-activation of the training forward is
// allowed), fp32 output, and the GeLU-backward form.
template <int EPI>
__host__ __device__ inline bool gemm_direct_ok(const GemmArgs& g) {
  if constexpr (EPI == kEpiSplitGelu)
    return g.bias == nullptr && g.rope_n == 0 && g.gelu_tanh == 0;
  else if constexpr (EPI == kEpiResidual)
    return g.bias == nullptr && g.resid == nullptr;
  else if constexpr (EPI == kEpiF32 || EPI == kEpiGeluBwd)
    return g.bias == nullptr;
  else
    return false;
}

// 8 consecutive columns n .. n+7 of row m for the direct epilogue's forms: Q|K|V columns stored
// as they are, FC1 columns through the exact GeLU (their pre-activation stored too when the
// training forward asks for it), the output GEMM's plain rounding, fp32, or the GeLU-backward
// form (FC1 columns scaled by GeLU' of the saved pre-activation).
template <int EPI>
__device__ __forceinline__ void store_plain8(const GemmArgs& g, int m, int n, const f32x4& lo, const f32x4& hi) {
  if constexpr (EPI == kEpiF32) {
    f32x4* o = reinterpret_cast<f32x4*>(g.out_f32 + int64_t(m) * g.ld0 + n);
    o[0] = lo;
    o[1] = hi;
    return;
  }
  float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  uint16_t* dst;
  if constexpr (EPI == kEpiSplitGelu) {
    if (n < g.nsplit) {
      dst = g.out0 + int64_t(m) * g.ld0 + n;
    } else {
      if (g.pre != nullptr) {
        const u32x4 pw = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                          pack_bf16x2(v[6], v[7])};
        *reinterpret_cast<u32x4*>(g.pre + int64_t(m) * g.ld_pre + (n - g.nsplit)) = pw;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = gelu_erf_bf16out(v[e]);
      dst = g.out1 + int64_t(m) * g.ld1 + g.off1 + (n - g.nsplit);
    }
  } else if constexpr (EPI == kEpiGeluBwd) {
    if (n < g.nsplit) {
      dst = g.out0 + int64_t(m) * g.ld0 + n;
    } else {
      const u32x4 fr = *reinterpret_cast<const u32x4*>(g.pre + int64_t(m) * g.ld_pre + (n - g.nsplit));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] *= gelu_erf_grad(__uint_as_float(fr[e] << 16));
        v[2 * e + 1] *= gelu_erf_grad(__uint_as_float(fr[e] & 0xFFFF0000u));
      }
      dst = g.out1 + int64_t(m) * g.ld1 + g.off1 + (n - g.nsplit);
    }
  } else {
    dst = g.out0 + int64_t(m) * g.ld0 + n;
  }
  const u32x4 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
  *reinterpret_cast<u32x4*>(dst) = o;
}

// Epilogue without LDS staging, for launches that gemm_direct_ok accepts (the host picks the
// kernel form: with both epilogues in one kernel the register allocator spills accumulators), and
// their split-K partials.
// For every 16-row block i and pair of 16-column blocks (2 jp, 2 jp + 1), one v_permlane16_swap
// per accumulator register exchanges 16-lane rows between the two blocks' accumulators: lane l
// of block j holds row l % 16, columns 4 (l / 16) + 0..3; after the swap the first register set
// holds columns 0..3 and the second 4..7 of one 8-column chunk, block 2 jp for lanes 0-15 and
// 32-47 (chunk columns 0 and 8), block 2 jp + 1 for lanes 16-31 and 48-63 (columns 16 and 24 of
// the pair).  Each lane then stores one 16-byte piece (a wave writes 64 contiguous bytes of each
// of 16 rows), or for a split-K chunk its fp32 partial (row-major BM x BN, 32-byte writes).
template <int EPI, int BM, int MI, int NJ, int BN>
__device__ __forceinline__ void gemm_epilogue_direct(const GemmArgs& g, f32x4 (&acc)[MI][NJ], float* part, int m0,
                                                     int n0, int wm, int wn) {
  static_assert(NJ % 2 == 0, "pairs of 16-column blocks");
  const int lane = threadIdx.x & 63;
  const int mrow = wm * (BM / 2) + (lane & 15);
  const int ncol = wn * (BN / 2) + 16 * ((lane >> 4) & 1) + 8 * (lane >> 5);
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int jp = 0; jp < NJ / 2; ++jp) {
      f32x4 lo, hi;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[i][2 * jp][k]),
                                                        __float_as_uint(acc[i][2 * jp + 1][k]), false, false);
        lo[k] = __uint_as_float(r[0]);
        hi[k] = __uint_as_float(r[1]);
      }
      const int ml = mrow + 16 * i, nl = ncol + 32 * jp;
      if (part != nullptr) {
        f32x4* dst = reinterpret_cast<f32x4*>(part + ml * BN + nl);
        dst[0] = lo;
        dst[1] = hi;
      } else if (m0 + ml < g.M && n0 + nl < g.N) {
        store_plain8<EPI>(g, m0 + ml, n0 + nl, lo, hi);
      }
    }
}

template <int EPI, int BM = kGemmBM, bool PUB = false, int BN = kGemmBN, bool DIRECT = false>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_bf16_kernel(GemmArgs g, GemmSched sk, RowPublish pub) {
  static_assert(BM == 256 || BM == 128, "tile height 256 or 128");
  static_assert(BN == 256 || (BN == 192 && BM == 256 && !PUB), "tile width 256, or 192 for whole waves");
  static_assert(!DIRECT || ((EPI == kEpiSplitGelu || EPI == kEpiResidual || EPI == kEpiF32) && !PUB),
                "direct epilogue forms");
  constexpr int BK = kGemmBK, NT = kGemmThreads;
  constexpr int MI = BM / 32, NJ = BN / 32;  // 16x16 MFMA tiles per wavefront (BM/2 x BN/2)
  constexpr int P = MI * NJ / 2;       // MFMAs per phase (half a 32-deep k-step)
  constexpr int NR = MI + NJ;          // fragment reads per k-step
  constexpr int NA = BM / 32;          // A copy instructions per wavefront and slab
  constexpr int NB = BN / 32;          // B copy instructions per wavefront and slab
  constexpr int NC = NA + NB;          // copy instructions per wavefront and slab
  constexpr int C12 = (2 * NC + 2) / 3;  // of them issued in phases 2 and 3 (see copy_pos)
  __shared__ __attribute__((aligned(1024))) uint16_t a0[kGemmHalf];
  __shared__ __attribute__((aligned(1024))) uint16_t b0[kGemmHalf];
  __shared__ __attribute__((aligned(1024))) uint16_t a1[kGemmHalf];
  __shared__ __attribute__((aligned(1024))) uint16_t b1[kGemmHalf];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  int L, kb, ke, tl = -1, chunk = 0;
  if (PUB) {
    // publication order wave by wave: wave w runs units [wG, wG + G), each XCD a contiguous run
    const int G = sk.wave_units;
    const int w0 = (int(blockIdx.x) / G) * G;
    L = w0 + xcd_remap(int(blockIdx.x) - w0, min(G, sk.dp_units - w0));
    kb = 0;
    ke = sk.KT;
  } else if (int(blockIdx.x) < sk.dp_units) {
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
  if constexpr (BM == 128) {
    // half-height tiles of the 256 x 256 tiling (tiles_m counts 256-row tiles)
    if (PUB) tile_coords_pub(sk.unit_base + L / 2, sk.tiles_m, sk.tiles_n, pub, &tm, &tn);
    else tile_coords(sk.unit_base + L / 2, sk.tiles_m, sk.tiles_n, &tm, &tn);
    tm = 2 * tm + (L & 1);
  } else {
    if (PUB) tile_coords_pub(L, sk.tiles_m, sk.tiles_n, pub, &tm, &tn);
    else tile_coords(L, sk.tiles_m, sk.tiles_n, &tm, &tn);
  }
  const int m0 = tm * BM, n0 = tn * BN;

  // Copies: B instruction i (0 .. NB-1) of wave w fills 1 KiB block NB w + i of the B tile =
  // rows (BN/4) w + 8i + l/8; lane l writes physical chunk l%8, fetched from logical chunk
  // (l%8) ^ ((row >> 1) & 7) = (l%8) ^ (4*(i&1) + l/16) (BN/4 is a multiple of 16).
  const uint32_t lda_b = uint32_t(g.lda) * 2u, ldb_b = uint32_t(g.ldb) * 2u;
  uint32_t offa[2], offb[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int lc = (lane & 7) ^ (4 * p + (lane >> 4));
    offa[p] = uint32_t(lane >> 3) * lda_b + uint32_t(lc << 4);
    offb[p] = uint32_t(lane >> 3) * ldb_b + uint32_t(lc << 4);
  }
  // A: wave w's NA instructions fill rows w*BM/4 .. +BM/4 (1 KiB block w*NA + i = rows
  // w*BM/4 + 8i + l/8: the same row swizzle, since BM/4 is a multiple of 16)
  const uint8_t* a_blk = reinterpret_cast<const uint8_t*>(g.a) + int64_t(m0 + wave * (BM / 4)) * lda_b;
  // copy instruction i of slab kt: A (i < NA) and B (i < NB)
  auto issue_a = [&](int kt, uint16_t* sa, int i) __attribute__((always_inline)) {
    const uint32_t kofs = uint32_t(kt) * (BK * 2);
    __builtin_amdgcn_global_load_lds(a_blk + int64_t(8 * i) * lda_b + kofs + offa[i & 1],
                                     (PBLK_LDS void*)(sa + (wave * NA + i) * 512), 16, 0, 0);
  };
  auto issue_b = [&](int kt, uint16_t* sb, int i) __attribute__((always_inline)) {
    const uint32_t kofs = uint32_t(kt) * (BK * 2);
    const int brow = min(n0 + wave * (BN / 4) + 8 * i, g.N - 8);
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(g.b) + int64_t(brow) * ldb_b + kofs + offb[i & 1],
                                     (PBLK_LDS void*)(sb + (wave * NB + i) * 512), 16, 0, 0);
  };
  // copy instructions i0 .. i1-1 of slab kt
  auto issue = [&](int kt, uint16_t* sa, uint16_t* sb, int i0, int i1) __attribute__((always_inline)) {
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      if (i < NA) issue_a(kt, sa, i);
      if (i < NB) issue_b(kt, sb, i);
    }
  };
  // Copy c (0 .. NC-1) of a slab: the A and B instructions of i = c / 2 alternately while both
  // have one, then the remaining instructions of the other operand.
  constexpr int NMIN = NA < NB ? NA : NB;
  auto copy1 = [&](int kt, uint16_t* sa, uint16_t* sb, int c) __attribute__((always_inline)) {
    if (c < 2 * NMIN) {
      if (c & 1) issue_b(kt, sb, c >> 1);
      else issue_a(kt, sa, c >> 1);
    } else if (NA > NB) {
      issue_a(kt, sa, c - NB);
    } else {
      issue_b(kt, sb, c - NA);
    }
  };

  // Fragment reads (16x16x32 operands): lane l reads row 16 * block + l % 16, the 8 k of
  // logical chunk 4 ks + l / 16 of k-step ks, at physical chunk (4 ks + l / 16) ^ ((l % 16 >> 1) & 7);
  // byte offsets within an operand tile.
  const int lr = lane & 15, lq = lane >> 4;
  uint32_t rda[2], rdb[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const uint32_t o = uint32_t(lr * 128 + (((4 * ks + lq) ^ ((lr >> 1) & 7)) << 4));
    rda[ks] = o + uint32_t(wm * (BM / 2) * 128);
    rdb[ks] = o + uint32_t(wn * (BN / 2) * 128);
  }

  f32x4 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 fa[2][MI], fb[2][NJ];  // one fragment buffer per k-step of a slab
  // Fragment read x (0 .. NR-1) of k-step ks into buffer buf, in the order the MFMAs consume
  // them: A row block 0, B column blocks 0 .. NJ-1, A row blocks 1 .. MI-1.
  auto rd1 = [&](int buf, const uint16_t* sa, const uint16_t* sb, int ks, int x) __attribute__((always_inline)) {
    const uint8_t* pa = reinterpret_cast<const uint8_t*>(sa);
    const uint8_t* pb = reinterpret_cast<const uint8_t*>(sb);
    if (x == 0) fa[buf][0] = *reinterpret_cast<const bf16x8*>(pa + rda[ks]);
    else if (x <= NJ) fb[buf][x - 1] = *reinterpret_cast<const bf16x8*>(pb + rdb[ks] + (x - 1) * 16 * 128);
    else fa[buf][x - NJ] = *reinterpret_cast<const bf16x8*>(pa + rda[ks] + (x - NJ) * 16 * 128);
  };
  // One phase: the P MFMAs of k-step buf over fragment rows [h MI/2, (h+1) MI/2) (all NJ column
  // blocks), with fragment read x (x < nr: k-step rks of stage (rsa, rsb) into buffer rbuf)
  // behind MFMA x.  In copy phase cq (1..3; 0: none) the copies of slab tc into stage (wa, wb)
  // are spread evenly: copy c goes behind MFMA position copy_pos(c) = c * 3P / NC of the three
  // phases' 3P MFMAs.  A CU's load path moves about 64 bytes per clock, so the 4 KiB that four
  // wavefronts' copies carry per MFMA position must not come in bursts: a wavefront whose copy
  // cannot issue holds back the MFMAs behind it.
  //
  // The MFMA is written as inline asm with its accumulator tied ("+a"): the builtin's untied
  // 16x16 form lets the register allocator rotate the accumulators through copies on every
  // loop trip.  Volatile asm also keeps every memory operation in program order around it,
  // which fixes the interleave written here.  The only hazards left to the code are those of
  // the accumulators (the fragment registers a read overwrites were last read at least 8
  // MFMAs earlier): the zeroing before the first MFMA and the epilogue's reads after the last
  // one are separated from them by explicit wait states.
  auto phase = [&](int buf, int h, int nr, int rbuf, const uint16_t* rsa, const uint16_t* rsb, int rks, int cq, int tc,
                   uint16_t* wa, uint16_t* wb) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < P; ++x) {
      const int i = h * (MI / 2) + x / NJ, j = x % NJ;
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[i][j]) : "v"(fb[buf][j]), "v"(fa[buf][i]));
      if (x < nr) rd1(rbuf, rsa, rsb, rks, x);
      if (cq > 0) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
          if (c * 3 * P / NC == (cq - 1) * P + x) copy1(tc, wa, wb, c);
      }
    }
  };

  // Slab t in stage (ca, cb), its k-step 0 fragments requested into buffer 0, the copies of
  // slab t+1 into stage (na, nb) in flight.  Four phases of P MFMAs: k-step 0 then k-step 1,
  // each in two halves of its fragment rows.
  //   1: k-step 1's fragments are read behind the first NR MFMAs; then the stage is consumed
  //      (own reads waited for, a barrier for everyone's) and is free for slab t+2;
  //   2, 3: copies 0 .. C12-1 of slab t+2 spread over the MFMAs;
  //   before 4: this wave's copies of slab t+1 landed, a barrier: slab t+1 is complete;
  //   4: the rest of the copies, and the reads of slab t+1's k-step 0 fragments behind the
  //      MFMAs.
  auto slab = [&](int t, const uint16_t* ca, const uint16_t* cb, uint16_t* na, uint16_t* nb) __attribute__((always_inline)) {
    uint16_t* wa = const_cast<uint16_t*>(ca);
    uint16_t* wb = const_cast<uint16_t*>(cb);
    const int tc = min(t + 2, ke - 1);  // branch-free: past the end the last slab is fetched again
    phase(0, 0, NR, 1, ca, cb, 1, 0, tc, wa, wb);
    wait_lgkm0();   // own reads of this stage done
    lds_barrier();  // everyone's: the stage is free
    phase(0, 1, 0, 0, ca, cb, 0, 1, tc, wa, wb);
    phase(1, 0, 0, 0, ca, cb, 0, 2, tc, wa, wb);
    wait_vm_lgkm0<C12>();  // own copies of slab t+1 landed (those of slab t+2 may be in flight)
    lds_barrier();         // everyone's: slab t+1 is complete
    phase(1, 1, NR, 0, na, nb, 0, 3, tc, wa, wb);
  };

  constexpr int NMAX = NA > NB ? NA : NB;
  issue(kb, a0, b0, 0, NMAX);
  issue(min(kb + 1, ke - 1), a1, b1, 0, NMAX);
  wait_vm_lgkm0<NC>();  // slab kb landed
  lds_barrier();
#pragma unroll
  for (int x = 0; x < NR; ++x) rd1(0, a0, b0, 0, x);
  // the accumulators' zeroing (VALU writes) before their first MFMA read
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 4");
  __builtin_amdgcn_sched_barrier(0);
  const int n = ke - kb;
  int kt = kb;
  for (int p = 0; p + 2 <= n; p += 2, kt += 2) {
    slab(kt, a0, b0, a1, b1);
    slab(kt + 1, a1, b1, a0, b0);
  }
  if (n & 1) slab(kt, a0, b0, a1, b1);
  // the last MFMAs' accumulator writes before any other instruction reads them
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0): no copy may still be writing this workgroup's LDS

  // Epilogue: split-K chunks store their fp32 partial tile, every other tile its outputs.
  float* part = tl >= 0 ? sk.partials + int64_t(tl * sk.split + chunk) * (BM * BN) : nullptr;
  if constexpr (DIRECT) {
    gemm_epilogue_direct<EPI, BM, MI, NJ, BN>(g, acc, part, m0, n0, wm, wn);
  } else {
    lds_barrier();  // every wave is past its last fragment read
    gemm_epilogue<EPI, BM, MI, NJ, BN>(g, acc, a0, b0, a1, b1, part, m0, n0, wm, wn);
  }
  if constexpr (PUB) {
    __builtin_amdgcn_s_waitcnt(0x0070);  // this thread's stores of the tile are done
    __syncthreads();
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // the tile's rows, written back
      uint64_t mask = chunk_mask(m0, min(m0 + BM, g.M), pub.S, pub.n);
      while (mask != 0) {
        const int k = __builtin_ctzll(mask);
        mask &= mask - 1;
        const uint32_t old = __hip_atomic_fetch_add(pub.counters + k, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old + 1 == pub.need[k]) {
          // the chunk's last tile: every other tile's release precedes its increment
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
          __hip_atomic_store(pub.counters + k, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(pub.flags + k, pub.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
}

// Sums the k-chunk partials of each tail tile in chunk order and applies the epilogue.
// grid = tail * 32 workgroups of 256 threads; workgroup (tile, b) handles rows 8b .. 8b+7
// of the tile, thread t row 8b + t/32 and columns 8*(t%32) .. +7: coalesced 32-byte
// partial reads and 16-byte output writes.
// Rows 8 blk .. 8 blk + 7 of the tail's tiles in order (32 row groups per tile).
template <int EPI>
__device__ __forceinline__ void tail_reduce_rows(const GemmArgs& g, const GemmSched& sk, int blk) {
  constexpr int BM = kGemmBM, BN = kGemmBN;
  const int tl = blk >> 5;
  const int r = (blk & 31) * 8 + (threadIdx.x >> 5);
  const int c = (threadIdx.x & 31) * 8;
  int tm, tn;
  tile_coords(sk.dp_units + tl, sk.tiles_m, sk.tiles_n, &tm, &tn);
  const int m = tm * BM + r, n = tn * BN + c;
  if (m >= g.M || n >= g.N) return;
  const f32x4* src = reinterpret_cast<const f32x4*>(sk.partials + int64_t(tl * sk.split) * (BM * BN) + r * BN + c);
  f32x4 lo = src[0], hi = src[1];
  for (int k = 1; k < sk.split; ++k) {
    src += (BM * BN) / 4;
    lo += src[0];
    hi += src[1];
  }
  store_chunk8<EPI>(g, m, n, lo, hi);
}

template <int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_tail_reduce_kernel(GemmArgs g, GemmSched sk) {
  tail_reduce_rows<EPI>(g, sk, blockIdx.x);
}

}  // namespace pblk
