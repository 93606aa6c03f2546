// Sliding-window causal attention on gfx950 matrix cores (bf16 in, fp32 math).
//
// Method: each query i attends to keys j in [max(0, i-W+1), i] (MegaScale
// guided reading, section 2: a fixed window of nearby tokens), with exact
// softmax weights (section 4: exact attention, FlashAttention-2).  The kernel
// is flash-style -- key/value tiles stream through LDS and the softmax is
// kept online in fp32 -- but it only visits the key tiles that intersect the
// window band of its query tile, so its cost is proportional to S*W.
//
// Work decomposition: one workgroup = one (sequence, head, 128-query tile),
// four wavefronts of 32 queries each, key/value tiles of 64.  Query tiles are
// dispatched last-first so that, for long causal windows, the longest tiles
// start first.  A launch may cover only the query positions [q_lo, q_hi) of
// each sequence (keys still reach back W-1 positions before q_lo).
//
// Data movement: K and V tiles are copied global -> LDS by the load unit
// (global_load_lds, 16 bytes per lane, 1 KiB per wave instruction) into two
// stages; tile t+1 is in flight while tile t is computed.  Both tiles keep
// their row-major [key][head-dim] layout; the 16-byte chunks of each row are
// XOR-permuted so that the fragment reads below hit distinct LDS banks.
//
// Per 64-key tile a wavefront computes S^T = K Q^T with the 32x32x16 bf16
// MFMA: the key fragment is the first operand and the query fragment (kept in
// registers for the whole kernel) the second, so each lane ends up owning one
// query (lane % 32) and 32 of the 64 keys.  That is exactly the operand layout
// the second product needs for P: O^T = V^T P^T takes P straight from the
// score registers.  The V^T fragments come from the row-major V tile through
// the LDS transpose read (ds_read_b64_tr_b16): within each 16-lane group,
// lane 4a+b receives element b of the 8-byte pieces addressed by lanes a,
// a+4, a+8, a+12, so four lanes addressing four consecutive keys at the same
// head-dim columns hand every lane four keys of one head-dim column.
// Row max / row sum are per lane plus one exchange with the lane 32 apart.
// Tiles wholly inside the band skip the mask; a wavefront whose 32 queries
// cannot see any key of the tile skips the tile's arithmetic.
#pragma once

#include "common.hpp"

namespace pblk {

struct AttnArgs {
  const uint16_t* qkv;  // [B*S, ld_qkv]: Q | K | V, head-major within each
  int64_t ld_qkv;
  uint16_t* o;          // [B*S, ld_o]: head h at columns [h*hd, (h+1)*hd)
  int64_t ld_o;
  int B, S, H, W;
  int q_lo, q_hi;       // query positions [q_lo, q_hi) of every sequence (0, S for all)
  float scale_log2;     // log2(e) / sqrt(hd)
  float* lse;           // optional [B, H, S]: log2 of each query's softmax denominator in the
                        // exponent's units, so that p_ij = 2^(s_ij * scale_log2 - lse) (backward pass)
};

constexpr int kAttnBQ = 128;
constexpr int kAttnBKV = 64;
constexpr int kAttnThreads = 256;
// Largest gap (log2 units) between a tile max and the reference max before rescaling.
constexpr float kRescaleSlack = 8.0f;
constexpr bf16x2 kOnesBf16x2 = {(__bf16)1.0f, (__bf16)1.0f};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Value held by the lane 32 apart (lanes l and l^32 exchange through a half-wave swap).
__device__ __forceinline__ float other_half(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  // lanes < 32: r[1] holds the upper half's value, r[0] its own; lanes >= 32 the reverse
  return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

// LDS chunk permutations (16-byte chunks within a row of HD bf16 values).
// K rows are read 16 rows x one chunk per pass: all 16 rows must land on distinct
// bank groups.  V rows are read (transposed) 4 rows x 4 consecutive chunks per pass.
template <int HD>
__device__ __forceinline__ int swz_k(int row) {
  return HD == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int HD>
__device__ __forceinline__ int swz_v(int row) {
  return HD == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

__device__ __forceinline__ void attn_wait_copies() {
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
}
__device__ __forceinline__ void attn_barrier() { asm volatile("s_barrier" ::: "memory"); }

// LDS of one attention workgroup: K and V tiles of 64 rows in two stages.
template <int HD>
struct AttnLds {
  static constexpr int TB = kAttnBKV * HD * 2;
  uint8_t k0[TB], v0[TB], k1[TB], v1[TB];
};

// One workgroup's (sequence, head, query tile) of the launch, blk in [0, B * H * tiles) (unsigned:
// a signed division here cost the kernel 40 registers and spills), with
// the calling kernel's own LDS (declared there: each kernel's LDS then sits at addresses known
// when it is compiled, which the fragment reads fold into their offsets).
template <int HD>
__device__ __forceinline__ void swa_attn_block(const AttnArgs& a, unsigned blk, AttnLds<HD>& lds) {
  constexpr int BQ = kAttnBQ, BKV = kAttnBKV;
  constexpr int NW = kAttnThreads / 64;
  constexpr int ROWB = HD * 2;         // bytes per K/V row
  constexpr int TB = BKV * ROWB;       // bytes per K or V tile
  constexpr int NI = TB / 1024;        // 1 KiB copy instructions per tile
  constexpr int NIW = NI / NW;         // ... issued by each wave
  constexpr int NH = HD / 32;          // 32-wide head-dim tiles of the output
  constexpr int NKK = HD / 16;         // 16-deep slices of the QK^T contraction
  static_assert(NIW * NW == NI, "copy instructions split evenly over the waves");
  uint8_t* const k_st0 = lds.k0;
  uint8_t* const v_st0 = lds.v0;
  uint8_t* const k_st1 = lds.k1;
  uint8_t* const v_st1 = lds.v1;

  const int S = a.S, W = a.W;
  const int nqt = (a.q_hi - a.q_lo + BQ - 1) / BQ;
  const int BH = a.B * a.H;
  const int bh = blk % BH;
  const int qt = nqt - 1 - blk / BH;
  const int b = bh / a.H, h = bh % a.H;
  const int A = a.H * HD;
  const uint16_t* qbase = a.qkv + int64_t(b) * S * a.ld_qkv + h * HD;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(qbase + A);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(qbase + 2 * A);
  const uint32_t ldb = uint32_t(a.ld_qkv) * 2u;  // row pitch in bytes

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: copy targets in SGPRs
  const int lr = lane & 31, lg = lane >> 5;
  const int q0 = a.q_lo + qt * BQ;
  const int wq0 = q0 + wave * 32;
  const int my_q = wq0 + lr;

  bf16x8 qf[NKK];
  {
    const uint16_t* qp = qbase + int64_t(min(my_q, S - 1)) * a.ld_qkv + lg * 8;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 16);
  }

  const int q_last = min(q0 + BQ, a.q_hi) - 1;
  const int t_begin = max(0, q0 - W + 1) / BKV;
  const int t_end = q_last / BKV;

  // Copies: instruction c of this wave fills LDS bytes [1024 i, 1024 i + 1024) of a tile,
  // i = wave * NIW + c; lane L writes 16 bytes at 1024 i + 16 L = row r, physical chunk pc,
  // and fetches the row's logical chunk pc ^ swz(r).  Offsets are relative to the tile's
  // first row; rows past the last query of the launch are clamped to it (masked anyway).
  auto copy_row = [&](int c) { return (1024 * (wave * NIW + c) + 16 * lane) / ROWB; };
  auto copy_pc = [&](int c) { return ((16 * lane) % ROWB) / 16; };
  // (fixed array bounds: the host compiler drops the kernel's launch stub when a lambda
  // captures an array whose bound depends on the template parameter)
  static_assert(NIW <= 4 && NKK <= 8 && NH <= 4, "offset arrays sized for hd <= 128");
  uint32_t koff[4], voff[4];
#pragma unroll
  for (int c = 0; c < NIW; ++c) {
    const int r = copy_row(c), pc = copy_pc(c);
    koff[c] = uint32_t(r) * ldb + uint32_t((pc ^ swz_k<HD>(r)) << 4);
    voff[c] = uint32_t(r) * ldb + uint32_t((pc ^ swz_v<HD>(r)) << 4);
  }
  // Key rows at or past q_hi are never attended by this launch's queries (causal), and in a
  // position-chunked forward they have not been projected yet: rows are clamped to q_hi - 1, so
  // no stale value (a NaN times a zero weight is NaN) reaches the P V product.
  const int kv_end = a.q_hi;
  auto issue = [&](int t, uint8_t* ks, uint8_t* vs) {
    const int j0 = t * BKV;
    const uint8_t* kt = kbase + int64_t(j0) * ldb;
    const uint8_t* vt = vbase + int64_t(j0) * ldb;
    if (j0 + BKV <= kv_end) {
#pragma unroll
      for (int c = 0; c < NIW; ++c) {
        __builtin_amdgcn_global_load_lds(kt + koff[c], (lds_void*)(ks + 1024 * (wave * NIW + c)), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vt + voff[c], (lds_void*)(vs + 1024 * (wave * NIW + c)), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int c = 0; c < NIW; ++c) {
        const int r = copy_row(c), pc = copy_pc(c);
        const uint32_t rb = uint32_t(min(j0 + r, kv_end - 1) - j0) * ldb;
        __builtin_amdgcn_global_load_lds(kt + rb + uint32_t((pc ^ swz_k<HD>(r)) << 4),
                                         (lds_void*)(ks + 1024 * (wave * NIW + c)), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vt + rb + uint32_t((pc ^ swz_v<HD>(r)) << 4),
                                         (lds_void*)(vs + 1024 * (wave * NIW + c)), 16, 0, 0);
      }
    }
  };

  // Fragment read offsets within a tile.  K: row t2*32 + lr, logical chunk 2kk + lg.
  // V (transpose read): lane 16G + j addresses key row 4*(G/2) + j/4 (+ tt*16 + 8*half) and
  // head-dim columns ht*32 + 16*(G%2) + 4*(j%4) .. +3; its swizzle depends on j/4 only.
  uint32_t kro[8], vro[4];
  {
    const int krow = lr;  // t2 adds 32 rows: same swizzle (swz_k depends on row % 16)
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) kro[kk] = uint32_t(krow * ROWB + (((2 * kk + lg) ^ swz_k<HD>(krow)) << 4));
    const int G = lane >> 4, j = lane & 15;
    const int vrow = 4 * (G >> 1) + (j >> 2);
#pragma unroll
    for (int ht = 0; ht < NH; ++ht) {
      const int lch = ht * 4 + 2 * (G & 1) + ((j & 3) >> 1);
      vro[ht] = uint32_t(vrow * ROWB + ((lch ^ swz_v<HD>(vrow)) << 4) + (j & 1) * 8);
    }
  }

  f32x16 oacc[NH];
#pragma unroll
  for (int t = 0; t < NH; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;
  float m_run = -INFINITY, l_part = 0.f;  // m_run: reference max in log2 units

  auto compute = [&](int t, const uint8_t* ks, const uint8_t* vs) {
    const int j0 = t * BKV;
    const bool active = (wq0 < a.q_hi) && (j0 <= wq0 + 31) && (j0 + BKV - 1 >= wq0 - W + 1);
    if (!active) return;
    f32x16 sacc[2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[t2][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + kro[kk] + t2 * 32 * ROWB);
        sacc[t2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], sacc[t2], 0, 0, 0);
      }
    }
    // lane owns query my_q and keys j0 + t2*32 + 8*(r/4) + 4*lg + (r%4); a key is in the
    // band iff 0 <= my_q - j < W, one unsigned compare against the lane's offset
    const bool full = (j0 + BKV - 1 <= wq0) && (j0 >= wq0 + 31 - W + 1);
    if (!full) {
      const int diff = my_q - j0 - 4 * lg;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int koff = t2 * 32 + 8 * (r >> 2) + (r & 3);
          sacc[t2][r] = (uint32_t(diff - koff) < uint32_t(W)) ? sacc[t2][r] : -INFINITY;
        }
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sacc[t2][r]);
    // the other 32 keys of this query sit in the lane 32 apart
    const float m_tile = fmaxf(mloc, other_half(mloc)) * a.scale_log2;
    // The running max (log2 units) only moves when a tile exceeds it by more than
    // kRescaleSlack: until then the unnormalised weights stay below 2^kRescaleSlack and
    // the accumulators need no rescaling.  The final division by the row sum makes the
    // result independent of which reference max was used.
    if (__builtin_amdgcn_ballot_w64(m_tile > m_run + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = __builtin_amdgcn_exp2f(m_run - ((m_new == -INFINITY) ? 0.f : m_new));
      m_run = m_new;
      l_part *= alpha;
#pragma unroll
      for (int ht = 0; ht < NH; ++ht)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[ht][r] *= alpha;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    // P in bf16, as the B operand of O^T = V^T P^T: fragment tt covers keys tt*16 .. tt*16+15
    // (lane group lg holds keys tt*16 + 4lg + 0..3 and tt*16 + 8 + 4lg + 0..3).  The row sum
    // adds the rounded weights, the same values the product uses.
    bf16x8 pf[4];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        bf16x2 w[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const f32x2 pp = {__builtin_amdgcn_exp2f(fmaf(sacc[t2][8 * hh + 2 * e2], a.scale_log2, -m_use)),
                            __builtin_amdgcn_exp2f(fmaf(sacc[t2][8 * hh + 2 * e2 + 1], a.scale_log2, -m_use))};
          w[e2] = __builtin_convertvector(pp, bf16x2);
          l_part = __builtin_amdgcn_fdot2_f32_bf16(w[e2], kOnesBf16x2, l_part, false);
        }
        pf[t2 * 2 + hh] = bf16x8{w[0][0], w[0][1], w[1][0], w[1][1], w[2][0], w[2][1], w[3][0], w[3][1]};
      }
    // V^T fragment (ht, tt): keys tt*16 + 4lg + 0..3 from the first transpose read, keys
    // tt*16 + 8 + 4lg + 0..3 from the second, head-dim ht*32 + lane%32.
#pragma unroll
    for (int ht = 0; ht < NH; ++ht)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const uint8_t* p = vs + vro[ht] + tt * 16 * ROWB;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 8 * ROWB));
        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
        const u32x4 u = {lo2.x, lo2.y, hi2.x, hi2.y};
        oacc[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, u), pf[tt], oacc[ht], 0, 0, 0);
      }
  };

  // Two stages, tile t in stage (t - t_begin) % 2.  Each step: wait for this wave's copies
  // of tile t (and, on the first step, the Q loads), barrier (all copies of tile t landed;
  // every wave is done with tile t-1, whose stage now takes tile t+1), copy tile t+1,
  // compute tile t.
  auto step = [&](int t, const uint8_t* ks, const uint8_t* vs, uint8_t* kn, uint8_t* vn) {
    attn_wait_copies();
    attn_barrier();
    if (t < t_end) issue(t + 1, kn, vn);
    compute(t, ks, vs);
  };
  issue(t_begin, k_st0, v_st0);
  const int n_tiles = t_end - t_begin + 1;
  int t = t_begin;
  for (int p = 0; p + 2 <= n_tiles; p += 2, t += 2) {
    step(t, k_st0, v_st0, k_st1, v_st1);
    step(t + 1, k_st1, v_st1, k_st0, v_st0);
  }
  if (n_tiles & 1) step(t, k_st0, v_st0, k_st1, v_st1);

  const float l = l_part + other_half(l_part);
  if (my_q < a.q_hi) {
    if (a.lse != nullptr && lg == 0)
      a.lse[(int64_t(b) * a.H + h) * S + my_q] = ((m_run == -INFINITY) ? 0.f : m_run) + log2f(l);
    const float inv = 1.0f / l;
    uint16_t* orow = a.o + (int64_t(b) * S + my_q) * a.ld_o + h * HD;
#pragma unroll
    for (int ht = 0; ht < NH; ++ht)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int hd = ht * 32 + 8 * r4 + 4 * lg;
        const f32x2 p0 = {oacc[ht][4 * r4 + 0] * inv, oacc[ht][4 * r4 + 1] * inv};
        const f32x2 p1 = {oacc[ht][4 * r4 + 2] * inv, oacc[ht][4 * r4 + 3] * inv};
        const u32x2 w = {__builtin_bit_cast(uint32_t, __builtin_convertvector(p0, bf16x2)),
                         __builtin_bit_cast(uint32_t, __builtin_convertvector(p1, bf16x2))};
        *reinterpret_cast<u32x2*>(orow + hd) = w;
      }
  }
}

template <int HD>
__global__ __launch_bounds__(kAttnThreads, 2) void swa_attn_bf16_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) AttnLds<HD> lds;
  swa_attn_block<HD>(a, blockIdx.x, lds);
}

}  // namespace pblk
