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
// start first.
//
// Per 64-key tile a wavefront computes S^T = K Q^T with the 32x32x16 bf16
// MFMA: the key fragment is the first operand and the query fragment (kept in
// registers for the whole kernel) the second, so each lane ends up owning one
// query (lane % 32) and 32 of the 64 keys.  That is exactly the operand layout
// the second product needs for P: O^T = V^T P^T takes P straight from the
// score registers, and V^T comes from an LDS copy of the value tile stored
// transposed (row = head dim, padded to keep the strided 8-byte reads on
// distinct banks).  Row max / row sum are per lane plus one exchange with the
// lane 32 apart.  Tiles wholly inside the band skip the mask; a wavefront
// whose 32 queries cannot see any key of the tile skips the tile.
#pragma once

#include "common.hpp"

namespace pblk {

struct AttnArgs {
  const uint16_t* qkv;  // [B*S, ld_qkv]: Q | K | V, head-major within each
  int64_t ld_qkv;
  uint16_t* o;          // [B*S, ld_o]: head h at columns [h*hd, (h+1)*hd)
  int64_t ld_o;
  int B, S, H, W;
  float scale_log2;     // log2(e) / sqrt(hd)
};

constexpr int kAttnBQ = 128;
constexpr int kAttnBKV = 64;
// Largest gap (log2 units) between a tile max and the reference max before rescaling.
constexpr float kRescaleSlack = 8.0f;
constexpr bf16x2 kOnesBf16x2 = {(__bf16)1.0f, (__bf16)1.0f};

// Value held by the lane 32 apart (lanes l and l^32 exchange through a half-wave swap).
__device__ __forceinline__ float other_half(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  // lanes < 32: r[1] holds the upper half's value, r[0] its own; lanes >= 32 the reverse
  return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

template <int HD>
__global__ __launch_bounds__(256, 2) void swa_attn_bf16_kernel(AttnArgs a) {
  constexpr int BQ = kAttnBQ, BKV = kAttnBKV;
  constexpr int KCH = HD / 8;          // 16-byte chunks per K row
  constexpr int VT_LD = BKV + 4;       // padded V^T row, in elements
  constexpr int K_RPP = 256 / KCH;     // K rows per load pass
  constexpr int K_LD = BKV / K_RPP;    // K load passes per tile
  constexpr int V_LD = KCH / 8;        // V row-pair chunks per thread per tile
  constexpr int NH = HD / 32;          // 32-wide head-dim tiles of the output
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][BKV * HD];
  __shared__ __attribute__((aligned(16))) uint16_t vt[2][HD * VT_LD];

  const int S = a.S, W = a.W;
  const int nqt = (S + BQ - 1) / BQ;
  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int qt = nqt - 1 - blockIdx.x / BH;
  const int b = bh / a.H, h = bh % a.H;
  const int A = a.H * HD;
  const uint16_t* qbase = a.qkv + int64_t(b) * S * a.ld_qkv + h * HD;
  const uint16_t* kbase = qbase + A;
  const uint16_t* vbase = qbase + 2 * A;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  const int q0 = qt * BQ;
  const int wq0 = q0 + wave * 32;
  const int my_q = wq0 + lr;

  bf16x8 qf[HD / 16];
  {
    const uint16_t* qp = qbase + int64_t(min(my_q, S - 1)) * a.ld_qkv + lg * 8;
#pragma unroll
    for (int kk = 0; kk < HD / 16; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 16);
  }

  const int q_last = min(q0 + BQ, S) - 1;
  const int t_begin = max(0, q0 - W + 1) / BKV;
  const int t_end = q_last / BKV;

  // K loader: chunk kc of row kr (+ pass * K_RPP); V loader: rows 2*vp, 2*vp+1, chunk vc (+ 8 * pass)
  const int kc = tid % KCH, kr = tid / KCH;
  const int vp = tid & 31, vc = tid >> 5;
  u32x4 rk[K_LD], rv[V_LD][2];
  auto load_kv = [&](int t) {
    const int j0 = t * BKV;
#pragma unroll
    for (int p = 0; p < K_LD; ++p) {
      const int j = min(j0 + kr + p * K_RPP, S - 1);
      rk[p] = *reinterpret_cast<const u32x4*>(kbase + int64_t(j) * a.ld_qkv + kc * 8);
    }
#pragma unroll
    for (int p = 0; p < V_LD; ++p) {
      const int c = vc + p * 8;
      const int j_a = min(j0 + 2 * vp, S - 1), j_b = min(j0 + 2 * vp + 1, S - 1);
      rv[p][0] = *reinterpret_cast<const u32x4*>(vbase + int64_t(j_a) * a.ld_qkv + c * 8);
      rv[p][1] = *reinterpret_cast<const u32x4*>(vbase + int64_t(j_b) * a.ld_qkv + c * 8);
    }
  };
  auto store_kv = [&](int st) {
#pragma unroll
    for (int p = 0; p < K_LD; ++p) {
      const int r = kr + p * K_RPP;
      *reinterpret_cast<u32x4*>(&ks[st][r * HD + ((kc ^ (r & 7)) << 3)]) = rk[p];
    }
#pragma unroll
    for (int p = 0; p < V_LD; ++p) {
      const int c = vc + p * 8;
      const uint32_t ra[4] = {rv[p][0].x, rv[p][0].y, rv[p][0].z, rv[p][0].w};
      const uint32_t rb[4] = {rv[p][1].x, rv[p][1].y, rv[p][1].z, rv[p][1].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // head-dim 8c+2e (low halves) and 8c+2e+1 (high halves) of keys 2vp, 2vp+1
        const uint32_t lo = (ra[e] & 0xFFFFu) | (rb[e] << 16);
        const uint32_t hi = (ra[e] >> 16) | (rb[e] & 0xFFFF0000u);
        *reinterpret_cast<uint32_t*>(&vt[st][(c * 8 + 2 * e) * VT_LD + 2 * vp]) = lo;
        *reinterpret_cast<uint32_t*>(&vt[st][(c * 8 + 2 * e + 1) * VT_LD + 2 * vp]) = hi;
      }
    }
  };

  f32x16 oacc[NH];
#pragma unroll
  for (int t = 0; t < NH; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;
  float m_run = -INFINITY, l_part = 0.f;  // m_run: reference max in log2 units

  load_kv(t_begin);
  store_kv(0);
  // Every load issued so far (Q fragments included) must be complete here: otherwise the
  // compiler carries the Q loads into the loop as pending and makes the first products of
  // every tile wait for that tile's prefetch as well.
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  __syncthreads();

  for (int t = t_begin; t <= t_end; ++t) {
    const int cur = (t - t_begin) & 1;
    if (t < t_end) load_kv(t + 1);
    const int j0 = t * BKV;
    const bool active = (wq0 < S) && (j0 <= wq0 + 31) && (j0 + BKV - 1 >= wq0 - W + 1);
    if (active) {
      f32x16 sacc[2];
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[t2][r] = 0.f;
        const int row = t2 * 32 + lr;
#pragma unroll
        for (int kk = 0; kk < HD / 16; ++kk) {
          const bf16x8 kf =
              *reinterpret_cast<const bf16x8*>(&ks[cur][row * HD + (((kk * 2 + lg) ^ (lr & 7)) << 3)]);
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
      // P in bf16, as the B operand of O^T = V^T P^T: fragment tt covers keys tt*16 .. tt*16+15.
      // The row sum adds the rounded weights, the same values the product uses.
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
#pragma unroll
      for (int ht = 0; ht < NH; ++ht) {
        const uint16_t* vrow = &vt[cur][(ht * 32 + lr) * VT_LD + 4 * lg];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + tt * 16);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + tt * 16 + 8);
          const u32x4 u = {lo.x, lo.y, hi.x, hi.y};
          oacc[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, u), pf[tt], oacc[ht], 0, 0, 0);
        }
      }
    }
    if (t < t_end) store_kv(cur ^ 1);
    __syncthreads();
  }

  const float l = l_part + other_half(l_part);
  if (my_q < S) {
    const float inv = 1.0f / l;
    uint16_t* orow = a.o + (int64_t(b) * S + my_q) * a.ld_o + h * HD;
#pragma unroll
    for (int ht = 0; ht < NH; ++ht)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int hd = ht * 32 + 8 * r4 + 4 * lg;
        u32x2 w;
        w.x = pack_bf16x2(oacc[ht][4 * r4 + 0] * inv, oacc[ht][4 * r4 + 1] * inv);
        w.y = pack_bf16x2(oacc[ht][4 * r4 + 2] * inv, oacc[ht][4 * r4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + hd) = w;
      }
  }
}

}  // namespace pblk
