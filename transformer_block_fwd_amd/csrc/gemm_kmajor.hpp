// GEMM with K-major operands, for the backward pass's gradient GEMMs: C[m, n] = sum_k A(m, k) B(n, k)
// with B stored K-major (element (n, k) at b[k * ldb + n]) and A row-major (a[m * lda + k]) or, with
// AK, K-major too (a[k * lda + m]).  Same tiling, copies-to-LDS pipeline, slab schedule, split-K
// tail and epilogues as the forward GEMM (gemm_bf16.hpp); a K-major operand tile sits in LDS as
// [64 k][256 m or n] and its MFMA fragments come from the LDS transpose read, so the backward
// needs no transposed copies of the weights or activations.  K is a multiple of 64; the K-major
// operands are read for k < K only, the row-major A to the end of its 256-row tile.
#pragma once

#include "attn_bf16.hpp"
#include "gemm_bf16.hpp"

namespace pblk {

// One workgroup's tile (or split-K chunk) bid of the schedule sk.
template <int EPI, bool AK, bool DIRECT>
__device__ __forceinline__ void gemm_kmajor_tile(const GemmArgs& g, const GemmSched& sk, const int bid) {
  constexpr int BM = kGemmBM, BN = kGemmBN, BK = kGemmBK, NT = kGemmThreads;
  constexpr int MI = 8, NJ = 8;   // 16x16 MFMA tiles per wavefront (128 x 128)
  constexpr int P = MI * NJ / 2;  // MFMAs per phase (half a 32-deep k-step)
  constexpr int NRF = MI + NJ;    // operand fragments per k-step
  constexpr int NC = 16;          // copy instructions per wavefront and slab (8 per operand)
  constexpr int C12 = (2 * NC + 2) / 3;  // of them issued in phases 2 and 3
  __shared__ __attribute__((aligned(1024))) uint16_t a0[kGemmHalf];
  __shared__ __attribute__((aligned(1024))) uint16_t b0[kGemmHalf];
  __shared__ __attribute__((aligned(1024))) uint16_t a1[kGemmHalf];
  __shared__ __attribute__((aligned(1024))) uint16_t b1[kGemmHalf];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  int L, kb, ke, tl = -1, chunk = 0;
  if (bid < sk.dp_units) {
    L = xcd_remap(bid, sk.dp_units);
    kb = 0;
    ke = sk.KT;
  } else {
    const int nu = sk.tail * sk.split;
    const int u = xcd_remap(bid - sk.dp_units, nu);
    chunk = u / sk.tail;
    tl = u % sk.tail;
    L = sk.dp_units + tl;
    kb = int((int64_t(chunk) * sk.KT) / sk.split);
    ke = int((int64_t(chunk + 1) * sk.KT) / sk.split);
  }
  int tm, tn;
  tile_coords(L, sk.tiles_m, sk.tiles_n, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // Copies.  Row-major A (as the forward GEMM): instruction i of wave w fills 1 KiB block 8w + i
  // = rows 64w + 8i + l/8, lane l physical chunk l%8 fetched from logical (l%8) ^ ((row >> 1) & 7).
  // K-major operands: block 8w + i = k rows 16w + 2i + l/32 of 512 bytes (256 m or n values),
  // lane l physical chunk l%32 fetched from logical (l%32) ^ (4 * (krow & 3)); columns past the
  // operand's extent are clamped (they feed rows or columns that are never stored).
  const uint32_t lda_b = uint32_t(g.lda) * 2u, ldb_b = uint32_t(g.ldb) * 2u;
  uint32_t offa[2], offb[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int lck = (lane & 31) ^ (4 * ((2 * p + (lane >> 5)) & 3));
    offb[p] = uint32_t(lane >> 5) * ldb_b + uint32_t(min(n0 + lck * 8, g.N - 8)) * 2u;
    if constexpr (AK) {
      offa[p] = uint32_t(lane >> 5) * lda_b + uint32_t(min(m0 + lck * 8, g.M - 8)) * 2u;
    } else {
      const int lc = (lane & 7) ^ (4 * p + (lane >> 4));
      offa[p] = uint32_t(lane >> 3) * lda_b + uint32_t(lc << 4);
    }
  }
  const uint8_t* a_blk = reinterpret_cast<const uint8_t*>(g.a) + (AK ? int64_t(0) : int64_t(m0 + wave * 64) * lda_b);
  // copy instruction i (0..7) of slab kt, A or B
  auto issue_a = [&](int kt, uint16_t* sa, int i) __attribute__((always_inline)) {
    const int64_t krow0 = int64_t(kt) * BK + 16 * wave + 2 * i;  // K-major: first k row of the block
    const uint8_t* ga = AK ? a_blk + krow0 * lda_b + offa[i & 1]
                           : a_blk + int64_t(8 * i) * lda_b + uint32_t(kt) * (BK * 2) + offa[i & 1];
    __builtin_amdgcn_global_load_lds(ga, (PBLK_LDS void*)(sa + (wave * 8 + i) * 512), 16, 0, 0);
  };
  auto issue_b = [&](int kt, uint16_t* sb, int i) __attribute__((always_inline)) {
    const int64_t krow0 = int64_t(kt) * BK + 16 * wave + 2 * i;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(g.b) + krow0 * ldb_b + offb[i & 1],
                                     (PBLK_LDS void*)(sb + (wave * 8 + i) * 512), 16, 0, 0);
  };
  auto issue = [&](int kt, uint16_t* sa, uint16_t* sb, int i0, int i1) __attribute__((always_inline)) {
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      issue_a(kt, sa, i);
      issue_b(kt, sb, i);
    }
  };

  // Fragment reads (16x16x32 operands: lane l holds row or column 16 * block + l % 16 and the
  // 8 k of k-group l / 16 of a 32-deep k-step ks).  Row-major A: row w*128 + 16 i + l % 16,
  // logical chunk 4 ks + l / 16 at physical chunk (4 ks + l / 16) ^ ((l % 16 >> 1) & 7).
  // K-major operand block t (m or n = w*128 + 16 t + l % 16): two transpose reads
  // (ds_read_b64_tr_b16) in which lane 16G + j addresses k row 32 ks + 8 G + j / 4 (+4 for the
  // second) and columns w*128 + 16 t + 4 (j % 4) .. +3, so lane 16G + j receives k =
  // 32 ks + 8 G + 0..3 (then 4..7) of column 16 t + j: the MFMA operand.
  const int lr = lane & 15, lq = lane >> 4;
  uint32_t rda[2], trb, tra;
  {
    const int G = lane >> 4, j = lane & 15;
    const int krow = 8 * G + (j >> 2);
    const int sw = 4 * ((j >> 2) & 3);            // 4 * (krow & 3)
    const int cb = (wn * 128 + 4 * (j & 3)) >> 3;  // logical chunk of the first column
    const int ca = (wm * 128 + 4 * (j & 3)) >> 3;
    trb = uint32_t(krow * 512 + (((cb) ^ sw) << 4) + 8 * (j & 1));
    tra = uint32_t(krow * 512 + (((ca) ^ sw) << 4) + 8 * (j & 1));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      rda[ks] = uint32_t(lr * 128 + (((4 * ks + lq) ^ ((lr >> 1) & 7)) << 4)) + uint32_t(wm * 128 * 128);
  }

  f32x4 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 fa[2][MI], fb[2][NJ];  // one fragment buffer per k-step of a slab
  // the K-major fragment of block t (16 columns) of k-step ks: the physical chunk of column
  // 16 t + c0 is (logical + 2t) ^ sw, the XOR touching only bits 2..3 of the chunk index
  auto trfrag = [&](const uint8_t* base, uint32_t off, int t, int ks) __attribute__((always_inline)) {
    const uint8_t* p = base + (off ^ uint32_t((2 * t) << 4)) + ks * 32 * 512;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * 512));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    const u32x4 u = {l2.x, l2.y, h2.x, h2.y};
    return __builtin_bit_cast(bf16x8, u);
  };
  // fragment x (0 .. NRF-1) of k-step ks into buffer buf, in the order the MFMAs consume them:
  // A block 0, B blocks 0 .. NJ-1, A blocks 1 .. MI-1
  auto rd1 = [&](int buf, const uint16_t* sa, const uint16_t* sb, int ks, int x) __attribute__((always_inline)) {
    const uint8_t* pa = reinterpret_cast<const uint8_t*>(sa);
    const uint8_t* pb = reinterpret_cast<const uint8_t*>(sb);
    const bool is_b = x >= 1 && x <= NJ;
    const int blk = is_b ? x - 1 : (x == 0 ? 0 : x - NJ);
    if (is_b) {
      fb[buf][blk] = trfrag(pb, trb, blk, ks);
    } else if constexpr (AK) {
      fa[buf][blk] = trfrag(pa, tra, blk, ks);
    } else {
      fa[buf][blk] = *reinterpret_cast<const bf16x8*>(pa + rda[ks] + blk * 16 * 128);
    }
  };
  // copy c (0 .. NC-1): the A and B instructions of i = c / 2 alternately
  auto copy1 = [&](int kt, uint16_t* sa, uint16_t* sb, int c) __attribute__((always_inline)) {
    if (c & 1) issue_b(kt, sb, c >> 1);
    else issue_a(kt, sa, c >> 1);
  };
  // One phase, as in the forward GEMM: the P MFMAs of k-step buf over fragment rows
  // [h MI/2, (h+1) MI/2), fragment read x behind MFMA x (x < nr), and in copy phase cq (1..3)
  // copy c behind MFMA position c * 3P / NC of the three phases.  Tied inline-asm MFMAs (see
  // gemm_bf16.hpp): memory operations keep their program order around them.
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
  // slab t+1 into stage (na, nb) in flight: the forward GEMM's four phases.
  auto slab = [&](int t, const uint16_t* ca, const uint16_t* cb, uint16_t* na, uint16_t* nb) __attribute__((always_inline)) {
    uint16_t* wa = const_cast<uint16_t*>(ca);
    uint16_t* wb = const_cast<uint16_t*>(cb);
    const int tc = min(t + 2, ke - 1);  // branch-free: past the end the last slab is fetched again
    phase(0, 0, NRF, 1, ca, cb, 1, 0, tc, wa, wb);
    wait_lgkm0();   // own reads of this stage done
    lds_barrier();  // everyone's: the stage is free
    phase(0, 1, 0, 0, ca, cb, 0, 1, tc, wa, wb);
    phase(1, 0, 0, 0, ca, cb, 0, 2, tc, wa, wb);
    wait_vm_lgkm0<C12>();  // own copies of slab t+1 landed (those of slab t+2 may be in flight)
    lds_barrier();         // everyone's: slab t+1 is complete
    phase(1, 1, NRF, 0, na, nb, 0, 3, tc, wa, wb);
  };

  issue(kb, a0, b0, 0, 8);
  issue(min(kb + 1, ke - 1), a1, b1, 0, 8);
  wait_vm_lgkm0<16>();  // slab kb landed
  lds_barrier();
#pragma unroll
  for (int x = 0; x < NRF; ++x) rd1(0, a0, b0, 0, x);
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
    gemm_epilogue<EPI, BM>(g, acc, a0, b0, a1, b1, part, m0, n0, wm, wn);
  }
}

template <int EPI, bool AK, bool DIRECT = false>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_kmajor_kernel(GemmArgs g, GemmSched sk) {
  gemm_kmajor_tile<EPI, AK, DIRECT>(g, sk, int(blockIdx.x));
}

// Two independent K-major GEMMs in one launch (the two weight gradients): workgroups
// 0 .. s0.dp_units-1 compute the first, the rest the second, so that the second's tiles fill the
// compute units the first's last partial wave leaves idle.  Both schedules hold whole tiles only.
template <int EPI, bool AK, bool DIRECT>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_kmajor_pair_kernel(GemmArgs g0, GemmSched s0, GemmArgs g1,
                                                                            GemmSched s1) {
  const int bid = int(blockIdx.x);
  if (bid < s0.dp_units)
    gemm_kmajor_tile<EPI, AK, DIRECT>(g0, s0, bid);
  else
    gemm_kmajor_tile<EPI, AK, DIRECT>(g1, s1, bid - s0.dp_units);
}

// Work decomposition of one K-major GEMM on G resident workgroups: whole waves of tiles, then the
// remaining tiles in k-chunks when they fill at most half a wave.
inline GemmSched gemm_kmajor_sched(const GemmArgs& g, float* partials, int G) {
  GemmSched sk;
  sk.partials = partials;
  sk.unit_base = 0;
  sk.wave_units = G;
  sk.tiles_m = int((g.M + kGemmBM - 1) / kGemmBM);
  sk.tiles_n = int((g.N + kGemmBN - 1) / kGemmBN);
  sk.KT = g.K / kGemmBK;
  const int64_t T = int64_t(sk.tiles_m) * sk.tiles_n;
  const int64_t waves = T / G;
  sk.tail = int(T - waves * G);
  sk.dp_units = int(waves * G);
  sk.split = sk.tail > 0 ? int(std::max<int64_t>(1, std::min<int64_t>(G / sk.tail, sk.KT))) : 1;
  if (sk.split == 1) {  // more than half a wave left over: cutting k would not add workgroups
    sk.dp_units = int(T);
    sk.tail = 0;
  }
  return sk;
}

template <int EPI, bool AK>
void launch_gemm_kmajor(const GemmArgs& g, float* partials, int G, hipStream_t s) {
  const GemmSched sk = gemm_kmajor_sched(g, partials, G);
  const unsigned grid = unsigned(sk.dp_units + sk.tail * sk.split);
  bool launched = false;
  if constexpr (EPI == kEpiResidual || EPI == kEpiF32 || EPI == kEpiGeluBwd) {
    if (gemm_direct_ok<EPI>(g)) {  // the lane-swap epilogue (every gradient GEMM without a bias)
      hipLaunchKernelGGL((gemm_kmajor_kernel<EPI, AK, true>), dim3(grid), dim3(kGemmThreads), 0, s, g, sk);
      launched = true;
    }
  }
  if (!launched) hipLaunchKernelGGL((gemm_kmajor_kernel<EPI, AK>), dim3(grid), dim3(kGemmThreads), 0, s, g, sk);
  if (sk.tail > 0)
    hipLaunchKernelGGL((gemm_bf16_tail_reduce_kernel<EPI>), dim3(unsigned(sk.tail * 32)), dim3(256), 0, s, g, sk);
}

// Two independent K-major GEMMs: one launch when neither leaves tiles to split along k, both take
// the direct epilogue and a partial wave is left over; otherwise one launch after the other.
template <int EPI, bool AK>
void launch_gemm_kmajor_pair(const GemmArgs& g0, const GemmArgs& g1, float* partials, int G, hipStream_t s) {
  if constexpr (EPI == kEpiResidual || EPI == kEpiF32 || EPI == kEpiGeluBwd) {
    const GemmSched s0 = gemm_kmajor_sched(g0, partials, G), s1 = gemm_kmajor_sched(g1, partials, G);
    if (s0.tail == 0 && s1.tail == 0 && gemm_direct_ok<EPI>(g0) && gemm_direct_ok<EPI>(g1) &&
        (s0.dp_units % G != 0 || s1.dp_units % G != 0)) {
      hipLaunchKernelGGL((gemm_kmajor_pair_kernel<EPI, AK, true>), dim3(unsigned(s0.dp_units + s1.dp_units)),
                         dim3(kGemmThreads), 0, s, g0, s0, g1, s1);
      return;
    }
  }
  launch_gemm_kmajor<EPI, AK>(g0, partials, G, s);
  launch_gemm_kmajor<EPI, AK>(g1, partials, G, s);
}

}  // namespace pblk
