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

template <int EPI, bool AK>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_kmajor_kernel(GemmArgs g, GemmSched sk) {
  constexpr int BM = kGemmBM, BN = kGemmBN, BK = kGemmBK, NT = kGemmThreads;
  constexpr int FM = 4, FN = 4;  // 32x32 MFMA tiles per wavefront (128 x 128)
  __shared__ __attribute__((aligned(1024))) uint16_t a0[kGemmHalf];
  __shared__ __attribute__((aligned(1024))) uint16_t b0[kGemmHalf];
  __shared__ __attribute__((aligned(1024))) uint16_t a1[kGemmHalf];
  __shared__ __attribute__((aligned(1024))) uint16_t b1[kGemmHalf];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lg = lane >> 5;

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
  auto issue = [&](int kt, uint16_t* sa, uint16_t* sb, int i0, int i1) __attribute__((always_inline)) {
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      const int64_t krow0 = int64_t(kt) * BK + 16 * wave + 2 * i;  // K-major: first k row of the block
      const uint8_t* ga = AK ? a_blk + krow0 * lda_b + offa[i & 1]
                             : a_blk + int64_t(8 * i) * lda_b + uint32_t(kt) * (BK * 2) + offa[i & 1];
      __builtin_amdgcn_global_load_lds(ga, (PBLK_LDS void*)(sa + (wave * 8 + i) * 512), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(g.b) + krow0 * ldb_b + offb[i & 1],
                                       (PBLK_LDS void*)(sb + (wave * 8 + i) * 512), 16, 0, 0);
    }
  };

  // Fragment reads.  Row-major A: row w*128 + i*32 + lr, logical chunk 2kk + lg at physical
  // (2kk + lg) ^ ((lr >> 1) & 7).  K-major operand tile t (m or n = w*128 + t*32 + lane%32):
  // two transpose reads (ds_read_b64_tr_b16) in which lane 16G + j addresses k row
  // kk*16 + 8*(G/2) + j/4 (+4 for the second) and columns w*128 + t*32 + 16*(G%2) + 4*(j%4) .. +3,
  // so lane L receives k = kk*16 + 8*(L/32) + 0..3 (then 4..7) of column L%32: the MFMA operand.
  uint32_t rda[4], trb[4], tra[4];
  {
    const int G = lane >> 4, j = lane & 15;
    const int krow = 8 * (G >> 1) + (j >> 2);
    const int sw = 4 * ((j >> 2) & 3);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int e = 2 * (G & 1) + ((j & 3) >> 1);
      trb[t] = uint32_t(krow * 512 + (((wn * 16 + 4 * t + e) ^ sw) << 4) + 8 * (j & 1));
      tra[t] = uint32_t(krow * 512 + (((wm * 16 + 4 * t + e) ^ sw) << 4) + 8 * (j & 1));
      rda[t] = uint32_t(lr * 128 + (((2 * t + lg) ^ ((lr >> 1) & 7)) << 4)) + uint32_t(wm * 128 * 128);
    }
  }

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  bf16x8 fa[4][FM], fb[4][FN];  // one fragment buffer per k-step of a slab
  auto trfrag = [&](const uint8_t* p) __attribute__((always_inline)) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * 512));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    const u32x4 u = {l2.x, l2.y, h2.x, h2.y};
    return __builtin_bit_cast(bf16x8, u);
  };
  auto rd = [&](int buf, const uint16_t* sa, const uint16_t* sb, int kk) __attribute__((always_inline)) {
    const uint8_t* pa = reinterpret_cast<const uint8_t*>(sa);
    const uint8_t* pb = reinterpret_cast<const uint8_t*>(sb);
    // in the order the MFMAs consume them
    if constexpr (AK) fa[buf][0] = trfrag(pa + tra[0] + kk * 16 * 512);
    else fa[buf][0] = *reinterpret_cast<const bf16x8*>(pa + rda[kk]);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[buf][j] = trfrag(pb + trb[j] + kk * 16 * 512);
#pragma unroll
    for (int i = 1; i < FM; ++i) {
      if constexpr (AK) fa[buf][i] = trfrag(pa + tra[i] + kk * 16 * 512);
      else fa[buf][i] = *reinterpret_cast<const bf16x8*>(pa + rda[kk] + i * 32 * 128);
    }
  };
  auto mm = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0);
  };
  // sched_group_barrier masks: 0x008 MFMA, 0x020 VMEM read, 0x100 DS read
  // LDS read instructions per k-step: 4 (row-major A) or 8 (K-major A) plus 8 for K-major B
  constexpr int RD = (AK ? 8 : 4) + 8;
  // 16 MFMAs with the 3 * RD fragment reads of the next three k-steps behind the first 12
  auto interleave_rd24 = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < 12; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, RD / 4, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };
  // 16 MFMAs with n copy instructions and nr fragment reads spread over them
  auto interleave_cp = [&](int n, int nr) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (x < nr) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (x < n) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
  };

  // Slab t in stage (ca, cb), its k-step 0 fragments requested into buffer 0, the copies of
  // slab t+1 into stage (na, nb) in flight.
  auto slab = [&](int t, const uint16_t* ca, const uint16_t* cb, uint16_t* na, uint16_t* nb) __attribute__((always_inline)) {
    uint16_t* wa = const_cast<uint16_t*>(ca);
    uint16_t* wb = const_cast<uint16_t*>(cb);
    const int tc = min(t + 2, ke - 1);  // branch-free: past the end the last slab is fetched again
    rd(1, ca, cb, 1);
    rd(2, ca, cb, 2);
    rd(3, ca, cb, 3);
    mm(0);
    interleave_rd24();
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkm0();   // own reads of this stage done
    lds_barrier();  // everyone's: the stage is free
    issue(tc, wa, wb, 0, 3);
    mm(1);
    interleave_cp(6, 0);
    __builtin_amdgcn_sched_barrier(0);
    issue(tc, wa, wb, 3, 5);
    mm(2);
    interleave_cp(4, 0);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm_lgkm0<10>();  // own copies of slab t+1 landed (10 of slab t+2 may be in flight)
    lds_barrier();        // everyone's: slab t+1 is complete
    issue(tc, wa, wb, 5, 8);
    rd(0, na, nb, 0);
    mm(3);
    interleave_cp(6, RD > 16 ? 16 : RD);
    __builtin_amdgcn_sched_barrier(0);
  };

  issue(kb, a0, b0, 0, 8);
  issue(min(kb + 1, ke - 1), a1, b1, 0, 8);
  wait_vm_lgkm0<16>();  // slab kb landed
  lds_barrier();
  rd(0, a0, b0, 0);
  const int n = ke - kb;
  int kt = kb;
  for (int p = 0; p + 2 <= n; p += 2, kt += 2) {
    slab(kt, a0, b0, a1, b1);
    slab(kt + 1, a1, b1, a0, b0);
  }
  if (n & 1) slab(kt, a0, b0, a1, b1);
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0): no copy may still be writing this workgroup's LDS

  // Epilogue through LDS, four rounds: in round i every wave stages its rows wm*128 + i*32 +
  // 0..31 as fp32 (stage pair i&1, the wm half in its own array, 16-byte chunks XOR-permuted
  // by row), then all threads store 64 full rows: bf16 outputs with 16-byte writes, or, for a
  // split-K chunk, its fp32 partial tile (row-major 256 x 256) with 32-byte writes.  Lane
  // (lr, lg) of MFMA tile (i, j) holds row lr and columns j*32 + 8*(r/4) + 4*lg + r%4.
  float* part = tl >= 0 ? sk.partials + int64_t(tl * sk.split + chunk) * (BM * BN) : nullptr;
  lds_barrier();  // every wave is past its last fragment read
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    float* mine = reinterpret_cast<float*>((i & 1) ? (wm ? b1 : a1) : (wm ? b0 : a0));
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int c = wn * 32 + j * 8 + r4 * 2 + lg;
        const f32x4 v = {acc[i][j][4 * r4], acc[i][j][4 * r4 + 1], acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3]};
        *reinterpret_cast<f32x4*>(mine + lr * 256 + ((c ^ (lr & 15)) << 2)) = v;
      }
    lds_barrier();
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int r = p * 8 + (tid >> 5);
      const int half = r >> 5, lrow = r & 31;
      const float* src = reinterpret_cast<const float*>((i & 1) ? (half ? b1 : a1) : (half ? b0 : a0));
      const int c0 = (tid & 31) * 2;
      const f32x4 lo = *reinterpret_cast<const f32x4*>(src + lrow * 256 + ((c0 ^ (lrow & 15)) << 2));
      const f32x4 hi = *reinterpret_cast<const f32x4*>(src + lrow * 256 + (((c0 + 1) ^ (lrow & 15)) << 2));
      const int ml = half * 128 + i * 32 + lrow, nl = (tid & 31) * 8;
      if (part != nullptr) {
        f32x4* dst = reinterpret_cast<f32x4*>(part + ml * BN + nl);
        dst[0] = lo;
        dst[1] = hi;
      } else if (m0 + ml < g.M && n0 + nl < g.N) {
        store_chunk8<EPI>(g, m0 + ml, n0 + nl, lo, hi);
      }
    }
  }
}

template <int EPI, bool AK>
void launch_gemm_kmajor(const GemmArgs& g, float* partials, int G, hipStream_t s) {
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
  const unsigned grid = unsigned(sk.dp_units + sk.tail * sk.split);
  hipLaunchKernelGGL((gemm_kmajor_kernel<EPI, AK>), dim3(grid), dim3(kGemmThreads), 0, s, g, sk);
  if (sk.tail > 0)
    hipLaunchKernelGGL((gemm_bf16_tail_reduce_kernel<EPI>), dim3(unsigned(sk.tail * 32)), dim3(256), 0, s, g, sk);
}

}  // namespace pblk
