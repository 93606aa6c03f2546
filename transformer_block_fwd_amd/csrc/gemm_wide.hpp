// bf16 GEMM in 256 x 384 tiles: C[m, n] = sum_k X[m, k] * Wt[n, k], for a GEMM whose 256 x 384
// tiles fill whole waves where 256 x 256 tiles would leave a partial one.  The 175B shard's
// output projection (2048 x 12288, k = 7680) is 8 x 32 = 256 such tiles: one tile per CU, one
// wave, against 384 tiles of 256 x 256 (a wave and a half) or two waves of 256 x 192.
//
// Operands, LDS layout within a stage, the copies (global_load_lds_dwordx4, 1 KiB = 8 rows of a
// 64-deep slab per instruction, 16-byte chunks XOR-permuted by (row >> 1) & 7), the fragment
// reads and the 16x16x32 MFMA operand order are those of gemm_bf16_kernel.  What differs:
//
// * Each of the 4 wavefronts owns 128 x 192 outputs, 8 x 12 MFMA tiles of 16 x 16: 384
//   accumulator registers per lane, column blocks 0..7 in the AGPR file (256 registers) and
//   8..11 in VGPRs (128).  The per-flop operand traffic is 5/6 of a 256 x 256 tile's: each slab
//   copies 80 KiB for 3/2 of the work.
// * The two stages are 80 KiB each (A 32 KiB, B 48 KiB): all 160 KiB of LDS.
// * Fragments: the A fragments of both 32-deep k-steps of a slab in two buffers (64 registers)
//   and the B fragments in a ring of 6 (24 registers).  The MFMAs run column block by column
//   block (the 8 row blocks of B block j back to back).  Reads go in pairs of columns: behind
//   the first MFMA of columns j, j+1 (j even) come B blocks j+2 and j+3 and, in k-step 0, two of
//   k-step 1's A fragments.  The compiler waits for all outstanding LDS reads (lgkmcnt(0): a
//   pending LDS copy makes it give up on partial counts) before the first MFMA that uses one,
//   so every read has the 16 MFMAs of a column pair to land.  A fragment register is rewritten
//   at least 17 MFMAs after the last MFMA that read it.
// * One barrier per slab, before the last two columns of k-step 1: this wavefront has read
//   everything it needs from the slab's stage and waited for its own copies of the next slab;
//   after everyone's, the stage is free for the slab after next and the next slab is complete.
//   The next slab's first fragments (A of k-step 0, B blocks 0 and 1) are read behind the last
//   16 MFMAs.  The 20 copies of the slab after next go 3 behind the barrier and 17 behind MFMAs
//   1, 6, .., 81 of the next slab: one every 5 MFMAs, so that a CU's copy path (about 64 bytes
//   per clock) never takes a burst, and the last one lands about 95 MFMAs before it is needed.
//
// Epilogue: the lane-swap one of gemm_bf16_kernel (no LDS) in the DIRECT form, which the host
// launches when there is no bias or residual (the 175B shard's partial output); otherwise the
// accumulators go through LDS in 8 rounds of 16 rows per wavefront row (fp32, 16-byte chunks
// XOR-permuted by row), and every thread stores 6 chunks of 8 columns with 16-byte writes,
// consecutive threads on consecutive chunks of a row.
//
// Requirements (checked by the launcher): N % 384 == 0, K % 64 == 0, A allocated in whole
// 256-row tiles, every tile whole (no k-split), EPI kEpiResidual; the DIRECT form only without
// bias or residual.
#pragma once

#include "gemm_bf16.hpp"

namespace pblk {

constexpr int kWideBN = 384;

template <int EPI, bool DIRECT = false>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_bf16_wide_kernel(GemmArgs g, GemmSched sk) {
  constexpr int BM = kGemmBM, BN = kWideBN, BK = kGemmBK;
  constexpr int MI = 8, NJ = 12, NJA = 8;  // per wavefront 128 x 192; column blocks < NJA in AGPRs
  constexpr int NA = 8, NB = 12, NC = NA + NB;  // copy instructions per wavefront and slab
  constexpr int NX = 2 * MI * NJ;               // MFMAs per wavefront and slab
  constexpr int XB = MI * NJ + MI * (NJ - 2);   // position of the barrier: k-step 1, column 10
  constexpr int C_EARLY = 3;                    // copies of the slab after next behind the barrier
  constexpr int C_STEP = 5;                     // MFMAs between copies
  static_assert(XB + 2 + C_STEP * (C_EARLY - 1) < NX && C_STEP * (NC - C_EARLY - 1) + 1 < XB, "copy positions");
  __shared__ __attribute__((aligned(1024))) uint16_t a0[BM * BK];
  __shared__ __attribute__((aligned(1024))) uint16_t b0[BN * BK];
  __shared__ __attribute__((aligned(1024))) uint16_t a1[BM * BK];
  __shared__ __attribute__((aligned(1024))) uint16_t b1[BN * BK];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_coords(xcd_remap(blockIdx.x, sk.dp_units), sk.tiles_m, sk.tiles_n, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int KT = sk.KT;

  // Copies: A instruction i (0..NA-1) of wave w fills rows 64 w + 8 i + l / 8 (1 KiB block
  // NA w + i), B instruction i (0..NB-1) rows 96 w + 8 i + l / 8 (block NB w + i); lane l writes
  // physical chunk l % 8, fetched from logical chunk (l % 8) ^ ((row >> 1) & 7) =
  // (l % 8) ^ (4 (i & 1) + l / 16) (64 w and 96 w are multiples of 16).
  const uint32_t lda_b = uint32_t(g.lda) * 2u, ldb_b = uint32_t(g.ldb) * 2u;
  uint32_t offa[2], offb[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int lc = (lane & 7) ^ (4 * p + (lane >> 4));
    offa[p] = uint32_t(lane >> 3) * lda_b + uint32_t(lc << 4);
    offb[p] = uint32_t(lane >> 3) * ldb_b + uint32_t(lc << 4);
  }
  const uint8_t* a_blk = reinterpret_cast<const uint8_t*>(g.a) + int64_t(m0 + wave * (BM / 4)) * lda_b;
  // copy c (0..NC-1) of slab kt: A and B instructions alternately, then the remaining B ones
  auto copy1 = [&](int kt, uint16_t* sa, uint16_t* sb, int c) __attribute__((always_inline)) {
    const uint32_t kofs = uint32_t(kt) * (BK * 2);
    if (c < 2 * NA && (c & 1) == 0) {
      const int i = c >> 1;
      __builtin_amdgcn_global_load_lds(a_blk + int64_t(8 * i) * lda_b + kofs + offa[i & 1],
                                       (PBLK_LDS void*)(sa + (wave * NA + i) * 512), 16, 0, 0);
    } else {
      const int i = c < 2 * NA ? (c >> 1) : c - NA;
      const int brow = min(n0 + wave * (BN / 4) + 8 * i, g.N - 8);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(g.b) + int64_t(brow) * ldb_b + kofs + offb[i & 1],
                                       (PBLK_LDS void*)(sb + (wave * NB + i) * 512), 16, 0, 0);
    }
  };

  // Fragment reads: lane l reads row 16 * block + l % 16, the 8 k of logical chunk
  // 4 ks + l / 16 of k-step ks, at physical chunk (4 ks + l / 16) ^ ((l % 16 >> 1) & 7).
  const int lr = lane & 15, lq = lane >> 4;
  uint32_t rda[2], rdb[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const uint32_t o = uint32_t(lr * 128 + (((4 * ks + lq) ^ ((lr >> 1) & 7)) << 4));
    rda[ks] = o + uint32_t(wm * (BM / 2) * 128);
    rdb[ks] = o + uint32_t(wn * (BN / 2) * 128);
  }
  auto rd_a = [&](const uint16_t* sa, int ks, int i) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const uint8_t*>(sa) + rda[ks] + i * 16 * 128);
  };
  auto rd_b = [&](const uint16_t* sb, int ks, int j) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const uint8_t*>(sb) + rdb[ks] + j * 16 * 128);
  };

  f32x4 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int NFB = 6;  // B fragment ring
  bf16x8 fa[2][MI], fb[NFB];

  // Slab t from stage (ca, cb), the next slab's stage (na, nb).  On entry fa[0] and fb[0..1] hold
  // k-step 0's A fragments and B blocks 0, 1 of slab t, and copies 0..C_EARLY-1 of slab t+1 are in
  // flight.  The MFMAs are inline asm with the accumulator tied ("+a" / "+v": the builtin lets
  // the register allocator rotate accumulators through copies); volatile asm keeps every memory
  // operation in program order around them, which fixes the interleave written here.
  auto slab = [&](int t, const uint16_t* ca, const uint16_t* cb, uint16_t* na, uint16_t* nb) __attribute__((always_inline)) {
    const int t1 = min(t + 1, KT - 1), t2 = min(t + 2, KT - 1);  // past the end: the last slab again
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const int x = ks * (MI * NJ) + j * MI + i;
          if (x == XB) {
            wait_vm_lgkm0<0>();  // own reads of this stage done, own copies of slab t+1 landed
            lds_barrier();       // everyone's: this stage is free, slab t+1 is complete
#pragma unroll
            for (int ii = 0; ii < MI; ++ii) fa[0][ii] = rd_a(na, 0, ii);
          }
          if (j < NJA)
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[i][j]) : "v"(fb[j % NFB]), "v"(fa[ks][i]));
          else
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc[i][j]) : "v"(fb[j % NFB]), "v"(fa[ks][i]));
          if (i == 0 && (j & 1) == 0) {
            // B blocks j + 2, j + 3, wrapping into the next k-step (or the next slab's k-step 0)
            if (j + 2 < NJ) {
              fb[(j + 2) % NFB] = rd_b(cb, ks, j + 2);
              fb[(j + 3) % NFB] = rd_b(cb, ks, j + 3);
            } else if (ks == 0) {
              fb[(j + 2) % NFB] = rd_b(cb, 1, j + 2 - NJ);
              fb[(j + 3) % NFB] = rd_b(cb, 1, j + 3 - NJ);
            } else {
              fb[(j + 2) % NFB] = rd_b(nb, 0, j + 2 - NJ);
              fb[(j + 3) % NFB] = rd_b(nb, 0, j + 3 - NJ);
            }
            // k-step 1's A fragments behind column pairs 1..4 of k-step 0
            if (ks == 0 && j >= 2 && j < 2 + MI) {
              fa[1][j - 2] = rd_a(ca, 1, j - 2);
              fa[1][j - 1] = rd_a(ca, 1, j - 1);
            }
          }
          if (x < XB) {
            // copies C_EARLY.. of slab t+1 behind MFMAs 1, 1 + C_STEP, ..
            if ((x - 1) % C_STEP == 0 && x >= 1 && (x - 1) / C_STEP + C_EARLY < NC)
              copy1(t1, na, nb, (x - 1) / C_STEP + C_EARLY);
          } else {
            // copies 0..C_EARLY-1 of slab t+2 into this stage, behind MFMAs XB + 2, XB + 2 + C_STEP, ..
            const int d = x - XB - 2;
            if (d >= 0 && d % C_STEP == 0 && d / C_STEP < C_EARLY)
              copy1(t2, const_cast<uint16_t*>(ca), const_cast<uint16_t*>(cb), d / C_STEP);
          }
        }
  };

#pragma unroll
  for (int c = 0; c < NC; ++c) copy1(0, a0, b0, c);
  wait_vm_lgkm0<0>();  // slab 0 landed
  lds_barrier();
#pragma unroll
  for (int ii = 0; ii < MI; ++ii) fa[0][ii] = rd_a(a0, 0, ii);
  fb[0] = rd_b(b0, 0, 0);
  fb[1] = rd_b(b0, 0, 1);
#pragma unroll
  for (int c = 0; c < C_EARLY; ++c) copy1(min(1, KT - 1), a1, b1, c);
  // the accumulators' zeroing (VALU writes) before their first MFMA read
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 4");
  __builtin_amdgcn_sched_barrier(0);
  int kt = 0;
  for (int p = 0; p + 2 <= KT; p += 2, kt += 2) {
    slab(kt, a0, b0, a1, b1);
    slab(kt + 1, a1, b1, a0, b0);
  }
  if (KT & 1) slab(kt, a0, b0, a1, b1);
  // the last MFMAs' accumulator writes before any other instruction reads them
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0): no copy may still be writing this workgroup's LDS
  if constexpr (DIRECT) {
    // no bias or residual: the lane-swap epilogue of gemm_bf16_kernel, no LDS
    gemm_epilogue_direct<EPI, BM, MI, NJ, BN>(g, acc, nullptr, m0, n0, wm, wn);
  } else {
    lds_barrier();  // every wave is past its last fragment read

    // Epilogue: round r stages MFMA row block r of every wavefront (rows 128 wm + 16 r + 0..15,
    // the wavefront's 192 columns) as fp32 into buffer pair r & 1 (a0 / a1 for even rounds, b0 / b1
    // for odd ones, the wm half in its own array; 16 rows x 384 columns = 24 KiB each), then the
    // 256 threads store the round's 32 rows x 48 chunks of 8 columns.
#pragma unroll
    for (int r = 0; r < MI; ++r) {
      float* mine = reinterpret_cast<float*>((r & 1) ? (wm ? b1 : b0) : (wm ? a1 : a0));
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int c = wn * (BN / 8) + 4 * j + lq;  // 16-byte chunk of the row (0..95)
        *reinterpret_cast<f32x4*>(mine + lr * BN + ((c ^ lr) << 2)) = acc[r][j];
      }
      lds_barrier();
#pragma unroll 1
      for (int p = 0; p < 6; ++p) {
        const int q = p * 256 + tid;
        const int row = q / 48, ch = q - row * 48;  // row of the round (0..31), 8-column chunk (0..47)
        const int half = row >> 4, lrow = row & 15;
        const float* src = reinterpret_cast<const float*>((r & 1) ? (half ? b1 : b0) : (half ? a1 : a0));
        const f32x4 lo = *reinterpret_cast<const f32x4*>(src + lrow * BN + (((2 * ch) ^ lrow) << 2));
        const f32x4 hi = *reinterpret_cast<const f32x4*>(src + lrow * BN + (((2 * ch + 1) ^ lrow) << 2));
        const int m = m0 + half * (BM / 2) + 16 * r + lrow, n = n0 + 8 * ch;
        if (m < g.M && n < g.N) store_chunk8<EPI>(g, m, n, lo, hi);
      }
    }
  }
}

}  // namespace pblk
