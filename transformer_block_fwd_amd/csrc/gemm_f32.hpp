// fp32 GEMM for the fp32 debug path: C[m, n] = sum_k X[m, k] * Wt[n, k] on the
// vector ALUs (exact fp32 FMAs, fixed k order), with the same two epilogues as
// the bf16 matrix-core GEMM.  Untimed; it exists so the whole block can be
// checked against the oracle at fp32 tolerance.
#pragma once

#include "common.hpp"

namespace pblk {

struct GemmArgsF32 {
  const float* a;
  int64_t lda;
  const float* b;
  int64_t ldb;
  int M, N, K;
  float* out0;
  int64_t ld0;
  float* out1;
  int64_t ld1;
  int64_t off1;
  int nsplit;
  const float* resid;
  int64_t ldr;
  // variant switches, as in the bf16 GEMM's epilogue (off when zero / null)
  const float* bias;
  const float* rope;
  int rope_n, seq, hd;
  int gelu_tanh;
};

// 64x64 tile, 256 threads, 4x4 outputs per thread, k slabs of 16 in LDS.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgsF32 g) {
  constexpr int T = 64, BK = 16;
  __shared__ float sa[BK][T + 4];
  __shared__ float sb[BK][T + 4];
  const int tiles_m = (g.M + T - 1) / T;
  const int m0 = (blockIdx.x % tiles_m) * T;
  const int n0 = (blockIdx.x / tiles_m) * T;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  // loader: each thread moves 4 consecutive k of one row for A and for B
  const int lrow = tid >> 2, lk = (tid & 3) * 4;
  const float* ap = g.a + int64_t(min(m0 + lrow, g.M - 1)) * g.lda + lk;
  const float* bp = g.b + int64_t(min(n0 + lrow, g.N - 1)) * g.ldb + lk;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += BK) {
    const float4 va = *reinterpret_cast<const float4*>(ap + k0);
    const float4 vb = *reinterpret_cast<const float4*>(bp + k0);
    sa[lk + 0][lrow] = va.x; sa[lk + 1][lrow] = va.y; sa[lk + 2][lrow] = va.z; sa[lk + 3][lrow] = va.w;
    sb[lk + 0][lrow] = vb.x; sb[lk + 1][lrow] = vb.y; sb[lk + 2][lrow] = vb.z; sb[lk + 3][lrow] = vb.w;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = sa[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = sb[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= g.M) continue;
    const int nb = n0 + tx * 4;  // 4 consecutive columns, nb a multiple of 4; N is a multiple of 64
    if (nb >= g.N) continue;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = acc[i][j] + (g.bias != nullptr ? g.bias[nb + j] : 0.f);
    if constexpr (EPI == kEpiSplitGelu) {
      if (nb < g.nsplit) {
        if (nb < g.rope_n) {
          const int c = nb & (g.hd - 1);
          const float* t = g.rope + (int64_t(m % g.seq) * (g.hd >> 1) + (c >> 1)) * 2;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const float e = v[2 * q], o = v[2 * q + 1], cv = t[2 * q], sv = t[2 * q + 1];
            v[2 * q] = e * cv - o * sv;
            v[2 * q + 1] = e * sv + o * cv;
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) g.out0[int64_t(m) * g.ld0 + nb + j] = v[j];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          g.out1[int64_t(m) * g.ld1 + g.off1 + (nb + j - g.nsplit)] = g.gelu_tanh ? gelu_tanh(v[j]) : gelu_erf(v[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float r = v[j];
        if (g.resid != nullptr) r += g.resid[int64_t(m) * g.ldr + nb + j];
        g.out0[int64_t(m) * g.ld0 + nb + j] = r;
      }
    }
  }
}

}  // namespace pblk
