// Elementwise and reduction kernels of the block's backward pass (bf16 storage, fp32 math):
//   zero_kernel             zeroes the token padding (rows M .. Mp-1) the weight-gradient GEMMs
//                           read as k rows;
//   layernorm_bwd_kernel    dx = (g - mean(g) - xhat mean(g xhat)) / sigma (+ dy), g = du gamma,
//                           from the forward's per-row mean and 1/sigma, with per-workgroup
//                           column partials of du xhat and du;
//   column_sum_kernel       dgamma, dbeta from those partials.
// The chain rule through LayerNorm, GeLU and attention is the one the MegaScale guided reading's
// section 3 implies for the backward pass (its forward-pass overlap carries over to it).
#pragma once

#include "common.hpp"

namespace pblk {

// d/dz of z * Phi(z): Phi(z) + z * phi(z), phi(z) = e^(-z^2/2) / sqrt(2 pi).  Phi comes from
// the erfc of Abramowitz and Stegun 7.1.26 (as gelu_erf_bf16out: absolute error of erf below
// 1.5e-7, so of Phi below 7.5e-8), erfc(x) = t (a1 + a2 t + .. + a5 t^4) e^(-x^2) with x = |z|/sqrt 2,
// whose e^(-x^2) is the same e^(-z^2/2) phi needs: one reciprocal and one exponential per value.
// The derivative scales a bf16 gradient and is stored as bf16, far coarser than this error.
__device__ __forceinline__ float gelu_erf_grad(float z) {
  const float x = fabsf(z) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
  // 0.5 * (a1 .. a5): h = erfc(x) / 2 directly
  float q = 0.5307027145f;
  q = fmaf(t, q, -0.7265760135f);
  q = fmaf(t, q, 0.7107068705f);
  q = fmaf(t, q, -0.142248368f);
  q = fmaf(t, q, 0.127414796f);
  const float e = __builtin_amdgcn_exp2f(x * x * -1.4426950408889634f);  // e^(-z^2/2)
  const float h = q * t * e;
  const float Phi = z >= 0.0f ? 1.0f - h : h;
  return fmaf(z * 0.3989422804014327f, e, Phi);
}

// Zeroes n 16-byte pieces at p (grid-stride).
__global__ __launch_bounds__(256) void zero_kernel(u32x4* __restrict__ p, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) p[i] = u32x4{0u, 0u, 0u, 0u};
}

__device__ __forceinline__ float2 block_sum2_256(float a, float b, float* red) {
  a = wave_sum(a);
  b = wave_sum(b);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();  // red[] may still be read from a previous reduction
  if (lane == 0) {
    red[wave] = a;
    red[4 + wave] = b;
  }
  __syncthreads();
  return make_float2(red[0] + red[1] + red[2] + red[3], red[4] + red[5] + red[6] + red[7]);
}

// One workgroup (256 threads) per `rows` consecutive rows of x [M, d] (bf16), du [M, d] (fp32),
// dy [M, d] (bf16, may be null: no residual), with each row's mean and 1/sigma from the forward
// (stats [M][2]).  Writes dx [M, d] (bf16) and, per workgroup, partial [blockIdx][0][d] = sum over
// its rows of du * xhat, partial [blockIdx][1][d] = sum du (fp32).  VPT 8-element pieces per
// thread cover d (d <= VPT * 2048).  One block reduction per row (sum g, sum g * xhat).
template <int VPT>
__global__ __launch_bounds__(256) void layernorm_bwd_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ gamma,
                                                            const float* __restrict__ du,
                                                            const uint16_t* __restrict__ dy,
                                                            const float* __restrict__ stats,
                                                            uint16_t* __restrict__ dx, float* __restrict__ partial,
                                                            int64_t M, int d, int rows) {
  __shared__ float red[8];
  const int nvec = d / 8;
  const int64_t row0 = int64_t(blockIdx.x) * rows;
  const int64_t row_end = min(row0 + rows, M);
  const float inv_d = 1.0f / float(d);
  float pg[VPT][8], pb[VPT][8];
#pragma unroll
  for (int i = 0; i < VPT; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) pg[i][e] = pb[i][e] = 0.f;
  for (int64_t row = row0; row < row_end; ++row) {
    const float mean = stats[2 * row], rstd = stats[2 * row + 1];
    // xhat and g = du * gamma; sums of g and g * xhat
    float xh[VPT][8], gv[VPT][8];
    float sg = 0.f, sgx = 0.f;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = threadIdx.x + i * 256;
      if (c < nvec) {
        const u32x4 xr = *reinterpret_cast<const u32x4*>(x + row * d + c * 8);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(du + row * d + c * 8);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(du + row * d + c * 8 + 4);
        const u32x4 gr = *reinterpret_cast<const u32x4*>(gamma + c * 8);
        const float dv[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t xw = xr[e >> 1], gw = gr[e >> 1];
          const float xe = (e & 1) ? __uint_as_float(xw & 0xFFFF0000u) : __uint_as_float(xw << 16);
          const float gm = (e & 1) ? __uint_as_float(gw & 0xFFFF0000u) : __uint_as_float(gw << 16);
          xh[i][e] = (xe - mean) * rstd;
          gv[i][e] = dv[e] * gm;
          sg += gv[i][e];
          sgx += gv[i][e] * xh[i][e];
          pg[i][e] += dv[e] * xh[i][e];
          pb[i][e] += dv[e];
        }
      }
    }
    const float2 sums = block_sum2_256(sg, sgx, red);
    const float mg = sums.x * inv_d, mgx = sums.y * inv_d;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = threadIdx.x + i * 256;
      if (c < nvec) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (gv[i][e] - mg - xh[i][e] * mgx) * rstd;
        if (dy != nullptr) {
          const u32x4 r = *reinterpret_cast<const u32x4*>(dy + row * d + c * 8);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[2 * e] += __uint_as_float(r[e] << 16);
            o[2 * e + 1] += __uint_as_float(r[e] & 0xFFFF0000u);
          }
        }
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f32x2 pr = {o[2 * e], o[2 * e + 1]};
          w[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
        }
        *reinterpret_cast<u32x4*>(dx + row * d + c * 8) = w;
      }
    }
  }
  float* pgo = partial + int64_t(blockIdx.x) * 2 * d;
  float* pbo = pgo + d;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int c = threadIdx.x + i * 256;
    if (c < nvec) {
      *reinterpret_cast<f32x4*>(pgo + c * 8) = f32x4{pg[i][0], pg[i][1], pg[i][2], pg[i][3]};
      *reinterpret_cast<f32x4*>(pgo + c * 8 + 4) = f32x4{pg[i][4], pg[i][5], pg[i][6], pg[i][7]};
      *reinterpret_cast<f32x4*>(pbo + c * 8) = f32x4{pb[i][0], pb[i][1], pb[i][2], pb[i][3]};
      *reinterpret_cast<f32x4*>(pbo + c * 8 + 4) = f32x4{pb[i][4], pb[i][5], pb[i][6], pb[i][7]};
    }
  }
}

// out[j] = sum over p < n_part of partial[p][j] for the 64 columns j of this workgroup (n a
// multiple of 64): thread (g, c) sums the rows p = g mod 4 of column c, then the four partial
// sums meet in LDS in a fixed order (bf16 result: j < half to out0, else out1).
__global__ __launch_bounds__(256) void column_sum_kernel(const float* __restrict__ partial, int n_part, int64_t n,
                                                         uint16_t* __restrict__ out0, uint16_t* __restrict__ out1,
                                                         int64_t half) {
  __shared__ float red[4][64];
  const int c = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int64_t j = int64_t(blockIdx.x) * 64 + c;
  // four independent running sums (rows g, g+4, g+8, g+12 mod 16) keep four loads in flight;
  // the order of every addition is fixed by n_part alone
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  int p = g;
  for (; p + 12 < n_part; p += 16) {
    s0 += partial[int64_t(p) * n + j];
    s1 += partial[int64_t(p + 4) * n + j];
    s2 += partial[int64_t(p + 8) * n + j];
    s3 += partial[int64_t(p + 12) * n + j];
  }
  for (; p < n_part; p += 4) s0 += partial[int64_t(p) * n + j];
  red[g][c] = (s0 + s1) + (s2 + s3);
  __syncthreads();
  if (g == 0) {
    const float t = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
    const f32x2 pr = {t, 0.f};
    const uint16_t v = uint16_t(__builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2)) & 0xFFFFu);
    if (j < half) out0[j] = v;
    else out1[j - half] = v;
  }
}

}  // namespace pblk
