// LayerNorm over the model dimension, one workgroup (4 wavefronts) per token.
//
// The MegaScale guided reading (section 4, "Operators") fuses LayerNorm into a
// single kernel to cut launches and memory traffic; here the row is read once
// with 16-byte vector loads, kept in registers, reduced twice (mean, then the
// centred second moment) with wavefront shuffles plus one LDS exchange, and
// written once.  Statistics are fp32; the biased variance is used.
#pragma once

#include "common.hpp"

namespace pblk {

constexpr int kLnThreads = 256;

template <typename T>
struct LnVec;
template <>
struct LnVec<uint16_t> {  // bf16: 8 elements per 16-byte vector
  static constexpr int N = 8;
  __device__ static void load(const uint16_t* p, float* v) {
    u32x4 r = *reinterpret_cast<const u32x4*>(p);
    uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ static void store(uint16_t* p, const float* v) {
    u32x4 r;
    r.x = pack_bf16x2(v[0], v[1]);
    r.y = pack_bf16x2(v[2], v[3]);
    r.z = pack_bf16x2(v[4], v[5]);
    r.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<u32x4*>(p) = r;
  }
};
template <>
struct LnVec<float> {  // fp32: 4 elements per 16-byte vector
  static constexpr int N = 4;
  __device__ static void load(const float* p, float* v) {
    float4 r = *reinterpret_cast<const float4*>(p);
    v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
  }
  __device__ static void store(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

__device__ __forceinline__ float block_sum_256(float v, float* red) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();  // red[] may still be read from a previous reduction
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// VPT = 16-byte vectors per thread; the host picks the smallest that covers d.
template <typename T, int VPT>
__global__ __launch_bounds__(kLnThreads) void layernorm_kernel(const T* __restrict__ x, const T* __restrict__ gamma,
                                                               const T* __restrict__ beta, T* __restrict__ u,
                                                               int d, float eps) {
  using V = LnVec<T>;
  constexpr int N = V::N;
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const T* xr = x + row * d;
  T* ur = u + row * d;
  const int nvec = d / N;
  float v[VPT][N];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int c = threadIdx.x + i * kLnThreads;
    if (c < nvec) {
      V::load(xr + c * N, v[i]);
#pragma unroll
      for (int e = 0; e < N; ++e) s += v[i][e];
    } else {
#pragma unroll
      for (int e = 0; e < N; ++e) v[i][e] = 0.f;
    }
  }
  const float inv_d = 1.0f / float(d);
  const float mean = block_sum_256(s, red) * inv_d;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int c = threadIdx.x + i * kLnThreads;
    if (c < nvec) {
#pragma unroll
      for (int e = 0; e < N; ++e) {
        const float t = v[i][e] - mean;
        q += t * t;
      }
    }
  }
  const float var = block_sum_256(q, red) * inv_d;
  const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int c = threadIdx.x + i * kLnThreads;
    if (c < nvec) {
      float g[N], b[N], o[N];
      V::load(gamma + c * N, g);
      V::load(beta + c * N, b);
#pragma unroll
      for (int e = 0; e < N; ++e) o[e] = (v[i][e] - mean) * rstd * g[e] + b[e];
      V::store(ur + c * N, o);
    }
  }
}

}  // namespace pblk
