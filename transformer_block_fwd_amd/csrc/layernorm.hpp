// LayerNorm over the model dimension, one workgroup (4 wavefronts) per group of
// consecutive tokens.
//
// The MegaScale guided reading (section 4, "Operators") fuses LayerNorm into a
// single kernel to cut launches and memory traffic; here each row is read once
// with 16-byte vector loads, kept in registers, reduced twice (mean, then the
// centred second moment) with wavefront shuffles plus one LDS exchange, and
// written once.  gamma and beta are loaded once per workgroup, and the next
// row's loads are in flight while the current row is reduced.  Statistics are
// fp32; the biased variance is used.
#pragma once

#include "common.hpp"

namespace pblk {

constexpr int kLnThreads = 256;
constexpr int kLnMaxRows = 4;  // rows per workgroup at most (host launch choice)

// Raw = the 16-byte vector as loaded (bf16 rows stay packed in registers until used).
template <typename T>
struct LnVec;
template <>
struct LnVec<uint16_t> {  // bf16: 8 elements per 16-byte vector
  static constexpr int N = 8;
  using Raw = u32x4;
  __device__ static Raw load(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
  __device__ static Raw zero() { return Raw{0u, 0u, 0u, 0u}; }
  __device__ static void unpack(const Raw& r, float* v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(r[i] << 16);
      v[2 * i + 1] = __uint_as_float(r[i] & 0xFFFF0000u);
    }
  }
  __device__ static void store(uint16_t* p, const float* v) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 pr = {v[2 * i], v[2 * i + 1]};
      r[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));  // RNE
    }
    *reinterpret_cast<u32x4*>(p) = r;
  }
};
template <>
struct LnVec<float> {  // fp32: 4 elements per 16-byte vector
  static constexpr int N = 4;
  using Raw = float4;
  __device__ static Raw load(const float* p) { return *reinterpret_cast<const float4*>(p); }
  __device__ static Raw zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ static void unpack(const Raw& r, float* v) {
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

// VPT = 16-byte vectors per thread (the host picks the smallest that covers d).  Each
// workgroup normalizes rows_per_wg consecutive rows; `stats` (optional, [M][2]) receives each
// row's mean and 1/sigma.  For rows of up to 2048 vectors
// (VPT <= 8) gamma and beta stay in registers across the rows and the next row's loads
// are in flight while the current one is reduced and written; wider rows are loaded one
// at a time (the host gives them one row per workgroup unless the grid would exceed the
// launch limit) and read gamma and beta per row.
template <typename T, int VPT>
__global__ __launch_bounds__(kLnThreads) void layernorm_kernel(const T* __restrict__ x, const T* __restrict__ gamma,
                                                               const T* __restrict__ beta, T* __restrict__ u,
                                                               int64_t M, int d, int rows_per_wg, float eps,
                                                               float* __restrict__ stats) {
  using V = LnVec<T>;
  using Raw = typename V::Raw;
  constexpr int N = V::N;
  constexpr bool kHold = VPT <= 8;
  __shared__ float red[4];
  const int nvec = d / N;
  const int64_t row0 = int64_t(blockIdx.x) * rows_per_wg;
  const int64_t row_end = min(row0 + rows_per_wg, M);
  Raw cur[VPT], nxt[VPT], g[kHold ? VPT : 1], b[kHold ? VPT : 1];
  auto load_row = [&](int64_t row, Raw (&v)[VPT]) __attribute__((always_inline)) {
    const T* xr = x + row * d;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = threadIdx.x + i * kLnThreads;
      v[i] = c < nvec ? V::load(xr + c * N) : V::zero();
    }
  };
  load_row(row0, cur);
  if constexpr (kHold) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = threadIdx.x + i * kLnThreads;
      if (c < nvec) {
        g[i] = V::load(gamma + c * N);
        b[i] = V::load(beta + c * N);
      }
    }
  }
  const float inv_d = 1.0f / float(d);
  for (int64_t row = row0; row < row_end; ++row) {
    if (kHold && row + 1 < row_end) load_row(row + 1, nxt);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      float v[N];
      V::unpack(cur[i], v);
#pragma unroll
      for (int e = 0; e < N; ++e) s += v[e];
    }
    const float mean = block_sum_256(s, red) * inv_d;
    // a bf16 row stays packed between the passes: unpacking it again is cheaper than holding
    // it as fp32 (twice the registers; at d = 12288 that is 165 VGPRs against 196)
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int i = 0; i < VPT; ++i) asm volatile("" : "+v"(cur[i]));
    }
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = threadIdx.x + i * kLnThreads;
      if (c < nvec) {
        float v[N];
        V::unpack(cur[i], v);
#pragma unroll
        for (int e = 0; e < N; ++e) {
          const float t = v[e] - mean;
          q += t * t;
        }
      }
    }
    const float var = block_sum_256(q, red) * inv_d;
    const float rstd = 1.0f / sqrtf(var + eps);
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int i = 0; i < VPT; ++i) asm volatile("" : "+v"(cur[i]));
    }
    if (stats != nullptr && threadIdx.x == 0) {  // mean and 1/sigma of the row, for the backward pass
      stats[2 * row] = mean;
      stats[2 * row + 1] = rstd;
    }
    T* ur = u + row * d;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = threadIdx.x + i * kLnThreads;
      if (c < nvec) {
        float v[N], gv[N], bv[N], o[N];
        V::unpack(cur[i], v);
        if constexpr (kHold) {
          V::unpack(g[i], gv);
          V::unpack(b[i], bv);
        } else {
          V::unpack(V::load(gamma + c * N), gv);
          V::unpack(V::load(beta + c * N), bv);
        }
#pragma unroll
        for (int e = 0; e < N; ++e) o[e] = (v[e] - mean) * rstd * gv[e] + bv[e];
        V::store(ur + c * N, o);
      }
    }
    if constexpr (kHold) {
#pragma unroll
      for (int i = 0; i < VPT; ++i) cur[i] = nxt[i];
    } else if (row + 1 < row_end) {
      load_row(row + 1, cur);
    }
  }
}

}  // namespace pblk
