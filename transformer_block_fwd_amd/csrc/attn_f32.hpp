// Sliding-window causal attention for the fp32 debug path: one thread per
// query walks its window j = max(0, i-W+1) .. i with an online softmax in
// fp32 (accurate expf).  Untimed; it exists to check the block at fp32
// tolerance.  A launch covers query positions [q_lo, q_hi) of each sequence.
#pragma once

#include "common.hpp"

namespace pblk {

template <int HD>
__global__ __launch_bounds__(64) void swa_attn_f32_kernel(const float* __restrict__ qkv, int64_t ld_qkv,
                                                          float* __restrict__ o, int64_t ld_o, int S, int H,
                                                          int W, float scale, int q_lo, int q_hi) {
  const int nqb = (q_hi - q_lo + 63) / 64;
  const int qb = blockIdx.x % nqb;
  const int h = (blockIdx.x / nqb) % H;
  const int b = blockIdx.x / (nqb * H);
  const int i = q_lo + qb * 64 + threadIdx.x;
  if (i >= q_hi) return;
  const int A = H * HD;
  const float* base = qkv + int64_t(b) * S * ld_qkv + h * HD;
  float q[HD], acc[HD];
#pragma unroll
  for (int e = 0; e < HD; ++e) {
    q[e] = base[int64_t(i) * ld_qkv + e] * scale;
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int j = max(0, i - W + 1); j <= i; ++j) {
    const float* kr = base + int64_t(j) * ld_qkv + A;
    const float* vr = kr + A;
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < HD; ++e) s = fmaf(q[e], kr[e], s);
    const float m_new = fmaxf(m, s);
    const float alpha = expf(m - m_new);
    const float p = expf(s - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int e = 0; e < HD; ++e) acc[e] = fmaf(p, vr[e], acc[e] * alpha);
    m = m_new;
  }
  float* orow = o + (int64_t(b) * S + i) * ld_o + h * HD;
  const float inv = 1.0f / l;
#pragma unroll
  for (int e = 0; e < HD; ++e) orow[e] = acc[e] * inv;
}

}  // namespace pblk
