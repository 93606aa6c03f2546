// Rotary position embedding of q and k (RoFormer, Su et al., section 3): in each head of hd
// features the pair (t[2i], t[2i+1]) at position p turns by the angle p * base^(-2i/hd).
// The angles' cosines and sines come from a table built once per base in fp64 and
// rounded to fp32, so a position of several thousand loses nothing to an fp32 angle.
#pragma once

#include "common.hpp"

namespace pblk {

// cs[(p * hd/2 + i) * 2 + {0, 1}] = cos, sin of p * base^(-2i/hd), p in [0, n_pos).
__global__ __launch_bounds__(256) void rope_table_kernel(float* __restrict__ cs, int n_pos, int hd, double base) {
  const int half = hd >> 1;
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= int64_t(n_pos) * half) return;
  const int p = int(t / half), i = int(t % half);
  const double ang = double(p) * pow(base, -2.0 * double(i) / double(hd));
  double sn, cn;
  sincos(ang, &sn, &cn);
  cs[2 * t] = float(cn);
  cs[2 * t + 1] = float(sn);
}

// Rotates the 4 pairs of v[0..7], head-local columns c .. c+7 (c a multiple of 8) at position p.
__device__ __forceinline__ void rope_rotate8(float* v, const float* __restrict__ cs, int p, int c, int hd) {
  const float* t = cs + (int64_t(p) * (hd >> 1) + (c >> 1)) * 2;
  const f32x4 a = *reinterpret_cast<const f32x4*>(t);
  const f32x4 b = *reinterpret_cast<const f32x4*>(t + 4);
  const float cosv[4] = {a[0], a[2], b[0], b[2]}, sinv[4] = {a[1], a[3], b[1], b[3]};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float e = v[2 * q], o = v[2 * q + 1];
    v[2 * q] = e * cosv[q] - o * sinv[q];
    v[2 * q + 1] = e * sinv[q] + o * cosv[q];
  }
}

}  // namespace pblk
