// Shared device helpers for the gfx950 kernels: bf16 storage conversions,
// vector types for the MFMA operands, wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pblk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Native clang vectors for 16- and 8-byte moves (HIP's uint4 is a struct, which
// keeps register arrays of it from being split into registers).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// GEMM epilogues (see gemm_bf16.hpp).
enum { kEpiSplitGelu = 0, kEpiResidual = 1, kEpiGeluBwd = 2, kEpiF32 = 3 };

// bf16 values are stored as raw uint16 bits (the upper half of an fp32).
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// Round-to-nearest-even fp32 -> bf16 (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even: one conversion
// instruction for the pair (the same bits as f32_to_bf16 on each, for finite inputs).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 pr = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
}

// Sum over the 64 lanes of a wavefront without LDS: quad butterflies and row rotations by DPP
// inside each 16-lane row, then the v_permlane16_swap / v_permlane32_swap exchanges across rows.
// Every lane ends with the total; the order of the additions differs between lanes, so lanes may
// differ in the last bit (callers read one lane).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_f32<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_f32<0x124>(v);  // row_ror 4
  v += dpp_f32<0x128>(v);  // row_ror 8
  const uint32_t u16 = __float_as_uint(v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u16, u16, false, false);  // rows 0 <-> 1, 2 <-> 3
  v += __uint_as_float((threadIdx.x & 16) ? r16[0] : r16[1]);
  const uint32_t u32 = __float_as_uint(v);
  const auto r32 = __builtin_amdgcn_permlane32_swap(u32, u32, false, false);  // lanes l <-> l ^ 32
  v += __uint_as_float((threadIdx.x & 32) ? r32[0] : r32[1]);
  return v;
}

// Exact GeLU z * Phi(z) = z/2 * (1 + erf(z / sqrt 2)) = z * (1 - erfc(z / sqrt 2) / 2), fp32.
// erfc from the Chebyshev-fitted formula of Numerical Recipes (2nd ed., section 6.2, erfcc):
// with x = |z| / sqrt 2 and t = 1 / (1 + x/2), erfc(x) = t * exp(-x^2 + P(t)), P a degree-9
// polynomial, fractional error below 1.2e-7 for every x >= 0; erfc(-x) = 2 - erfc(x).  The
// result differs from the exact value by at most ~1e-6 absolute (as an fp32 erff-based GeLU
// does).  Branch-free: z >= 0 gives z * (1 - h), z < 0 gives z * h, h = erfc(|z|/sqrt 2) / 2.
__device__ __forceinline__ float gelu_erf(float z) {
  const float x = fabsf(z) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, x, 1.0f));
  float p = 0.17087277f;
  p = fmaf(t, p, -0.82215223f);
  p = fmaf(t, p, 1.48851587f);
  p = fmaf(t, p, -1.13520398f);
  p = fmaf(t, p, 0.27886807f);
  p = fmaf(t, p, -0.18628806f);
  p = fmaf(t, p, 0.09678418f);
  p = fmaf(t, p, 0.37409196f);
  p = fmaf(t, p, 1.00002368f);
  const float arg = fmaf(-x, x, fmaf(t, p, -1.26551223f));
  const float h = 0.5f * t * __builtin_amdgcn_exp2f(arg * 1.4426950408889634f);
  return z * (z >= 0.0f ? 1.0f - h : h);
}

// Exact-erf GeLU for the bf16 path: erfc(x) = t (a1 + a2 t + a3 t^2 + a4 t^3 + a5 t^4) e^(-x^2),
// t = 1 / (1 + p x), from Abramowitz and Stegun, Handbook of Mathematical Functions, formula
// 7.1.26 (absolute error of erf below 1.5e-7 for x >= 0).  With x = |z| / sqrt 2 and
// h = erfc(x) / 2, z Phi(z) = max(z, 0) - |z| h for either sign of z; the 1 / sqrt 2 is folded
// into p and the exponent is 2^(z^2 (-log2(e) / 2)): 12 VALU instructions plus one reciprocal
// and one exp2.  The GeLU it gives differs from the exact one by at most 7.5e-8 |z| plus its
// fp32 evaluation, far below half an ulp of the bf16 value it is stored as; five polynomial
// terms instead of the ten of gelu_erf, the one the fp32 path keeps.
__device__ __forceinline__ float gelu_erf_bf16out(float z) {
  const float az = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.2316418883f, az, 1.0f));  // p / sqrt 2, p = 0.3275911
  // 0.5 * (a1 .. a5): h = erfc(x) / 2 directly
  float q = 0.5307027145f;
  q = fmaf(t, q, -0.7265760135f);
  q = fmaf(t, q, 0.7107068705f);
  q = fmaf(t, q, -0.142248368f);
  q = fmaf(t, q, 0.127414796f);
  const float h = q * t * __builtin_amdgcn_exp2f(z * z * -0.72134752044448169f);
  return fmaf(-az, h, fmaxf(z, 0.0f));
}

// GeLU's tanh approximation (Hendrycks and Gimpel, "Gaussian Error Linear Units", section 2):
// z/2 (1 + tanh y), y = sqrt(2/pi) (z + 0.044715 z^3), evaluated as z * sigmoid(2y) =
// z / (1 + 2^(-2y log2 e)); both tails are exact limits (2^+inf = inf gives -0 for z << 0).
__device__ __forceinline__ float gelu_tanh(float z) {
  const float y = 0.7978845608028654f * fmaf(0.044715f * z, z * z, z);
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-2.8853900817779268f * y));
}

}  // namespace pblk
