// C ABI of the parallel-block forward (declared in include/pblock.h).
//
// pblock_forward enqueues four kernels on the caller's stream:
//   1. layernorm_kernel          x -> u
//   2. GEMM (split/GeLU epi)     u . W_in^T -> Q|K|V into `qkv`, GeLU(FC1) into ag[:, A:]
//   3. swa_attn kernel           qkv -> attention heads into ag[:, :A]
//   4. GEMM (residual epi)       ag . W_out^T (+ x) -> out
// The attention output and the GeLU activations share one K-contiguous buffer
// (ag), so the out-projection and FC2 run as a single GEMM: the two branches
// of the parallel block are summed inside its accumulators.
// pblock_forward_variant runs the same launches with epilogue switches (biases,
// rotary embedding of q and k, tanh GeLU), and with a second LayerNorm for the
// MLP branch splits the input GEMM in two around it.
#include <hip/hip_runtime.h>

#include <array>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/pblock.h"
#include "attn_bf16.hpp"
#include "attn_bwd_bf16.hpp"
#include "attn_f32.hpp"
#include "attn_tail.hpp"
#include "backward.hpp"
#include "gemm_bf16.hpp"
#include "gemm_f32.hpp"
#include "gemm_kmajor.hpp"
#include "gemm_wide.hpp"
#include "layernorm.hpp"
#include "rowchunks.hpp"

using namespace pblk;

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int elem_size(int32_t dtype) { return dtype == PBLOCK_BF16 ? 2 : 4; }

bool mult64(int64_t v) { return v > 0 && (v % 64) == 0; }

int validate(const pblock_cfg* c) {
  if (!c) return fail(PBLOCK_ERR_NULL, "cfg is NULL");
  if (c->dtype != PBLOCK_F32 && c->dtype != PBLOCK_BF16) return fail(PBLOCK_ERR_DTYPE, "dtype must be F32 or BF16");
  if (c->B < 1 || c->S < 1) return fail(PBLOCK_ERR_SHAPE, "B and S must be >= 1");
  if (int64_t(c->B) * c->S > (int64_t(1) << 24)) return fail(PBLOCK_ERR_SHAPE, "B*S exceeds 2^24");
  if (c->W < 1) return fail(PBLOCK_ERR_SHAPE, "W must be >= 1");
  if (c->hd != 64 && c->hd != 128) return fail(PBLOCK_ERR_SHAPE, "hd must be 64 or 128");
  if (c->H < 1 || c->H > 4096) return fail(PBLOCK_ERR_SHAPE, "H must be in [1, 4096]");
  if (!mult64(c->d) || c->d > 32768) return fail(PBLOCK_ERR_SHAPE, "d must be a positive multiple of 64, <= 32768");
  if (!mult64(c->ffn) || c->ffn > (1 << 20)) return fail(PBLOCK_ERR_SHAPE, "ffn must be a positive multiple of 64, <= 2^20");
  if (int64_t(c->H) * c->hd > (1 << 20)) return fail(PBLOCK_ERR_SHAPE, "H*hd exceeds 2^20");
  if (c->add_residual != 0 && c->add_residual != 1) return fail(PBLOCK_ERR_ARG, "add_residual must be 0 or 1");
  if (!(c->ln_eps > 0.f) || !std::isfinite(c->ln_eps)) return fail(PBLOCK_ERR_ARG, "ln_eps must be finite and > 0");
  return PBLOCK_OK;
}

struct Dims {
  int64_t M, A, n_in, k_out;
};
Dims dims(const pblock_cfg* c) {
  Dims d;
  d.M = int64_t(c->B) * c->S;
  d.A = int64_t(c->H) * c->hd;
  d.n_in = 3 * d.A + c->ffn;
  d.k_out = d.A + c->ffn;
  return d;
}

int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }


struct WsLayout {
  int64_t u, qkv, ag, partials, rope, counters, total;
};
// G = persistent GEMM workgroups (the device's CU count); 0 for a host-only estimate at 256.
WsLayout ws_layout(const pblock_cfg* c, int G) {
  const Dims dm = dims(c);
  const int es = elem_size(c->dtype);
  if (G <= 0) G = 256;
  // u and ag are the GEMMs' row operands: the bf16 GEMM reads its A operand up to the end of
  // the last 256-row tile it covers (rows past M are never stored), and a row-chunked
  // forward starts GEMMs at any row, so both get M rounded up to 256 plus one more tile
  const int64_t m_tiles = (dm.M + kGemmBM - 1) / kGemmBM * kGemmBM + kGemmBM;
  WsLayout w;
  w.u = 0;
  w.qkv = align256(m_tiles * c->d * es);
  w.ag = w.qkv + align256(dm.M * 3 * dm.A * es);
  w.partials = w.ag + align256(m_tiles * dm.k_out * es);
  int64_t part_bytes = 0;
  if (c->dtype == PBLOCK_BF16) {
    // the split-K tail holds at most G chunks (one wave)
    part_bytes = int64_t(G) * kGemmBM * kGemmBN * 4;
  }
  w.rope = w.partials + align256(part_bytes);
  // rotary-embedding table: (cos, sin) fp32 for hd/2 pairs at positions 0 .. M-1 (any S <= M)
  w.counters = w.rope + align256(dm.M * c->hd * 4);
  // per-chunk tile counters of the row-chunk publication (zeroed at creation)
  w.total = w.counters + align256(kMaxChunks * 4);
  return w;
}

// Per-device cache of "is this a gfx950": 0 unknown, 1 yes, -1 no (threads may fill it
// concurrently; they all store the same value).
std::atomic<int> g_arch_ok[64];

int check_device(int* dev_out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PBLOCK_ERR_DEVICE, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(PBLOCK_ERR_DEVICE, "device index out of range");
  if (g_arch_ok[dev].load(std::memory_order_relaxed) == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(PBLOCK_ERR_DEVICE, std::string("hipGetDeviceProperties: ") + hipGetErrorString(e));
    g_arch_ok[dev].store((std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1, std::memory_order_relaxed);
  }
  if (g_arch_ok[dev].load(std::memory_order_relaxed) != 1) return fail(PBLOCK_ERR_DEVICE, "current device is not gfx950");
  if (dev_out) *dev_out = dev;
  return PBLOCK_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + uintptr_t(nb) && b0 < a0 + uintptr_t(na);
}

int launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PBLOCK_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return PBLOCK_OK;
}

// Register-only MFMA loops (measurement aid): operands drawn from the thread id by an
// integer hash so the datapath sees non-trivial bf16 values.
template <int NOPS>
__device__ __forceinline__ void hashed_operands(uint32_t s, bf16x8 (&a)[NOPS], bf16x8 (&b)[NOPS]) {
#pragma unroll
  for (int i = 0; i < NOPS; ++i) {
    u32x4 ua, ub;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t h = (s * 16u + uint32_t(i) * 4u + uint32_t(e)) * 2654435761u;
      h ^= h >> 15;
      h *= 0x2c1b3c6du;
      h ^= h >> 12;
      ua[e] = h & 0x3F7F3F7Fu;  // two bf16 values in [0, 1) (sign and top exponent bits cleared)
      ub[e] = (h >> 1) & 0x3F7F3F7Fu;
    }
    a[i] = __builtin_bit_cast(bf16x8, ua);
    b[i] = __builtin_bit_cast(bf16x8, ub);
  }
}

// 32x32x16 form: 16 independent accumulators of 16, 16 MFMAs per iteration.
__global__ __launch_bounds__(256, 1) void mfma_loop32_kernel(int iters, float* sink) {
  const uint32_t s = blockIdx.x * 256u + threadIdx.x;
  bf16x8 a[4], b[4];
  hashed_operands<4>(s, a, b);
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) t += acc[i][j][r];
  sink[s] = t;
}

// 16x16x32 form (the GEMMs' instruction): 64 accumulators of 4, 32 MFMAs per iteration (the
// same flops as the 32x32x16 form's 16), run as all 64 every two iterations.  The MFMA is the
// GEMM's tied inline-asm form, with the same explicit wait states around the loop.
__global__ __launch_bounds__(256, 1) void mfma_loop16_kernel(int iters, float* sink) {
  const uint32_t s = blockIdx.x * 256u + threadIdx.x;
  bf16x8 a[8], b[8];
  hashed_operands<8>(s, a, b);
  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 4");
  __builtin_amdgcn_sched_barrier(0);
  auto rows = [&](int i0, int i1) __attribute__((always_inline)) {
#pragma unroll
    for (int i = i0; i < i1; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[i][j]) : "v"(b[j]), "v"(a[i]));
  };
  for (int it = 0; it + 2 <= iters; it += 2) rows(0, 8);
  if (iters & 1) rows(0, 4);
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
  __builtin_amdgcn_sched_barrier(0);
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) t += acc[i][j][r];
  sink[s] = t;
}

// The device GeLU forms of the GEMM epilogues, evaluated on their own (test entry):
// out[i] = f(z[i]) in fp32, before any bf16 rounding.  Grid-stride over n values.
__global__ __launch_bounds__(256) void activation_kernel(const float* __restrict__ z, float* __restrict__ out,
                                                         int64_t n, int form) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    const float v = z[i];
    float r;
    if (form == PBLOCK_ACT_GELU_ERF_F32) r = gelu_erf(v);
    else if (form == PBLOCK_ACT_GELU_ERF_BF16) r = gelu_erf_bf16out(v);
    else if (form == PBLOCK_ACT_GELU_TANH) r = gelu_tanh(v);
    else r = gelu_erf_grad(v);
    out[i] = r;
  }
}

// ------------------------------------------------------------------------ launches

constexpr int64_t kMaxGridWgs = (int64_t(1) << 24) - 1;  // workgroups of 256 in one launch
constexpr int64_t kMaxAttnLd = int64_t(1) << 24;          // row stride (elements) of the attention entry point
constexpr unsigned long long kPackTimeoutTicks = 200000000ull;  // 2 s of the 100 MHz device real-time clock

template <typename T>
void launch_layernorm(const T* x, const T* g, const T* b, T* u, int64_t M, int d, float eps, hipStream_t s,
                      float* stats = nullptr) {
  const int per = 16 / int(sizeof(T));
  const int need = (d / per + kLnThreads - 1) / kLnThreads;
  // Rows per workgroup: wide rows (>= 16 KiB) gain from gamma/beta reuse and the next-row
  // prefetch, narrow ones from more workgroups; at least 512 workgroups either way.  Rows
  // wider than 8 vectors per thread go one per workgroup.
  const int64_t row_bytes = int64_t(d) * int64_t(sizeof(T));
  const int want = row_bytes >= 16384 ? kLnMaxRows : (row_bytes >= 4096 ? 2 : 1);
  int rows = need > 8 ? 1 : int(std::max<int64_t>(1, std::min<int64_t>(want, M / 512)));
  // a launch holds fewer than 2^32 work-items: at most 2^24 - 1 workgroups of 256
  rows = int(std::max<int64_t>(rows, (M + kMaxGridWgs - 1) / kMaxGridWgs));
  const dim3 grid{static_cast<unsigned>((M + rows - 1) / rows)}, block{kLnThreads};
#define PBLK_LN(V) hipLaunchKernelGGL((layernorm_kernel<T, V>), grid, block, 0, s, x, g, b, u, M, d, rows, eps, stats)
  if (need <= 1) PBLK_LN(1);
  else if (need <= 2) PBLK_LN(2);
  else if (need <= 3) PBLK_LN(3);
  else if (need <= 4) PBLK_LN(4);
  else if (need <= 6) PBLK_LN(6);
  else if (need <= 8) PBLK_LN(8);
  else if (need <= 12) PBLK_LN(12);
  else if (need <= 16) PBLK_LN(16);
  else PBLK_LN(32);
#undef PBLK_LN
}

// GEMM scratch: fp32 partial tiles of the split-K tail (at most one wave of chunks).
struct SkScratch {
  float* partials;
  int G;  // workgroups resident at once (one per CU)
};

// Split of a T-tile GEMM over G resident workgroups: whole tiles in full waves,
// the remainder cut into k-chunks so that the last wave is (nearly) full.
struct Split {
  int dp_units, tail, split;
};
Split plan_split(int64_t T, int KT, int G) {
  Split p;
  const int64_t waves = T / G;
  p.tail = int(T - waves * G);
  p.dp_units = int(waves * G);
  p.split = 1;
  if (p.tail > 0) p.split = int(std::max<int64_t>(1, std::min<int64_t>(G / p.tail, KT)));
  if (p.split == 1) {  // more than half a wave left over: cutting k would not add workgroups
    p.dp_units = int(T);
    p.tail = 0;
  }
  return p;
}

// A split-K reduce left for the attention launch to run (see attn_tail.hpp).
struct TailPending {
  bool valid = false;
  GemmArgs g;
  GemmSched sk;
};

// One launch of gemm_bf16_kernel<EPI, BM, false, BN> in its direct-epilogue form when `direct`.
template <int EPI, int BM, int BN>
void launch_gemm_form(bool direct, unsigned grid, hipStream_t s, const GemmArgs& g, const GemmSched& sk) {
  if constexpr (EPI == kEpiSplitGelu || EPI == kEpiResidual) {
    if (direct) {
      hipLaunchKernelGGL((gemm_bf16_kernel<EPI, BM, false, BN, true>), dim3(grid), dim3(kGemmThreads), 0, s, g, sk,
                         RowPublish{});
      return;
    }
  }
  hipLaunchKernelGGL((gemm_bf16_kernel<EPI, BM, false, BN>), dim3(grid), dim3(kGemmThreads), 0, s, g, sk, RowPublish{});
}

template <int EPI>
void launch_gemm_bf16(const GemmArgs& g, const SkScratch& scr, hipStream_t s, TailPending* defer = nullptr) {
  const bool direct = gemm_direct_ok<EPI>(g);
  GemmSched sk;
  sk.partials = scr.partials;
  sk.wave_units = scr.G;
  sk.tiles_m = int((g.M + kGemmBM - 1) / kGemmBM);
  sk.tiles_n = int((g.N + kGemmBN - 1) / kGemmBN);
  sk.KT = g.K / kGemmBK;
  sk.unit_base = 0;
  const Split p = plan_split(int64_t(sk.tiles_m) * sk.tiles_n, sk.KT, scr.G);
  if constexpr (EPI == kEpiResidual) {
    const int tiles_nw = g.N / kWideBN;
    if (p.tail > 0 && g.N % kWideBN == 0 && int64_t(sk.tiles_m) * tiles_nw % scr.G == 0) {
      // 256 x 256 tiles leave a partial wave, 256 x 384 tiles fill whole waves: those, every
      // tile whole (3/2 of the work per tile at 5/4 of the operand traffic)
      sk.tiles_n = tiles_nw;
      sk.dp_units = sk.tiles_m * tiles_nw;
      sk.tail = 0;
      sk.split = 1;
      if (direct)
        hipLaunchKernelGGL((gemm_bf16_wide_kernel<EPI, true>), dim3(unsigned(sk.dp_units)), dim3(kGemmThreads), 0, s, g, sk);
      else
        hipLaunchKernelGGL((gemm_bf16_wide_kernel<EPI>), dim3(unsigned(sk.dp_units)), dim3(kGemmThreads), 0, s, g, sk);
      return;
    }
  }
  const int tiles_n192 = (g.N + 191) / 192;
  if (p.tail > 0 && int64_t(sk.tiles_m) * tiles_n192 % scr.G == 0) {
    // 256 x 256 tiles leave a partial wave, 256 x 192 tiles fill whole waves: those, every tile
    // whole (three quarters of the work per tile at seven eighths of the operand traffic)
    sk.tiles_n = tiles_n192;
    sk.dp_units = sk.tiles_m * tiles_n192;
    sk.tail = 0;
    sk.split = 1;
    launch_gemm_form<EPI, 256, 192>(direct, unsigned(sk.dp_units), s, g, sk);
    return;
  }
  if (p.tail > 0 && p.split == 2 && p.dp_units > 0) {
    // after whole waves, the remainder as 2 * tail half-height tiles (at most one wave): whole
    // tiles, no partials, no reduce (measured: 5% off the 4096 x 14336 x 2048 input GEMM, 1.3%
    // off the 2048 x 12288 x 7680 output GEMM; a GEMM that is one partial wave in all keeps the
    // k-split, whose halved k loops are faster there)
    sk.dp_units = p.dp_units;
    sk.tail = 0;
    sk.split = 1;
    launch_gemm_form<EPI, 256, 256>(direct, unsigned(p.dp_units), s, g, sk);
    GemmSched sh = sk;
    sh.dp_units = 2 * p.tail;
    sh.unit_base = p.dp_units;
    launch_gemm_form<EPI, 128, 256>(direct, unsigned(sh.dp_units), s, g, sh);
    return;
  }
  sk.dp_units = p.dp_units;
  sk.tail = p.tail;
  sk.split = p.split;
  const unsigned grid = unsigned(p.dp_units + p.tail * p.split);
  launch_gemm_form<EPI, 256, 256>(direct, grid, s, g, sk);
  if (p.tail > 0) {
    if (EPI == kEpiSplitGelu && defer != nullptr) {
      // the reduce writes only FC1 columns when every tail tile starts at or past nsplit
      bool fc1_only = true;
      for (int tl = 0; tl < p.tail && fc1_only; ++tl) {
        int tm, tn;
        tile_coords(p.dp_units + tl, sk.tiles_m, sk.tiles_n, &tm, &tn);
        fc1_only = tn * kGemmBN >= g.nsplit;
      }
      if (fc1_only) {
        defer->valid = true;
        defer->g = g;
        defer->sk = sk;
        return;
      }
    }
    hipLaunchKernelGGL((gemm_bf16_tail_reduce_kernel<EPI>), dim3(unsigned(p.tail * 32)), dim3(256), 0, s, g, sk);
  }
}

// The output GEMM with row-chunk publication (pub.n, S, B, flags, counters, epoch set by the
// caller): tiles in publication order, whole waves of 256 x 256 tiles, then a remainder of at
// most half a wave as 128 x 256 half-height tiles (no k-split: every tile publishes itself).
template <int EPI>
void launch_gemm_bf16_publish(const GemmArgs& g, const SkScratch& scr, RowPublish pub, hipStream_t s) {
  GemmSched sk{};
  sk.partials = nullptr;
  sk.tiles_m = int((g.M + kGemmBM - 1) / kGemmBM);
  sk.tiles_n = int((g.N + kGemmBN - 1) / kGemmBN);
  sk.KT = g.K / kGemmBK;
  sk.split = 1;
  sk.wave_units = scr.G;
  const int64_t T = int64_t(sk.tiles_m) * sk.tiles_n;
  const int64_t dp = (T / scr.G) * scr.G, tail = T - dp;
  const bool halves = tail > 0 && 2 * tail <= scr.G;
  const int64_t whole = halves ? dp : T;
  // tiles touching each chunk, unit by unit as the kernels will count them
  for (int k = 0; k < kMaxChunks; ++k) pub.need[k] = 0;
  auto count = [&](int r0, int r1) {
    for (uint64_t m = chunk_mask(r0, std::min(r1, g.M), pub.S, pub.n); m != 0; m &= m - 1) ++pub.need[__builtin_ctzll(m)];
  };
  for (int64_t L = 0; L < T; ++L) {
    int tm, tn;
    tile_coords_pub(int(L), sk.tiles_m, sk.tiles_n, pub, &tm, &tn);
    if (L < whole) {
      count(tm * 256, tm * 256 + 256);
    } else {
      count(tm * 256, tm * 256 + 128);
      count(tm * 256 + 128, tm * 256 + 256);
    }
  }
  if (whole > 0) {
    sk.dp_units = int(whole);
    hipLaunchKernelGGL((gemm_bf16_kernel<EPI, 256, true>), dim3(unsigned(whole)), dim3(kGemmThreads), 0, s, g, sk, pub);
  }
  if (halves) {
    GemmSched sh = sk;
    sh.dp_units = int(2 * tail);
    sh.unit_base = int(dp);
    hipLaunchKernelGGL((gemm_bf16_kernel<EPI, 128, true>), dim3(unsigned(2 * tail)), dim3(kGemmThreads), 0, s, g, sh,
                       pub);
  }
}

template <int EPI>
void launch_gemm_f32(const GemmArgsF32& g, hipStream_t s) {
  const unsigned grid = unsigned(((g.M + 63) / 64) * ((g.N + 63) / 64));
  hipLaunchKernelGGL((gemm_f32_kernel<EPI>), dim3(grid), dim3(256), 0, s, g);
}

// Attention for query positions [q_lo, q_hi) of each of the B sequences.
void launch_attention(const void* qkv, int64_t ld_qkv, void* o, int64_t ld_o, int B, int S, int H, int hd, int W,
                      int dtype, hipStream_t s, int q_lo = 0, int q_hi = -1, float* lse = nullptr,
                      const TailPending* tail = nullptr) {
  if (q_hi < 0) q_hi = S;
  // W >= S is full causal attention; clamping keeps every window sum in the kernels' int range
  W = std::min(W, S);
  const float scale = 1.0f / std::sqrt(float(hd));
  if (dtype == PBLOCK_BF16) {
    AttnArgs a{};
    a.lse = lse;
    a.qkv = static_cast<const uint16_t*>(qkv);
    a.ld_qkv = ld_qkv;
    a.o = static_cast<uint16_t*>(o);
    a.ld_o = ld_o;
    a.B = B; a.S = S; a.H = H; a.W = W;
    a.q_lo = q_lo; a.q_hi = q_hi;
    a.scale_log2 = scale * 1.4426950408889634f;
    const unsigned grid = unsigned(((q_hi - q_lo + kAttnBQ - 1) / kAttnBQ) * int64_t(B) * H);
    if (tail != nullptr && tail->valid) {
      // the input GEMM's split-K reduce in the same launch: 8 row groups (64 rows) per workgroup
      constexpr int kRpw = 8;
      const int n_groups = tail->sk.tail * 32;
      const unsigned total = grid + unsigned((n_groups + kRpw - 1) / kRpw);
      if (hd == 128)
        hipLaunchKernelGGL((swa_attn_tail_kernel<128>), dim3(total), dim3(256), 0, s, a, int(grid), tail->g, tail->sk,
                           kRpw, n_groups);
      else
        hipLaunchKernelGGL((swa_attn_tail_kernel<64>), dim3(total), dim3(256), 0, s, a, int(grid), tail->g, tail->sk,
                           kRpw, n_groups);
    } else if (hd == 128) {
      hipLaunchKernelGGL((swa_attn_bf16_kernel<128>), dim3(grid), dim3(256), 0, s, a);
    } else {
      hipLaunchKernelGGL((swa_attn_bf16_kernel<64>), dim3(grid), dim3(256), 0, s, a);
    }
  } else {
    const dim3 grid{unsigned(int64_t((q_hi - q_lo + 63) / 64) * H * B)};
    const float* q = static_cast<const float*>(qkv);
    float* out = static_cast<float*>(o);
    if (hd == 128)
      hipLaunchKernelGGL((swa_attn_f32_kernel<128>), grid, dim3(64), 0, s, q, ld_qkv, out, ld_o, S, H, W, scale, q_lo, q_hi);
    else
      hipLaunchKernelGGL((swa_attn_f32_kernel<64>), grid, dim3(64), 0, s, q, ld_qkv, out, ld_o, S, H, W, scale, q_lo, q_hi);
  }
}

// timing categories: layernorm, gemm_in, attention, gemm_out (forward); prep (dy staged into
// whole tiles, token padding zeroed), gemm_dgrad, attention, gemm_wgrad, layernorm (backward)
constexpr int kTimedKernels = 9;
constexpr int kMaxLaunches = 12;  // launches (or launch groups) of one call that get their own event pair
constexpr size_t kEventPool = 256;

// Events of one timed forward: ev[k] .. ev[k+1] brackets launch k, of category cat[k].
struct EventSet {
  std::array<hipEvent_t, kMaxLaunches + 1> ev;
  int n;
  int cat[kMaxLaunches];
};

}  // namespace

struct pblock_s {
  pblock_cfg cfg;
  int device;
  int64_t m_cap;
  int64_t last_m;  // B*S of the most recent forward (0: none yet)
  int n_cu;        // compute units: persistent GEMM workgroups
  void* ws;
  WsLayout lay;
  bool timing;
  std::vector<EventSet> events;
  size_t ev_used;
  double ms_sum[kTimedKernels];
  int n_forwards;
  double rope_base;         // base the rotary table in the workspace was built for (NaN: none yet)
  hipStream_t rope_stream;  // stream it was built on (a call on another stream rebuilds it there)
};

namespace {

void destroy_events(pblock_s* h) {
  for (auto& set : h->events)
    for (auto e : set.ev) (void)hipEventDestroy(e);
  h->events.clear();
  h->ev_used = 0;
}

int drain_events(pblock_s* h) {
  for (size_t i = 0; i < h->ev_used; ++i) {
    auto& set = h->events[i];
    hipError_t e = hipEventSynchronize(set.ev[set.n]);
    if (e != hipSuccess) return fail(PBLOCK_ERR_HIP, std::string("hipEventSynchronize: ") + hipGetErrorString(e));
    for (int k = 0; k < set.n; ++k) {
      float ms = 0.f;
      e = hipEventElapsedTime(&ms, set.ev[k], set.ev[k + 1]);
      if (e != hipSuccess) return fail(PBLOCK_ERR_HIP, std::string("hipEventElapsedTime: ") + hipGetErrorString(e));
      h->ms_sum[set.cat[k]] += ms;
    }
    h->n_forwards += 1;
  }
  h->ev_used = 0;
  return PBLOCK_OK;
}

// Argument checks of the block forward that need no handle (all before any launch): pointers
// and cfg (part 1), alignment and aliasing (part 2).
int check_block_ptrs(const void* x, const pblock_weights* w, const pblock_cfg* cfg, void* out) {
  if (!x || !w || !out || !w->ln_gamma || !w->ln_beta || !w->w_in || !w->w_out)
    return fail(PBLOCK_ERR_NULL, "x, out, weights or a weight pointer is NULL");
  return validate(cfg);
}
int check_block_layout(const void* x, const pblock_weights* w, const pblock_cfg& c, const Dims& dm, void* out) {
  if (!aligned16(x) || !aligned16(out) || !aligned16(w->ln_gamma) || !aligned16(w->ln_beta) ||
      !aligned16(w->w_in) || !aligned16(w->w_out))
    return fail(PBLOCK_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  const int es = elem_size(c.dtype);
  const int64_t xb = dm.M * c.d * es;
  if (overlap(out, xb, x, xb) || overlap(out, xb, w->w_in, dm.n_in * c.d * es) ||
      overlap(out, xb, w->w_out, int64_t(c.d) * dm.k_out * es) || overlap(out, xb, w->ln_gamma, c.d * es) ||
      overlap(out, xb, w->ln_beta, c.d * es))
    return fail(PBLOCK_ERR_ALIAS, "out overlaps x or a weight");
  return PBLOCK_OK;
}

// Argument checks shared by the handle's block forms (all before any launch).
int check_forward(pblock_t h, const void* x, const pblock_weights* w, const pblock_cfg* cfg, void* out, Dims* dm_out) {
  if (!h) return fail(PBLOCK_ERR_NULL, "handle is NULL");
  int st = check_block_ptrs(x, w, cfg, out);
  if (st != PBLOCK_OK) return st;
  const pblock_cfg& c = *cfg;
  const pblock_cfg& hc = h->cfg;
  if (c.d != hc.d || c.H != hc.H || c.hd != hc.hd || c.ffn != hc.ffn || c.dtype != hc.dtype)
    return fail(PBLOCK_ERR_CFG_MISMATCH, "d, H, hd, ffn and dtype must equal the handle's");
  const Dims dm = dims(&c);
  if (dm.M > h->m_cap) return fail(PBLOCK_ERR_CFG_MISMATCH, "B*S exceeds the handle's B*S");
  st = check_block_layout(x, w, c, dm, out);
  if (st != PBLOCK_OK) return st;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev != h->device) return fail(PBLOCK_ERR_DEVICE, "current device differs from the handle's");
  *dm_out = dm;
  return PBLOCK_OK;
}

struct Ws {
  void *u, *qkv, *ag;
  float* rope;
  SkScratch scr;
};
Ws workspace(pblock_s* h) {
  char* base = static_cast<char*>(h->ws);
  Ws w;
  w.u = base + h->lay.u;
  w.qkv = base + h->lay.qkv;
  w.ag = base + h->lay.ag;
  w.rope = reinterpret_cast<float*>(base + h->lay.rope);
  w.scr.partials = reinterpret_cast<float*>(base + h->lay.partials);
  w.scr.G = h->n_cu;
  return w;
}

// HIP events around the launches of one forward when the handle's timing is on.
struct Timer {
  EventSet* set = nullptr;
  hipStream_t s = nullptr;
  int begin(pblock_s* h, hipStream_t stream) {
    s = stream;
    if (!h->timing) return PBLOCK_OK;
    if (h->ev_used == h->events.size()) {
      int st = drain_events(h);
      if (st != PBLOCK_OK) return st;
    }
    set = &h->events[h->ev_used++];
    set->n = 0;
    (void)hipEventRecord(set->ev[0], s);
    return PBLOCK_OK;
  }
  void mark(int category) {
    if (!set || set->n >= kMaxLaunches) return;
    set->cat[set->n] = category;
    (void)hipEventRecord(set->ev[++set->n], s);
  }
};

void run_layernorm(const void* x, const void* g, const void* b, void* u, int64_t M, const pblock_cfg& c, hipStream_t s,
                   float* stats = nullptr) {
  if (c.dtype == PBLOCK_BF16)
    launch_layernorm(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(g), static_cast<const uint16_t*>(b),
                     static_cast<uint16_t*>(u), M, c.d, c.ln_eps, s, stats);
  else
    launch_layernorm(static_cast<const float*>(x), static_cast<const float*>(g), static_cast<const float*>(b),
                     static_cast<float*>(u), M, c.d, c.ln_eps, s);
}

// Variant steps of the input GEMM's epilogue (all off by default).
struct InEpi {
  const void* bias = nullptr;  // [N] per output column
  const float* rope = nullptr;  // rotary table; columns [0, rope_n) are q and k heads
  int rope_n = 0;
  int seq = 1;  // positions per sequence: row m is at position m % seq
  int hd = 64;
  int gelu_tanh = 0;
  void* pre = nullptr;  // FC1 pre-activation store [M, N - nsplit] (row stride ld_pre), bf16 only
  int64_t ld_pre = 0;
};

// out0[m, n] = Z[m, n] for n < nsplit; out1[m, off1 + n - nsplit] = GeLU(Z[m, n]) otherwise;
// Z = A B^T, A [M, K] (row stride lda), B [N, K] (row stride ldb).
void run_gemm_in(const void* a, int64_t lda, const void* b, int64_t ldb, int64_t M, int64_t N, int64_t K, void* out0,
                 int64_t ld0, void* out1, int64_t ld1, int64_t off1, int64_t nsplit, int dtype, const SkScratch& scr,
                 hipStream_t s, const InEpi& ep = InEpi{}, TailPending* defer = nullptr) {
  if (dtype == PBLOCK_BF16) {
    GemmArgs g{};
    g.a = static_cast<const uint16_t*>(a); g.lda = lda;
    g.b = static_cast<const uint16_t*>(b); g.ldb = ldb;
    g.M = int(M); g.N = int(N); g.K = int(K);
    g.out0 = static_cast<uint16_t*>(out0); g.ld0 = ld0;
    g.out1 = static_cast<uint16_t*>(out1); g.ld1 = ld1; g.off1 = off1;
    g.nsplit = int(nsplit);
    g.bias = static_cast<const uint16_t*>(ep.bias);
    g.rope = ep.rope; g.rope_n = ep.rope_n; g.seq = ep.seq; g.hd = ep.hd;
    g.gelu_tanh = ep.gelu_tanh;
    g.pre = static_cast<uint16_t*>(ep.pre);
    g.ld_pre = ep.ld_pre;
    launch_gemm_bf16<kEpiSplitGelu>(g, scr, s, defer);
  } else {
    GemmArgsF32 g{};
    g.a = static_cast<const float*>(a); g.lda = lda;
    g.b = static_cast<const float*>(b); g.ldb = ldb;
    g.M = int(M); g.N = int(N); g.K = int(K);
    g.out0 = static_cast<float*>(out0); g.ld0 = ld0;
    g.out1 = static_cast<float*>(out1); g.ld1 = ld1; g.off1 = off1;
    g.nsplit = int(nsplit);
    g.bias = static_cast<const float*>(ep.bias);
    g.rope = ep.rope; g.rope_n = ep.rope_n; g.seq = ep.seq; g.hd = ep.hd;
    g.gelu_tanh = ep.gelu_tanh;
    launch_gemm_f32<kEpiSplitGelu>(g, s);
  }
}

// out [M, N] (row stride N) = A B^T (+ bias [N]) (+ resid [M, N], row stride N); resid may be
// out itself (each element is read by the thread that then writes it).
void run_gemm_out(const void* a, int64_t lda, const void* b, int64_t ldb, int64_t M, int64_t N, int64_t K, void* out,
                  const void* resid, int dtype, const SkScratch& scr, hipStream_t s, const void* bias = nullptr) {
  if (dtype == PBLOCK_BF16) {
    GemmArgs g{};
    g.a = static_cast<const uint16_t*>(a); g.lda = lda;
    g.b = static_cast<const uint16_t*>(b); g.ldb = ldb;
    g.M = int(M); g.N = int(N); g.K = int(K);
    g.out0 = static_cast<uint16_t*>(out); g.ld0 = N;
    g.resid = static_cast<const uint16_t*>(resid); g.ldr = N;
    g.bias = static_cast<const uint16_t*>(bias);
    launch_gemm_bf16<kEpiResidual>(g, scr, s);
  } else {
    GemmArgsF32 g{};
    g.a = static_cast<const float*>(a); g.lda = lda;
    g.b = static_cast<const float*>(b); g.ldb = ldb;
    g.M = int(M); g.N = int(N); g.K = int(K);
    g.out0 = static_cast<float*>(out); g.ld0 = N;
    g.resid = static_cast<const float*>(resid); g.ldr = N;
    g.bias = static_cast<const float*>(bias);
    launch_gemm_f32<kEpiResidual>(g, s);
  }
}

// ------------------------------------------------------------------------ training

// Caller-owned training workspace: the activations pblock_forward_train saves (u, q|k|v,
// [attention | GeLU], the FC1 pre-activation F, the softmax log-sum-exp) and the backward
// pass's scratch.  Offsets depend on the call's B*S, so forward_train and backward must be
// called with the same cfg.
struct TrainLayout {
  int64_t u, qkv, ag, f, lse, stats, delta, dyp, dO, dz, du, part, total;
  int64_t Mp, ln_rows, ln_grid;
};
TrainLayout train_layout(const pblock_cfg* c) {
  const Dims dm = dims(c);
  const int64_t es = 2, M = dm.M, d = c->d;
  const int64_t m256 = (M + kGemmBM - 1) / kGemmBM * kGemmBM;
  const int64_t Mt = m256 + kGemmBM;
  TrainLayout t;
  t.Mp = (M + kGemmBK - 1) / kGemmBK * kGemmBK;  // token count padded to the GEMM's k slab
  t.ln_rows = std::max<int64_t>(1, (M + 511) / 512);  // about two LayerNorm-backward workgroups per CU
  t.ln_grid = (M + t.ln_rows - 1) / t.ln_rows;
  int64_t o = 0;
  auto take = [&](int64_t bytes) {
    const int64_t at = o;
    o += align256(bytes);
    return at;
  };
  t.u = take(Mt * d * es);  // GEMM row operands: whole 256-row tiles (+ one, as the forward's)
  t.qkv = take(M * 3 * dm.A * es);
  t.ag = take(Mt * dm.k_out * es);
  t.f = take(M * c->ffn * es);
  t.lse = take(M * c->H * 4);
  t.stats = take(M * 2 * 4);
  t.delta = take(M * c->H * 4);
  t.dyp = take(m256 * d * es);
  t.dO = take(M * dm.A * es);
  t.dz = take(m256 * dm.n_in * es);
  t.du = take(M * d * 4);
  t.part = take(t.ln_grid * 2 * d * 4);
  t.total = o;
  return t;
}

// Zeroes rows [r0, r1) of a row-major bf16 matrix with ld columns (ld a multiple of 8): the token
// padding the weight-gradient GEMMs read as k rows.
void launch_zero_rows(void* base, int64_t ld, int64_t r0, int64_t r1, hipStream_t s) {
  if (r1 <= r0) return;
  const int64_t n16 = (r1 - r0) * ld / 8;  // 16-byte pieces
  hipLaunchKernelGGL(zero_kernel, dim3(unsigned(std::min<int64_t>((n16 + 255) / 256, 1024))), dim3(256), 0, s,
                     reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + r0 * ld), n16);
}

constexpr int kBwdMaxD = 16384;  // LayerNorm backward holds up to 8 vectors of 8 per thread

int check_train(pblock_t h, const void* x, const pblock_weights* w, const pblock_cfg* cfg, void* ws, int64_t ws_bytes,
                Dims* dm, TrainLayout* lay) {
  if (!ws) return fail(PBLOCK_ERR_NULL, "training workspace is NULL");
  // the shared checks, with the workspace in the place of out (the real out is checked by the caller)
  int st = check_forward(h, x, w, cfg, ws, dm);
  if (st != PBLOCK_OK) return st;
  if (cfg->dtype != PBLOCK_BF16) return fail(PBLOCK_ERR_DTYPE, "the training path is bf16 only");
  if (cfg->d > kBwdMaxD) return fail(PBLOCK_ERR_SHAPE, "the backward pass supports d <= 16384");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(PBLOCK_ERR_ALIGN, "training workspace must be 256-byte aligned");
  *lay = train_layout(cfg);
  if (ws_bytes < lay->total) return fail(PBLOCK_ERR_ARG, "training workspace too small (pblock_train_workspace_bytes)");
  const int64_t es = 2;
  const int64_t xb = dm->M * cfg->d * es;
  if (overlap(ws, lay->total, x, xb) || overlap(ws, lay->total, w->w_in, dm->n_in * cfg->d * es) ||
      overlap(ws, lay->total, w->w_out, int64_t(cfg->d) * dm->k_out * es) ||
      overlap(ws, lay->total, w->ln_gamma, cfg->d * es) || overlap(ws, lay->total, w->ln_beta, cfg->d * es))
    return fail(PBLOCK_ERR_ALIAS, "training workspace overlaps x or a weight");
  return PBLOCK_OK;
}

// ------------------------------------------------------------------------ static workspace
// The no-allocation forward keeps its intermediates in this file-scope device array: one copy
// per GPU the library runs on, held until the process ends.  Host code never passes `scratch`
// itself to a kernel (in host code it names a host-side stand-in); it uses the device address
// hipGetSymbolAddress returns for the current device, looked up once per device.
constexpr int64_t kStaticScratchBytes = int64_t(256) << 20;

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // device address of `scratch` per device (nullptr: not looked up yet)
int g_scratch_cus[64];    // compute units of that device

}  // namespace

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

int static_scratch(int dev, void** ptr, int* n_cu) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(PBLOCK_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    }
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || cus <= 0) return fail(PBLOCK_ERR_DEVICE, "cannot query the compute-unit count");
    g_scratch_cus[dev] = cus;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *n_cu = g_scratch_cus[dev];
  return PBLOCK_OK;
}

// The four launches of the block forward on stream s, intermediates in ws.
void enqueue_forward(const Ws& ws, const void* x, const pblock_weights* w, const pblock_cfg& c, const Dims& dm,
                     void* out, hipStream_t s, Timer* tm) {
  const int64_t A = dm.A;
  run_layernorm(x, w->ln_gamma, w->ln_beta, ws.u, dm.M, c, s);
  tm->mark(0);
  // Z = u W_in^T: Q|K|V columns to QKV, FC1 columns through GeLU to AG[:, A:]
  // (a split-K reduce of FC1-only tail tiles runs inside the attention launch)
  TailPending tail;
  run_gemm_in(ws.u, c.d, w->w_in, c.d, dm.M, dm.n_in, c.d, ws.qkv, 3 * A, ws.ag, dm.k_out, A, 3 * A, c.dtype, ws.scr,
              s, InEpi{}, &tail);
  tm->mark(1);
  launch_attention(ws.qkv, 3 * A, ws.ag, dm.k_out, c.B, c.S, c.H, c.hd, c.W, c.dtype, s, 0, -1, nullptr, &tail);
  tm->mark(2);
  // y = [attention | GeLU] W_out^T (+ x): both branches summed in one accumulator
  run_gemm_out(ws.ag, dm.k_out, w->w_out, dm.k_out, dm.M, c.d, dm.k_out, out, c.add_residual ? x : nullptr, c.dtype,
               ws.scr, s);
  tm->mark(3);
}

}  // namespace

extern "C" {

int pblock_validate_cfg(const pblock_cfg* cfg) {
  try {
    return validate(cfg);
  } catch (...) {
    return fail(PBLOCK_ERR_ARG, "internal error");
  }
}

int64_t pblock_workspace_bytes(const pblock_cfg* cfg) {
  const int st = validate(cfg);
  if (st != PBLOCK_OK) return st;
  return ws_layout(cfg, 0).total;
}

double pblock_flops(const pblock_cfg* cfg) {
  if (validate(cfg) != PBLOCK_OK) return -1.0;
  const Dims dm = dims(cfg);
  const int64_t S = cfg->S, w = std::min<int64_t>(cfg->W, cfg->S);
  const double keys = double(S * w - w * (w - 1) / 2);
  return 2.0 * dm.M * cfg->d * dm.n_in + 2.0 * dm.M * dm.k_out * cfg->d + 4.0 * cfg->B * cfg->H * cfg->hd * keys;
}

int pblock_create(const pblock_cfg* cfg, pblock_t* out_handle) {
  try {
    if (!out_handle) return fail(PBLOCK_ERR_NULL, "out_handle is NULL");
    int st = validate(cfg);
    if (st != PBLOCK_OK) return st;
    int dev = -1;
    st = check_device(&dev);
    if (st != PBLOCK_OK) return st;
    pblock_s* h = new pblock_s();
    h->cfg = *cfg;
    h->device = dev;
    h->m_cap = int64_t(cfg->B) * cfg->S;
    h->last_m = 0;
    int n_cu = 0;
    hipError_t ea = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (ea != hipSuccess || n_cu <= 0) {
      delete h;
      return fail(PBLOCK_ERR_DEVICE, "cannot query the compute-unit count");
    }
    h->n_cu = n_cu;
    h->lay = ws_layout(cfg, n_cu);
    h->ws = nullptr;
    h->timing = false;
    h->ev_used = 0;
    h->n_forwards = 0;
    h->rope_base = std::nan("");
    h->rope_stream = nullptr;
    for (double& v : h->ms_sum) v = 0.0;
    hipError_t e = hipMalloc(&h->ws, size_t(h->lay.total));
    if (e != hipSuccess) {
      delete h;
      (void)hipGetLastError();
      return fail(PBLOCK_ERR_NOMEM, std::string("hipMalloc workspace: ") + hipGetErrorString(e));
    }
    e = hipMemset(static_cast<char*>(h->ws) + h->lay.counters, 0, size_t(kMaxChunks * 4));
    if (e != hipSuccess) {
      (void)hipFree(h->ws);
      delete h;
      (void)hipGetLastError();
      return fail(PBLOCK_ERR_HIP, std::string("hipMemset chunk counters: ") + hipGetErrorString(e));
    }
    *out_handle = h;
    return PBLOCK_OK;
  } catch (...) {
    return fail(PBLOCK_ERR_NOMEM, "host allocation failed");
  }
}

int pblock_destroy(pblock_t h) {
  if (!h) return PBLOCK_OK;
  destroy_events(h);
  hipError_t e = hipFree(h->ws);
  delete h;
  if (e != hipSuccess) return fail(PBLOCK_ERR_HIP, std::string("hipFree: ") + hipGetErrorString(e));
  return PBLOCK_OK;
}

int pblock_intermediates(pblock_t h, void** u, void** qkv, void** ag) {
  if (!h) return fail(PBLOCK_ERR_NULL, "handle is NULL");
  char* base = static_cast<char*>(h->ws);
  if (u) *u = base + h->lay.u;
  if (qkv) *qkv = base + h->lay.qkv;
  if (ag) *ag = base + h->lay.ag;
  return PBLOCK_OK;
}

int pblock_copy_intermediates(pblock_t h, void* u, void* qkv, void* ag, void* stream) {
  if (!h) return fail(PBLOCK_ERR_NULL, "handle is NULL");
  if (h->last_m == 0) return fail(PBLOCK_ERR_ARG, "no forward has run on this handle");
  const Dims dm = dims(&h->cfg);
  const int64_t es = elem_size(h->cfg.dtype), M = h->last_m;
  const char* base = static_cast<const char*>(h->ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  struct Item { void* dst; int64_t off, bytes; } items[3] = {
      {u, h->lay.u, M * h->cfg.d * es}, {qkv, h->lay.qkv, M * 3 * dm.A * es}, {ag, h->lay.ag, M * dm.k_out * es}};
  for (const Item& it : items) {
    if (!it.dst) continue;
    hipError_t e = hipMemcpyAsync(it.dst, base + it.off, size_t(it.bytes), hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return fail(PBLOCK_ERR_HIP, std::string("hipMemcpyAsync: ") + hipGetErrorString(e));
  }
  return PBLOCK_OK;
}

int pblock_set_timing(pblock_t h, int enable) {
  try {
    if (!h) return fail(PBLOCK_ERR_NULL, "handle is NULL");
    destroy_events(h);
    for (double& v : h->ms_sum) v = 0.0;
    h->n_forwards = 0;
    h->timing = enable != 0;
    if (h->timing) {
      h->events.resize(kEventPool);
      for (auto& set : h->events)
        for (auto& ev : set.ev) {
          hipError_t e = hipEventCreate(&ev);
          if (e != hipSuccess) {
            h->timing = false;
            return fail(PBLOCK_ERR_HIP, std::string("hipEventCreate: ") + hipGetErrorString(e));
          }
        }
    }
    return PBLOCK_OK;
  } catch (...) {
    return fail(PBLOCK_ERR_NOMEM, "host allocation failed");
  }
}

int pblock_kernel_times(pblock_t h, float* ms, int n, int* n_forwards) {
  if (!h || !ms) return fail(PBLOCK_ERR_NULL, "handle or ms is NULL");
  if (n < 4) return fail(PBLOCK_ERR_ARG, "n must be >= 4");
  int st = drain_events(h);
  if (st != PBLOCK_OK) return st;
  for (int k = 0; k < std::min(n, kTimedKernels); ++k) ms[k] = float(h->ms_sum[k]);
  if (n_forwards) *n_forwards = h->n_forwards;
  return PBLOCK_OK;
}

int pblock_forward(pblock_t h, const void* x, const pblock_weights* w, const pblock_cfg* cfg, void* out,
                   void* stream) {
  try {
    Dims dm;
    int st = check_forward(h, x, w, cfg, out, &dm);
    if (st != PBLOCK_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Timer tm;
    st = tm.begin(h, s);
    if (st != PBLOCK_OK) return st;
    enqueue_forward(workspace(h), x, w, *cfg, dm, out, s, &tm);
    h->last_m = dm.M;
    return launch_status("pblock_forward launch");
  } catch (...) {
    return fail(PBLOCK_ERR_ARG, "internal error");
  }
}

int pblock_forward_static(const void* x, const pblock_weights* w, const pblock_cfg* cfg, void* out, void* stream) {
  try {
    int st = check_block_ptrs(x, w, cfg, out);
    if (st != PBLOCK_OK) return st;
    const pblock_cfg& c = *cfg;
    const Dims dm = dims(&c);
    st = check_block_layout(x, w, c, dm, out);
    if (st != PBLOCK_OK) return st;
    int dev = -1;
    st = check_device(&dev);
    if (st != PBLOCK_OK) return st;
    void* base = nullptr;
    int n_cu = 0;
    st = static_scratch(dev, &base, &n_cu);
    if (st != PBLOCK_OK) return st;
    const WsLayout lay = ws_layout(&c, n_cu);
    if (lay.rope > kStaticScratchBytes)
      return fail(PBLOCK_ERR_SHAPE, "cfg needs " + std::to_string(lay.rope) + " bytes of workspace; the static one holds " +
                                        std::to_string(kStaticScratchBytes));
    char* b = static_cast<char*>(base);
    Ws ws;
    ws.u = b + lay.u;
    ws.qkv = b + lay.qkv;
    ws.ag = b + lay.ag;
    ws.rope = nullptr;
    ws.scr.partials = reinterpret_cast<float*>(b + lay.partials);
    ws.scr.G = n_cu;
    Timer tm;  // no timing: no handle
    enqueue_forward(ws, x, w, c, dm, out, static_cast<hipStream_t>(stream), &tm);
    return launch_status("pblock_forward_static launch");
  } catch (...) {
    return fail(PBLOCK_ERR_ARG, "internal error");
  }
}

int pblock_forward_rowchunks(pblock_t h, const void* x, const pblock_weights* w, const pblock_cfg* cfg, void* out,
                             int32_t n_chunks, uint32_t* flags, uint32_t epoch, void* stream) {
  try {
    Dims dm;
    int st = check_forward(h, x, w, cfg, out, &dm);
    if (st != PBLOCK_OK) return st;
    const pblock_cfg& c = *cfg;
    if (c.dtype != PBLOCK_BF16) return fail(PBLOCK_ERR_DTYPE, "the row-chunk publication is bf16 only");
    if (n_chunks < 1 || n_chunks > std::min(c.S, kMaxChunks))
      return fail(PBLOCK_ERR_ARG, "n_chunks must be in [1, min(S, 64)]");
    if (!flags) return fail(PBLOCK_ERR_NULL, "flags is NULL");
    if ((reinterpret_cast<uintptr_t>(flags) & 3u) != 0) return fail(PBLOCK_ERR_ALIGN, "flags must be 4-byte aligned");
    if (epoch == 0) return fail(PBLOCK_ERR_ARG, "epoch must be nonzero");
    const int64_t xb = dm.M * c.d * 2;
    if (overlap(flags, n_chunks * 4, out, xb) || overlap(flags, n_chunks * 4, x, xb) ||
        overlap(flags, n_chunks * 4, w->w_in, dm.n_in * c.d * 2) ||
        overlap(flags, n_chunks * 4, w->w_out, int64_t(c.d) * dm.k_out * 2))
      return fail(PBLOCK_ERR_ALIAS, "flags overlap out, x or a weight");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Ws ws = workspace(h);
    Timer tm;
    st = tm.begin(h, s);
    if (st != PBLOCK_OK) return st;
    const int64_t A = dm.A;
    run_layernorm(x, w->ln_gamma, w->ln_beta, ws.u, dm.M, c, s);
    tm.mark(0);
    run_gemm_in(ws.u, c.d, w->w_in, c.d, dm.M, dm.n_in, c.d, ws.qkv, 3 * A, ws.ag, dm.k_out, A, 3 * A, c.dtype, ws.scr,
                s);
    tm.mark(1);
    launch_attention(ws.qkv, 3 * A, ws.ag, dm.k_out, c.B, c.S, c.H, c.hd, c.W, c.dtype, s);
    tm.mark(2);
    GemmArgs g{};
    g.a = static_cast<const uint16_t*>(ws.ag); g.lda = dm.k_out;
    g.b = static_cast<const uint16_t*>(w->w_out); g.ldb = dm.k_out;
    g.M = int(dm.M); g.N = c.d; g.K = int(dm.k_out);
    g.out0 = static_cast<uint16_t*>(out); g.ld0 = c.d;
    g.resid = c.add_residual ? static_cast<const uint16_t*>(x) : nullptr; g.ldr = c.d;
    RowPublish pub{};
    pub.counters = reinterpret_cast<uint32_t*>(static_cast<char*>(h->ws) + h->lay.counters);
    pub.flags = flags;
    pub.epoch = epoch;
    pub.n = n_chunks;
    pub.S = c.S;
    pub.B = c.B;
    // M-tiles per group of the publication order (M fastest inside a group): each XCD's 32
    // concurrent tiles then span 2 M-tiles and 16 N-tiles.  Measured at the 175B shard shape in
    // alternating rounds against pblock_forward: 2 costs 0.1-0.3% at 4 and 8 chunks, 1, 4 or 8
    // cost 0.7-1.2%.
    pub.group_m = 2;
    launch_gemm_bf16_publish<kEpiResidual>(g, ws.scr, pub, s);
    tm.mark(3);
    h->last_m = dm.M;
    return launch_status("pblock_forward_rowchunks launch");
  } catch (...) {
    return fail(PBLOCK_ERR_ARG, "internal error");
  }
}

int pblock_pack_chunks(const void* out, const pblock_cfg* cfg, int32_t n_chunks, const uint32_t* flags, uint32_t epoch,
                       void* send, uint64_t* stamps, void* stream) {
  try {
    if (!out || !flags || !send || !stamps) return fail(PBLOCK_ERR_NULL, "out, flags, send or stamps is NULL");
    int st = validate(cfg);
    if (st != PBLOCK_OK) return st;
    const pblock_cfg& c = *cfg;
    if (c.dtype != PBLOCK_BF16) return fail(PBLOCK_ERR_DTYPE, "the row-chunk publication is bf16 only");
    if (n_chunks < 1 || n_chunks > std::min(c.S, kMaxChunks))
      return fail(PBLOCK_ERR_ARG, "n_chunks must be in [1, min(S, 64)]");
    if (!aligned16(out) || !aligned16(send) || (reinterpret_cast<uintptr_t>(flags) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(stamps) & 7u) != 0)
      return fail(PBLOCK_ERR_ALIGN, "out and send 16-byte, flags 4-byte, stamps 8-byte aligned");
    const int64_t bytes = int64_t(c.B) * c.S * c.d * 2;
    if (overlap(send, bytes, out, bytes) || overlap(stamps, n_chunks * 8, out, bytes) ||
        overlap(stamps, n_chunks * 8, send, bytes) || overlap(flags, n_chunks * 4, send, bytes) ||
        overlap(stamps, n_chunks * 8, flags, n_chunks * 4))
      return fail(PBLOCK_ERR_ALIAS, "send, stamps, flags and out must not overlap");
    st = check_device(nullptr);
    if (st != PBLOCK_OK) return st;
    PackArgs a{};
    a.out = static_cast<const uint16_t*>(out);
    a.send = static_cast<uint16_t*>(send);
    a.flags = flags;
    a.stamps = reinterpret_cast<unsigned long long*>(stamps);
    a.epoch = epoch;
    a.B = c.B; a.S = c.S; a.d = c.d; a.n = n_chunks;
    a.wgs_per_chunk = std::max(1, 32 / n_chunks);  // at most 32 workgroups (n <= 32): one per CU of a small mask
    a.timeout_ticks = kPackTimeoutTicks;
    hipLaunchKernelGGL(pack_chunks_kernel, dim3(unsigned(n_chunks * a.wgs_per_chunk)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), a);
    return launch_status("pblock_pack_chunks launch");
  } catch (...) {
    return fail(PBLOCK_ERR_ARG, "internal error");
  }
}

int pblock_forward_serial(pblock_t h, const void* x, const pblock_weights* w, const void* ln2_gamma,
                          const void* ln2_beta, const pblock_cfg* cfg, void* out, void* stream) {
  try {
    Dims dm;
    int st = check_forward(h, x, w, cfg, out, &dm);
    if (st != PBLOCK_OK) return st;
    const pblock_cfg& c = *cfg;
    if (!ln2_gamma || !ln2_beta) return fail(PBLOCK_ERR_NULL, "ln2_gamma or ln2_beta is NULL");
    if (!aligned16(ln2_gamma) || !aligned16(ln2_beta)) return fail(PBLOCK_ERR_ALIGN, "LN2 parameters must be 16-byte aligned");
    const int es = elem_size(c.dtype);
    const int64_t xb = dm.M * c.d * es;
    if (overlap(out, xb, ln2_gamma, c.d * es) || overlap(out, xb, ln2_beta, c.d * es))
      return fail(PBLOCK_ERR_ALIAS, "out overlaps an LN2 parameter");
    if (!c.add_residual) return fail(PBLOCK_ERR_ARG, "the serial form needs add_residual = 1 (its residual stream)");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Ws ws = workspace(h);
    Timer tm;
    st = tm.begin(h, s);
    if (st != PBLOCK_OK) return st;
    const int64_t A = dm.A;
    const char* w_in = static_cast<const char*>(w->w_in);
    const char* w_out = static_cast<const char*>(w->w_out);
    char* ag = static_cast<char*>(ws.ag);

    // attention sub-layer: h = x + Attn(LN1(x)), h kept in out
    run_layernorm(x, w->ln_gamma, w->ln_beta, ws.u, dm.M, c, s);
    tm.mark(0);
    run_gemm_in(ws.u, c.d, w_in, c.d, dm.M, 3 * A, c.d, ws.qkv, 3 * A, nullptr, 0, 0, 3 * A, c.dtype, ws.scr, s);
    tm.mark(1);
    launch_attention(ws.qkv, 3 * A, ws.ag, dm.k_out, c.B, c.S, c.H, c.hd, c.W, c.dtype, s);
    tm.mark(2);
    run_gemm_out(ws.ag, dm.k_out, w_out, dm.k_out, dm.M, c.d, A, out, x, c.dtype, ws.scr, s);
    tm.mark(3);
    // feed-forward sub-layer on h: y = h + W2 GeLU(W1 LN2(h)), the residual read from out in place
    run_layernorm(out, ln2_gamma, ln2_beta, ws.u, dm.M, c, s);
    tm.mark(0);
    run_gemm_in(ws.u, c.d, w_in + 3 * A * c.d * es, c.d, dm.M, c.ffn, c.d, nullptr, 0, ws.ag, dm.k_out, A, 0, c.dtype,
                ws.scr, s);
    tm.mark(1);
    run_gemm_out(ag + A * es, dm.k_out, w_out + A * es, dm.k_out, dm.M, c.d, c.ffn, out, out, c.dtype, ws.scr, s);
    tm.mark(3);
    h->last_m = dm.M;
    return launch_status("pblock_forward_serial launch");
  } catch (...) {
    return fail(PBLOCK_ERR_ARG, "internal error");
  }
}

int pblock_forward_chunked(pblock_t h, const void* x, const pblock_weights* w, const pblock_cfg* cfg, void* out,
                           int32_t n_chunks, void* const* ready_events, void* const* done_events, void* stream) {
  try {
    Dims dm;
    int st = check_forward(h, x, w, cfg, out, &dm);
    if (st != PBLOCK_OK) return st;
    const pblock_cfg& c = *cfg;
    if (n_chunks < 1 || n_chunks > c.S) return fail(PBLOCK_ERR_ARG, "n_chunks must be in [1, S]");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Ws ws = workspace(h);
    const int64_t A = dm.A;
    const int es = elem_size(c.dtype);
    const char* xb = static_cast<const char*>(x);
    char* ob = static_cast<char*>(out);
    char* ub = static_cast<char*>(ws.u);
    char* qb = static_cast<char*>(ws.qkv);
    char* ab = static_cast<char*>(ws.ag);
    if (!ready_events) {
      // the input is whole: LayerNorm, the input GEMM and attention run once over every row, and
      // only the output GEMM goes chunk by chunk (the reduce-scatter side of the overlap)
      run_layernorm(x, w->ln_gamma, w->ln_beta, ws.u, dm.M, c, s);
      run_gemm_in(ws.u, c.d, w->w_in, c.d, dm.M, dm.n_in, c.d, ws.qkv, 3 * A, ws.ag, dm.k_out, A, 3 * A, c.dtype,
                  ws.scr, s);
      launch_attention(ws.qkv, 3 * A, ws.ag, dm.k_out, c.B, c.S, c.H, c.hd, c.W, c.dtype, s);
    }
    for (int ck = 0; ck < n_chunks; ++ck) {
      const int p0 = int(int64_t(ck) * c.S / n_chunks), p1 = int(int64_t(ck + 1) * c.S / n_chunks);
      const int64_t rows = p1 - p0;
      if (ready_events) {
        if (ready_events[ck]) {
          hipError_t e = hipStreamWaitEvent(s, static_cast<hipEvent_t>(ready_events[ck]), 0);
          if (e != hipSuccess) return fail(PBLOCK_ERR_HIP, std::string("hipStreamWaitEvent: ") + hipGetErrorString(e));
        }
        for (int b = 0; b < c.B; ++b) {
          const int64_t r0 = int64_t(b) * c.S + p0;
          run_layernorm(xb + r0 * c.d * es, w->ln_gamma, w->ln_beta, ub + r0 * c.d * es, rows, c, s);
        }
        for (int b = 0; b < c.B; ++b) {
          const int64_t r0 = int64_t(b) * c.S + p0;
          run_gemm_in(ub + r0 * c.d * es, c.d, w->w_in, c.d, rows, dm.n_in, c.d, qb + r0 * 3 * A * es, 3 * A,
                      ab + r0 * dm.k_out * es, dm.k_out, A, 3 * A, c.dtype, ws.scr, s);
        }
        // queries of this chunk; their keys reach back into earlier chunks, already projected
        launch_attention(ws.qkv, 3 * A, ws.ag, dm.k_out, c.B, c.S, c.H, c.hd, c.W, c.dtype, s, p0, p1);
      }
      for (int b = 0; b < c.B; ++b) {
        const int64_t r0 = int64_t(b) * c.S + p0;
        run_gemm_out(ab + r0 * dm.k_out * es, dm.k_out, w->w_out, dm.k_out, rows, c.d, dm.k_out, ob + r0 * c.d * es,
                     c.add_residual ? xb + r0 * c.d * es : nullptr, c.dtype, ws.scr, s);
      }
      if (done_events && done_events[ck]) {
        hipError_t e = hipEventRecord(static_cast<hipEvent_t>(done_events[ck]), s);
        if (e != hipSuccess) return fail(PBLOCK_ERR_HIP, std::string("hipEventRecord: ") + hipGetErrorString(e));
      }
    }
    h->last_m = dm.M;
    return launch_status("pblock_forward_chunked launch");
  } catch (...) {
    return fail(PBLOCK_ERR_ARG, "internal error");
  }
}

int pblock_forward_variant(pblock_t h, const void* x, const pblock_weights* w, const pblock_variant_weights* vw,
                           const pblock_cfg* cfg, const pblock_variant* var, void* out, void* stream) {
  try {
    Dims dm;
    int st = check_forward(h, x, w, cfg, out, &dm);
    if (st != PBLOCK_OK) return st;
    const pblock_cfg& c = *cfg;
    if (!var) return fail(PBLOCK_ERR_NULL, "variant is NULL");
    const pblock_variant& v = *var;
    if ((v.gelu_tanh != 0 && v.gelu_tanh != 1) || (v.rope != 0 && v.rope != 1) || (v.two_ln != 0 && v.two_ln != 1))
      return fail(PBLOCK_ERR_ARG, "gelu_tanh, rope and two_ln must be 0 or 1");
    if (v.rope && !(std::isfinite(v.rope_base) && v.rope_base > 0.f))
      return fail(PBLOCK_ERR_ARG, "rope_base must be finite and > 0");
    const pblock_variant_weights none{};
    const pblock_variant_weights& e = vw ? *vw : none;
    if (v.two_ln && (!e.ln2_gamma || !e.ln2_beta)) return fail(PBLOCK_ERR_NULL, "two_ln needs ln2_gamma and ln2_beta");
    const int es = elem_size(c.dtype);
    const int64_t xb = dm.M * c.d * es;
    const void* ln2g = v.two_ln ? e.ln2_gamma : nullptr;
    const void* ln2b = v.two_ln ? e.ln2_beta : nullptr;
    const struct { const void* p; int64_t bytes; } extra[4] = {
        {e.b_in, dm.n_in * es}, {e.b_out, int64_t(c.d) * es}, {ln2g, int64_t(c.d) * es}, {ln2b, int64_t(c.d) * es}};
    for (const auto& t : extra) {
      if (!t.p) continue;
      if (!aligned16(t.p)) return fail(PBLOCK_ERR_ALIGN, "bias and LN2 pointers must be 16-byte aligned");
      if (overlap(out, xb, t.p, t.bytes)) return fail(PBLOCK_ERR_ALIAS, "out overlaps a bias or an LN2 parameter");
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Ws ws = workspace(h);
    const int64_t A = dm.A;
    if (v.rope && (!(double(v.rope_base) == h->rope_base) || s != h->rope_stream)) {
      // (cos, sin) for every position the handle can see; rebuilt when the base changes, and
      // on the calling stream whenever it is not the stream the table was built on, so that
      // every call reads a table its own stream ordered before it
      const int64_t n = h->m_cap * (c.hd / 2);
      hipLaunchKernelGGL(rope_table_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, ws.rope, int(h->m_cap),
                         c.hd, double(v.rope_base));
      st = launch_status("rope table launch");
      if (st != PBLOCK_OK) return st;
      h->rope_base = double(v.rope_base);
      h->rope_stream = s;
    }
    Timer tm;
    st = tm.begin(h, s);
    if (st != PBLOCK_OK) return st;
    InEpi ep;
    ep.bias = e.b_in;
    ep.rope = v.rope ? ws.rope : nullptr;
    ep.rope_n = v.rope ? int(2 * A) : 0;
    ep.seq = c.S;
    ep.hd = c.hd;
    ep.gelu_tanh = v.gelu_tanh;
    run_layernorm(x, w->ln_gamma, w->ln_beta, ws.u, dm.M, c, s);
    tm.mark(0);
    if (!v.two_ln) {
      run_gemm_in(ws.u, c.d, w->w_in, c.d, dm.M, dm.n_in, c.d, ws.qkv, 3 * A, ws.ag, dm.k_out, A, 3 * A, c.dtype,
                  ws.scr, s, ep);
      tm.mark(1);
    } else {
      // the MLP branch has its own LayerNorm: q|k|v from LN(x), then FC1 from LN2(x) in the same u buffer
      run_gemm_in(ws.u, c.d, w->w_in, c.d, dm.M, 3 * A, c.d, ws.qkv, 3 * A, nullptr, 0, 0, 3 * A, c.dtype, ws.scr, s,
                  ep);
      tm.mark(1);
      run_layernorm(x, ln2g, ln2b, ws.u, dm.M, c, s);
      tm.mark(0);
      InEpi ep2 = ep;
      ep2.bias = e.b_in ? static_cast<const char*>(e.b_in) + 3 * A * es : nullptr;
      ep2.rope = nullptr;
      ep2.rope_n = 0;
      run_gemm_in(ws.u, c.d, static_cast<const char*>(w->w_in) + 3 * A * c.d * es, c.d, dm.M, c.ffn, c.d, nullptr, 0,
                  ws.ag, dm.k_out, A, 0, c.dtype, ws.scr, s, ep2);
      tm.mark(1);
    }
    launch_attention(ws.qkv, 3 * A, ws.ag, dm.k_out, c.B, c.S, c.H, c.hd, c.W, c.dtype, s);
    tm.mark(2);
    run_gemm_out(ws.ag, dm.k_out, w->w_out, dm.k_out, dm.M, c.d, dm.k_out, out, c.add_residual ? x : nullptr, c.dtype,
                 ws.scr, s, e.b_out);
    tm.mark(3);
    h->last_m = dm.M;
    return launch_status("pblock_forward_variant launch");
  } catch (...) {
    return fail(PBLOCK_ERR_ARG, "internal error");
  }
}

int64_t pblock_train_workspace_bytes(const pblock_cfg* cfg) {
  const int st = validate(cfg);
  if (st != PBLOCK_OK) return st;
  if (cfg->dtype != PBLOCK_BF16) return fail(PBLOCK_ERR_DTYPE, "the training path is bf16 only");
  if (cfg->d > kBwdMaxD) return fail(PBLOCK_ERR_SHAPE, "the backward pass supports d <= 16384");
  return train_layout(cfg).total;
}

int pblock_forward_train(pblock_t h, const void* x, const pblock_weights* w, const pblock_cfg* cfg, void* out,
                         void* ws, int64_t ws_bytes, void* stream) {
  try {
    Dims dm;
    TrainLayout T;
    int st = check_train(h, x, w, cfg, ws, ws_bytes, &dm, &T);
    if (st != PBLOCK_OK) return st;
    st = check_forward(h, x, w, cfg, out, &dm);
    if (st != PBLOCK_OK) return st;
    const pblock_cfg& c = *cfg;
    if (overlap(out, dm.M * c.d * 2, ws, T.total)) return fail(PBLOCK_ERR_ALIAS, "out overlaps the training workspace");
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* base = static_cast<char*>(ws);
    const Ws hw = workspace(h);
    const int64_t A = dm.A;
    Timer tm;
    st = tm.begin(h, s);
    if (st != PBLOCK_OK) return st;
    run_layernorm(x, w->ln_gamma, w->ln_beta, base + T.u, dm.M, c, s, reinterpret_cast<float*>(base + T.stats));
    tm.mark(0);
    InEpi ep;
    ep.pre = base + T.f;
    ep.ld_pre = c.ffn;
    // as in the plain forward, a split-K reduce of FC1-only tail tiles (which also stores their
    // pre-activation) runs inside the attention launch
    TailPending tail;
    run_gemm_in(base + T.u, c.d, w->w_in, c.d, dm.M, dm.n_in, c.d, base + T.qkv, 3 * A, base + T.ag, dm.k_out, A, 3 * A,
                c.dtype, hw.scr, s, ep, &tail);
    tm.mark(1);
    launch_attention(base + T.qkv, 3 * A, base + T.ag, dm.k_out, c.B, c.S, c.H, c.hd, c.W, c.dtype, s, 0, -1,
                     reinterpret_cast<float*>(base + T.lse), &tail);
    tm.mark(2);
    run_gemm_out(base + T.ag, dm.k_out, w->w_out, dm.k_out, dm.M, c.d, dm.k_out, out, c.add_residual ? x : nullptr,
                 c.dtype, hw.scr, s);
    tm.mark(3);
    h->last_m = dm.M;
    return launch_status("pblock_forward_train launch");
  } catch (...) {
    return fail(PBLOCK_ERR_ARG, "internal error");
  }
}

int pblock_backward(pblock_t h, const void* x, const pblock_weights* w, const pblock_cfg* cfg, const void* dy,
                    const pblock_grads* grads, void* ws, int64_t ws_bytes, void* stream) {
  try {
    Dims dm;
    TrainLayout T;
    int st = check_train(h, x, w, cfg, ws, ws_bytes, &dm, &T);
    if (st != PBLOCK_OK) return st;
    const pblock_cfg& c = *cfg;
    if (!dy || !grads || !grads->dx || !grads->dln_gamma || !grads->dln_beta || !grads->dw_in || !grads->dw_out)
      return fail(PBLOCK_ERR_NULL, "dy, grads or a gradient pointer is NULL");
    const int64_t es = 2, A = dm.A, M = dm.M, d = c.d;
    const struct { const void* p; int64_t bytes; } outs[5] = {
        {grads->dx, M * d * es}, {grads->dln_gamma, d * es}, {grads->dln_beta, d * es},
        {grads->dw_in, dm.n_in * d * es}, {grads->dw_out, d * dm.k_out * es}};
    const struct { const void* p; int64_t bytes; } ins[7] = {
        {x, M * d * es}, {dy, M * d * es}, {w->w_in, dm.n_in * d * es}, {w->w_out, d * dm.k_out * es},
        {w->ln_gamma, d * es}, {w->ln_beta, d * es}, {ws, T.total}};
    if (!aligned16(dy)) return fail(PBLOCK_ERR_ALIGN, "dy must be 16-byte aligned");
    // dy may be read in place while the backward writes its scratch into ws
    if (overlap(dy, M * d * es, ws, T.total)) return fail(PBLOCK_ERR_ALIAS, "dy overlaps the training workspace");
    for (int i = 0; i < 5; ++i) {
      if (!aligned16(outs[i].p)) return fail(PBLOCK_ERR_ALIGN, "gradient pointers must be 16-byte aligned");
      for (const auto& in : ins)
        if (overlap(outs[i].p, outs[i].bytes, in.p, in.bytes))
          return fail(PBLOCK_ERR_ALIAS, "a gradient overlaps an input, a weight or the workspace");
      for (int j = 0; j < i; ++j)
        if (overlap(outs[i].p, outs[i].bytes, outs[j].p, outs[j].bytes))
          return fail(PBLOCK_ERR_ALIAS, "gradients overlap each other");
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* base = static_cast<char*>(ws);
    const Ws hw = workspace(h);
    Timer tm;
    st = tm.begin(h, s);
    if (st != PBLOCK_OK) return st;

    // dy as the GEMMs' row operand: read in place when B*S fills whole 256-row tiles (no row
    // past M is read then), else copied into whole tiles with its token padding zeroed
    const void* dy_rows = dy;
    if (M % kGemmBM != 0) {
      hipError_t e = hipMemcpyAsync(base + T.dyp, dy, size_t(M * d * es), hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return fail(PBLOCK_ERR_HIP, std::string("hipMemcpyAsync: ") + hipGetErrorString(e));
      launch_zero_rows(base + T.dyp, d, M, T.Mp, s);
      dy_rows = base + T.dyp;
    }
    launch_zero_rows(base + T.ag, dm.k_out, M, T.Mp, s);
    launch_zero_rows(base + T.u, d, M, T.Mp, s);
    launch_zero_rows(base + T.dz, dm.n_in, M, T.Mp, s);
    tm.mark(4);
    // [dO | dG] = dy W_out (W_out read K-major in place); dF = dG * GeLU'(F) straight into dz's
    // FC1 columns
    {
      GemmArgs g{};
      g.a = static_cast<const uint16_t*>(dy_rows); g.lda = d;
      g.b = static_cast<const uint16_t*>(w->w_out); g.ldb = dm.k_out;
      g.M = int(M); g.N = int(dm.k_out); g.K = int(d);
      g.out0 = reinterpret_cast<uint16_t*>(base + T.dO); g.ld0 = A;
      g.out1 = reinterpret_cast<uint16_t*>(base + T.dz); g.ld1 = dm.n_in; g.off1 = 3 * A;
      g.nsplit = int(A);
      g.pre = reinterpret_cast<uint16_t*>(base + T.f); g.ld_pre = c.ffn;
      launch_gemm_kmajor<kEpiGeluBwd, false>(g, hw.scr.partials, hw.scr.G, s);
    }
    tm.mark(5);
    // attention backward: dQ (and D), then dK, dV, into dz's Q|K|V columns
    {
      AttnBwdArgs ab{};
      ab.qkv = reinterpret_cast<const uint16_t*>(base + T.qkv); ab.ld_qkv = 3 * A;
      ab.o = reinterpret_cast<const uint16_t*>(base + T.ag); ab.ld_o = dm.k_out;
      ab.dout = reinterpret_cast<const uint16_t*>(base + T.dO); ab.ld_do = A;
      ab.lse = reinterpret_cast<const float*>(base + T.lse);
      ab.delta = reinterpret_cast<float*>(base + T.delta);
      ab.dqkv = reinterpret_cast<uint16_t*>(base + T.dz); ab.ld_dqkv = dm.n_in;
      ab.B = c.B; ab.S = c.S; ab.H = c.H;
      ab.W = std::min(c.W, c.S);  // W >= S is full causal; the dK/dV band sums stay in int range
      ab.scale = 1.0f / std::sqrt(float(c.hd));
      ab.scale_log2 = ab.scale * 1.4426950408889634f;
      const unsigned gq = unsigned(int64_t((c.S + kAttnBQ - 1) / kAttnBQ) * c.B * c.H);
      const unsigned gk = unsigned(int64_t((c.S + 127) / 128) * c.B * c.H);
      if (c.hd == 128) {
        hipLaunchKernelGGL((swa_attn_bwd_dq_kernel<128>), dim3(gq), dim3(kAttnThreads), 0, s, ab);
        hipLaunchKernelGGL((swa_attn_bwd_dkdv_kernel<128>), dim3(gk), dim3(kAttnThreads), 0, s, ab);
      } else {
        hipLaunchKernelGGL((swa_attn_bwd_dq_kernel<64>), dim3(gq), dim3(kAttnThreads), 0, s, ab);
        hipLaunchKernelGGL((swa_attn_bwd_dkdv_kernel<64>), dim3(gk), dim3(kAttnThreads), 0, s, ab);
      }
    }
    tm.mark(6);
    // du = dz W_in (W_in read K-major in place; fp32 out)
    {
      GemmArgs g{};
      g.a = reinterpret_cast<const uint16_t*>(base + T.dz); g.lda = dm.n_in;
      g.b = static_cast<const uint16_t*>(w->w_in); g.ldb = d;
      g.M = int(M); g.N = int(d); g.K = int(dm.n_in);
      g.ld0 = d;
      g.out_f32 = reinterpret_cast<float*>(base + T.du);
      launch_gemm_kmajor<kEpiF32, false>(g, hw.scr.partials, hw.scr.G, s);
    }
    tm.mark(5);
    // LayerNorm backward (+ dy for the residual), dgamma and dbeta
    {
      const int need = int((d / 8 + 255) / 256);
      const dim3 grid{unsigned(T.ln_grid)}, block{256};
      const auto* xp = static_cast<const uint16_t*>(x);
      const auto* gp = static_cast<const uint16_t*>(w->ln_gamma);
      const auto* dup = reinterpret_cast<const float*>(base + T.du);
      const auto* stp = reinterpret_cast<const float*>(base + T.stats);
      const auto* dyr = c.add_residual ? static_cast<const uint16_t*>(dy) : nullptr;
      auto* dxp = static_cast<uint16_t*>(grads->dx);
      auto* part = reinterpret_cast<float*>(base + T.part);
      const int rows = int(T.ln_rows);
#define PBLK_LNB(V) hipLaunchKernelGGL((layernorm_bwd_kernel<V>), grid, block, 0, s, xp, gp, dup, dyr, stp, dxp, part, M, int(d), rows)
      if (need <= 1) PBLK_LNB(1);
      else if (need <= 2) PBLK_LNB(2);
      else if (need <= 3) PBLK_LNB(3);
      else if (need <= 4) PBLK_LNB(4);
      else if (need <= 6) PBLK_LNB(6);
      else PBLK_LNB(8);
#undef PBLK_LNB
      hipLaunchKernelGGL(column_sum_kernel, dim3(unsigned(2 * d / 64)), dim3(256), 0, s, part, int(T.ln_grid), 2 * d,
                         static_cast<uint16_t*>(grads->dln_gamma), static_cast<uint16_t*>(grads->dln_beta), d);
    }
    tm.mark(8);
    // dW_out = dy^T [A | G], dW_in = dz^T u: contractions over the Mp tokens, both operands read
    // K-major in place (token rows M .. Mp-1 zeroed above)
    {
      GemmArgs go{}, gi{};
      go.a = static_cast<const uint16_t*>(dy_rows); go.lda = d;
      go.b = reinterpret_cast<const uint16_t*>(base + T.ag); go.ldb = dm.k_out;
      go.M = int(d); go.N = int(dm.k_out); go.K = int(T.Mp);
      go.out0 = static_cast<uint16_t*>(grads->dw_out); go.ld0 = dm.k_out;
      gi.a = reinterpret_cast<const uint16_t*>(base + T.dz); gi.lda = dm.n_in;
      gi.b = reinterpret_cast<const uint16_t*>(base + T.u); gi.ldb = d;
      gi.M = int(dm.n_in); gi.N = int(d); gi.K = int(T.Mp);
      gi.out0 = static_cast<uint16_t*>(grads->dw_in); gi.ld0 = d;
      launch_gemm_kmajor_pair<kEpiResidual, true>(go, gi, hw.scr.partials, hw.scr.G, s);
    }
    tm.mark(7);
    return launch_status("pblock_backward launch");
  } catch (...) {
    return fail(PBLOCK_ERR_ARG, "internal error");
  }
}

int pblock_swa_attention(const void* qkv, int64_t ld_qkv, void* o, int64_t ld_o, int32_t B, int32_t S, int32_t H,
                         int32_t hd, int32_t W, int32_t dtype, void* stream) {
  try {
    if (!qkv || !o) return fail(PBLOCK_ERR_NULL, "qkv or o is NULL");
    if (dtype != PBLOCK_F32 && dtype != PBLOCK_BF16) return fail(PBLOCK_ERR_DTYPE, "dtype must be F32 or BF16");
    if (B < 1 || S < 1 || H < 1 || W < 1 || int64_t(B) * S > (int64_t(1) << 24) || H > 4096)
      return fail(PBLOCK_ERR_SHAPE, "B, S, H, W must be >= 1 (B*S <= 2^24, H <= 4096)");
    if (hd != 64 && hd != 128) return fail(PBLOCK_ERR_SHAPE, "hd must be 64 or 128");
    const int64_t A = int64_t(H) * hd;
    if (ld_qkv < 3 * A || ld_o < A || (ld_qkv % 8) != 0 || (ld_o % 8) != 0)
      return fail(PBLOCK_ERR_SHAPE, "ld_qkv >= 3*H*hd and ld_o >= H*hd, both multiples of 8");
    // the kernels address a 64-row tile with 32-bit byte offsets from its first row
    if (ld_qkv > kMaxAttnLd || ld_o > kMaxAttnLd)
      return fail(PBLOCK_ERR_SHAPE, "ld_qkv and ld_o must be <= 2^24 elements");
    if (!aligned16(qkv) || !aligned16(o)) return fail(PBLOCK_ERR_ALIGN, "qkv and o must be 16-byte aligned");
    const int es = elem_size(dtype);
    const int64_t M = int64_t(B) * S;
    if (overlap(qkv, ((M - 1) * ld_qkv + 3 * A) * es, o, ((M - 1) * ld_o + A) * es))
      return fail(PBLOCK_ERR_ALIAS, "o overlaps qkv");
    int st = check_device(nullptr);
    if (st != PBLOCK_OK) return st;
    launch_attention(qkv, ld_qkv, o, ld_o, B, S, H, hd, W, dtype, static_cast<hipStream_t>(stream));
    return launch_status("pblock_swa_attention launch");
  } catch (...) {
    return fail(PBLOCK_ERR_ARG, "internal error");
  }
}

const char* pblock_strerror(int code) {
  switch (code) {
    case PBLOCK_OK: return "ok";
    case PBLOCK_ERR_NULL: return "a required pointer is NULL";
    case PBLOCK_ERR_SHAPE: return "a dimension is out of the supported range";
    case PBLOCK_ERR_DTYPE: return "unsupported dtype";
    case PBLOCK_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case PBLOCK_ERR_ALIAS: return "output overlaps an input";
    case PBLOCK_ERR_CFG_MISMATCH: return "cfg does not match the handle";
    case PBLOCK_ERR_DEVICE: return "no gfx950 device is current";
    case PBLOCK_ERR_NOMEM: return "out of memory";
    case PBLOCK_ERR_HIP: return "HIP runtime error";
    case PBLOCK_ERR_ARG: return "invalid argument";
    default: return "unknown status";
  }
}

const char* pblock_last_error(void) { return g_last_error.c_str(); }

int pblock_activation(const float* z, float* out, int64_t n, int32_t form, void* stream) {
  try {
    if (!z || !out) return fail(PBLOCK_ERR_NULL, "z or out is NULL");
    if (n < 0 || n > (int64_t(1) << 40)) return fail(PBLOCK_ERR_SHAPE, "n must be in [0, 2^40]");
    if (form != PBLOCK_ACT_GELU_ERF_F32 && form != PBLOCK_ACT_GELU_ERF_BF16 && form != PBLOCK_ACT_GELU_TANH &&
        form != PBLOCK_ACT_GELU_ERF_GRAD)
      return fail(PBLOCK_ERR_ARG, "unknown activation form");
    if (overlap(z, n * 4, out, n * 4) && z != out) return fail(PBLOCK_ERR_ALIAS, "out partly overlaps z");
    int st = check_device(nullptr);
    if (st != PBLOCK_OK) return st;
    if (n == 0) return PBLOCK_OK;
    const unsigned grid = unsigned(std::min<int64_t>((n + 255) / 256, 4096));
    hipLaunchKernelGGL(activation_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), z, out, n,
                       int(form));
    return launch_status("pblock_activation launch");
  } catch (...) {
    return fail(PBLOCK_ERR_ARG, "internal error");
  }
}

int pblock_mfma_loop(int32_t workgroups, int32_t iterations, int32_t form, float* sink, void* stream) {
  try {
    if (!sink) return fail(PBLOCK_ERR_NULL, "sink is NULL");
    if (workgroups < 1 || iterations < 1) return fail(PBLOCK_ERR_ARG, "workgroups and iterations must be >= 1");
    if (form != PBLOCK_MFMA_16X16X32 && form != PBLOCK_MFMA_32X32X16) return fail(PBLOCK_ERR_ARG, "unknown MFMA form");
    int st = check_device(nullptr);
    if (st != PBLOCK_OK) return st;
    hipLaunchKernelGGL(form == PBLOCK_MFMA_16X16X32 ? mfma_loop16_kernel : mfma_loop32_kernel, dim3(unsigned(workgroups)),
                       dim3(256), 0, static_cast<hipStream_t>(stream), int(iterations), sink);
    return launch_status("pblock_mfma_loop launch");
  } catch (...) {
    return fail(PBLOCK_ERR_ARG, "internal error");
  }
}

}  // extern "C"
