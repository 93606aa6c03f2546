// Consumer side of the row-chunk publication (the local half of a reduce-scatter): copies each
// chunk of the block's output into its piece of a send buffer as soon as the output GEMM has
// published it.
//
// Chunk k holds positions [floor(k S / n), floor((k+1) S / n)) of every sequence (MegaScale
// guided reading, section 3: with sequence parallelism each of the n ranks keeps one slice of
// the sequence after the reduce-scatter, and the GEMM next to the collective is cut into chunks
// so that one chunk's communication overlaps the next chunk's computation).  Piece k of the
// send buffer is chunk k's rows, sequence by sequence, pieces in chunk order: the piece rank k
// receives.
#pragma once

#include "common.hpp"

namespace pblk {

struct PackArgs {
  const uint16_t* out;        // bf16 [B*S, d]
  uint16_t* send;             // bf16, B*S*d elements: n pieces
  const uint32_t* flags;      // [n]: chunk k is published when flags[k] == epoch
  unsigned long long* stamps;  // [n]: device real-time clock when the flag was seen, or ~0 on timeout
  uint32_t epoch;
  int B, S, d, n;
  int wgs_per_chunk;
  unsigned long long timeout_ticks;  // bound of each wait, in real-time clock ticks
};

// grid = n * wgs_per_chunk workgroups of 256: workgroup (k, part) waits for chunk k (thread 0
// polls the flag with a bounded wait), then copies its share of the chunk in 16-byte pieces.
__global__ __launch_bounds__(256) void pack_chunks_kernel(PackArgs a) {
  const int k = blockIdx.x / a.wgs_per_chunk, part = blockIdx.x % a.wgs_per_chunk;
  __shared__ int seen;
  if (threadIdx.x == 0) {
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    unsigned long long t = t0;
    int ok = 0;
    for (;;) {
      if (__hip_atomic_load(a.flags + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.epoch) {
        ok = 1;
        t = __builtin_amdgcn_s_memrealtime();
        break;
      }
      if (__builtin_amdgcn_s_memrealtime() - t0 > a.timeout_ticks) break;
      __builtin_amdgcn_s_sleep(8);
    }
    // the producer's release, then this workgroup's reads: drop any stale cached copy of out
    if (ok) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    seen = ok;
    if (part == 0) a.stamps[k] = ok ? t : ~0ull;
  }
  __syncthreads();
  if (!seen) return;
  const int p0 = int(int64_t(k) * a.S / a.n), p1 = int(int64_t(k + 1) * a.S / a.n);
  const int64_t rows = int64_t(p1 - p0);
  const int64_t vec_per_row = a.d / 8;
  const int64_t total = int64_t(a.B) * rows * vec_per_row;
  const u32x4* src = reinterpret_cast<const u32x4*>(a.out);
  u32x4* dst = reinterpret_cast<u32x4*>(a.send) + int64_t(a.B) * p0 * vec_per_row;
  for (int64_t i = int64_t(part) * 256 + threadIdx.x; i < total; i += int64_t(a.wgs_per_chunk) * 256) {
    const int64_t j = i / vec_per_row, c = i % vec_per_row;
    const int64_t b = j / rows, p = p0 + j % rows;
    dst[i] = src[(b * a.S + p) * vec_per_row + c];
  }
}

}  // namespace pblk
