// Attention launched together with the input GEMM's split-K reduce.
//
// When the tail tiles of the input GEMM (the tiles it computes as k-chunks after its whole
// waves) all lie in the FC1 columns, attention does not read what their reduce writes: the
// reduce (summing the chunks' partials, GeLU, store to the FC1 part of AG) and attention
// (reading Q, K, V, writing the attention part of AG) touch disjoint data.  Both then run as
// one launch: workgroups [0, n_attn) are attention's, the rest each reduce rpw row groups of
// 8 tail-tile rows.  Attention alone leaves compute units idle at the 175B shard shape (192
// workgroups of a 128-query tile on 256 units) and is bound by its per-tile chain rather than
// by memory, while the reduce is a pass over the partials: the two overlap instead of running
// back to back.
#pragma once

#include "attn_bf16.hpp"
#include "gemm_bf16.hpp"

namespace pblk {

template <int HD>
__global__ __launch_bounds__(kAttnThreads, 2) void swa_attn_tail_kernel(AttnArgs a, int n_attn, GemmArgs g,
                                                                       GemmSched sk, int rpw, int n_groups) {
  __shared__ __attribute__((aligned(1024))) AttnLds<HD> lds;
  if (blockIdx.x < unsigned(n_attn)) {
    swa_attn_block<HD>(a, blockIdx.x, lds);
    return;
  }
  const int g0 = (int(blockIdx.x) - n_attn) * rpw;
  for (int k = 0; k < rpw && g0 + k < n_groups; ++k) tail_reduce_rows<kEpiSplitGelu>(g, sk, g0 + k);
}

}  // namespace pblk
