// Embedding row gather of the vocab-parallel embedding: the first op of
// forward_batch.
//
// "Mini-SGLang 完整剖析" sections 4.9.2-4.9.3 (VocabParallelEmbedding calls
// indexing(weights, ids, vocab_range); the index kernel copies one weight row
// per token). A shard holds the rows of ids in [vocab_start, vocab_end) (row
// id - vocab_start of its weight); any other id gives an all-zero row, so the
// shards' outputs add up to the whole table's gather. Like store_kv, a row is
// cut into 16-byte packets spread over the grid; table rows use ordinary
// loads, since the same id recurs across tokens and steps.
#pragma once

#include "common.hpp"

namespace pkv {

template <int PK>
__global__ void __launch_bounds__(256) embed_gather_kernel(
    const u32x4* __restrict__ w, int64_t w_row_pk, const int32_t* __restrict__ ids, int64_t n,
    int64_t vocab_start, int64_t vocab_end, u32x4* __restrict__ out, int64_t out_row_pk,
    int32_t packets_per_row) {
  const int32_t groups_per_row = packets_per_row / PK;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / groups_per_row;
  if (row >= n) return;
  const int32_t p0 = (int32_t)(gid - row * groups_per_row) * PK;
  const int64_t id = (int64_t)ids[row];
  u32x4 x[PK];
  if (id >= vocab_start && id < vocab_end) {
#pragma unroll
    for (int i = 0; i < PK; ++i) x[i] = w[(id - vocab_start) * w_row_pk + p0 + i];
  } else {
#pragma unroll
    for (int i = 0; i < PK; ++i) x[i] = u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < PK; ++i) out[row * out_row_pk + p0 + i] = x[i];
}

}  // namespace pkv
