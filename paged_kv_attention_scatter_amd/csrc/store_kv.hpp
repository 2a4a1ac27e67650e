// store_kv: scatter this step's K/V rows into the paged pool.
//
// "Mini-SGLang 完整剖析", sections 4.4.3 and 4.9.4-4.9.5: row i of k (and v)
// is copied to pool slot out_loc[i]; rows are kv_heads * head_dim elements.
// The reference moves a row with one 32-lane warp in 16-byte packets. Here a
// row is split into 16-byte packets spread over all lanes of the grid, so one
// wave64 instruction moves 1 KiB, and K and V of the same row are handled by
// the same thread to share the slot lookup.
#pragma once

#include "common.hpp"

namespace pkv {

// Every thread copies PK consecutive 16-byte packets of one row of K and the
// same packets of V. `packets_per_row` = row bytes / 16.
template <typename IdxT, int PK>
__global__ void __launch_bounds__(256) store_kv_kernel(
    u32x4* __restrict__ k_pool, u32x4* __restrict__ v_pool, int64_t pool_row_pk,
    int64_t num_slots, const IdxT* __restrict__ out_loc, int64_t n,
    const u32x4* __restrict__ k, int64_t k_row_pk, const u32x4* __restrict__ v,
    int64_t v_row_pk, int32_t packets_per_row, uint32_t* faults) {
  const int32_t groups_per_row = packets_per_row / PK;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / groups_per_row;
  if (row >= n) return;
  const int32_t p0 = (int32_t)(gid - row * groups_per_row) * PK;
  const int64_t slot = (int64_t)out_loc[row];
  if (slot < 0 || slot >= num_slots) {
    if (p0 == 0) raise_fault(faults, 0x1u);
    return;
  }
  u32x4 kb[PK], vb[PK];
#pragma unroll
  for (int i = 0; i < PK; ++i) {
    kb[i] = __builtin_nontemporal_load(k + row * k_row_pk + p0 + i);
    vb[i] = __builtin_nontemporal_load(v + row * v_row_pk + p0 + i);
  }
#pragma unroll
  for (int i = 0; i < PK; ++i) {
    k_pool[slot * pool_row_pk + p0 + i] = kb[i];
    v_pool[slot * pool_row_pk + p0 + i] = vb[i];
  }
}

}  // namespace pkv
