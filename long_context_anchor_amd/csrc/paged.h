// Block-table addressing of paged K/V caches, shared by the paged decode and
// prefill kernels.  Key j of batch b is row j mod 2^blk_shift of physical
// block table[b * table_stride + (j >> blk_shift)]; physical row R of head g
// starts at element g * kv_stride_h + R * kv_stride_n of the cache, with
// R = block * blk_rows + row (blk_rows = block stride / kv_stride_n).
//
// Only stdint is needed, so a host compiler can build this header too
// (with __host__ and __device__ defined empty) to check the arithmetic.
#pragma once
#include <stdint.h>

namespace kc {

// Physical row of logical position j: j is clamped into [0, n_ctx) and the
// block number read from the table into [0, num_blocks), so neither a bad list
// nor a bad table can leave the cache.
__host__ __device__ inline uint32_t paged_row(const int32_t* table, int64_t table_stride, int b, int j,
                                              int n_ctx, int blk_shift, int num_blocks,
                                              uint32_t blk_rows) {
  j = j < 0 ? 0 : (j > n_ctx - 1 ? n_ctx - 1 : j);
  int blk = table[(int64_t)b * table_stride + (j >> blk_shift)];
  blk = blk < 0 ? 0 : (blk > num_blocks - 1 ? num_blocks - 1 : blk);
  return (uint32_t)blk * blk_rows + (uint32_t)(j & ((1 << blk_shift) - 1));
}

// The last physical row a head may read: row 2^blk_shift - 1 of the last
// block.  With the host's check that every head's block rows lie inside the
// block stride, head g's bytes of this row end inside the cache.
__host__ __device__ inline uint32_t paged_max_row(int num_blocks, uint32_t blk_rows, int blk_shift) {
  return (uint32_t)(num_blocks - 1) * blk_rows + (uint32_t)((1 << blk_shift) - 1);
}

}  // namespace kc
