// Host check of the paged-cache addressing that the paged decode and prefill
// kernels use (long_context_anchor_amd/csrc/paged.h), built with a host C++
// compiler: for random caches that pass the library's documented paged-cache
// constraints, every row address a kernel can form -- from listed positions
// (in range, negative, past the context), from the padding entries of a
// staged list (row 0), for every KV head, with random block tables holding
// out-of-range block numbers and a ragged last block -- stays inside the
// cache, and in-range positions land on the row the block table names.
// Prints "ok <cases>" and exits 0, or prints the failing case and exits 1.
#define __host__
#define __device__
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../long_context_anchor_amd/csrc/paged.h"

int main() {
  std::mt19937_64 rng(20251203);
  auto uni = [&](int64_t lo, int64_t hi) {   // inclusive
    return lo + (int64_t)(rng() % (uint64_t)(hi - lo + 1));
  };
  long cases = 0;
  for (int iter = 0; iter < 4000; ++iter) {
    const int d = 128, es = 2;                       // bf16 / fp16 rows of 256 bytes
    const int Hkv = (int)uni(1, 8);
    const int shift = (int)uni(0, 8);                // block sizes 1 .. 256
    const int bs = 1 << shift;
    const bool heads_outer = (iter & 1) == 0;        // [nb, Hkv, bs, d] or [nb, bs, Hkv, d]
    const int64_t pad = 8 * uni(0, 2);               // padded rows, 16-byte multiples
    int64_t kv_sn, kv_sh, block_stride;
    if (heads_outer) {
      kv_sn = d + pad;
      kv_sh = bs * kv_sn;
      block_stride = Hkv * kv_sh;
    } else {
      kv_sh = d + pad;
      kv_sn = Hkv * kv_sh;
      block_stride = bs * kv_sn;
    }
    block_stride += kv_sn * uni(0, 2);               // spare rows at the end of a block
    // the library's constraint: every head's bs rows inside the block
    if ((int64_t)(Hkv - 1) * kv_sh + (int64_t)(bs - 1) * kv_sn + d > block_stride) {
      std::printf("generator broke the constraint\n");
      return 1;
    }
    const int B = (int)uni(1, 3);
    const int n_ctx = (int)uni(1, 3000);             // ragged last block in general
    const int nblk_b = (n_ctx + bs - 1) / bs;
    const int num_blocks = (int)uni(1, B * nblk_b + 3);
    const int64_t table_stride = nblk_b + uni(0, 2);
    std::vector<int32_t> table(B * table_stride);
    for (auto& t : table) {
      const int64_t r = uni(0, 9);
      t = r == 0 ? -(int32_t)uni(1, 100) : r == 1 ? num_blocks + (int32_t)uni(0, 100)
                                                  : (int32_t)uni(0, num_blocks - 1);
    }
    const uint32_t blk_rows = (uint32_t)(block_stride / kv_sn);
    const uint32_t max_row = kc::paged_max_row(num_blocks, blk_rows, shift);
    const int64_t cache_bytes = (int64_t)num_blocks * block_stride * es;
    const int64_t row_bytes = kv_sn * es;
    for (int c = 0; c < 64; ++c) {
      const int b = (int)uni(0, B - 1);
      const int64_t r = uni(0, 5);
      const int j = r == 0 ? -(int)uni(1, 1000) : r == 1 ? n_ctx + (int)uni(0, 1000)
                                                       : (int)uni(0, n_ctx - 1);
      // a staged list entry, one of the padding entries after it (row 0), or
      // an arbitrary 32-bit value (what an unwritten LDS entry could hold):
      // the kernel's clamp to max_row must keep even that inside every head
      const int64_t kind = uni(0, 7);
      const bool padding = kind == 0, garbage = kind == 1;
      uint32_t row = padding ? 0u
                     : garbage ? (uint32_t)rng()
                               : kc::paged_row(table.data(), table_stride, b, j, n_ctx, shift, num_blocks,
                                               blk_rows);
      if (!garbage && row > max_row) {
        std::printf("row %u above max_row %u (iter %d)\n", row, max_row, iter);
        return 1;
      }
      if (!padding && !garbage && j >= 0 && j < n_ctx) {
        const int32_t t = table[b * table_stride + (j >> shift)];
        if (t >= 0 && t < num_blocks && row != (uint32_t)t * blk_rows + (uint32_t)(j & (bs - 1))) {
          std::printf("row %u is not the table's (iter %d)\n", row, iter);
          return 1;
        }
      }
      // the decode kernel clamps staged rows to max_row before forming offsets
      row = row < max_row ? row : max_row;
      for (int g = 0; g < Hkv; ++g) {
        const int64_t first = (int64_t)g * kv_sh * es + (int64_t)row * row_bytes;
        const int64_t last = first + 15 * 16 + 16;   // 16 lanes of 16 bytes
        if (first < 0 || last > cache_bytes) {
          std::printf("head %d row %u bytes [%lld, %lld) outside the cache of %lld (iter %d)\n", g, row,
                      (long long)first, (long long)last, (long long)cache_bytes, iter);
          return 1;
        }
        ++cases;
      }
    }
  }
  std::printf("ok %ld\n", cases);
  return 0;
}
