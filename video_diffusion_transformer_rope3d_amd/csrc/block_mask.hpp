// Key-tile lists from a block bit mask: for each (b, head, 256-query block),
// the ascending indices of the 64-key blocks whose bit is set. The lists feed
// the block-sparse attention kernel unchanged.
#pragma once

#include "common.hpp"

namespace vidattn {

// One thread per list row r (r < rows): mask words mask[r * words ..] (bit
// j % 32 of word j / 32 is key block j; bits at or past nkb are ignored)
// -> kv_blocks[r * nkb ..] (ascending, at most nkb entries) and kv_count[r].
__global__ __launch_bounds__(256) void block_mask_lists_kernel(const uint32_t* __restrict__ mask,
                                                               int32_t* __restrict__ kv_blocks,
                                                               int32_t* __restrict__ kv_count, int64_t rows,
                                                               int words, int nkb) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const uint32_t* m = mask + r * words;
  int32_t* out = kv_blocks + r * nkb;
  int n = 0;
  for (int w = 0; w < words; ++w) {
    uint32_t bits = m[w];
    const int left = nkb - 32 * w;  // key blocks this word covers: min(32, left)
    if (left < 32) bits &= (1u << left) - 1u;
    while (bits) {
      out[n++] = 32 * w + __builtin_ctz(bits);
      bits &= bits - 1u;
    }
  }
  kv_count[r] = n;
}

}  // namespace vidattn
