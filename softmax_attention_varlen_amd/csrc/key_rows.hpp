// Where the key rows of one document live, for the prefill kernels.
#pragma once
#include "attn_common.hpp"

namespace attn {

// Element offset of key row `key` (this kv head's row starts at +hk*D, added by
// the caller): contiguous keys of one document (rows `stride` elements apart),
// or a paged cache whose 128-token blocks the sequence's table row names (a
// 64-key tile aligned to 64 never crosses a block).
template <bool PAGED>
struct KeyRows {
  long stride;           // elements between consecutive keys (Hkv * D)
  const int32_t* table;  // paged: this sequence's block-table row
  int num_blocks;
  __device__ __forceinline__ long row(int key) const {
    if (!PAGED) return (long)key * stride;
    const int blk = clampi(table[key >> 7], 0, num_blocks - 1);
    return ((long)blk * 128 + (key & 127)) * stride;
  }
};

}  // namespace attn
