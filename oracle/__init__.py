"""Plain fp64 CPU oracle for the attention forward path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or link
anything in this package: only the tests, the smoke check and the CPU-baseline
leg of the benchmark use it. It shares no code with the HIP library and never
imports its binding.

Every function is a direct, slow statement of what the pages define, written
with numpy in float64 (inputs of any float dtype, including bf16 torch tensors,
are upcast exactly). The one library primitive used for the attention itself is
a matrix product; there is no online softmax, no blocking and no reordering.

Sources (three web pages, each a Python source file):

* [FA]  vLLM-Omni diffusion attention backend ``flash_attn.py``
        (FlashAttentionImpl: the varlen/dense/packed forwards, the NPU causal
        branch, the prefix-KV slicing and laser pre-scale notes).
* [ASC] vLLM-Ascend ``attention_v1.py`` (cache shape and block size,
        AscendMetadata block tables / slot mapping, paged attention).
* [VSA] vLLM-Omni diffusion attention backend ``fastvideo_vsa.py``
        (tile geometry, pooled scores, top-k block map, block-sparse call).

Pin status of each function is listed in its docstring; every function here is
pinned by tests in ``tests/test_oracle_*.py`` against closed forms, invariants,
brute force on tiny inputs, a library SDPA in float64, or the pages' worked
example.
"""

from .attention import (  # noqa: F401
    NEG_INF,
    varlen_attention,
    dense_attention,
    paged_decode_attention,
    paged_kv_write,
    paged_prefill_attention,
    block_sparse_attention,
    merge_partials,
    slot_to_block_offset,
)
from .tiles import (  # noqa: F401
    tile_partition_indices,
    variable_block_sizes,
    non_pad_index,
    tile_metadata,
    to_tile_order,
    from_tile_order,
    h3_tile_metadata,
    h3_to_tile_order,
    h3_from_tile_order,
)
from .blockmap import (  # noqa: F401
    pool_tiles,
    pooled_scores,
    topk_block_map,
    h3_block_map,
    map_to_index,
    compressed_branch,
)
from .variants import (  # noqa: F401
    sliding_window_decode_attention,
    padded_prefix_attention,
    masked_attention,
)
