// Host-side launch plans shared between the C ABI layer and the kernel files.
// Every struct holds already-validated arguments; the launchers only enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/attn_mi355x.h"

namespace attn {

struct VarlenArgs {
  const void* q;
  const void* k;  // contiguous: [total_k][Hkv][D]; paged: the K plane of the cache
  const void* v;  // contiguous: [total_k][Hkv][D]; paged: the V plane of the cache
  const int32_t* cu_q;
  const int32_t* cu_k;  // contiguous only
  int batch, total_q, total_k, max_seqlen_q, max_seqlen_k;
  int num_heads, num_kv_heads, head_dim;
  float scale;
  int causal;
  void* out;
  float* lse;
  // paged keys (multi-token attention over a paged cache): key t of document b
  // is cache row (block_tables[b][t / 128], t % 128); its length is
  // context_lens[b] clamped to max_seqlen_k
  bool paged = false;
  const int32_t* block_tables = nullptr;
  const int32_t* context_lens = nullptr;
  int max_blocks_per_seq = 0, num_blocks = 0;
  // padded documents (nullable): document b keeps only the first q_used[b]
  // query rows and k_used[b] key rows of its cu_q / cu_k range
  const int32_t* q_used = nullptr;
  const int32_t* k_used = nullptr;
};

hipError_t launch_varlen_fwd(const VarlenArgs& a, hipStream_t stream);

// Padded batch (padding.hip): base carries q, k, v, out, lse, batch, heads,
// head_dim, scale and causal; q_lens / k_lens are the valid prefix lengths
// (q_lens null: every row is padding). Workspace: the two strided cu arrays.
size_t padded_workspace_bytes(int batch);
hipError_t launch_padded_fwd(const VarlenArgs& base, const int32_t* q_lens, const int32_t* k_lens, int seqlen_q,
                             int seqlen_k, void* workspace, hipStream_t stream);

// Key-padding mask (padding.hip): byte offsets of the workspace pieces.
struct MaskedLayout {
  size_t cu_q, cu_k, count, idx, inv, k, v;  // always
  size_t q, o, lse;                          // mask over the queries too
  size_t bytes;
};
MaskedLayout plan_masked(int batch, int seqlen_q, int seqlen_k, int num_heads, int num_kv_heads, int head_dim,
                         bool mask_queries);
hipError_t launch_masked_fwd(const VarlenArgs& base, const uint8_t* key_mask, int seqlen_q, int seqlen_k,
                             bool mask_queries, const MaskedLayout& l, void* workspace, hipStream_t stream);
// head_dims 96 to 256, and 64 without the causal mask: pipelined
// direct-to-LDS prefill (prefill_pipe.hip)
bool prefill_pipe_supported(const VarlenArgs& a);
hipError_t launch_prefill_pipe(const VarlenArgs& a, hipStream_t stream);
long varlen_grid_size(int batch, int max_seqlen_q, int num_heads);

struct DecodeArgs {
  const void* q;
  const void* kv_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int num_seqs, num_blocks, max_blocks_per_seq, max_context_len;
  int num_heads, num_kv_heads, head_dim, block_size;
  float scale;
  void* out;
  float* lse;
  void* workspace;
  // multi-token queries: q is packed by cu_q, sequence b
  // has cu_q[b+1] - cu_q[b] <= max_q new tokens; nullptr = one token each
  const int32_t* cu_q = nullptr;
  int total_q = 0;
  // sliding window (single-token queries only): the query at position L - 1
  // sees keys t >= L - 1 - window; -1 = no window
  int window = -1;
};

// The library's own decode scratch (decode_scratch.hip): a fixed device array
// of kDecodeScratchBytes per GPU, held until the process ends, for the
// allocation-free decode entry point. Its device address on the current
// device is looked up once per device and cached.
constexpr size_t kDecodeScratchBytes = ATTN_DECODE_SCRATCH_BYTES;
hipError_t decode_scratch_address(void** ptr);

// Paged decode (every head dim): balanced streaming decode
// (paged_decode_stream.hip). The token stream of all sequences is cut into
// n_seg equal segments per kv head (and query-head chunk); one wave streams one
// segment. The plan does not depend on the context lengths.
struct DecodeStreamPlan {
  int max_q, q_chunks, n_seg;
  size_t prefix_bytes;  // int32 [num_seqs + 1] token prefix sums
  size_t skip_bytes;    // int32 [num_seqs] first streamed position (sliding window)
  size_t lse_bytes;     // fp32 [n_seg + num_seqs][max_q][num_heads] partial LSE
  size_t o_bytes;       // fp32 [n_seg + num_seqs][max_q][num_heads][head_dim] partial O
  size_t workspace_bytes;
};
// max_q: new query tokens per sequence at most (1 for decode)
DecodeStreamPlan plan_decode_stream(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int max_q = 1);
// multi-token queries take the streaming path when their (token, head)
// columns per kv head fit in kSpecMaxCols (at most that many / 16 passes over K/V)
constexpr int kSpecMaxCols = 64;
hipError_t launch_decode_stream(const DecodeArgs& a, const DecodeStreamPlan& p, hipStream_t stream);

// Scatter new tokens' K/V rows into the paged cache by slot (negative or
// out-of-range slots are skipped). row_elems = Hkv * D.
hipError_t launch_paged_kv_write(const void* k, const void* v, const int32_t* slots, int num_tokens, int row_elems,
                                 int num_blocks, void* kv_cache, hipStream_t stream);

// Block map -> ascending index lists.
// With sizes != nullptr: tiles of size 0 are dropped, entries are (size << 24) | tile.
hipError_t launch_map_to_index(const uint8_t* map, int rows, int n_cols, const int32_t* sizes, int32_t* idx,
                               int32_t* num, hipStream_t stream);

struct SparseArgs {
  const void* q;
  const void* k;
  const void* v;
  const uint8_t* block_map;
  const int32_t* tile_sizes;
  int batch, num_tiles, num_heads, num_kv_heads, head_dim;
  float scale;
  void* out;
  float* lse;
  int32_t* idx;  // workspace: [batch*num_heads*num_tiles][num_tiles]
  int32_t* num;  // workspace: [batch*num_heads*num_tiles]
  int32_t* order;  // workspace: [batch*num_heads*num_tiles], the order the pipelined kernel runs items in
};

size_t sparse_workspace_bytes(int batch, int num_heads, int num_tiles);
hipError_t launch_block_sparse_fwd(const SparseArgs& a, hipStream_t stream);
// Pipelined block-sparse kernel (block_sparse_pipe.hip): head_dims 96 to 256
// with at most kSparsePipeMaxTiles tiles (its kept-tile list is staged in
// LDS); expects the packed, size-filtered lists in a.idx / a.num.
constexpr int kSparsePipeMaxTiles = 3072;
bool sparse_pipe_supported(int head_dim, int num_tiles);
hipError_t launch_block_sparse_pipe(const SparseArgs& a, hipStream_t stream);

// Video tile geometry (raster (t, h, w) cut into (tile_t, tile_h, tile_w) boxes),
// optionally behind prefix segments (host array of num_segments lengths >= 0):
// the H3 layout, whose prefix rows come first and are cut into 64-row tiles
// segment by segment.
constexpr int kMaxPrefixSegments = 16;
struct VsaGeometry {
  int t, h, w, tile_t, tile_h, tile_w;
  const int32_t* prefix_segments = nullptr;
  int num_segments = 0;
};

int vsa_num_tiles(const VsaGeometry& g);  // prefix tiles included
int vsa_prefix_tiles(const VsaGeometry& g);
hipError_t launch_tile_gather(const void* x, const VsaGeometry& g, int batch, int row_elems, void* y,
                              int32_t* sizes, hipStream_t stream);
hipError_t launch_untile(const void* y, const VsaGeometry& g, int batch, int row_elems, void* x, hipStream_t stream);
size_t vsa_map_workspace_bytes(int batch, int heads, int kv_heads, int n_tiles, int head_dim);
// n_prefix > 0: the first n_prefix tiles are H3 prefix tiles (their rows and
// columns of the map are kept; top-k ranks the video columns only)
hipError_t launch_vsa_block_map(const void* q_tiled, const void* k_tiled, const int32_t* sizes, int batch,
                                int n_tiles, int heads, int kv_heads, int head_dim, float scale, int topk,
                                uint8_t* map, void* workspace, hipStream_t stream, int n_prefix = 0);
// Tile gather of raster q and k and the block map from their tile means in
// one pass over the raster rows (the tile-order copies are written, not read
// back); same workspace layout and map as launch_vsa_block_map.
hipError_t launch_vsa_gather_block_map(const void* q, const void* k, const VsaGeometry& g, int batch, int heads,
                                       int kv_heads, int head_dim, float scale, int topk, void* q_tiled,
                                       void* k_tiled, int32_t* sizes, uint8_t* map, void* workspace,
                                       hipStream_t stream);

// VSA compressed branch: out (tile order, bf16) += broadcast_rows(softmax(pooled
// scores) @ value tile means) * gate. Workspace: fp32 means of q, k, v and c.
size_t vsa_compressed_workspace_bytes(int batch, int heads, int kv_heads, int n_tiles, int head_dim);
hipError_t launch_vsa_compressed_add(const void* q_tiled, const void* k_tiled, const void* v_tiled,
                                     const int32_t* sizes, const void* gate, int batch, int n_tiles, int heads,
                                     int kv_heads, int head_dim, float scale, void* out, void* workspace,
                                     hipStream_t stream);

}  // namespace attn
