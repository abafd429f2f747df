// C ABI entry points: host-side validation, launch planning and dispatch.
// Nothing here reads device memory, allocates, or synchronises.
#include "../../include/attn_mi355x.h"

#include <cmath>
#include <cstdint>

#include "launch.hpp"

namespace {

bool supported_head_dim(int d) { return d == 64 || d == 96 || d == 128 || d == 192 || d == 256; }

bool valid_scale(float s) { return std::isfinite(s) && s > 0.f; }

// Signed byte counts stay far inside size_t; this guards 32-bit index math in
// the kernels, which address tensors with 64-bit offsets but 32-bit row ids.
constexpr long long kMaxRows = 0x7fffffffLL;

attn_status_t from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH; }

// Shape checks shared by the padded-batch and key-padding-mask entry points.
attn_status_t check_padded_shape(int batch, int seqlen_q, int seqlen_k, int num_heads, int num_kv_heads,
                                 int head_dim, float scale) {
  if (batch < 0 || seqlen_q < 0 || seqlen_k < 0 || num_heads <= 0 || num_kv_heads <= 0) return ATTN_ERR_INVALID_ARG;
  if (!valid_scale(scale)) return ATTN_ERR_INVALID_ARG;
  if (!supported_head_dim(head_dim)) return ATTN_ERR_UNSUPPORTED;
  if (num_heads % num_kv_heads != 0) return ATTN_ERR_UNSUPPORTED;
  if ((long long)batch * seqlen_q * num_heads > kMaxRows || (long long)batch * seqlen_k * num_kv_heads > kMaxRows) {
    return ATTN_ERR_UNSUPPORTED;
  }
  if (attn::varlen_grid_size(batch, seqlen_q, num_heads) > kMaxRows) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

attn_status_t attn_varlen_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, int32_t batch, int32_t total_q, int32_t total_k,
                              int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_heads,
                              int32_t num_kv_heads, int32_t head_dim, float softmax_scale, int32_t causal,
                              void* out, float* lse, void* stream) {
  if (batch < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0) return ATTN_ERR_INVALID_ARG;
  if (num_heads <= 0 || num_kv_heads <= 0) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (!valid_scale(softmax_scale)) return ATTN_ERR_INVALID_ARG;
  if (!supported_head_dim(head_dim)) return ATTN_ERR_UNSUPPORTED;
  if (num_heads % num_kv_heads != 0) return ATTN_ERR_UNSUPPORTED;
  if (max_seqlen_q > total_q || max_seqlen_k > total_k) return ATTN_ERR_INVALID_ARG;
  if (batch == 0 || total_q == 0) return ATTN_OK;
  if (max_seqlen_q == 0) return ATTN_ERR_INVALID_ARG;  // rows exist but no document could own them
  if (q == nullptr || out == nullptr || cu_seqlens_q == nullptr || cu_seqlens_k == nullptr) {
    return ATTN_ERR_INVALID_ARG;
  }
  if (total_k > 0 && (k == nullptr || v == nullptr)) return ATTN_ERR_INVALID_ARG;
  if ((long long)total_q * num_heads > kMaxRows || (long long)total_k * num_kv_heads > kMaxRows) {
    return ATTN_ERR_UNSUPPORTED;
  }
  if (attn::varlen_grid_size(batch, max_seqlen_q, num_heads) > kMaxRows) return ATTN_ERR_UNSUPPORTED;
  attn::VarlenArgs a{q, k, v, cu_seqlens_q, cu_seqlens_k, batch, total_q, total_k, max_seqlen_q, max_seqlen_k,
                     num_heads, num_kv_heads, head_dim, softmax_scale, causal, out, lse};
  return from_hip(attn::launch_varlen_fwd(a, (hipStream_t)stream));
}

attn_status_t attn_paged_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                               int32_t head_dim, int32_t max_context_len, size_t* bytes) {
  if (bytes == nullptr) return ATTN_ERR_INVALID_ARG;
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0) return ATTN_ERR_INVALID_ARG;
  if (!supported_head_dim(head_dim)) return ATTN_ERR_UNSUPPORTED;
  if (num_heads % num_kv_heads != 0) return ATTN_ERR_UNSUPPORTED;
  *bytes = attn::plan_decode_stream(num_seqs, num_heads, num_kv_heads, head_dim).workspace_bytes;
  return ATTN_OK;
}

}  // extern "C"

namespace {

attn_status_t paged_decode_impl(const void* q, const void* kv_cache, const int32_t* block_tables,
                                const int32_t* context_lens, int32_t num_seqs, int32_t num_blocks,
                                int32_t max_blocks_per_seq, int32_t max_context_len, int32_t num_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t window,
                                float softmax_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                                void* stream, bool use_scratch = false) {
  if (num_seqs < 0 || num_blocks < 0 || max_blocks_per_seq < 0 || max_context_len < 0) return ATTN_ERR_INVALID_ARG;
  if (num_heads <= 0 || num_kv_heads <= 0) return ATTN_ERR_INVALID_ARG;
  if (!valid_scale(softmax_scale)) return ATTN_ERR_INVALID_ARG;
  if (!supported_head_dim(head_dim)) return ATTN_ERR_UNSUPPORTED;
  if (num_heads % num_kv_heads != 0) return ATTN_ERR_UNSUPPORTED;
  if (block_size != 128) return ATTN_ERR_UNSUPPORTED;
  if ((long long)max_context_len > (long long)max_blocks_per_seq * block_size) return ATTN_ERR_INVALID_ARG;
  if (num_seqs == 0) return ATTN_OK;
  if (q == nullptr || out == nullptr || context_lens == nullptr) return ATTN_ERR_INVALID_ARG;
  if (max_context_len > 0 && (kv_cache == nullptr || block_tables == nullptr || num_blocks == 0)) {
    return ATTN_ERR_INVALID_ARG;
  }
  if ((long long)num_blocks * block_size * num_kv_heads > kMaxRows) return ATTN_ERR_UNSUPPORTED;
  if ((long long)num_seqs * max_context_len >= (1LL << 30)) return ATTN_ERR_UNSUPPORTED;  // int32 token prefix
  const attn::DecodeStreamPlan plan = attn::plan_decode_stream(num_seqs, num_heads, num_kv_heads, head_dim);
  if (use_scratch) {
    // the library's fixed scratch: refuse what does not fit it, then resolve
    // its address on this device
    if (plan.workspace_bytes > attn::kDecodeScratchBytes) return ATTN_ERR_WORKSPACE_TOO_SMALL;
    if (attn::decode_scratch_address(&workspace) != hipSuccess) return ATTN_ERR_LAUNCH;
  } else {
    if (workspace_bytes < plan.workspace_bytes) return ATTN_ERR_WORKSPACE_TOO_SMALL;
    if (plan.workspace_bytes > 0 && workspace == nullptr) return ATTN_ERR_INVALID_ARG;
  }
  attn::DecodeArgs a{q, kv_cache, block_tables, context_lens, num_seqs, num_blocks, max_blocks_per_seq,
                     max_context_len, num_heads, num_kv_heads, head_dim, block_size, softmax_scale, out, lse,
                     workspace};
  // a window at least as long as the context is no window
  a.window = window >= 0 && window < max_context_len ? window : -1;
  return from_hip(attn::launch_decode_stream(a, plan, (hipStream_t)stream));
}

}  // namespace

extern "C" {

attn_status_t attn_paged_decode(const void* q, const void* kv_cache, const int32_t* block_tables,
                                const int32_t* context_lens, int32_t num_seqs, int32_t num_blocks,
                                int32_t max_blocks_per_seq, int32_t max_context_len, int32_t num_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float softmax_scale,
                                void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return paged_decode_impl(q, kv_cache, block_tables, context_lens, num_seqs, num_blocks, max_blocks_per_seq,
                           max_context_len, num_heads, num_kv_heads, head_dim, block_size, -1, softmax_scale, out,
                           lse, workspace, workspace_bytes, stream);
}

attn_status_t attn_paged_decode_scratch(const void* q, const void* kv_cache, const int32_t* block_tables,
                                        const int32_t* context_lens, int32_t num_seqs, int32_t num_blocks,
                                        int32_t max_blocks_per_seq, int32_t max_context_len, int32_t num_heads,
                                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                        float softmax_scale, void* out, float* lse, void* stream) {
  return paged_decode_impl(q, kv_cache, block_tables, context_lens, num_seqs, num_blocks, max_blocks_per_seq,
                           max_context_len, num_heads, num_kv_heads, head_dim, block_size, -1, softmax_scale, out,
                           lse, nullptr, 0, stream, true);
}

attn_status_t attn_paged_decode_sliding_window(const void* q, const void* kv_cache, const int32_t* block_tables,
                                               const int32_t* context_lens, int32_t num_seqs, int32_t num_blocks,
                                               int32_t max_blocks_per_seq, int32_t max_context_len,
                                               int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                               int32_t block_size, int32_t window, float softmax_scale, void* out,
                                               float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (window < 0) return ATTN_ERR_INVALID_ARG;
  return paged_decode_impl(q, kv_cache, block_tables, context_lens, num_seqs, num_blocks, max_blocks_per_seq,
                           max_context_len, num_heads, num_kv_heads, head_dim, block_size, window, softmax_scale,
                           out, lse, workspace, workspace_bytes, stream);
}

attn_status_t attn_padded_fwd_workspace_size(int32_t batch, size_t* bytes) {
  if (bytes == nullptr || batch < 0) return ATTN_ERR_INVALID_ARG;
  *bytes = attn::padded_workspace_bytes(batch);
  return ATTN_OK;
}

attn_status_t attn_padded_fwd(const void* q, const void* k, const void* v, const int32_t* q_lens,
                              const int32_t* k_lens, int32_t batch, int32_t seqlen_q, int32_t seqlen_k,
                              int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, float softmax_scale,
                              int32_t causal, void* out, float* lse, void* workspace, size_t workspace_bytes,
                              void* stream) {
  const attn_status_t st = check_padded_shape(batch, seqlen_q, seqlen_k, num_heads, num_kv_heads, head_dim,
                                              softmax_scale);
  if (st != ATTN_OK) return st;
  if (batch == 0 || seqlen_q == 0) return ATTN_OK;
  if (q == nullptr || out == nullptr || q_lens == nullptr || k_lens == nullptr) return ATTN_ERR_INVALID_ARG;
  if (seqlen_k > 0 && (k == nullptr || v == nullptr)) return ATTN_ERR_INVALID_ARG;
  if (workspace_bytes < attn::padded_workspace_bytes(batch)) return ATTN_ERR_WORKSPACE_TOO_SMALL;
  if (workspace == nullptr) return ATTN_ERR_INVALID_ARG;
  attn::VarlenArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.batch = batch;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.scale = softmax_scale;
  a.causal = causal != 0;
  a.out = out;
  a.lse = lse;
  return from_hip(attn::launch_padded_fwd(a, q_lens, k_lens, seqlen_q, seqlen_k, workspace, (hipStream_t)stream));
}

attn_status_t attn_masked_fwd_workspace_size(int32_t batch, int32_t seqlen_q, int32_t seqlen_k, int32_t num_heads,
                                             int32_t num_kv_heads, int32_t head_dim, int32_t mask_queries,
                                             size_t* bytes) {
  if (bytes == nullptr) return ATTN_ERR_INVALID_ARG;
  if (batch < 0 || seqlen_q < 0 || seqlen_k < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0) {
    return ATTN_ERR_INVALID_ARG;
  }
  *bytes = attn::plan_masked(batch, seqlen_q, seqlen_k, num_heads, num_kv_heads, head_dim, mask_queries != 0).bytes;
  return ATTN_OK;
}

attn_status_t attn_masked_fwd(const void* q, const void* k, const void* v, const uint8_t* key_mask, int32_t batch,
                              int32_t seqlen_q, int32_t seqlen_k, int32_t num_heads, int32_t num_kv_heads,
                              int32_t head_dim, float softmax_scale, int32_t causal, int32_t mask_queries, void* out,
                              float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  const attn_status_t st = check_padded_shape(batch, seqlen_q, seqlen_k, num_heads, num_kv_heads, head_dim,
                                              softmax_scale);
  if (st != ATTN_OK) return st;
  if (mask_queries != 0 && seqlen_q != seqlen_k) return ATTN_ERR_INVALID_ARG;
  if (batch == 0 || seqlen_q == 0) return ATTN_OK;
  if (q == nullptr || out == nullptr) return ATTN_ERR_INVALID_ARG;
  if (seqlen_k > 0 && (k == nullptr || v == nullptr || key_mask == nullptr)) return ATTN_ERR_INVALID_ARG;
  const attn::MaskedLayout l =
      attn::plan_masked(batch, seqlen_q, seqlen_k, num_heads, num_kv_heads, head_dim, mask_queries != 0);
  if (workspace_bytes < l.bytes) return ATTN_ERR_WORKSPACE_TOO_SMALL;
  if (workspace == nullptr) return ATTN_ERR_INVALID_ARG;
  attn::VarlenArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.batch = batch;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.scale = softmax_scale;
  a.causal = causal != 0;
  a.out = out;
  a.lse = lse;
  if (seqlen_k == 0) {  // no key anywhere: every row is a padding row of length 0
    return from_hip(attn::launch_padded_fwd(a, nullptr, nullptr, seqlen_q, 0, workspace, (hipStream_t)stream));
  }
  return from_hip(attn::launch_masked_fwd(a, key_mask, seqlen_q, seqlen_k, mask_queries != 0, l, workspace,
                                          (hipStream_t)stream));
}

attn_status_t attn_paged_kv_write(const void* k, const void* v, const int32_t* slot_mapping, int32_t num_tokens,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks, int32_t block_size,
                                  void* kv_cache, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0) return ATTN_ERR_INVALID_ARG;
  if (!supported_head_dim(head_dim)) return ATTN_ERR_UNSUPPORTED;
  if (block_size != 128) return ATTN_ERR_UNSUPPORTED;
  if (num_tokens == 0) return ATTN_OK;
  if (k == nullptr || v == nullptr || slot_mapping == nullptr || kv_cache == nullptr || num_blocks == 0) {
    return ATTN_ERR_INVALID_ARG;
  }
  if ((long long)num_blocks * block_size * num_kv_heads > kMaxRows) return ATTN_ERR_UNSUPPORTED;
  return from_hip(attn::launch_paged_kv_write(k, v, slot_mapping, num_tokens, num_kv_heads * head_dim, num_blocks,
                                              kv_cache, (hipStream_t)stream));
}

}  // extern "C"

namespace {
// Short multi-token queries (speculative decoding) stream the paged cache like
// decode, with (query token, head) columns; longer ones run the prefill kernels.
bool paged_prefill_streams(int batch, int num_heads, int num_kv_heads, int max_seqlen_q, int max_context_len) {
  return (long long)max_seqlen_q * (num_heads / num_kv_heads) <= attn::kSpecMaxCols &&
         (long long)batch * max_context_len < (1LL << 30);
}
}  // namespace

extern "C" {

attn_status_t attn_paged_prefill_workspace_size(int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                                int32_t head_dim, int32_t max_seqlen_q, int32_t max_context_len,
                                                size_t* bytes) {
  if (bytes == nullptr) return ATTN_ERR_INVALID_ARG;
  if (batch < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_seqlen_q < 0 || max_context_len < 0) {
    return ATTN_ERR_INVALID_ARG;
  }
  if (!supported_head_dim(head_dim)) return ATTN_ERR_UNSUPPORTED;
  if (num_heads % num_kv_heads != 0) return ATTN_ERR_UNSUPPORTED;
  *bytes = paged_prefill_streams(batch, num_heads, num_kv_heads, max_seqlen_q, max_context_len)
               ? attn::plan_decode_stream(batch, num_heads, num_kv_heads, head_dim, max_seqlen_q).workspace_bytes
               : 0;
  return ATTN_OK;
}

attn_status_t attn_paged_prefill(const void* q, const void* kv_cache, const int32_t* block_tables,
                                 const int32_t* cu_seqlens_q, const int32_t* context_lens, int32_t batch,
                                 int32_t total_q, int32_t max_seqlen_q, int32_t max_context_len, int32_t num_blocks,
                                 int32_t max_blocks_per_seq, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, float softmax_scale, void* out, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (batch < 0 || total_q < 0 || max_seqlen_q < 0 || max_context_len < 0) return ATTN_ERR_INVALID_ARG;
  if (num_blocks < 0 || max_blocks_per_seq < 0 || num_heads <= 0 || num_kv_heads <= 0) return ATTN_ERR_INVALID_ARG;
  if (!valid_scale(softmax_scale)) return ATTN_ERR_INVALID_ARG;
  if (!supported_head_dim(head_dim)) return ATTN_ERR_UNSUPPORTED;
  if (num_heads % num_kv_heads != 0) return ATTN_ERR_UNSUPPORTED;
  if (block_size != 128) return ATTN_ERR_UNSUPPORTED;
  if ((long long)max_context_len > (long long)max_blocks_per_seq * block_size) return ATTN_ERR_INVALID_ARG;
  if (max_seqlen_q > total_q) return ATTN_ERR_INVALID_ARG;
  if (batch == 0 || total_q == 0) return ATTN_OK;
  if (max_seqlen_q == 0) return ATTN_ERR_INVALID_ARG;  // rows exist but no sequence could own them
  if (q == nullptr || out == nullptr || cu_seqlens_q == nullptr || context_lens == nullptr) {
    return ATTN_ERR_INVALID_ARG;
  }
  if (max_context_len > 0 && (kv_cache == nullptr || block_tables == nullptr || num_blocks == 0)) {
    return ATTN_ERR_INVALID_ARG;
  }
  if ((long long)total_q * num_heads > kMaxRows) return ATTN_ERR_UNSUPPORTED;
  if ((long long)num_blocks * block_size * num_kv_heads > kMaxRows) return ATTN_ERR_UNSUPPORTED;
  if (attn::varlen_grid_size(batch, max_seqlen_q, num_heads) > kMaxRows) return ATTN_ERR_UNSUPPORTED;
  if (paged_prefill_streams(batch, num_heads, num_kv_heads, max_seqlen_q, max_context_len)) {
    const attn::DecodeStreamPlan plan =
        attn::plan_decode_stream(batch, num_heads, num_kv_heads, head_dim, max_seqlen_q);
    if (workspace_bytes < plan.workspace_bytes) return ATTN_ERR_WORKSPACE_TOO_SMALL;
    if (workspace == nullptr) return ATTN_ERR_INVALID_ARG;
    attn::DecodeArgs d{q, kv_cache, block_tables, context_lens, batch, num_blocks, max_blocks_per_seq,
                       max_context_len, num_heads, num_kv_heads, head_dim, block_size, softmax_scale, out, lse,
                       workspace};
    d.cu_q = cu_seqlens_q;
    d.total_q = total_q;
    return from_hip(attn::launch_decode_stream(d, plan, (hipStream_t)stream));
  }
  const long long plane = (long long)num_blocks * block_size * num_kv_heads * head_dim;  // elements
  attn::VarlenArgs a{q, kv_cache, (const uint16_t*)kv_cache + plane, cu_seqlens_q, nullptr, batch, total_q, 0,
                     max_seqlen_q, max_context_len, num_heads, num_kv_heads, head_dim, softmax_scale, 1, out, lse};
  a.paged = true;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  return from_hip(attn::launch_varlen_fwd(a, (hipStream_t)stream));
}

attn_status_t attn_block_map_to_index(const uint8_t* block_map, int32_t rows, int32_t n_cols, int32_t* idx,
                                      int32_t* num, void* stream) {
  if (rows < 0 || n_cols <= 0) return ATTN_ERR_INVALID_ARG;
  if (rows == 0) return ATTN_OK;
  if (block_map == nullptr || idx == nullptr || num == nullptr) return ATTN_ERR_INVALID_ARG;
  if ((long long)rows * n_cols > kMaxRows) return ATTN_ERR_UNSUPPORTED;
  return from_hip(attn::launch_map_to_index(block_map, rows, n_cols, nullptr, idx, num, (hipStream_t)stream));
}

attn_status_t attn_block_sparse_workspace_size(int32_t batch, int32_t num_heads, int32_t num_tiles, size_t* bytes) {
  if (bytes == nullptr) return ATTN_ERR_INVALID_ARG;
  if (batch < 0 || num_heads <= 0 || num_tiles < 0) return ATTN_ERR_INVALID_ARG;
  *bytes = attn::sparse_workspace_bytes(batch, num_heads, num_tiles);
  return ATTN_OK;
}

attn_status_t attn_block_sparse_fwd(const void* q, const void* k, const void* v, const uint8_t* block_map,
                                    const int32_t* tile_sizes, int32_t batch, int32_t num_tiles, int32_t num_heads,
                                    int32_t num_kv_heads, int32_t head_dim, float softmax_scale, void* out,
                                    float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (batch < 0 || num_tiles < 0 || num_heads <= 0 || num_kv_heads <= 0) return ATTN_ERR_INVALID_ARG;
  if (!valid_scale(softmax_scale)) return ATTN_ERR_INVALID_ARG;
  if (!supported_head_dim(head_dim)) return ATTN_ERR_UNSUPPORTED;
  if (num_heads % num_kv_heads != 0) return ATTN_ERR_UNSUPPORTED;
  if (batch == 0 || num_tiles == 0) return ATTN_OK;
  if (q == nullptr || k == nullptr || v == nullptr || block_map == nullptr || tile_sizes == nullptr ||
      out == nullptr) {
    return ATTN_ERR_INVALID_ARG;
  }
  if ((long long)batch * num_tiles * 64 * num_heads > kMaxRows) return ATTN_ERR_UNSUPPORTED;
  if ((long long)batch * num_heads * num_tiles * num_tiles > kMaxRows) return ATTN_ERR_UNSUPPORTED;
  const size_t need = attn::sparse_workspace_bytes(batch, num_heads, num_tiles);
  if (workspace_bytes < need) return ATTN_ERR_WORKSPACE_TOO_SMALL;
  if (workspace == nullptr) return ATTN_ERR_INVALID_ARG;
  const size_t rows = (size_t)batch * num_heads * num_tiles;
  int32_t* idx = (int32_t*)workspace;
  int32_t* num = idx + rows * (size_t)num_tiles;
  int32_t* order = num + rows;
  attn::SparseArgs a{q, k, v, block_map, tile_sizes, batch, num_tiles, num_heads, num_kv_heads, head_dim,
                     softmax_scale, out, lse, idx, num, order};
  return from_hip(attn::launch_block_sparse_fwd(a, (hipStream_t)stream));
}

static attn_status_t check_vsa_geometry(int32_t batch, int32_t t, int32_t h, int32_t w, int32_t tile_t,
                                        int32_t tile_h, int32_t tile_w, int32_t row_elems) {
  if (batch < 0 || t < 0 || h < 0 || w < 0 || row_elems <= 0) return ATTN_ERR_INVALID_ARG;
  if (tile_t <= 0 || tile_h <= 0 || tile_w <= 0) return ATTN_ERR_INVALID_ARG;
  if ((long long)tile_t * tile_h * tile_w > 64) return ATTN_ERR_UNSUPPORTED;
  if (row_elems % 8 != 0) return ATTN_ERR_UNSUPPORTED;
  const long long n = (long long)t * h * w;
  const long long tiles = (long long)((t + tile_t - 1) / tile_t) * ((h + tile_h - 1) / tile_h) *
                          ((w + tile_w - 1) / tile_w);
  if ((long long)batch * (n > tiles * 64 ? n : tiles * 64) > kMaxRows) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

attn_status_t attn_vsa_tile_gather(const void* x, int32_t batch, int32_t t, int32_t h, int32_t w, int32_t tile_t,
                                   int32_t tile_h, int32_t tile_w, int32_t row_elems, void* x_tiled,
                                   int32_t* tile_sizes, void* stream) {
  const attn_status_t st = check_vsa_geometry(batch, t, h, w, tile_t, tile_h, tile_w, row_elems);
  if (st != ATTN_OK) return st;
  if (batch == 0 || (long long)t * h * w == 0) return ATTN_OK;
  if (x == nullptr || x_tiled == nullptr) return ATTN_ERR_INVALID_ARG;
  const attn::VsaGeometry g{t, h, w, tile_t, tile_h, tile_w};
  return from_hip(attn::launch_tile_gather(x, g, batch, row_elems, x_tiled, tile_sizes, (hipStream_t)stream));
}

attn_status_t attn_vsa_untile(const void* x_tiled, int32_t batch, int32_t t, int32_t h, int32_t w, int32_t tile_t,
                              int32_t tile_h, int32_t tile_w, int32_t row_elems, void* x, void* stream) {
  const attn_status_t st = check_vsa_geometry(batch, t, h, w, tile_t, tile_h, tile_w, row_elems);
  if (st != ATTN_OK) return st;
  if (batch == 0 || (long long)t * h * w == 0) return ATTN_OK;
  if (x == nullptr || x_tiled == nullptr) return ATTN_ERR_INVALID_ARG;
  const attn::VsaGeometry g{t, h, w, tile_t, tile_h, tile_w};
  return from_hip(attn::launch_untile(x_tiled, g, batch, row_elems, x, (hipStream_t)stream));
}

static attn_status_t check_prefix(const int32_t* prefix_segments, int32_t num_segments, long long* rows) {
  if (num_segments < 0 || num_segments > attn::kMaxPrefixSegments) return ATTN_ERR_UNSUPPORTED;
  if (num_segments > 0 && prefix_segments == nullptr) return ATTN_ERR_INVALID_ARG;
  long long n = 0;
  for (int i = 0; i < num_segments; ++i) {
    if (prefix_segments[i] < 0) return ATTN_ERR_INVALID_ARG;
    n += prefix_segments[i];
  }
  *rows = n;
  return ATTN_OK;
}

// H3 layout checks: the prefix rows and their 64-row tiles added to the video's.
static attn_status_t check_h3_geometry(const int32_t* prefix_segments, int32_t num_segments, int32_t batch,
                                       int32_t t, int32_t h, int32_t w, int32_t tile_t, int32_t tile_h,
                                       int32_t tile_w, int32_t row_elems) {
  attn_status_t st = check_vsa_geometry(batch, t, h, w, tile_t, tile_h, tile_w, row_elems);
  if (st != ATTN_OK) return st;
  long long prefix = 0;
  st = check_prefix(prefix_segments, num_segments, &prefix);
  if (st != ATTN_OK) return st;
  const long long tiles = (long long)((t + tile_t - 1) / tile_t) * ((h + tile_h - 1) / tile_h) *
                              ((w + tile_w - 1) / tile_w) + prefix / 64 + num_segments;
  if ((long long)batch * (prefix + (long long)t * h * w + tiles * 64) > kMaxRows) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

attn_status_t attn_vsa_h3_num_tiles(const int32_t* prefix_segments, int32_t num_segments, int32_t t, int32_t h,
                                    int32_t w, int32_t tile_t, int32_t tile_h, int32_t tile_w,
                                    int32_t* num_prefix_tiles, int32_t* num_tiles) {
  if (num_prefix_tiles == nullptr || num_tiles == nullptr) return ATTN_ERR_INVALID_ARG;
  const attn_status_t st = check_h3_geometry(prefix_segments, num_segments, 1, t, h, w, tile_t, tile_h, tile_w, 8);
  if (st != ATTN_OK) return st;
  attn::VsaGeometry g{t, h, w, tile_t, tile_h, tile_w};
  g.prefix_segments = prefix_segments;
  g.num_segments = num_segments;
  *num_prefix_tiles = attn::vsa_prefix_tiles(g);
  *num_tiles = attn::vsa_num_tiles(g);
  return ATTN_OK;
}

attn_status_t attn_vsa_h3_tile_gather(const void* x, const int32_t* prefix_segments, int32_t num_segments,
                                      int32_t batch, int32_t t, int32_t h, int32_t w, int32_t tile_t, int32_t tile_h,
                                      int32_t tile_w, int32_t row_elems, void* x_tiled, int32_t* tile_sizes,
                                      void* stream) {
  const attn_status_t st =
      check_h3_geometry(prefix_segments, num_segments, batch, t, h, w, tile_t, tile_h, tile_w, row_elems);
  if (st != ATTN_OK) return st;
  attn::VsaGeometry g{t, h, w, tile_t, tile_h, tile_w};
  g.prefix_segments = prefix_segments;
  g.num_segments = num_segments;
  if (batch == 0 || attn::vsa_num_tiles(g) == 0) return ATTN_OK;
  if (x == nullptr || x_tiled == nullptr) return ATTN_ERR_INVALID_ARG;
  return from_hip(attn::launch_tile_gather(x, g, batch, row_elems, x_tiled, tile_sizes, (hipStream_t)stream));
}

attn_status_t attn_vsa_h3_untile(const void* x_tiled, const int32_t* prefix_segments, int32_t num_segments,
                                 int32_t batch, int32_t t, int32_t h, int32_t w, int32_t tile_t, int32_t tile_h,
                                 int32_t tile_w, int32_t row_elems, void* x, void* stream) {
  const attn_status_t st =
      check_h3_geometry(prefix_segments, num_segments, batch, t, h, w, tile_t, tile_h, tile_w, row_elems);
  if (st != ATTN_OK) return st;
  attn::VsaGeometry g{t, h, w, tile_t, tile_h, tile_w};
  g.prefix_segments = prefix_segments;
  g.num_segments = num_segments;
  if (batch == 0 || attn::vsa_num_tiles(g) == 0) return ATTN_OK;
  if (x == nullptr || x_tiled == nullptr) return ATTN_ERR_INVALID_ARG;
  return from_hip(attn::launch_untile(x_tiled, g, batch, row_elems, x, (hipStream_t)stream));
}

attn_status_t attn_vsa_block_map_workspace_size(int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                                int32_t num_tiles, int32_t head_dim, size_t* bytes) {
  if (bytes == nullptr) return ATTN_ERR_INVALID_ARG;
  if (batch < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_tiles < 0 || head_dim <= 0) {
    return ATTN_ERR_INVALID_ARG;
  }
  *bytes = attn::vsa_map_workspace_bytes(batch, num_heads, num_kv_heads, num_tiles, head_dim);
  return ATTN_OK;
}

static attn_status_t vsa_block_map_impl(const void* q_tiled, const void* k_tiled, const int32_t* tile_sizes,
                                        int32_t batch, int32_t num_tiles, int32_t num_prefix_tiles,
                                        int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                        float softmax_scale, int32_t topk, uint8_t* block_map, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  if (batch < 0 || num_tiles < 0 || num_heads <= 0 || num_kv_heads <= 0 || topk < 1) return ATTN_ERR_INVALID_ARG;
  if (num_prefix_tiles < 0 || num_prefix_tiles > num_tiles) return ATTN_ERR_INVALID_ARG;
  if (!valid_scale(softmax_scale)) return ATTN_ERR_INVALID_ARG;
  if (!supported_head_dim(head_dim)) return ATTN_ERR_UNSUPPORTED;
  if (num_heads % num_kv_heads != 0) return ATTN_ERR_UNSUPPORTED;
  if (num_tiles > 16384) return ATTN_ERR_UNSUPPORTED;
  if (batch == 0 || num_tiles == 0) return ATTN_OK;
  if (q_tiled == nullptr || k_tiled == nullptr || tile_sizes == nullptr || block_map == nullptr) {
    return ATTN_ERR_INVALID_ARG;
  }
  if ((long long)batch * num_heads * num_tiles * num_tiles > kMaxRows) return ATTN_ERR_UNSUPPORTED;
  const size_t need = attn::vsa_map_workspace_bytes(batch, num_heads, num_kv_heads, num_tiles, head_dim);
  if (workspace_bytes < need) return ATTN_ERR_WORKSPACE_TOO_SMALL;
  if (workspace == nullptr) return ATTN_ERR_INVALID_ARG;
  return from_hip(attn::launch_vsa_block_map(q_tiled, k_tiled, tile_sizes, batch, num_tiles, num_heads, num_kv_heads,
                                             head_dim, softmax_scale, topk, block_map, workspace, (hipStream_t)stream,
                                             num_prefix_tiles));
}

attn_status_t attn_vsa_block_map(const void* q_tiled, const void* k_tiled, const int32_t* tile_sizes,
                                 int32_t batch, int32_t num_tiles, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, float softmax_scale, int32_t topk, uint8_t* block_map,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return vsa_block_map_impl(q_tiled, k_tiled, tile_sizes, batch, num_tiles, 0, num_heads, num_kv_heads, head_dim,
                            softmax_scale, topk, block_map, workspace, workspace_bytes, stream);
}

attn_status_t attn_vsa_h3_block_map(const void* q_tiled, const void* k_tiled, const int32_t* tile_sizes,
                                    int32_t batch, int32_t num_tiles, int32_t num_prefix_tiles, int32_t num_heads,
                                    int32_t num_kv_heads, int32_t head_dim, float softmax_scale, int32_t topk,
                                    uint8_t* block_map, void* workspace, size_t workspace_bytes, void* stream) {
  return vsa_block_map_impl(q_tiled, k_tiled, tile_sizes, batch, num_tiles, num_prefix_tiles, num_heads,
                            num_kv_heads, head_dim, softmax_scale, topk, block_map, workspace, workspace_bytes,
                            stream);
}

attn_status_t attn_vsa_h3_gather_block_map(const void* q, const void* k, const int32_t* prefix_segments,
                                           int32_t num_segments, int32_t batch, int32_t t, int32_t h, int32_t w,
                                           int32_t tile_t, int32_t tile_h, int32_t tile_w, int32_t num_heads,
                                           int32_t num_kv_heads, int32_t head_dim, float softmax_scale, int32_t topk,
                                           void* q_tiled, void* k_tiled, int32_t* tile_sizes, uint8_t* block_map,
                                           void* workspace, size_t workspace_bytes, void* stream) {
  if (num_heads <= 0 || num_kv_heads <= 0 || topk < 1) return ATTN_ERR_INVALID_ARG;
  if (!valid_scale(softmax_scale)) return ATTN_ERR_INVALID_ARG;
  if (!supported_head_dim(head_dim)) return ATTN_ERR_UNSUPPORTED;
  if (num_heads % num_kv_heads != 0) return ATTN_ERR_UNSUPPORTED;
  const attn_status_t st = check_h3_geometry(prefix_segments, num_segments, batch, t, h, w, tile_t, tile_h, tile_w,
                                             num_heads * head_dim);
  if (st != ATTN_OK) return st;
  attn::VsaGeometry g{t, h, w, tile_t, tile_h, tile_w};
  g.prefix_segments = prefix_segments;
  g.num_segments = num_segments;
  const int num_tiles = attn::vsa_num_tiles(g);
  if (num_tiles > 16384) return ATTN_ERR_UNSUPPORTED;
  if (batch == 0 || num_tiles == 0) return ATTN_OK;
  if (q == nullptr || k == nullptr || q_tiled == nullptr || k_tiled == nullptr || block_map == nullptr) {
    return ATTN_ERR_INVALID_ARG;
  }
  if ((long long)batch * num_heads * num_tiles * num_tiles > kMaxRows) return ATTN_ERR_UNSUPPORTED;
  const size_t need = attn::vsa_map_workspace_bytes(batch, num_heads, num_kv_heads, num_tiles, head_dim);
  if (workspace_bytes < need) return ATTN_ERR_WORKSPACE_TOO_SMALL;
  if (workspace == nullptr) return ATTN_ERR_INVALID_ARG;
  return from_hip(attn::launch_vsa_gather_block_map(q, k, g, batch, num_heads, num_kv_heads, head_dim, softmax_scale,
                                                    topk, q_tiled, k_tiled, tile_sizes, block_map, workspace,
                                                    (hipStream_t)stream));
}

attn_status_t attn_vsa_compressed_workspace_size(int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                                 int32_t num_tiles, int32_t head_dim, size_t* bytes) {
  if (bytes == nullptr) return ATTN_ERR_INVALID_ARG;
  if (batch < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_tiles < 0 || head_dim <= 0) {
    return ATTN_ERR_INVALID_ARG;
  }
  *bytes = attn::vsa_compressed_workspace_bytes(batch, num_heads, num_kv_heads, num_tiles, head_dim);
  return ATTN_OK;
}

attn_status_t attn_vsa_compressed_add(const void* q_tiled, const void* k_tiled, const void* v_tiled,
                                      const int32_t* tile_sizes, const void* gate_tiled, int32_t batch,
                                      int32_t num_tiles, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                      float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  if (batch < 0 || num_tiles < 0 || num_heads <= 0 || num_kv_heads <= 0) return ATTN_ERR_INVALID_ARG;
  if (!valid_scale(softmax_scale)) return ATTN_ERR_INVALID_ARG;
  if (!supported_head_dim(head_dim)) return ATTN_ERR_UNSUPPORTED;
  if (num_heads % num_kv_heads != 0) return ATTN_ERR_UNSUPPORTED;
  if (num_tiles > 16384) return ATTN_ERR_UNSUPPORTED;
  if (batch == 0 || num_tiles == 0) return ATTN_OK;
  if (q_tiled == nullptr || k_tiled == nullptr || v_tiled == nullptr || tile_sizes == nullptr ||
      gate_tiled == nullptr || out == nullptr) {
    return ATTN_ERR_INVALID_ARG;
  }
  if ((long long)batch * num_tiles * 64 * num_heads > kMaxRows) return ATTN_ERR_UNSUPPORTED;
  const size_t need = attn::vsa_compressed_workspace_bytes(batch, num_heads, num_kv_heads, num_tiles, head_dim);
  if (workspace_bytes < need) return ATTN_ERR_WORKSPACE_TOO_SMALL;
  if (workspace == nullptr) return ATTN_ERR_INVALID_ARG;
  return from_hip(attn::launch_vsa_compressed_add(q_tiled, k_tiled, v_tiled, tile_sizes, gate_tiled, batch,
                                                  num_tiles, num_heads, num_kv_heads, head_dim, softmax_scale, out,
                                                  workspace, (hipStream_t)stream));
}

}  // extern "C"
