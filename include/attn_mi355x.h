/*
 * attn_mi355x.h - C ABI of the MI355X (gfx950) attention forward library.
 *
 * Operation (all entry points): fused scaled-dot-product attention forward
 *
 *     O_i   = sum_j exp(z_ij) v_j / sum_j exp(z_ij),   z_ij = scale * <q_i, k_j>
 *     LSE_i = ln sum_j exp(z_ij)
 *
 * over the keys j allowed for query i. This is the contract of the fused kernels
 * that the vLLM-Omni diffusion backend page (flash_attn.py, FlashAttentionImpl)
 * calls with a softmax scale and a causal flag and that return out or
 * (out, lse); its laser-attention note names S = Q K^T, and the fastvideo_vsa.py
 * page writes tile attention as softmax(scale * q k^T) v. A query row with no
 * allowed key gets O = 0 and LSE = -inf.
 *
 * Conventions shared by every call:
 *   - Pointers are DEVICE pointers unless marked (host). Tensors are dense,
 *     row-major, with no padding between rows. Q/K/V/O and the KV cache are
 *     bf16 (passed as void*), index arrays int32, LSE fp32.
 *   - Output buffers belong to the caller (the pages' backends all declare
 *     accept_output_buffer and the Ascend forward requires an output tensor).
 *     The library allocates nothing, never synchronises the host, keeps no
 *     state besides cached launch parameters (and the fixed device array of
 *     attn_paged_decode_scratch, part of the loaded code), and enqueues its kernels on
 *     `stream` (a hipStream_t; NULL = the default stream). Every call is
 *     therefore capturable in a HIP graph.
 *   - Host-side sizes (batch, totals, max lengths) plan the launch; device-side
 *     index arrays are never read by the host (the pages pass max_seqlen as host
 *     ints so no device sync is needed).
 *   - Validation: every argument the host can check is checked before any HIP
 *     call; on failure nothing is enqueued and an ATTN_ERR_* code is returned.
 *     Device-resident index values (cu_seqlens, block tables, context lengths,
 *     tile sizes) are preconditions; the kernels clamp them into the buffers
 *     they index, so a bad value yields wrong numbers, never an out-of-bounds
 *     access.
 *   - Determinism: results are bitwise identical run to run (fixed reduction
 *     order, no atomics).
 *   - softmax_scale must be finite and > 0 (the pages use head_dim^-0.5).
 *   - head_dim must be one of 64, 96, 128, 192, 256 (the flash backend's
 *     get_supported_head_sizes list).
 *   - Grouped-query heads: num_heads % num_kv_heads == 0; query head h reads kv
 *     head h / (num_heads / num_kv_heads) (the Ascend backend's
 *     num_queries_per_kv grouping).
 */
#ifndef ATTN_MI355X_H
#define ATTN_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 1

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1,          /* null pointer, negative size, inconsistent shape */
  ATTN_ERR_UNSUPPORTED = 2,          /* head_dim, block_size or GQA ratio not supported */
  ATTN_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes below the size query's answer */
  ATTN_ERR_LAUNCH = 4                /* the HIP runtime rejected a kernel launch */
} attn_status_t;

/* Static, human-readable name of a status code (never NULL). */
const char* attn_status_string(int status);

/* ATTN_ABI_VERSION of the built library. */
int attn_abi_version(void);

/*
 * Packed variable-length prefill (vLLM-Omni flash_attn.py page:
 * FlashAttentionImpl._forward_varlen_packed and _forward_varlen_dense, which
 * flatten [B, S, H, D] to [total, H, D] and pass cumulative cu_seqlens;
 * vLLM-Ascend attention_v1.py page: _forward_encoder_attention / TND layout).
 *
 *   q            [total_q, num_heads, head_dim]     bf16
 *   k, v         [total_k, num_kv_heads, head_dim]  bf16
 *   cu_seqlens_q [batch + 1] int32, cu_seqlens_q[0] = 0, non-decreasing,
 *                cu_seqlens_q[batch] = total_q; document b owns rows
 *                [cu_seqlens_q[b], cu_seqlens_q[b+1]). Same for cu_seqlens_k.
 *   max_seqlen_q (host) >= every document's query length; sizes the grid.
 *   max_seqlen_k (host) >= every document's key length.
 *   causal       0 = every key of the document; 1 = bottom-right aligned causal
 *                (key j is allowed for query i iff j <= i + Lk - Lq, the
 *                alignment the flash backend's NPU causal branch spells out).
 *   out          [total_q, num_heads, head_dim] bf16 (caller-owned)
 *   lse          nullable; [num_heads, total_q] fp32 natural-log LSE.
 * A query never attends a key of another document. batch == 0 or
 * total_q == 0 is a no-op returning ATTN_OK.
 */
attn_status_t attn_varlen_fwd(const void* q, const void* k, const void* v,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int32_t batch, int32_t total_q, int32_t total_k,
                              int32_t max_seqlen_q, int32_t max_seqlen_k,
                              int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                              float softmax_scale, int32_t causal,
                              void* out, float* lse, void* stream);

/*
 * Workspace bytes that attn_paged_decode needs for these host sizes
 * (the Ascend page sizes its paged-attention workspace with a query call,
 * _npu_paged_attention_get_workspace). Written to *bytes (host pointer). The
 * size does not depend on max_context_len (kept for that call's shape): two
 * int32 arrays of num_seqs + 1 plus fp32 partials (O and LSE) for
 * num_seqs + n_seg slots of every head, n_seg = 256 * W / (num_kv_heads *
 * ceil(num_heads / num_kv_heads / 16)) with W = 8, 4, 4, 2, 2 waves per CU at
 * head_dim 64, 96, 128, 192, 256.
 */
attn_status_t attn_paged_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                               int32_t head_dim, int32_t max_context_len, size_t* bytes);

/*
 * Single-token decode over a paged KV cache (vLLM-Ascend attention_v1.py page:
 * get_kv_cache_shape, get_supported_block_size, AscendMetadata.block_tables /
 * seq_lens, forward_paged_attention).
 *
 *   q             [num_seqs, num_heads, head_dim] bf16, one query token per sequence
 *   kv_cache      [2, num_blocks, block_size, num_kv_heads, head_dim] bf16;
 *                 [0] = K, [1] = V
 *   block_tables  [num_seqs, max_blocks_per_seq] int32 physical block ids;
 *                 token t of sequence b lives in block block_tables[b][t / block_size]
 *                 at offset t % block_size. Entries at or past
 *                 ceil(context_lens[b] / block_size) are never read.
 *   context_lens  [num_seqs] int32, 0 <= len <= max_blocks_per_seq * block_size
 *                 (the cache already holds the new token: the query attends all
 *                 context_lens[b] keys). len 0 gives O = 0, LSE = -inf.
 *   max_context_len (host) >= every context_lens[b].
 *   block_size    must be 128.
 *   out           [num_seqs, num_heads, head_dim] bf16
 *   lse           nullable; [num_heads, num_seqs] fp32
 *   workspace     device buffer of at least attn_paged_decode_workspace_size()
 *                 bytes (token prefix sums and partials; contents on return
 *                 are unspecified).
 * The contexts of all sequences, end to end, are cut into equal segments, one
 * per wave, whatever the mix of lengths; a sequence that spans segments has its
 * partial (O, LSE) pairs merged in ascending segment order by a second kernel,
 * so the result is deterministic.
 * num_seqs == 0 is a no-op.
 */
attn_status_t attn_paged_decode(const void* q, const void* kv_cache,
                                const int32_t* block_tables, const int32_t* context_lens,
                                int32_t num_seqs, int32_t num_blocks, int32_t max_blocks_per_seq,
                                int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, float softmax_scale,
                                void* out, float* lse, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * Single-token decode with a sliding window (vLLM-Ascend attention_v1.py page:
 * AscendAttentionBackendImpl._forward_fia_slidingwindow, the decode-only route
 * of a layer with a sliding window, which hands the window to the fused kernel
 * as pre_tokens). The query of sequence b sits at position L - 1
 * (L = context_lens[b]) and sees keys t with L - 1 - window <= t <= L - 1:
 * the window counts the tokens before the query that stay visible.
 *
 * Arguments as for attn_paged_decode, plus
 *   window        (host) >= 0; window >= max_context_len - 1 is plain decode.
 * The workspace is the one attn_paged_decode_workspace_size() reports for the
 * same sizes. Errors: window < 0 gives ATTN_ERR_INVALID_ARG; otherwise as for
 * attn_paged_decode.
 */
attn_status_t attn_paged_decode_sliding_window(const void* q, const void* kv_cache,
                                               const int32_t* block_tables, const int32_t* context_lens,
                                               int32_t num_seqs, int32_t num_blocks, int32_t max_blocks_per_seq,
                                               int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads,
                                               int32_t head_dim, int32_t block_size, int32_t window,
                                               float softmax_scale, void* out, float* lse, void* workspace,
                                               size_t workspace_bytes, void* stream);

/* Bytes of the device scratch array behind attn_paged_decode_scratch (per GPU). */
#define ATTN_DECODE_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * attn_paged_decode without a workspace, for callers that cannot allocate
 * device memory or pass one in: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation. Arguments, layouts and results are
 * those of attn_paged_decode minus workspace / workspace_bytes; the call
 * allocates nothing.
 *
 * The workspace of attn_paged_decode (token prefix sums and partials) lives in
 * the library's own device array of ATTN_DECODE_SCRATCH_BYTES, one per GPU,
 * which stays allocated from the first use until the process ends. A call
 * whose workspace (attn_paged_decode_workspace_size) exceeds the array
 * returns ATTN_ERR_WORKSPACE_TOO_SMALL before any HIP call (about 1900
 * sequences at 32/8 heads and head_dim 128). Nothing in the array needs
 * clearing: every call writes each partial before it reads it.
 * Every call on one GPU shares that GPU's array and leaves its partials there,
 * so calls that overlap on one GPU (other streams, other host threads) race:
 * issue them in order on one stream. The first call on each device looks the
 * array's device address up in the HIP runtime (no allocation) and caches it;
 * a failed lookup returns ATTN_ERR_LAUNCH. The result equals
 * attn_paged_decode's bit for bit.
 */
attn_status_t attn_paged_decode_scratch(const void* q, const void* kv_cache,
                                        const int32_t* block_tables, const int32_t* context_lens,
                                        int32_t num_seqs, int32_t num_blocks, int32_t max_blocks_per_seq,
                                        int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size, float softmax_scale,
                                        void* out, float* lse, void* stream);

/*
 * Workspace bytes attn_padded_fwd needs (two int32 arrays of batch + 1).
 */
attn_status_t attn_padded_fwd_workspace_size(int32_t batch, size_t* bytes);

/*
 * Attention over the valid prefix of each entry of a padded batch (vLLM-Omni
 * fastvideo_vsa.py page: FastVideoVSAImpl._fallback and forward_cuda with
 * packed_padding: the first q_length query rows and kv_length key rows are
 * real, attention runs on those prefixes and the output rows past q_length are
 * zero).
 *
 *   q             [batch, seqlen_q, num_heads, head_dim] bf16
 *   k, v          [batch, seqlen_k, num_kv_heads, head_dim] bf16
 *   q_lens        [batch] int32 (device), 0 <= q_lens[b] <= seqlen_q (clamped)
 *   k_lens        [batch] int32 (device), 0 <= k_lens[b] <= seqlen_k (clamped)
 *   causal        bottom-right on (q_lens[b], k_lens[b]), as attn_varlen_fwd
 *   out           [batch, seqlen_q, num_heads, head_dim] bf16; rows at or past
 *                 q_lens[b] are written as zeros
 *   lse           nullable; [num_heads, batch * seqlen_q] fp32, -inf on pad rows
 *                 and on rows that see no key
 *   workspace     >= attn_padded_fwd_workspace_size() bytes
 * The contents of pad rows of q, k and v are never read into the result.
 * batch == 0 or seqlen_q == 0 is a no-op. Errors: negative sizes, a bad
 * scale or null pointers give ATTN_ERR_INVALID_ARG; an unsupported head_dim
 * or head ratio ATTN_ERR_UNSUPPORTED; a short workspace
 * ATTN_ERR_WORKSPACE_TOO_SMALL.
 */
attn_status_t attn_padded_fwd(const void* q, const void* k, const void* v, const int32_t* q_lens,
                              const int32_t* k_lens, int32_t batch, int32_t seqlen_q, int32_t seqlen_k,
                              int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, float softmax_scale,
                              int32_t causal, void* out, float* lse, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * Workspace bytes attn_masked_fwd needs: packed copies of k and v (and of q and
 * the output when mask_queries is set) plus the per-entry index arrays.
 */
attn_status_t attn_masked_fwd_workspace_size(int32_t batch, int32_t seqlen_q, int32_t seqlen_k,
                                             int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                             int32_t mask_queries, size_t* bytes);

/*
 * Attention under a 2-D key-padding mask (vLLM-Omni flash_attn.py page:
 * FlashAttentionImpl._forward_varlen_masked, which unpads by the mask, runs
 * varlen attention and pads the result back).
 *
 *   q             [batch, seqlen_q, num_heads, head_dim] bf16
 *   k, v          [batch, seqlen_k, num_kv_heads, head_dim] bf16
 *   key_mask      [batch, seqlen_k] uint8 (device), nonzero = real token
 *   mask_queries  nonzero: self-attention, the mask also selects the query rows
 *                 (needs seqlen_q == seqlen_k); the real tokens of an entry, in
 *                 order, form one document and padding rows come back as
 *                 zeros. Zero: cross-attention, the mask covers keys only and
 *                 every query row attends the real keys of its entry.
 *   causal        bottom-right on the real-token counts, as attn_varlen_fwd
 *   out           [batch, seqlen_q, num_heads, head_dim] bf16
 *   lse           nullable; [num_heads, batch * seqlen_q] fp32, -inf on
 *                 padding rows and on rows that see no key
 *   workspace     >= attn_masked_fwd_workspace_size() bytes (same mask_queries)
 * batch == 0 or seqlen_q == 0 is a no-op. Errors as for attn_padded_fwd, and
 * mask_queries with seqlen_q != seqlen_k gives ATTN_ERR_INVALID_ARG.
 */
attn_status_t attn_masked_fwd(const void* q, const void* k, const void* v, const uint8_t* key_mask,
                              int32_t batch, int32_t seqlen_q, int32_t seqlen_k, int32_t num_heads,
                              int32_t num_kv_heads, int32_t head_dim, float softmax_scale, int32_t causal,
                              int32_t mask_queries, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * Paged KV cache write (vLLM-Ascend attention_v1.py page:
 * AscendAttentionImpl.reshape_and_cache with AscendMetadata.slot_mapping).
 * New token i's K and V rows are stored at cache slot slot_mapping[i]: block
 * slot / block_size, offset slot % block_size, in both planes.
 *
 *   k, v          [num_tokens, num_kv_heads, head_dim] bf16
 *   slot_mapping  [num_tokens] int32; a negative slot (a padding token) or one
 *                 at or past num_blocks * block_size is skipped. Slots must be
 *                 unique (two tokens writing one slot race).
 *   kv_cache      [2, num_blocks, block_size, num_kv_heads, head_dim] bf16,
 *                 written in place (only the named slots change)
 *   block_size    must be 128.
 * num_tokens == 0 is a no-op.
 */
attn_status_t attn_paged_kv_write(const void* k, const void* v, const int32_t* slot_mapping,
                                  int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t num_blocks, int32_t block_size, void* kv_cache, void* stream);

/*
 * Multi-token attention over a paged KV cache: prefix-cache-hit prefill,
 * chunked prefill and speculative decoding (vLLM-Ascend attention_v1.py page:
 * AscendAttentionState and _get_fia_params, which read keys and values from
 * the paged cache through block_table with actual_seq_lengths_kv = seq_lens and
 * take the queries packed by cumulative query lengths). The cache already
 * holds each sequence's new tokens (reshape_and_cache runs first), so the
 * Lq = cu_seqlens_q[b+1] - cu_seqlens_q[b] queries of sequence b are its last
 * Lq positions among Lk = context_lens[b] keys, with bottom-right causal
 * masking: key j is visible to query i iff j <= i + Lk - Lq. A query that sees
 * no key gets O = 0, LSE = -inf.
 *
 *   q             [total_q, num_heads, head_dim] bf16, packed by cu_seqlens_q
 *   kv_cache      [2, num_blocks, block_size, num_kv_heads, head_dim] bf16
 *   block_tables  [batch, max_blocks_per_seq] int32, as for attn_paged_decode
 *   cu_seqlens_q  [batch + 1] int32, leading 0, non-decreasing
 *   context_lens  [batch] int32 keys per sequence (new tokens included),
 *                 0 <= len <= max_context_len
 *   max_seqlen_q, max_context_len (host) bound the lengths; they size the grid.
 *   block_size    must be 128.
 *   out           [total_q, num_heads, head_dim] bf16
 *   lse           nullable; [num_heads, total_q] fp32
 *   workspace     device buffer of at least attn_paged_prefill_workspace_size()
 *                 bytes (nullable when that is 0). Short query runs (speculative
 *                 decoding: max_seqlen_q * num_heads/num_kv_heads <= 64)
 *                 stream the cache once per kv head like decode and keep fp32
 *                 partials there; longer ones need none.
 * batch == 0 or total_q == 0 is a no-op.
 */
attn_status_t attn_paged_prefill(const void* q, const void* kv_cache, const int32_t* block_tables,
                                 const int32_t* cu_seqlens_q, const int32_t* context_lens,
                                 int32_t batch, int32_t total_q, int32_t max_seqlen_q,
                                 int32_t max_context_len, int32_t num_blocks, int32_t max_blocks_per_seq,
                                 int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, float softmax_scale, void* out, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes that attn_paged_prefill needs for these host sizes (0 when
 * the call runs the prefill kernels). Written to *bytes (host pointer). */
attn_status_t attn_paged_prefill_workspace_size(int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                                int32_t head_dim, int32_t max_seqlen_q,
                                                int32_t max_context_len, size_t* bytes);

/*
 * Block map -> ascending index lists (vLLM-Omni fastvideo_vsa.py page: the
 * native route converts the boolean block map with map_to_index into per-row
 * kept key-tile indices and counts).
 *
 *   block_map [rows, n_cols] uint8, nonzero = keep
 *   idx       [rows, n_cols] int32: row r's kept columns in ascending order in
 *             idx[r][0 .. num[r]-1]; entries past num[r] are left untouched
 *   num       [rows] int32
 * Bit-exact. rows == 0 is a no-op.
 */
attn_status_t attn_block_map_to_index(const uint8_t* block_map, int32_t rows, int32_t n_cols,
                                      int32_t* idx, int32_t* num, void* stream);

/* Workspace bytes for attn_block_sparse_fwd: the kept-tile index lists it
 * builds, their lengths, and the order in which it runs the query tiles. */
attn_status_t attn_block_sparse_workspace_size(int32_t batch, int32_t num_heads, int32_t num_tiles,
                                               size_t* bytes);

/*
 * 64-token-tile block-sparse attention (vLLM-Omni fastvideo_vsa.py page:
 * _fastvideo_h3_vsa_bhsd_op / block_sparse_attn with block_map and
 * variable_block_sizes; FastVideoVSAImpl._forward_h3 prepares tile order).
 *
 *   q            [batch, num_tiles * 64, num_heads, head_dim]    bf16, tile order
 *   k, v         [batch, num_tiles * 64, num_kv_heads, head_dim] bf16, tile order
 *   block_map    [batch, num_heads, num_tiles, num_tiles] uint8; nonzero = query
 *                tile a attends key tile c
 *   tile_sizes   [num_tiles] int32 in [0, 64]: rows >= tile_sizes[c] of tile c
 *                are padding (neither queries nor keys)
 *   out          [batch, num_tiles * 64, num_heads, head_dim] bf16; padding rows
 *                and rows whose map row is empty are written 0
 *   lse          nullable; [batch, num_heads, num_tiles * 64] fp32 (-inf there)
 *   workspace    >= attn_block_sparse_workspace_size() bytes
 * Non-causal only and Sq == Skv, as the page's VSA preconditions require;
 * the same tile_sizes serve queries and keys.
 */
attn_status_t attn_block_sparse_fwd(const void* q, const void* k, const void* v,
                                    const uint8_t* block_map, const int32_t* tile_sizes,
                                    int32_t batch, int32_t num_tiles, int32_t num_heads,
                                    int32_t num_kv_heads, int32_t head_dim, float softmax_scale,
                                    void* out, float* lse, void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * Raster -> padded tile order (vLLM-Omni fastvideo_vsa.py page:
 * _get_tile_partition_indices, _construct_variable_block_sizes,
 * _get_non_pad_index; FastVideoVSAImpl._forward_h3 gathers q/k/v this way).
 * A raster (t, h, w) latent is cut into (tile_t, tile_h, tile_w) boxes,
 * enumerated t-box slowest, then h, then w, tokens inside a box in raster
 * order, edge boxes clipped; box c owns rows [64c, 64c + 64).
 *   x          [batch, t*h*w, row_elems] bf16 in raster order
 *              (row_elems = heads * head_dim, a multiple of 8)
 *   x_tiled    [batch, num_tiles * 64, row_elems] bf16; rows past a box's size
 *              are written 0
 *   tile_sizes nullable; [num_tiles] int32, real rows of each box
 * num_tiles = ceil(t/tile_t) * ceil(h/tile_h) * ceil(w/tile_w);
 * tile_t * tile_h * tile_w must be <= 64. Pure data movement (bit-exact).
 */
attn_status_t attn_vsa_tile_gather(const void* x, int32_t batch, int32_t t, int32_t h, int32_t w, int32_t tile_t,
                                   int32_t tile_h, int32_t tile_w, int32_t row_elems, void* x_tiled,
                                   int32_t* tile_sizes, void* stream);

/* Inverse of attn_vsa_tile_gather: padded tile order -> raster order (the
 * page's untile gather, non_pad[argsort(partition)]). Padding rows are
 * dropped. Same argument meaning; x [batch, t*h*w, row_elems] is written. */
attn_status_t attn_vsa_untile(const void* x_tiled, int32_t batch, int32_t t, int32_t h, int32_t w, int32_t tile_t,
                              int32_t tile_h, int32_t tile_w, int32_t row_elems, void* x, void* stream);

/* Workspace bytes for attn_vsa_block_map (fp32 tile means of q and k). */
attn_status_t attn_vsa_block_map_workspace_size(int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                                int32_t num_tiles, int32_t head_dim, size_t* bytes);

/*
 * Per-query-tile top-k block map from tile means (vLLM-Omni fastvideo_vsa.py
 * page: _pool_h3_tiles, the pooled score matmul and _build_h3_block_map in
 * FastVideoVSAImpl._forward_h3).
 *   q_tiled     [batch, num_tiles * 64, num_heads, head_dim] bf16 tile order
 *   k_tiled     [batch, num_tiles * 64, num_kv_heads, head_dim] bf16 tile order
 *   tile_sizes  [num_tiles] int32 in [0, 64]
 *   block_map   [batch, num_heads, num_tiles, num_tiles] uint8 (1 = keep)
 * Each tile's mean is taken in fp32 over its real rows (divided by
 * max(size, 1)); score[a][c] = scale * qmean_a . kmean_c in fp32; row a keeps
 * the min(topk, num_tiles) largest scores, a tie going to the lower tile index;
 * topk >= num_tiles keeps every tile. num_tiles <= 16384, topk >= 1.
 */
attn_status_t attn_vsa_block_map(const void* q_tiled, const void* k_tiled, const int32_t* tile_sizes,
                                 int32_t batch, int32_t num_tiles, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, float softmax_scale, int32_t topk, uint8_t* block_map,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * H3 layout (vLLM-Omni fastvideo_vsa.py page: _get_h3_tile_metadata): prefix
 * rows (the segments before the target video, e.g. text and reference frames)
 * come first, each segment cut into 64-row tiles with its remainder as a last,
 * partial tile; the video's (tile_t, tile_h, tile_w) boxes follow (the page
 * uses (4, 4, 4)). The raster input holds the prefix rows, then the video in
 * (t, h, w) raster order.
 *
 *   prefix_segments  (host) int32 [num_segments] row counts >= 0 (empty segments
 *                    add no tile); num_segments <= 16
 *   num_prefix_tiles, num_tiles (host outputs of attn_vsa_h3_num_tiles)
 * Tile gather / untile: as attn_vsa_tile_gather / attn_vsa_untile with
 *   x  [batch, prefix rows + t*h*w, row_elems] bf16 raster
 *   x_tiled [batch, num_tiles * 64, row_elems], tile_sizes [num_tiles] int32
 *   (nullable), prefix tiles first.
 * Errors: more than 16 segments gives ATTN_ERR_UNSUPPORTED; a negative segment
 * or a null prefix_segments with num_segments > 0 ATTN_ERR_INVALID_ARG;
 * otherwise as for the video-only calls.
 */
attn_status_t attn_vsa_h3_num_tiles(const int32_t* prefix_segments, int32_t num_segments, int32_t t, int32_t h,
                                    int32_t w, int32_t tile_t, int32_t tile_h, int32_t tile_w,
                                    int32_t* num_prefix_tiles, int32_t* num_tiles);
attn_status_t attn_vsa_h3_tile_gather(const void* x, const int32_t* prefix_segments, int32_t num_segments,
                                      int32_t batch, int32_t t, int32_t h, int32_t w, int32_t tile_t,
                                      int32_t tile_h, int32_t tile_w, int32_t row_elems, void* x_tiled,
                                      int32_t* tile_sizes, void* stream);
attn_status_t attn_vsa_h3_untile(const void* x_tiled, const int32_t* prefix_segments, int32_t num_segments,
                                 int32_t batch, int32_t t, int32_t h, int32_t w, int32_t tile_t, int32_t tile_h,
                                 int32_t tile_w, int32_t row_elems, void* x, void* stream);

/*
 * H3 block map (vLLM-Omni fastvideo_vsa.py page: _build_h3_block_map): as
 * attn_vsa_block_map, except that the first num_prefix_tiles tiles are prefix
 * tiles: prefix query tiles keep every key tile, every query tile keeps the
 * prefix key tiles, and a video query tile keeps min(topk, video tiles) video
 * key tiles by pooled score (ties: lower tile index). When that is every video
 * tile the map is all ones. Workspace: attn_vsa_block_map_workspace_size().
 * Errors: num_prefix_tiles outside [0, num_tiles] gives ATTN_ERR_INVALID_ARG;
 * otherwise as attn_vsa_block_map.
 */
attn_status_t attn_vsa_h3_block_map(const void* q_tiled, const void* k_tiled, const int32_t* tile_sizes,
                                    int32_t batch, int32_t num_tiles, int32_t num_prefix_tiles, int32_t num_heads,
                                    int32_t num_kv_heads, int32_t head_dim, float softmax_scale, int32_t topk,
                                    uint8_t* block_map, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Tile gather and block map in one call (vLLM-Omni fastvideo_vsa.py page:
 * _get_tile_partition_indices and the tile gather, then _pool_h3_tiles, the
 * pooled score matmul and _build_h3_block_map). Raster q and k go to tile
 * order exactly as attn_vsa_h3_tile_gather writes them, and the map equals
 * attn_vsa_h3_block_map's on those copies, bit for bit: the tile means are
 * summed in the same fp32 order while the rows are copied, so the copies are
 * not read back. num_segments == 0 is the plain video layout
 * (attn_vsa_tile_gather + attn_vsa_block_map).
 *   q           [batch, prefix rows + t*h*w, num_heads, head_dim] bf16 raster
 *   k           [batch, prefix rows + t*h*w, num_kv_heads, head_dim] bf16 raster
 *   q_tiled     [batch, num_tiles * 64, num_heads, head_dim] bf16, written
 *   k_tiled     [batch, num_tiles * 64, num_kv_heads, head_dim] bf16, written
 *   tile_sizes  [num_tiles] int32, written (nullable)
 *   block_map   [batch, num_heads, num_tiles, num_tiles] uint8, written
 *   workspace   >= attn_vsa_block_map_workspace_size() bytes for num_tiles
 *               (attn_vsa_h3_num_tiles gives num_tiles)
 * batch == 0 or num_tiles == 0 is a no-op. Errors: as attn_vsa_h3_tile_gather
 * (with row_elems = num_heads * head_dim) and attn_vsa_h3_block_map.
 */
attn_status_t attn_vsa_h3_gather_block_map(const void* q, const void* k, const int32_t* prefix_segments,
                                           int32_t num_segments, int32_t batch, int32_t t, int32_t h, int32_t w,
                                           int32_t tile_t, int32_t tile_h, int32_t tile_w, int32_t num_heads,
                                           int32_t num_kv_heads, int32_t head_dim, float softmax_scale, int32_t topk,
                                           void* q_tiled, void* k_tiled, int32_t* tile_sizes, uint8_t* block_map,
                                           void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for attn_vsa_compressed_add (fp32 tile means of q, k, v and
 * the per-tile compressed rows). Written to *bytes (host pointer). */
attn_status_t attn_vsa_compressed_workspace_size(int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                                 int32_t num_tiles, int32_t head_dim, size_t* bytes);

/*
 * VSA compressed branch (vLLM-Omni fastvideo_vsa.py page:
 * FastVideoVSAImpl._forward_h3, the gate branch): with the fp32 tile means of
 * q, k and v (as attn_vsa_block_map pools them) and the pooled scores
 * S = softmax_scale * qbar kbar^T, each query tile a gets
 * c_a = softmax(S[a, :]) @ vbar over all key tiles, and every row r of the
 * tile adds c_a * gate: out[b][64a + r][h][:] += c_a[:] * gate[b][64a + r][h][:]
 * (computed in fp32, rounded to bf16 once). The page's gate is zero on padding
 * rows, which then stay unchanged.
 *
 *   q_tiled     [batch, num_tiles * 64, num_heads, head_dim] bf16, tile order
 *   k/v_tiled   [batch, num_tiles * 64, num_kv_heads, head_dim] bf16
 *   tile_sizes  [num_tiles] int32 in [0, 64]
 *   gate_tiled  like q_tiled (the gate in tile order)
 *   out         like q_tiled, updated in place (the block-sparse output)
 *   workspace   >= attn_vsa_compressed_workspace_size() bytes
 * batch == 0 or num_tiles == 0 is a no-op.
 */
attn_status_t attn_vsa_compressed_add(const void* q_tiled, const void* k_tiled, const void* v_tiled,
                                      const int32_t* tile_sizes, const void* gate_tiled, int32_t batch,
                                      int32_t num_tiles, int32_t num_heads, int32_t num_kv_heads,
                                      int32_t head_dim, float softmax_scale, void* out, void* workspace,
                                      size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_H */
