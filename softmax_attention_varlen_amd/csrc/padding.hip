// Padded batches and key-padding masks, around the varlen attention kernels.
//
// Padded batch ([VSA] FastVideoVSAImpl._fallback / forward_cuda with packed
// padding): q [B][Sq][Hq][D] and k, v [B][Sk][Hkv][D] hold a valid prefix of
// q_lens[b] / k_lens[b] rows per batch entry. Batch entry b becomes varlen
// document b with rows [b*Sq, (b+1)*Sq) cut to its valid prefix (the kernels'
// used-length arguments), and the rows past the prefix are written as zeros
// with LSE = -inf.
//
// Key-padding mask ([FA] FlashAttentionImpl._forward_varlen_masked): mask
// [B][Sk], nonzero = real token. Each batch entry's real tokens are packed,
// in order, to the front of its own slot of a workspace copy (one workgroup
// per entry ranks them with wave ballots), which is the padded form above with
// the real-token counts as valid lengths: no global scan and no host read.
// When the mask also selects the queries (self-attention), the packed output
// rows are scattered back to their positions and the other rows are zeros.
//
// Every kernel moves whole rows, one wave per row, 16 bytes per lane.
#include "attn_common.hpp"
#include "launch.hpp"

namespace attn {
namespace {

// The strided document bounds of a padded batch: cu_q[b] = b * seqlen_q,
// cu_k[b] = b * seqlen_k for b = 0..batch (written by the first threads of the
// kernels below, ahead of the attention launch on the same stream).
__device__ __forceinline__ void write_strided_cu(long t, int32_t* cu_q, int32_t* cu_k, int batch, int seqlen_q,
                                                 int seqlen_k) {
  if (t <= batch) {
    cu_q[t] = (int32_t)(t * seqlen_q);
    cu_k[t] = (int32_t)(t * seqlen_k);
  }
}

__device__ __forceinline__ void zero_row(uint16_t* row, int elems, int lane) {
  for (int e = lane * 8; e < elems; e += 64 * 8) *reinterpret_cast<u32x4*>(row + e) = u32x4{0u, 0u, 0u, 0u};
}

__device__ __forceinline__ void copy_row(const uint16_t* src, uint16_t* dst, int elems, int lane) {
  for (int e = lane * 8; e < elems; e += 64 * 8) *reinterpret_cast<u32x4*>(dst + e) = ld_global16(src + e);
}

// Rows at or past the valid prefix of their batch entry (every row when used
// is null): zero output and LSE = -inf (LSE layout [Hq][batch * seqlen]).
__global__ __launch_bounds__(256) void pad_rows_kernel(const int32_t* __restrict__ used, int batch, int seqlen,
                                                       int hq, int head_dim, uint16_t* __restrict__ out,
                                                       float* __restrict__ lse, int32_t* __restrict__ cu_q,
                                                       int32_t* __restrict__ cu_k, int seqlen_k) {
  write_strided_cu((long)blockIdx.x * 256 + threadIdx.x, cu_q, cu_k, batch, seqlen, seqlen_k);
  const int lane = threadIdx.x & 63;
  const long rows = (long)batch * seqlen;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int b = (int)(row / seqlen), i = (int)(row % seqlen);
  if (used != nullptr && i < clampi(used[b], 0, seqlen)) return;
  zero_row(out + row * hq * head_dim, hq * head_dim, lane);
  if (lse != nullptr) {
    for (int h = lane; h < hq; h += 64) lse[(long)h * rows + row] = kNegInf;
  }
}

// One workgroup per batch entry: idx[b*s + j] = position of the j-th real
// token (j < count[b]), inv[b*s + p] = rank of position p among the real
// tokens or -1.
__global__ __launch_bounds__(256) void mask_compact_kernel(const uint8_t* __restrict__ mask, int s,
                                                           int32_t* __restrict__ idx, int32_t* __restrict__ inv,
                                                           int32_t* __restrict__ count, int32_t* __restrict__ cu_q,
                                                           int32_t* __restrict__ cu_k, int batch, int seqlen_q) {
  __shared__ int wave_count[4];
  const long b = blockIdx.x;
  if (threadIdx.x == 0) write_strided_cu(b, cu_q, cu_k, batch, seqlen_q, s);
  if (threadIdx.x == 1 && b + 1 == batch) write_strided_cu(batch, cu_q, cu_k, batch, seqlen_q, s);
  const uint8_t* m = mask + b * s;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int carry = 0;  // real tokens before this pass (the same in every thread)
  for (int base = 0; base < s; base += 256) {
    const int p = base + tid;
    const bool keep = p < s && m[p] != 0;
    const unsigned long long bal = __ballot(keep);
    const int before = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (lane == 0) wave_count[w] = __popcll(bal);
    __syncthreads();
    int rank = carry + before;
    for (int i = 0; i < w; ++i) rank += wave_count[i];
    if (p < s) {
      inv[b * s + p] = keep ? rank : -1;
      if (keep) idx[b * s + rank] = p;
    }
    carry += wave_count[0] + wave_count[1] + wave_count[2] + wave_count[3];
    __syncthreads();
  }
  if (tid == 0) count[b] = carry;
}

// dst row b*s + j = src row b*s + idx[b*s + j] for j < count[b]; blockIdx.y
// picks the (src, dst) pair, so k and v move in one launch.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ src0,
                                                          const uint16_t* __restrict__ src1,
                                                          const int32_t* __restrict__ idx,
                                                          const int32_t* __restrict__ count, int batch, int s,
                                                          int row_elems, uint16_t* __restrict__ dst0,
                                                          uint16_t* __restrict__ dst1) {
  const uint16_t* src = blockIdx.y == 0 ? src0 : src1;
  uint16_t* dst = blockIdx.y == 0 ? dst0 : dst1;
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long)batch * s) return;
  const int b = (int)(row / s), j = (int)(row % s);
  if (j >= clampi(count[b], 0, s)) return;
  const int p = clampi(idx[row], 0, s - 1);
  copy_row(src + ((long)b * s + p) * row_elems, dst + row * row_elems, row_elems, lane);
}

// out row b*s + p = packed row b*s + inv[b*s + p] (its LSE too), or zeros and
// LSE = -inf where inv < 0.
__global__ __launch_bounds__(256) void scatter_rows_kernel(const uint16_t* __restrict__ src,
                                                           const float* __restrict__ lse_src,
                                                           const int32_t* __restrict__ inv, int batch, int s, int hq,
                                                           int head_dim, uint16_t* __restrict__ out,
                                                           float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const long rows = (long)batch * s;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int b = (int)(row / s);
  const int j = inv[row] < s ? inv[row] : -1;
  const int elems = hq * head_dim;
  if (j < 0) {
    zero_row(out + row * elems, elems, lane);
  } else {
    copy_row(src + ((long)b * s + j) * elems, out + row * elems, elems, lane);
  }
  if (lse != nullptr) {
    for (int h = lane; h < hq; h += 64) lse[(long)h * rows + row] = j < 0 ? kNegInf : lse_src[(long)h * rows + (long)b * s + j];
  }
}

unsigned row_grid(long rows) { return (unsigned)((rows + 3) / 4); }

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

}  // namespace

size_t padded_workspace_bytes(int batch) { return 2 * align256((size_t)(batch + 1) * sizeof(int32_t)); }

hipError_t launch_padded_fwd(const VarlenArgs& base, const int32_t* q_lens, const int32_t* k_lens, int seqlen_q,
                             int seqlen_k, void* workspace, hipStream_t stream) {
  int32_t* cu_q = (int32_t*)workspace;
  int32_t* cu_k = (int32_t*)((char*)workspace + align256((size_t)(base.batch + 1) * sizeof(int32_t)));
  hipLaunchKernelGGL(pad_rows_kernel, dim3(row_grid((long)base.batch * seqlen_q)), dim3(256), 0, stream, q_lens,
                     base.batch, seqlen_q, base.num_heads, base.head_dim, (uint16_t*)base.out, base.lse, cu_q, cu_k,
                     seqlen_k);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || q_lens == nullptr) return e;  // no valid prefix: padding rows only
  VarlenArgs a = base;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.total_q = base.batch * seqlen_q;
  a.total_k = base.batch * seqlen_k;
  a.max_seqlen_q = seqlen_q;
  a.max_seqlen_k = seqlen_k;
  a.q_used = q_lens;
  a.k_used = k_lens;
  return launch_varlen_fwd(a, stream);
}

MaskedLayout plan_masked(int batch, int seqlen_q, int seqlen_k, int num_heads, int num_kv_heads, int head_dim,
                         bool mask_queries) {
  MaskedLayout l{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  const size_t rows_k = (size_t)batch * seqlen_k, rows_q = (size_t)batch * seqlen_q;
  l.cu_q = take((size_t)(batch + 1) * sizeof(int32_t));
  l.cu_k = take((size_t)(batch + 1) * sizeof(int32_t));
  l.count = take((size_t)batch * sizeof(int32_t));
  l.idx = take(rows_k * sizeof(int32_t));
  l.inv = take(rows_k * sizeof(int32_t));
  l.k = take(rows_k * num_kv_heads * head_dim * 2);
  l.v = take(rows_k * num_kv_heads * head_dim * 2);
  if (mask_queries) {
    l.q = take(rows_q * num_heads * head_dim * 2);
    l.o = take(rows_q * num_heads * head_dim * 2);
    l.lse = take(rows_q * num_heads * sizeof(float));
  }
  l.bytes = off;
  return l;
}

hipError_t launch_masked_fwd(const VarlenArgs& base, const uint8_t* key_mask, int seqlen_q, int seqlen_k,
                             bool mask_queries, const MaskedLayout& l, void* workspace, hipStream_t stream) {
  char* ws = (char*)workspace;
  int32_t* cu_q = (int32_t*)(ws + l.cu_q);
  int32_t* cu_k = (int32_t*)(ws + l.cu_k);
  int32_t* count = (int32_t*)(ws + l.count);
  int32_t* idx = (int32_t*)(ws + l.idx);
  int32_t* inv = (int32_t*)(ws + l.inv);
  uint16_t* kc = (uint16_t*)(ws + l.k);
  uint16_t* vc = (uint16_t*)(ws + l.v);
  const int batch = base.batch;
  const int kv_elems = base.num_kv_heads * base.head_dim, q_elems = base.num_heads * base.head_dim;
  hipLaunchKernelGGL(mask_compact_kernel, dim3((unsigned)batch), dim3(256), 0, stream, key_mask, seqlen_k, idx, inv,
                     count, cu_q, cu_k, batch, seqlen_q);
  hipLaunchKernelGGL(gather_rows_kernel, dim3(row_grid((long)batch * seqlen_k), 2), dim3(256), 0, stream,
                     (const uint16_t*)base.k, (const uint16_t*)base.v, idx, count, batch, seqlen_k, kv_elems, kc, vc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  VarlenArgs a = base;
  a.k = kc;
  a.v = vc;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.total_q = batch * seqlen_q;
  a.total_k = batch * seqlen_k;
  a.max_seqlen_q = seqlen_q;
  a.max_seqlen_k = seqlen_k;
  a.k_used = count;
  if (!mask_queries) return launch_varlen_fwd(a, stream);  // every query row is real
  uint16_t* qc = (uint16_t*)(ws + l.q);
  uint16_t* oc = (uint16_t*)(ws + l.o);
  float* lc = (float*)(ws + l.lse);
  hipLaunchKernelGGL(gather_rows_kernel, dim3(row_grid((long)batch * seqlen_q), 1), dim3(256), 0, stream,
                     (const uint16_t*)base.q, (const uint16_t*)base.q, idx, count, batch, seqlen_q, q_elems, qc, qc);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  a.q = qc;
  a.out = oc;
  a.lse = base.lse != nullptr ? lc : nullptr;
  a.q_used = count;
  e = launch_varlen_fwd(a, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scatter_rows_kernel, dim3(row_grid((long)batch * seqlen_q)), dim3(256), 0, stream, oc, lc, inv,
                     batch, seqlen_q, base.num_heads, base.head_dim, (uint16_t*)base.out, base.lse);
  return hipGetLastError();
}

}  // namespace attn
