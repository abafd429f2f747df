// Packed variable-length attention prefill for gfx950, register-staged: it
// serves head_dim 64 under the causal mask (every other call takes the
// pipelined kernels of prefill_pipe.hip, which measured faster there).
//
// Work unit: one workgroup of 4 waves owns a 128-row query tile of one
// document and one query head; each wave owns 32 query rows. K/V tiles of 64
// keys are staged through LDS (K row-major, V transposed) and the wave runs
//   S^T = K Q^T   (32x32x16 bf16 MFMA, fp32 accumulate)
//   online softmax in registers (row reductions in-lane + one lane exchange)
//   O^T += V^T P^T (32x32x16 bf16 MFMA, P rounded to bf16)
// Causal masking is bottom-right aligned (key j allowed for query i iff
// j <= i + Lk - Lq) and applied only on tiles that straddle the diagonal or the
// document end; tiles wholly above the diagonal are never loaded.
#include "attn_common.hpp"
#include "key_rows.hpp"
#include "launch.hpp"

namespace attn {

constexpr int kVarlenBM = 128;
constexpr int kVarlenBN = 64;
constexpr int kVarlenThreads = 256;

// PAGED: keys come from a paged cache (k, v = its K and V planes) through
// block_tables, with context_lens[doc] (clamped to max_len_k) keys per
// document; otherwise from contiguous rows delimited by cu_k. q_used / k_used
// (nullable) cut each document to a valid prefix of its rows.
template <int D, bool CAUSAL, bool PAGED>
__global__ __launch_bounds__(kVarlenThreads, (D <= 128 ? 2 : 1)) void varlen_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch, int total_q, int total_k,
    int tiles_per_doc, int hq, int hkv, float c, uint16_t* __restrict__ out, float* __restrict__ lse,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens, int max_blocks_per_seq,
    int num_blocks, int max_len_k, const int32_t* __restrict__ q_used, const int32_t* __restrict__ k_used) {
  using Tile = KVTile<D, kVarlenBN, kVarlenThreads>;
  __shared__ __attribute__((aligned(16))) char smem[Tile::BYTES];

  // heads fastest, then documents, then query tiles from the last (heaviest
  // under causal masking) to the first
  const int id = blockIdx.x;
  const int h = id % hq;
  const int y = id / hq;
  const int doc = y % batch;
  const int tile = tiles_per_doc - 1 - y / batch;

  const int q0 = clampi(cu_q[doc], 0, total_q);
  int q1 = clampi(cu_q[doc + 1], q0, total_q);
  if (q_used != nullptr) q1 = q0 + clampi(q_used[doc], 0, q1 - q0);  // valid prefix of the slot
  int k0 = 0, len_k;
  if (PAGED) {
    len_k = clampi(context_lens[doc], 0, max_len_k);
  } else {
    k0 = clampi(cu_k[doc], 0, total_k);
    len_k = clampi(cu_k[doc + 1], k0, total_k) - k0;
    if (k_used != nullptr) len_k = clampi(k_used[doc], 0, len_k);
  }
  const int len_q = q1 - q0;
  const int m0 = tile * kVarlenBM;
  if (m0 >= len_q) return;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, n = lane & 31;
  const int hk = h / (hq / hkv);
  const int diag = len_k - len_q;  // key j allowed iff j <= i + diag

  const int row = m0 + w * 32 + n;  // this lane's query row (doc-relative)
  const int row_c = row < len_q ? row : len_q - 1;
  const int wave_row0 = m0 + w * 32;
  const bool wave_live = wave_row0 < len_q;

  WaveRows32<D> st;
  st.init(q + ((long)(q0 + row_c) * hq + h) * D, g);

  int n_end = len_k;
  if (CAUSAL) {
    const int lim = m0 + kVarlenBM + diag;  // exclusive bound over the whole tile
    n_end = lim < n_end ? lim : n_end;
    n_end = n_end < 0 ? 0 : n_end;
  }
  const int ntiles = (n_end + kVarlenBN - 1) / kVarlenBN;
  const long kv_stride = (long)hkv * D;
  const uint16_t* kb0 = k + (long)k0 * kv_stride + hk * D;
  const uint16_t* vb0 = v + (long)k0 * kv_stride + hk * D;
  const KeyRows<PAGED> rows{kv_stride, PAGED ? block_tables + (long)doc * max_blocks_per_seq : nullptr, num_blocks};

  Tile tl;
  if (ntiles > 0) tl.load(kb0 + rows.row(0), vb0 + rows.row(0), kv_stride, len_k, tid);

  for (int j = 0; j < ntiles; ++j) {
    const int n0 = j * kVarlenBN;
    __syncthreads();
    tl.store(smem, tid);
    __syncthreads();
    if (j + 1 < ntiles) {
      const int n1 = n0 + kVarlenBN;
      tl.load(kb0 + rows.row(n1), vb0 + rows.row(n1), kv_stride, len_k - n1, tid);
    }
    // waves whose rows are all past the end or all above this tile's keys skip it
    bool active = wave_live;
    if (CAUSAL) active = active && (n0 <= wave_row0 + 31 + diag);
    if (active) {
      f32x16 s[2];
      st.template scores<Tile::K_STRIDE>(smem, lane, s);
      const bool need_mask =
          (n0 + kVarlenBN > len_k) || (CAUSAL && (n0 + kVarlenBN - 1 > wave_row0 + diag));
      if (need_mask) {
        const int lim = CAUSAL ? row + diag : 0x7fffffff;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = n0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key >= len_k || key > lim) s[kb][r] = kNegInf;
          }
        }
      }
      st.template update<Tile::V_STRIDE>(smem + Tile::K_BYTES, lane, s, c);
    }
  }

  if (row < len_q) {
    float* lp = lse != nullptr ? lse + (long)h * total_q + q0 + row : nullptr;
    st.finish(out + ((long)(q0 + row) * hq + h) * D, lp, lane, c);
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_varlen(const VarlenArgs& a, hipStream_t stream) {
  const int tiles = (a.max_seqlen_q + kVarlenBM - 1) / kVarlenBM;
  const long grid = (long)tiles * a.batch * a.num_heads;
  const float c = a.scale * kLog2e;
  if (a.paged) {
    hipLaunchKernelGGL((varlen_fwd_kernel<D, CAUSAL, true>), dim3((unsigned)grid), dim3(kVarlenThreads), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.cu_q, a.cu_k, a.batch,
                       a.total_q, a.total_k, tiles, a.num_heads, a.num_kv_heads, c, (uint16_t*)a.out, a.lse,
                       a.block_tables, a.context_lens, a.max_blocks_per_seq, a.num_blocks, a.max_seqlen_k, a.q_used,
                       nullptr);
  } else {
    hipLaunchKernelGGL((varlen_fwd_kernel<D, CAUSAL, false>), dim3((unsigned)grid), dim3(kVarlenThreads), 0,
                       stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.cu_q, a.cu_k,
                       a.batch, a.total_q, a.total_k, tiles, a.num_heads, a.num_kv_heads, c, (uint16_t*)a.out,
                       a.lse, nullptr, nullptr, 0, 0, 0, a.q_used, a.k_used);
  }
  return hipGetLastError();
}

hipError_t launch_varlen_fwd(const VarlenArgs& a, hipStream_t stream) {
  if (prefill_pipe_supported(a)) return launch_prefill_pipe(a, stream);
  // what the pipelined kernels leave: head_dim 64 under the causal mask
  if (a.head_dim == 64 && a.causal) return launch_varlen<64, true>(a, stream);
  return hipErrorInvalidValue;
}

long varlen_grid_size(int batch, int max_seqlen_q, int num_heads) {
  const long tiles = (max_seqlen_q + kVarlenBM - 1) / kVarlenBM;
  return tiles * batch * num_heads;
}

}  // namespace attn
