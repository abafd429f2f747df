// Single-token decode over a paged KV cache, split over the context (split-KV),
// for head dims 96 and 192 (head dims 64, 128 and 256 stream balanced
// segments instead: paged_decode_stream.hip).
//
// Cache layout [2][num_blocks][128][num_kv_heads][D] (K plane, then V plane).
// Work item (one wave): (sequence, split, kv head, chunk of <=16 query heads of
// that kv head's group). The wave streams its split 32 tokens at a time, all
// inside one 128-token block, so one block-table entry serves a chunk:
//   S^T[token][qhead] = K Q^T     16x16x32 bf16 MFMA (K rows straight from HBM
//                                  into the A operand: 16 bytes per lane)
//   online softmax in registers
//   O^T[d][qhead]   += V^T P^T    16x16x32 bf16 MFMA (V transposed through a
//                                  wave-private LDS slab)
// The next chunk's K and V are in flight while the current one is computed.
// A split writes a normalised fp32 partial (O_s, LSE_s); a second kernel merges
// the splits of each (sequence, head) in ascending order. A sequence that fits
// in one split writes its final bf16 output directly.
//
// Sliding window: the splits cover the keys from the 32-token chunk holding
// the window's first key to the end; keys below the window are masked.
#include "attn_common.hpp"
#include "launch.hpp"

namespace attn {

constexpr int kDecodeWaves = 4;
constexpr int kDecodeChunk = 32;       // tokens per inner step
constexpr int kDecodeBlock = 128;      // cache block size
// Work items the split plan aims for (at most 64 splits per sequence): each
// wave keeps one 32-token chunk in flight, so the grid needs many waves to
// cover HBM latency. On 64 sequences of 1k-32k tokens, 4096 items (4096-token
// splits) streamed 3.4 TB/s at D=64 and 4.5 at D=256; 32768 items (512-token
// splits) 4.7 and 5.3.
constexpr int kDecodeTargetItems = 32768;

// LDS slot of token t (0..31) in a transposed V row: t = 16a + 4g + r sits at
// 8g + 4a + r, so the 8 tokens one lane feeds into a PV MFMA (4g+{0..3} and
// 16+4g+{0..3}, as the S^T accumulator leaves them) are 8 consecutive slots.
__device__ __forceinline__ int vt_pos_decode(int t) {
  return ((t >> 2) & 3) * 8 + ((t >> 4) & 1) * 4 + (t & 3);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D>
struct DecodeChunk {
  static constexpr int KB = D / 32;                 // 32-wide d blocks of the QK^T contraction
  static constexpr int V_UNITS = (kDecodeChunk / 4) * (D / 8);
  static constexpr int V_PER_LANE = (V_UNITS + 63) / 64;  // (4 tokens x 8 d) units per lane
  u32x4 kr[2][KB];
  u32x4 vr[V_PER_LANE][4];

  // kbase/vbase: element address of token 0 of this chunk (K and V planes, this
  // kv head). n_valid >= 1 tokens are real; later rows re-read the last one.
  __device__ __forceinline__ void load(const uint16_t* kbase, const uint16_t* vbase, long tok_stride,
                                       int n_valid, int lane) {
    const int last = n_valid - 1;
    const int t16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      int t = kb * 16 + t16;
      t = t < last ? t : last;
#pragma unroll
      for (int b = 0; b < KB; ++b) kr[kb][b] = ld_global16(kbase + (long)t * tok_stride + b * 32 + g * 8);
    }
#pragma unroll
    for (int j = 0; j < V_PER_LANE; ++j) {
      const int u = lane + j * 64;
      if (V_UNITS % 64 != 0 && u >= V_UNITS) continue;
      const int tq = u % (kDecodeChunk / 4), ch = u / (kDecodeChunk / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int t = tq * 4 + r;
        t = t < last ? t : last;
        vr[j][r] = ld_global16(vbase + (long)t * tok_stride + ch * 8);
      }
    }
  }

  __device__ __forceinline__ void store_v(char* vt, int lane) const {
    constexpr int VS = kDecodeChunk * 2 + 16;  // bytes per transposed row
#pragma unroll
    for (int j = 0; j < V_PER_LANE; ++j) {
      const int u = lane + j * 64;
      if (V_UNITS % 64 != 0 && u >= V_UNITS) continue;
      const int tq = u % (kDecodeChunk / 4), ch = u / (kDecodeChunk / 4);
      const int pos = vt_pos_decode(tq * 4);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t a0 = vr[j][0][w], a1 = vr[j][1][w], a2 = vr[j][2][w], a3 = vr[j][3][w];
        u32x2 lo, hi;
        lo[0] = (a0 & 0xffffu) | (a1 << 16);
        lo[1] = (a2 & 0xffffu) | (a3 << 16);
        hi[0] = (a0 >> 16) | (a1 & 0xffff0000u);
        hi[1] = (a2 >> 16) | (a3 & 0xffff0000u);
        const int d = ch * 8 + 2 * w;
        *reinterpret_cast<u32x2*>(vt + d * VS + pos * 2) = lo;
        *reinterpret_cast<u32x2*>(vt + (d + 1) * VS + pos * 2) = hi;
      }
    }
  }
};

// First key the single query at position ctx - 1 sees under a sliding window
// of `window` preceding tokens (window < 0: no window).
__device__ __forceinline__ int window_start(int ctx, int window) {
  if (window < 0) return 0;
  const int lo = ctx - 1 - window;
  return lo > 0 ? lo : 0;
}

template <int D>
__global__ __launch_bounds__(64 * kDecodeWaves) void paged_decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int num_seqs, int num_blocks, int max_blocks_per_seq,
    int max_context_len, int hq, int hkv, int split_tokens, int max_splits, int q_chunks, float c, uint16_t* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_lse, int window) {
  constexpr int VS = kDecodeChunk * 2 + 16;
  constexpr int VT_BYTES = D * VS;
  constexpr int OB = D / 16;  // 16-wide d blocks of the PV output
  __shared__ __attribute__((aligned(16))) char smem[kDecodeWaves * VT_BYTES];

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  long item = (long)blockIdx.x * kDecodeWaves + wv;
  const int qc = item % q_chunks;
  item /= q_chunks;
  const int hk = item % hkv;
  item /= hkv;
  const int split = item % max_splits;
  const int seq = (int)(item / max_splits);
  if (seq >= num_seqs) return;

  // the host bound (<= max_blocks_per_seq * 128, checked on the host) keeps
  // every split index inside the workspace and every table index in the row
  const int ctx = clampi(context_lens[seq], 0, max_context_len);
  // keys [lo, ctx) are visible; the splits start at the 32-token chunk holding lo
  const int lo = window_start(ctx, window);
  const int skip = lo & ~(kDecodeChunk - 1);
  const int n = ctx - skip;
  if (split * split_tokens >= n) return;
  const int t_begin = skip + split * split_tokens;
  const int t_end = ctx - t_begin < split_tokens ? ctx : t_begin + split_tokens;
  const int nsplit = (n + split_tokens - 1) / split_tokens;

  const int group = hq / hkv;
  const int n16 = lane & 15, g = lane >> 4;
  const int qh_local = qc * 16 + n16;            // head within the group
  const bool q_real = qh_local < group;
  const int h = hk * group + (q_real ? qh_local : 0);

  // Q^T as the B operand: lane holds query n16, d = 32*b + 8*g .. +7
  bf16x8 qb[D / 32];
  {
    const uint16_t* qrow = q + ((long)seq * hq + h) * D;
#pragma unroll
    for (int b = 0; b < D / 32; ++b) {
      u32x4 x = ld_global16(qrow + b * 32 + g * 8);
      if (!q_real) x = u32x4{0u, 0u, 0u, 0u};
      qb[b] = as_bf16x8(x);
    }
  }

  f32x4 o[OB];
#pragma unroll
  for (int b = 0; b < OB; ++b) o[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, l = 0.f;

  const long tok_stride = (long)hkv * D;             // elements between tokens of a block
  const long block_elems = (long)kDecodeBlock * tok_stride;
  const long v_plane = (long)num_blocks * block_elems;
  const int32_t* table = block_tables + (long)seq * max_blocks_per_seq;
  char* vt = smem + wv * VT_BYTES;

  auto chunk_base = [&](int t0) -> const uint16_t* {
    int blk = table[t0 / kDecodeBlock];
    blk = clampi(blk, 0, num_blocks - 1);
    return kv + (long)blk * block_elems + (long)(t0 % kDecodeBlock) * tok_stride + hk * D;
  };

  DecodeChunk<D> cur;
  {
    const uint16_t* base = chunk_base(t_begin);
    const int nv = t_end - t_begin;
    cur.load(base, base + v_plane, tok_stride, nv < kDecodeChunk ? nv : kDecodeChunk, lane);
  }

  for (int t0 = t_begin; t0 < t_end; t0 += kDecodeChunk) {
    const int nvalid = t_end - t0 < kDecodeChunk ? t_end - t0 : kDecodeChunk;
    wave_lds_sync();  // previous chunk's V^T reads are done
    cur.store_v(vt, lane);
    // S^T = K Q^T from the registers of this chunk
    f32x4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < D / 32; ++b) s[kb] = mfma16x16x32(as_bf16x8(cur.kr[kb][b]), qb[b], s[kb]);
    }
    // next chunk in flight while this one is finished
    const int t1 = t0 + kDecodeChunk;
    if (t1 < t_end) {
      const uint16_t* base = chunk_base(t1);
      const int nv = t_end - t1;
      cur.load(base, base + v_plane, tok_stride, nv < kDecodeChunk ? nv : kDecodeChunk, lane);
    }
    if (nvalid < kDecodeChunk || t0 < lo) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = kb * 16 + 4 * g + r;
          if (i >= nvalid || t0 + i < lo) s[kb][r] = kNegInf;
        }
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = wave_xor_max(mx, 16);
    mx = wave_xor_max(mx, 32);
    const float m_new = fmaxf(m, mx);
    const float alpha = hw_exp2((m - m_new) * c);  // m_new is finite: every chunk has a visible token
    const float ms = m_new * c;
    f32x8 pt;
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pt[r] = hw_exp2(__builtin_fmaf(s[0][r], c, -ms));
      pt[4 + r] = hw_exp2(__builtin_fmaf(s[1][r], c, -ms));
      rs += pt[r] + pt[4 + r];
    }
    const bf16x8 p = to_bf16x8(pt);
    l = l * alpha + rs;
    m = m_new;
    wave_lds_sync();  // V^T of this chunk is visible to the whole wave
#pragma unroll
    for (int b = 0; b < OB; ++b) {
      const bf16x8 a = ld_lds16(vt, (b * 16 + n16) * VS + g * 16);
      o[b] = o[b] * alpha;
      o[b] = mfma16x16x32(a, p, o[b]);
    }
  }

  // this lane's query is n16; its partial row sum lives in 4 lanes (g = 0..3)
  l = wave_xor_sum(l, 16);
  l = wave_xor_sum(l, 32);
  if (!q_real) return;
  const float inv = 1.f / l;
  const float lse_s = (m * c + hw_log2(l)) * kLn2;
  if (nsplit == 1) {
    uint16_t* orow = out + ((long)seq * hq + h) * D;
#pragma unroll
    for (int b = 0; b < OB; ++b) {
      f32x4 t = o[b] * inv;
      *reinterpret_cast<bf16x4*>(orow + b * 16 + 4 * g) = to_bf16x4(t);
    }
    if (lse != nullptr && g == 0) lse[(long)h * num_seqs + seq] = lse_s;
  } else {
    const long slot = ((long)seq * max_splits + split) * hq + h;
    float* orow = part_o + slot * D;
#pragma unroll
    for (int b = 0; b < OB; ++b) *reinterpret_cast<f32x4*>(orow + b * 16 + 4 * g) = o[b] * inv;
    if (g == 0) part_lse[slot] = lse_s;
  }
}

// Merge split partials: LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s,
// splits in ascending order. One wave per (sequence, head).
template <int D>
__global__ __launch_bounds__(256) void paged_decode_combine_kernel(
    const int32_t* __restrict__ context_lens, int num_seqs, int max_context_len, int hq, int split_tokens,
    int max_splits, const float* __restrict__ part_o, const float* __restrict__ part_lse,
    uint16_t* __restrict__ out, float* __restrict__ lse, int window) {
  const int lane = threadIdx.x & 63;
  const long pair = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= (long)num_seqs * hq) return;
  const int seq = (int)(pair / hq), h = (int)(pair % hq);
  const int ctx = clampi(context_lens[seq], 0, max_context_len);
  const int n = ctx - (window_start(ctx, window) & ~(kDecodeChunk - 1));
  const int nsplit = (n + split_tokens - 1) / split_tokens;
  uint16_t* orow = out + pair * D;
  if (ctx == 0) {
    for (int d = lane; d < D; d += 64) orow[d] = 0;
    if (lse != nullptr && lane == 0) lse[(long)h * num_seqs + seq] = kNegInf;
    return;
  }
  if (nsplit == 1) return;  // written by the split kernel
  const long base = (long)seq * max_splits * hq + h;
  auto slot = [&](int sp) { return base + (long)sp * hq; };
  // The splits' LSEs are read lane-parallel (lane i holds split c0 + i of a
  // 64-split chunk) and reduced across the wave; the weighted sum of the
  // partial O takes each split's weight from its lane with v_readlane, in
  // ascending split order.
  float mx = kNegInf;
  for (int c0 = 0; c0 < nsplit; c0 += 64) {
    if (c0 + lane < nsplit) mx = fmaxf(mx, part_lse[slot(c0 + lane)]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = wave_xor_max(mx, o);
  float tot = 0.f;
  for (int c0 = 0; c0 < nsplit; c0 += 64) {
    if (c0 + lane < nsplit) tot += hw_exp2((part_lse[slot(c0 + lane)] - mx) * kLog2e);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) tot = wave_xor_sum(tot, o);
  const float lse_all = mx + hw_log2(tot) * kLn2;
  constexpr int NC = (D + 63) / 64;  // columns lane + 64k of the output row
  float acc[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) acc[k] = 0.f;
  for (int c0 = 0; c0 < nsplit; c0 += 64) {
    const float wl = c0 + lane < nsplit ? hw_exp2((part_lse[slot(c0 + lane)] - lse_all) * kLog2e) : 0.f;
    const int cnt = nsplit - c0 < 64 ? nsplit - c0 : 64;
    for (int i = 0; i < cnt; ++i) {
      const float wi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), i));
      const float* po = part_o + slot(c0 + i) * D;
#pragma unroll
      for (int k = 0; k < NC; ++k) {
        if (lane + 64 * k < D) acc[k] += wi * po[lane + 64 * k];
      }
    }
  }
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    if (lane + 64 * k < D) orow[lane + 64 * k] = __builtin_bit_cast(uint16_t, (__bf16)acc[k]);
  }
  if (lse != nullptr && lane == 0) lse[(long)h * num_seqs + seq] = lse_all;
}

DecodePlan plan_paged_decode(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int max_context_len,
                             size_t max_partial_bytes) {
  DecodePlan p{};
  const int group = num_heads / num_kv_heads;
  p.q_chunks = (group + 15) / 16;
  const long pairs = (long)num_seqs * num_kv_heads * p.q_chunks;
  long want = pairs > 0 ? (kDecodeTargetItems + pairs - 1) / pairs : 1;
  if (want < 1) want = 1;
  if (want > 64) want = 64;
  // fewer splits when their partials (O and LSE of every sequence and head)
  // must fit a fixed buffer; one split per sequence at the least
  const size_t per_split = (size_t)num_seqs * num_heads * (head_dim + 1) * sizeof(float);
  if (!decode_stream_supported(head_dim) && per_split > 0 && (size_t)want * per_split > max_partial_bytes) {
    const size_t cap = max_partial_bytes / per_split;
    want = cap > 0 ? (long)cap : 1;
  }
  const int ctx = max_context_len > 0 ? max_context_len : 1;
  long split = (ctx + want - 1) / want;
  split = ((split + kDecodeBlock - 1) / kDecodeBlock) * kDecodeBlock;
  if (split < kDecodeBlock) split = kDecodeBlock;
  p.split_tokens = (int)split;
  p.max_splits = (int)((ctx + split - 1) / split);
  p.o_bytes = (size_t)num_seqs * p.max_splits * num_heads * head_dim * sizeof(float);
  p.lse_bytes = (size_t)num_seqs * p.max_splits * num_heads * sizeof(float);
  p.workspace_bytes = p.o_bytes + p.lse_bytes;
  if (decode_stream_supported(head_dim)) {
    p.workspace_bytes = plan_decode_stream(num_seqs, num_heads, num_kv_heads, head_dim).workspace_bytes;
  }
  return p;
}

DecodePlan plan_paged_decode_window(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int max_context_len,
                                    int window) {
  const DecodePlan full = plan_paged_decode(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len);
  if (window < 0 || window >= max_context_len) return full;
  // the splits start at the 32-token chunk holding the window's first key, so
  // a sequence streams at most window + 32 keys
  const long streamed_l = (long)window + kDecodeChunk < max_context_len ? (long)window + kDecodeChunk : max_context_len;
  const int streamed = (int)streamed_l;
  DecodePlan p = plan_paged_decode(num_seqs, num_heads, num_kv_heads, head_dim, streamed);
  if (p.max_splits > full.max_splits) {
    // Splits round up to whole blocks, so the shorter stream can plan more
    // splits than the full context did; cap them at the full plan's count so
    // the partials fit the workspace that plan sized.
    long split = (streamed + full.max_splits - 1) / full.max_splits;
    split = ((split + kDecodeBlock - 1) / kDecodeBlock) * kDecodeBlock;
    p.split_tokens = (int)split;
    p.max_splits = (int)((streamed + split - 1) / split);
    p.o_bytes = (size_t)num_seqs * p.max_splits * num_heads * head_dim * sizeof(float);
    p.lse_bytes = (size_t)num_seqs * p.max_splits * num_heads * sizeof(float);
  }
  p.workspace_bytes = full.workspace_bytes;
  return p;
}

template <int D>
static hipError_t launch_decode_d(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream) {
  const float c = a.scale * kLog2e;
  float* part_o = (float*)a.workspace;
  float* part_lse = (float*)((char*)a.workspace + p.o_bytes);
  const long items = (long)a.num_seqs * p.max_splits * a.num_kv_heads * p.q_chunks;
  const long grid = (items + kDecodeWaves - 1) / kDecodeWaves;
  hipLaunchKernelGGL((paged_decode_split_kernel<D>), dim3((unsigned)grid), dim3(64 * kDecodeWaves), 0, stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.kv_cache, a.block_tables, a.context_lens,
                     a.num_seqs, a.num_blocks, a.max_blocks_per_seq, a.max_context_len, a.num_heads, a.num_kv_heads,
                     p.split_tokens, p.max_splits, p.q_chunks, c, (uint16_t*)a.out, a.lse, part_o, part_lse,
                     a.window);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long pairs = (long)a.num_seqs * a.num_heads;
  hipLaunchKernelGGL((paged_decode_combine_kernel<D>), dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, stream,
                     a.context_lens, a.num_seqs, a.max_context_len, a.num_heads, p.split_tokens,
                     p.max_splits, part_o, part_lse, (uint16_t*)a.out, a.lse, a.window);
  return hipGetLastError();
}

hipError_t launch_paged_decode(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream) {
  switch (a.head_dim) {
    case 64:
    case 128:
    case 256:
      return launch_decode_stream(a, plan_decode_stream(a.num_seqs, a.num_heads, a.num_kv_heads, a.head_dim), stream);
    case 96: return launch_decode_d<96>(a, p, stream);
    case 192: return launch_decode_d<192>(a, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
