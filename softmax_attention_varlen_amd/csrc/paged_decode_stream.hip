// Streaming single-token decode over a paged KV cache, head_dims 64, 96, 128,
// 192 and 256, gfx950.
//
// Work balance. The contexts of all sequences, laid end to end, form one token
// stream of T = sum(context_lens) positions. For each kv head (and chunk of
// <= 16 query heads of its group) the stream is cut into n_seg segments of
// L = max(ceil(T / n_seg), kMinSeg) positions; one wave owns one segment, so
// every wave reads the same number of K/V bytes whatever the mix of lengths.
// A segment may cover the end of one sequence, whole sequences and the start
// of another: each such piece is finished separately. A sequence that lies in
// one segment gets its final bf16 output from that wave; otherwise each piece
// writes a normalised fp32 partial (O, LSE) to slot (segment + sequence),
// which is unique because segments and sequences are both contiguous ranges
// of the stream, and the combine kernel merges the pieces of each sequence in
// ascending segment order. The token prefix sums come from a one-workgroup
// scan kernel, so the host never reads the lengths.
//
// Streaming. Each wave keeps a two-stage LDS ring of 32-token chunks (K and V
// of its kv head, 32 rows of 2*D bytes each) filled by direct-to-LDS loads,
// and issues chunk j+2 as soon as chunk j is consumed (its K half right after
// chunk j's S^T, its V half after the PV): one chunk is always in flight,
// which is what keeps HBM busy (a wave that waits for its whole chunk before
// issuing the next leaves gaps). A token row takes R = 2D bytes of LDS, padded
// to the next power of two at D = 96 and 192 (256 and 512 bytes; the pad lanes
// of a load re-read the row's last real 16 bytes, in the same cache line). A
// load writes 1 KB, i.e. 1024 / R token rows, so a chunk half is NB = R / 32
// load blocks: block b holds tokens b, b + NB, b + 2NB, ...; blocks sit 1056
// bytes apart, which makes the transposing V reads conflict-free at R = 256
// and the K reads at most 2-way. Workgroups hold 1024 / R * 4 waves (8, 4, 4,
// 2, 2 for D = 64, 96, 128, 192, 256), so every head dim uses about the same
// LDS per CU and keeps the same row bytes in flight per CU.
//
// Queries. The 16 MFMA columns of a wave are (query token, head) pairs of its
// kv head's group: column n of chunk qc is token (16qc + n) / group, head
// (16qc + n) % group, so a sequence's max_q new tokens (speculative decoding:
// the last max_q positions, bottom-right causal) share one pass over its K/V;
// plain decode is max_q = 1.
//
// Sliding window ([ASC] AscendAttentionBackendImpl._forward_fia_slidingwindow,
// decode only): a sequence streams only its last window + 1 keys, from the
// 32-token chunk that holds the first of them; the keys of that chunk below
// the window are masked like the causal limit.
//
// Math per chunk (16x16x32 bf16 MFMA): S^T = K Q^T with K from LDS (A) and the
// (token, head) columns (B); online softmax per column; O^T += V^T P^T
// with V^T from transposing LDS reads (A) and P straight from the S^T
// accumulator (B): the lane's 8 tokens 4G..4G+3 and 16+4G..16+4G+3 are the
// k-slots of its B operand, and the two transposing reads fetch exactly those
// V rows.
#include "attn_common.hpp"
#include "launch.hpp"

namespace attn {
namespace {

constexpr int kSChunk = 32;
constexpr int kSBlk = 1056;                  // one 1 KB load block + 32 B pad
constexpr int kMinSeg = 256;                 // shortest segment (positions)

// Per head dim: the chunk layout in LDS and the workgroup shape.
template <int D>
struct StreamShape {
  static_assert(D == 64 || D == 96 || D == 128 || D == 192 || D == 256, "head dims 64, 96, 128, 192, 256");
  static constexpr int kRow = D <= 64 ? 128 : D <= 128 ? 256 : 512;  // LDS bytes of one token row of one kv head
  static constexpr int kLanesPerRow = kRow / 16;       // 16-byte pieces of an LDS row: 8, 16, 32
  static constexpr int kRowPieces = D / 8;             // the real ones (fewer at D = 96, 192)
  static constexpr int kNB = kRow / 32;                // load blocks per chunk half: 4, 8, 16
  static constexpr int kHalf = kNB * kSBlk;            // K (or V) of one chunk
  static constexpr int kStage = 2 * kHalf;             // K, then V
  static constexpr int kWaveLds = 2 * kStage;          // two-stage ring per wave
  static constexpr int kWaves = 4 * 256 / kRow;        // waves per workgroup (one workgroup per CU by LDS)
  static constexpr int kLoads = 2 * kNB;               // direct-to-LDS loads per chunk per wave
  // byte offset of token t (0..31) of a chunk half: block t % NB, row t / NB
  __device__ __forceinline__ static uint32_t tok_off(uint32_t t) {
    return (t % (uint32_t)kNB) * kSBlk + (t / (uint32_t)kNB) * (uint32_t)kRow;
  }
};

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// sbase and lds are the same in every lane; readfirstlane tells the compiler
// so where it cannot see it (it would otherwise hand the scalar operands a
// vector register)
__device__ __forceinline__ void load_lds16(const void* sbase, uint32_t voff, uint32_t lds) {
  const uint64_t b = (uint64_t)(uintptr_t)sbase;
  const uint64_t bu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"((const void*)(uintptr_t)bu), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Index of the sequence holding stream position pos: the largest s with
// prefix[s] <= pos (prefix non-decreasing, prefix[0] = 0 <= pos < prefix[n]).
// A 64-way search: each round the lanes probe 64 evenly spaced entries.
__device__ __forceinline__ int find_seq(const int32_t* prefix, int n, int pos, int lane) {
  int lo = 0, hi = n;  // answer in [lo, hi)
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) / 64;
    const int idx = lo + lane * step;
    const bool ok = idx < hi && prefix[idx] <= pos;
    const int cnt = __popcll(__ballot(ok));  // >= 1: prefix[lo] <= pos
    lo = lo + (cnt - 1) * step;
    hi = lo + step < hi ? lo + step : hi;
  }
  return lo;
}

// Tokens a sequence puts on the stream. With a sliding window (window >= 0)
// the single query at position L - 1 sees keys t >= L - 1 - window; the stream
// then starts at that key rounded down to a whole 32-token chunk (*skip), so
// chunks stay inside one 128-token cache block, and the keys below the window
// in that first chunk are masked by the kernel.
constexpr int kNoLowerLimit = -(1 << 30);  // below every key index (windows are at most 2^30)

__device__ __forceinline__ int stream_tokens(int ctx_raw, int max_context_len, int window, int* skip) {
  const int len = clampi(ctx_raw, 0, max_context_len);
  int sk = 0;
  if (window >= 0) {
    const int lo = len - 1 - window;
    sk = lo > 0 ? (lo & ~(kSChunk - 1)) : 0;
  }
  *skip = sk;
  return len - sk;
}

// Exclusive prefix sums of the streamed token counts, prefix[num_seqs] = T;
// skip[s] (when windowed) is the first streamed position of sequence s.
__global__ __launch_bounds__(1024) void decode_prefix_kernel(const int32_t* __restrict__ context_lens, int num_seqs,
                                                             int max_context_len, int window,
                                                             int32_t* __restrict__ prefix, int32_t* __restrict__ skip) {
  __shared__ int part[1024];
  const int t = threadIdx.x;
  const int per = (num_seqs + 1023) / 1024;
  const int b = t * per < num_seqs ? t * per : num_seqs;
  const int e = b + per < num_seqs ? b + per : num_seqs;
  int sum = 0, sk;
  for (int i = b; i < e; ++i) sum += stream_tokens(context_lens[i], max_context_len, window, &sk);
  part[t] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
    const int add = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += add;
    __syncthreads();
  }
  int run = part[t] - sum;
  for (int i = b; i < e; ++i) {
    prefix[i] = run;
    run += stream_tokens(context_lens[i], max_context_len, window, &sk);
    if (skip != nullptr) skip[i] = sk;
  }
  if (t == 1023) prefix[num_seqs] = part[1023];
}

__device__ __forceinline__ int seg_len(int total, int n_seg) {
  const int l = (total + n_seg - 1) / n_seg;
  return l > kMinSeg ? l : kMinSeg;
}

template <int D>
__global__ __launch_bounds__(64 * StreamShape<D>::kWaves) void paged_decode_stream_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ prefix, int num_seqs, int num_blocks, int max_blocks_per_seq, int hq, int hkv,
    int q_chunks, int n_seg, float c, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse, const int32_t* __restrict__ cu_q, int max_q,
    int total_q, const int32_t* __restrict__ skip, int window) {
  using S = StreamShape<D>;
  constexpr int kSWaves = S::kWaves, kSWaveLds = S::kWaveLds, kSStage = S::kStage, kSHalf = S::kHalf;
  constexpr int kSLoads = S::kLoads;
  __shared__ __attribute__((aligned(1024))) char smem[kSWaves * kSWaveLds];
  // every cursor below is wave-uniform (scalar registers, scalar loads): no
  // compiler-visible vector load may sit in the streaming loop, since the
  // compiler's wait for it would also drain the ring
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = blockIdx.x * kSWaves + wv;
  if (w >= n_seg * hkv * q_chunks) return;  // no workgroup barriers below
  const int qc = w % q_chunks;
  const int hk = (w / q_chunks) % hkv;
  const int g = w / (q_chunks * hkv);

  const int total = prefix[num_seqs];
  if (total <= 0) return;
  const int L = seg_len(total, n_seg);
  const int seg_begin = g * L;
  if (seg_begin >= total) return;
  const int seg_end = total - seg_begin < L ? total : seg_begin + L;

  const int group = hq / hkv;
  const int n16 = lane & 15, G = lane >> 4;
  const int col = qc * 16 + n16;           // (query token, head) column of this kv head
  const bool col_real = col < max_q * group;
  const int qi = col_real ? col / group : 0;
  const int h = hk * group + (col_real ? col % group : 0);

  const long row_elems = (long)hkv * D;                  // elements between tokens of a block
  const long blk_elems = 128L * row_elems;
  const long v_plane = (long)num_blocks * blk_elems;
  const uint32_t row_bytes = (uint32_t)row_elems * 2u;
  const uint32_t ring = lds_addr(smem + wv * kSWaveLds);
  const char* ring_p = smem + wv * kSWaveLds;

  // per-lane LDS offsets: K A operand (token 16kb + n16, d = 32b + 8G) and the
  // transposing V reads (token 4G + s/4, columns 16db + 4(s%4))
  // (token 16kb + n16 sits 512 bytes after token n16 for every D)
  const uint32_t k_lane = S::tok_off((uint32_t)n16) + (uint32_t)G * 16u;
  const uint32_t v_lane = S::tok_off(4u * (uint32_t)G + ((uint32_t)n16 >> 2)) + ((uint32_t)n16 & 3u) * 8u;

  const int s0 = __builtin_amdgcn_readfirstlane(find_seq(prefix, num_seqs, seg_begin, lane));
  // the loader's cursor: sequence ls, chunk lc (32 tokens), its last chunk lc_end
  int ls = s0;
  int lbase = prefix[ls];
  int lctx = prefix[ls + 1] - lbase;
  int lskip = skip != nullptr ? skip[ls] : 0;  // cache position of stream token 0
  int lc = (seg_begin - lbase) / kSChunk;
  int lc_end = ((seg_end < lbase + lctx ? seg_end : lbase + lctx) - lbase - 1) / kSChunk;
  bool lvalid = true;

  // issue the loader's chunk into `stage` in two halves: K as soon as the
  // stage's K has been read (after this chunk's S^T), then V and the cursor
  // advance once its V has been read (after the PV)
  const uint16_t* lkb = kv;  // K base of the block being issued, kept between the halves
  auto issue_half = [&](int stage, bool v_half) __attribute__((always_inline)) {
    const int t0 = lc * kSChunk;
    if (!v_half) {
      int blk = block_tables[(long)ls * max_blocks_per_seq + ((t0 + lskip) >> 7)];
      blk = clampi(blk, 0, num_blocks - 1);
      lkb = kv + (long)blk * blk_elems + (long)hk * D;
    }
    const uint16_t* src = v_half ? lkb + v_plane : lkb;
    const uint32_t st = ring + stage * kSStage + (v_half ? kSHalf : 0);
#pragma unroll
    for (int b = 0; b < S::kNB; ++b) {
      // lane l writes 16 bytes at st + b * kSBlk + 16 l: row l / kLanesPerRow
      // of the block (token b + kNB * row), piece l % kLanesPerRow of it (a
      // pad piece re-reads the row's last real one)
      int t = t0 + b + S::kNB * (lane / S::kLanesPerRow);
      t = t < lctx ? t : lctx - 1;  // rows past the context re-read the last one (same block)
      const int piece = lane % S::kLanesPerRow;
      const uint32_t voff = (uint32_t)((t + lskip) & 127) * row_bytes +
                            (uint32_t)(piece < S::kRowPieces ? piece : S::kRowPieces - 1) * 16u;
      load_lds16(src, voff, st + b * kSBlk);
    }
    if (!v_half) return;
    if (lc < lc_end) {
      ++lc;
    } else {
      // next non-empty sequence starting before the segment end
      do {
        ls = __builtin_amdgcn_readfirstlane(ls + 1);
        lbase = prefix[ls];
        lctx = ls < num_seqs ? prefix[ls + 1] - lbase : 0;
      } while (ls < num_seqs && lctx == 0 && lbase < seg_end);
      lvalid = ls < num_seqs && lbase < seg_end;
      if (lvalid) {
        lskip = skip != nullptr ? skip[ls] : 0;
        lc = 0;
        lc_end = ((seg_end < lbase + lctx ? seg_end : lbase + lctx) - lbase - 1) / kSChunk;
      }
    }
  };
  auto issue = [&](int stage) __attribute__((always_inline)) {
    issue_half(stage, false);
    issue_half(stage, true);
  };

  issue(0);
  bool second = lvalid;
  if (second) issue(1);

  // the consumer's cursor mirrors the loader's
  int cs = s0;
  int cbase = prefix[cs];
  int cctx = prefix[cs + 1] - cbase;
  int cc = (seg_begin - cbase) / kSChunk;
  int t_lo = seg_begin - cbase;                                               // first token of the piece
  int t_hi = (seg_end < cbase + cctx ? seg_end : cbase + cctx) - cbase;       // one past its last
  int cc_end = (t_hi - 1) / kSChunk;
  bool fresh = true;

  constexpr int QB = D / 32;  // 32-wide d steps of S^T
  constexpr int OB = D / 16;  // 16-wide d blocks of O^T
  bf16x8 qb[QB];
  f32x4 o[OB];
  float m = kNegInf, l = 0.f;
  int q_row = 0, lim = 0, lim_min = 0, lo_lim = 0, lo_max = 0;
  bool live = false;
  for (int j = 0;; ++j) {
    if (fresh) {
      // a new piece: its queries (the compiler's wait for these loads also
      // drains the ring, once per piece), and a reset softmax state. Query
      // token qi of the sequence's lq sees keys t <= qi + cctx - lq.
      int q_first = cs, lq = 1;
      if (cu_q != nullptr) {
        q_first = clampi(cu_q[cs], 0, total_q);
        lq = clampi(cu_q[cs + 1], q_first, total_q) - q_first;
        lq = lq > max_q ? max_q : lq;
      }
      live = col_real && qi < lq;
      q_row = live ? q_first + qi : 0;  // row 0 exists whenever this kernel runs
      lim = qi + cctx - lq;
      lim_min = cctx - lq;
      // sliding window: keys below lim - window are hidden (the stream's first
      // chunk may start up to 31 keys early); lo_max is the largest such bound
      lo_lim = window >= 0 ? lim - window : kNoLowerLimit;
      lo_max = window >= 0 ? cctx - 1 - window : kNoLowerLimit;
      const uint16_t* qrow = q + ((long)q_row * hq + h) * D;
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        const u32x4 x = ld_global16(qrow + b * 32 + G * 8);  // unconditional: no branch per load
        qb[b] = as_bf16x8(live ? x : u32x4{0u, 0u, 0u, 0u});
      }
#pragma unroll
      for (int b = 0; b < QB; ++b) asm volatile("" : : "v"(qb[b]));
#pragma unroll
      for (int b = 0; b < OB; ++b) o[b] = f32x4{0.f, 0.f, 0.f, 0.f};
      m = kNegInf;
      l = 0.f;
      fresh = false;
    }
    // chunk j has landed once at most the next chunk's loads are in flight
    if (second) {
      wait_vm<kSLoads>();
    } else {
      wait_vm<0>();
    }
    const int stage = j & 1;
    const char* kt = ring_p + stage * kSStage;
    f32x4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        const bf16x8 a = ld_lds16(kt, (int)(k_lane + (uint32_t)kb * 512u + (uint32_t)b * 64u));
        s[kb] = mfma16x16x32(a, qb[b], s[kb]);
      }
    }
    if (lvalid) {
      asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");  // this chunk's K reads are done
      issue_half(stage, false);
    }
    const int t0 = cc * kSChunk;
    if (t0 < t_lo || t0 + kSChunk > t_hi || t0 + kSChunk - 1 > lim_min || t0 < lo_max) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = t0 + kb * 16 + 4 * G + r;
          if (t < t_lo || t >= t_hi || t > lim || t < lo_lim) s[kb][r] = kNegInf;
        }
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = wave_xor_max(mx, 16);
    mx = wave_xor_max(mx, 32);
    // a column may see no key of this chunk (causal limit) or of the piece yet
    const float m_new = fmaxf(m, mx);
    const float alpha = m_new == kNegInf ? 1.f : hw_exp2((m - m_new) * c);
    const float ms = m_new == kNegInf ? 0.f : m_new * c;
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
    const lds_bf16x4* vb = (const lds_bf16x4*)(ring + stage * kSStage + kSHalf + v_lane);
#pragma unroll
    for (int db = 0; db < OB; ++db) {
      // byte offsets 32db (columns) and 512 for tokens 16..31, in 8-byte units
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vb + 4 * db));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vb + 64 + 4 * db));
      const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      o[db] = o[db] * alpha;
      o[db] = mfma16x16x32(a, p, o[db]);
    }

    if (cc == cc_end) {
      // piece done: the lane's column sum lives in 4 lanes (G = 0..3)
      float lt = wave_xor_sum(l, 16);
      lt = wave_xor_sum(lt, 32);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const float lse_p = lt > 0.f ? (m * c + hw_log2(lt)) * kLn2 : kNegInf;
      if (live) {
        if (t_lo == 0 && t_hi == cctx) {
          uint16_t* orow = out + ((long)q_row * hq + h) * D;
#pragma unroll
          for (int db = 0; db < OB; ++db) {
            const f32x4 t = o[db] * inv;
            *reinterpret_cast<bf16x4*>(orow + db * 16 + 4 * G) = to_bf16x4(t);
          }
          if (lse != nullptr && G == 0) lse[(long)h * total_q + q_row] = lse_p;
        } else {
          const long slot = ((long)(g + cs) * max_q + qi) * hq + h;
          float* orow = part_o + slot * D;
#pragma unroll
          for (int db = 0; db < OB; ++db) *reinterpret_cast<f32x4*>(orow + db * 16 + 4 * G) = o[db] * inv;
          if (G == 0) part_lse[slot] = lse_p;
        }
      }
      // next non-empty sequence of the segment
      do {
        cs = __builtin_amdgcn_readfirstlane(cs + 1);
        cbase = prefix[cs];
        cctx = cs < num_seqs ? prefix[cs + 1] - cbase : 0;
      } while (cs < num_seqs && cctx == 0 && cbase < seg_end);
      if (cs >= num_seqs || cbase >= seg_end) break;
      cc = 0;
      t_lo = 0;
      t_hi = (seg_end < cbase + cctx ? seg_end : cbase + cctx) - cbase;
      cc_end = (t_hi - 1) / kSChunk;
      fresh = true;
    } else {
      ++cc;
    }
    // this chunk's V reads are done before the V half of its stage is refilled
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
    second = lvalid;
    if (lvalid) issue_half(stage, true);
  }
}

// Merge the pieces of each (sequence, query token, head) in ascending segment
// order: LSE = ln sum_i exp(LSE_i), O = sum_i exp(LSE_i - LSE) O_i. A sequence
// that lies in one segment was finished by the streaming kernel; an empty one
// gets zeros and LSE = -inf.
template <int D>
__global__ __launch_bounds__(256) void paged_decode_stream_combine_kernel(
    const int32_t* __restrict__ prefix, int num_seqs, int hq, int n_seg, const float* __restrict__ part_o,
    const float* __restrict__ part_lse, uint16_t* __restrict__ out, float* __restrict__ lse,
    const int32_t* __restrict__ cu_q, int max_q, int total_q) {
  const int lane = threadIdx.x & 63;
  const long pair = (long)blockIdx.x * 4 + (threadIdx.x >> 6);  // (s * max_q + qi) * hq + h
  if (pair >= (long)num_seqs * max_q * hq) return;
  const int h = (int)(pair % hq);
  const int qi = (int)((pair / hq) % max_q);
  const int s = (int)(pair / ((long)hq * max_q));
  int q_first = s, lq = 1;
  if (cu_q != nullptr) {
    q_first = clampi(cu_q[s], 0, total_q);
    lq = clampi(cu_q[s + 1], q_first, total_q) - q_first;
    lq = lq > max_q ? max_q : lq;
  }
  if (qi >= lq) return;
  const long row = q_first + qi;
  const int total = prefix[num_seqs];
  const int b0 = prefix[s], b1 = prefix[s + 1];
  uint16_t* orow = out + (row * hq + h) * D;
  if (b1 <= b0) {
    for (int d = lane; d < D; d += 64) orow[d] = 0;
    if (lse != nullptr && lane == 0) lse[(long)h * total_q + row] = kNegInf;
    return;
  }
  const int L = seg_len(total, n_seg);
  const int first = b0 / L, last = (b1 - 1) / L;
  if (first == last) return;
  auto slot = [&](int gg) { return ((long)(gg + s) * max_q + qi) * hq + h; };
  // The pieces' LSEs are read lane-parallel (lane i holds piece c0 + i of a
  // 64-piece chunk) and reduced across the wave; the weighted sum of the
  // partial O then takes each piece's weight from its lane with v_readlane, in
  // ascending piece order (the same order on every run).
  float mx = kNegInf;
  for (int c0 = first; c0 <= last; c0 += 64) {
    const int gg = c0 + lane;
    if (gg <= last) mx = fmaxf(mx, part_lse[slot(gg)]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = wave_xor_max(mx, o);
  if (mx == kNegInf) {  // no key visible to this query in any piece
    for (int d = lane; d < D; d += 64) orow[d] = 0;
    if (lse != nullptr && lane == 0) lse[(long)h * total_q + row] = kNegInf;
    return;
  }
  float tot = 0.f;
  for (int c0 = first; c0 <= last; c0 += 64) {
    const int gg = c0 + lane;
    if (gg <= last) tot += hw_exp2((part_lse[slot(gg)] - mx) * kLog2e);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) tot = wave_xor_sum(tot, o);
  const float lse_all = mx + hw_log2(tot) * kLn2;
  constexpr int NC = (D + 63) / 64;  // columns lane + 64k (< D) of the output row
  float acc[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) acc[k] = 0.f;
  for (int c0 = first; c0 <= last; c0 += 64) {
    const int gg = c0 + lane;
    const float wl = gg <= last ? hw_exp2((part_lse[slot(gg)] - lse_all) * kLog2e) : 0.f;
    const int n = last - c0 + 1 < 64 ? last - c0 + 1 : 64;
    for (int i = 0; i < n; ++i) {
      const float wi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), i));
      const float* po = part_o + slot(c0 + i) * D;
#pragma unroll
      for (int k = 0; k < NC; ++k) {
        if (D % 64 == 0 || lane + 64 * k < D) acc[k] += wi * po[lane + 64 * k];
      }
    }
  }
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    if (D % 64 == 0 || lane + 64 * k < D) orow[lane + 64 * k] = __builtin_bit_cast(uint16_t, (__bf16)acc[k]);
  }
  if (lse != nullptr && lane == 0) lse[(long)h * total_q + row] = lse_all;
}

}  // namespace

// stream waves: 256 CUs x the workgroup's waves
static int decode_stream_waves(int head_dim) {
  switch (head_dim) {
    case 64: return 256 * StreamShape<64>::kWaves;
    case 96: return 256 * StreamShape<96>::kWaves;
    case 128: return 256 * StreamShape<128>::kWaves;
    case 192: return 256 * StreamShape<192>::kWaves;
    default: return 256 * StreamShape<256>::kWaves;
  }
}

DecodeStreamPlan plan_decode_stream(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int max_q) {
  DecodeStreamPlan p{};
  const int group = num_heads / num_kv_heads;
  p.max_q = max_q > 1 ? max_q : 1;
  p.q_chunks = (p.max_q * group + 15) / 16;
  const int lanes = num_kv_heads * p.q_chunks;
  const int waves = decode_stream_waves(head_dim);
  p.n_seg = waves / lanes > 1 ? waves / lanes : 1;
  p.prefix_bytes = ((size_t)(num_seqs + 1) * sizeof(int32_t) + 255) & ~(size_t)255;
  p.skip_bytes = ((size_t)num_seqs * sizeof(int32_t) + 255) & ~(size_t)255;
  const size_t slots = (size_t)(p.n_seg + num_seqs) * p.max_q * num_heads;
  p.lse_bytes = (slots * sizeof(float) + 255) & ~(size_t)255;
  p.o_bytes = slots * (size_t)head_dim * sizeof(float);
  p.workspace_bytes = p.prefix_bytes + p.skip_bytes + p.lse_bytes + p.o_bytes;
  return p;
}

template <int D>
static hipError_t launch_decode_stream_d(const DecodeArgs& a, const DecodeStreamPlan& p, hipStream_t stream) {
  constexpr int kSWaves = StreamShape<D>::kWaves;
  int32_t* prefix = (int32_t*)a.workspace;
  int32_t* skip = a.window >= 0 ? (int32_t*)((char*)a.workspace + p.prefix_bytes) : nullptr;
  float* part_lse = (float*)((char*)a.workspace + p.prefix_bytes + p.skip_bytes);
  float* part_o = (float*)((char*)a.workspace + p.prefix_bytes + p.skip_bytes + p.lse_bytes);
  const int total_q = a.cu_q != nullptr ? a.total_q : a.num_seqs;
  hipLaunchKernelGGL(decode_prefix_kernel, dim3(1), dim3(1024), 0, stream, a.context_lens, a.num_seqs,
                     a.max_context_len, a.window, prefix, skip);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long waves = (long)p.n_seg * a.num_kv_heads * p.q_chunks;
  hipLaunchKernelGGL((paged_decode_stream_kernel<D>), dim3((unsigned)((waves + kSWaves - 1) / kSWaves)),
                     dim3(64 * kSWaves), 0, stream, (const uint16_t*)a.q, (const uint16_t*)a.kv_cache,
                     a.block_tables, prefix, a.num_seqs, a.num_blocks, a.max_blocks_per_seq, a.num_heads,
                     a.num_kv_heads, p.q_chunks, p.n_seg, a.scale * kLog2e, (uint16_t*)a.out, a.lse, part_o,
                     part_lse, a.cu_q, p.max_q, total_q, skip, a.window);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long pairs = (long)a.num_seqs * p.max_q * a.num_heads;
  hipLaunchKernelGGL((paged_decode_stream_combine_kernel<D>), dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0,
                     stream, prefix, a.num_seqs, a.num_heads, p.n_seg, part_o, part_lse, (uint16_t*)a.out, a.lse,
                     a.cu_q, p.max_q, total_q);
  return hipGetLastError();
}

hipError_t launch_decode_stream(const DecodeArgs& a, const DecodeStreamPlan& p, hipStream_t stream) {
  if (a.window >= 0 && a.cu_q != nullptr) return hipErrorInvalidValue;  // windows: one query token each
  switch (a.head_dim) {
    case 64: return launch_decode_stream_d<64>(a, p, stream);
    case 96: return launch_decode_stream_d<96>(a, p, stream);
    case 128: return launch_decode_stream_d<128>(a, p, stream);
    case 192: return launch_decode_stream_d<192>(a, p, stream);
    case 256: return launch_decode_stream_d<256>(a, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
