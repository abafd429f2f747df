// Pipelined block-sparse attention over 64-token tiles, head_dims 96, 128, 192
// and 256, gfx950.
//
// Work unit: one workgroup of 4 waves owns one (batch, head, query tile).
// Wave w owns query rows 32*(w%2) .. +31 of the tile and key half w/2 (keys
// 32*(w/2) .. +31 of every kept key tile), so all four waves consume each K/V
// tile the ring brings in, and the two key halves of a row are merged once at
// the end, through LDS, with the usual max/rescale combination of partial
// softmax sums.
//
// The kept key tiles come from the block map as ascending lists with empty
// tiles dropped, each entry packed as (size << 24) | tile. K and V stream
// through separate two-stage LDS rings (direct-to-LDS loads, the
// conflict-free layout of pipe.hpp): step j runs the softmax of tile j
// under the S^T MFMAs of tile j+1 and the PV MFMAs of tile j-1, reading K of
// tile j+1 and V of tile j-1, while K of tile j+2 and V of tile j are in
// flight. At head_dims 96 and 128 (256-byte LDS rows, 96 padded) two
// workgroups share a CU (66.5 KB of LDS each), so a SIMD holds two waves; at
// 192 and 256 (512-byte rows, 192 padded) the rings take 130 KB and one
// workgroup runs per CU.
//
// Padding keys (at or past a tile's size) are masked; padding query rows are
// written as zeros with LSE = -inf; a query tile with no kept key gets zeros
// and -inf as well.
//
// Item order: workgroup slot s of XCD x runs item order[x*per_xcd + s]. A small
// kernel fills order per XCD chunk (the items that XCD runs, so its L2 keeps
// serving the same heads) with the longest items first: a map can keep every
// key tile for a few query tiles (the dense prefix rows of the H3 layout) and
// far fewer for the rest, and a long item dispatched late in its chunk would
// set the end of the launch. Items fall into 16 classes by kept-tile count;
// the order is stable within a class, so a map with equal counts keeps the
// plain order. The order changes when an item runs, never what it computes.
#include <type_traits>

#include "launch.hpp"
#include "pipe.hpp"

namespace attn {
namespace {

using namespace pipe;

constexpr int kSW = 4;                             // waves per workgroup
constexpr int kListCap = kSparsePipeMaxTiles;      // the whole kept-tile list is staged in LDS

template <int D>
struct SparseShape {
  static constexpr int kTileBytes = Geom<D>::kTileBytes;
  static constexpr int kSIPW = Geom<D>::kBlocks / kSW;  // load blocks per wave per K (or V) tile
  static constexpr int kLds = 4 * kTileBytes;           // K stages 0, 1, then V stages 0, 1
  static constexpr int kMergeOBytes = 32 * D * 4;        // one wave's fp32 O^T block
  static constexpr int kWgPerCu = D <= 128 ? 2 : 1;
  static_assert(2 * kMergeOBytes + 2 * 512 <= kLds, "merge area must fit in the ring");
};

constexpr int kOrderThreads = 1024;
constexpr int kOrderWaves = kOrderThreads / 64;
constexpr int kOrderBins = 16;
constexpr int kOrderStaged = 4 * kOrderThreads;  // counts held in LDS; the rest of a chunk is re-read

// One workgroup per XCD chunk [x*per_xcd, min((x+1)*per_xcd, n_items)):
// writes a permutation of the chunk's item ids into the same range of order,
// class by class (class 0 holds the longest items), in item order within a
// class.
__global__ __launch_bounds__(kOrderThreads) void order_items_kernel(const int32_t* __restrict__ num, int n_items,
                                                                    int per_xcd, int32_t* __restrict__ order) {
  __shared__ int wave_max[kOrderWaves];
  __shared__ int wave_cnt[kOrderWaves][kOrderBins];
  __shared__ int next[kOrderBins];  // bin sizes, then the next free position of each class
  __shared__ int staged[kOrderStaged];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int base = blockIdx.x * per_xcd;
  const int len = clampi(n_items - base, 0, per_xcd);
  const unsigned long long below = (1ull << lane) - 1ull;

  // one pass over the counts (all loads in flight together), the first
  // kOrderStaged of them kept in LDS
  int m = 0;
  for (int i = tid; i < len; i += kOrderThreads) {
    const int c = num[base + i];
    if (i < kOrderStaged) staged[i] = c;
    m = max(m, c);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, __shfl_xor(m, o, 64));
  if (lane == 0) wave_max[w] = m;
  if (tid < kOrderBins) next[tid] = 0;
  __syncthreads();
  int mx = 0;
#pragma unroll
  for (int j = 0; j < kOrderWaves; ++j) mx = max(mx, wave_max[j]);
  // class of item i of the chunk (-1 past the end): non-increasing in the count
  auto cls = [&](int i) -> int {
    if (i >= len) return -1;
    const int c = clampi(i < kOrderStaged ? staged[i] : num[base + i], 0, mx);
    return (kOrderBins - 1) - (int)(((long)c * kOrderBins) / ((long)mx + 1));
  };

  for (int i0 = 0; i0 < len; i0 += kOrderThreads) {
    const int k = cls(i0 + tid);
#pragma unroll
    for (int b = 0; b < kOrderBins; ++b) {
      const unsigned long long bits = __ballot(k == b);
      if (lane == 0 && bits != 0ull) atomicAdd(&next[b], __popcll(bits));
    }
  }
  __syncthreads();
  if (tid == 0) {
    int sum = 0;
    for (int b = 0; b < kOrderBins; ++b) {
      const int t = next[b];
      next[b] = sum;
      sum += t;
    }
  }
  __syncthreads();

  for (int i0 = 0; i0 < len; i0 += kOrderThreads) {
    const int k = cls(i0 + tid);
    int rank = 0;
#pragma unroll
    for (int b = 0; b < kOrderBins; ++b) {
      const unsigned long long bits = __ballot(k == b);
      if (k == b) rank = __popcll(bits & below);
      if (lane == 0) wave_cnt[w][b] = __popcll(bits);
    }
    __syncthreads();
    if (k >= 0) {
      int pos = next[k] + rank;
      for (int j = 0; j < w; ++j) pos += wave_cnt[j][k];
      order[base + pos] = base + i0 + tid;
    }
    __syncthreads();
    if (tid < kOrderBins) {
      int add = 0;
      for (int j = 0; j < kOrderWaves; ++j) add += wave_cnt[j][tid];
      next[tid] += add;
    }
    __syncthreads();
  }
}

struct Entry {
  int tile, size;
};

__device__ __forceinline__ Entry unpack(int32_t v, int num_tiles) {
  Entry e;
  e.tile = clampi(v & 0xffffff, 0, num_tiles - 1);
  e.size = clampi((int)((uint32_t)v >> 24), 1, kBN);
  return e;
}

template <int D>
__global__ __launch_bounds__(64 * kSW, SparseShape<D>::kWgPerCu) void block_sparse_pipe_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ tile_sizes, const int32_t* __restrict__ kidx, const int32_t* __restrict__ knum,
    const int32_t* __restrict__ order, int num_tiles, int hq, int hkv, int n_items, int per_xcd, float c,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  using SS = SparseShape<D>;
  using G = Geom<D>;
  constexpr int kD = D, kTileBytes = SS::kTileBytes, kSIPW = SS::kSIPW, kMergeOBytes = SS::kMergeOBytes;
  constexpr int QB = G::kQB, OB = G::kOB;
  __shared__ __attribute__((aligned(1024))) char smem[SS::kLds];
  __shared__ int32_t lst[kListCap];

  // XCD-aware order: XCD x runs the items of [x*per_xcd, (x+1)*per_xcd) (query
  // tiles fastest, so one XCD's L2 serves the K/V of few heads), longest first.
  const int hw = blockIdx.x;
  const int slot = (hw & 7) * per_xcd + (hw >> 3);
  if (slot >= n_items) return;
  const int item = clampi(order[slot], 0, n_items - 1);
  const int a = item % num_tiles;
  const int bh = item / num_tiles;
  const int h = bh % hq;
  const int b = bh / hq;
  const int hk = h / (hq / hkv);
  const long seq = (long)num_tiles * kBN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // the same in every lane of a wave
  const int rh = w & 1, kh = w >> 1;
  const Lane L = make_lane<kD>(lane, 32 * kh);
  const int qsize = clampi(tile_sizes[a], 0, kBN);
  const int r = 32 * rh + L.n;
  const int r_c = r < qsize ? r : (qsize > 0 ? qsize - 1 : 0);
  const bool wave_live = 32 * rh < qsize;
  const int32_t* list = kidx + (long)item * num_tiles;
  const int count = qsize > 0 ? clampi(knum[item], 0, num_tiles) : 0;

  const long kv_stride = (long)hkv * kD;
  const uint32_t stride_bytes = (uint32_t)kv_stride * 2u;
  const uint16_t* kbatch = k + (long)b * seq * kv_stride + hk * kD;
  const uint16_t* vbatch = v + (long)b * seq * kv_stride + hk * kD;
  const uint32_t ring = lds_u32(smem);
  const long qrow0 = (long)b * seq + (long)a * kBN;

  bf16x8 qr[QB];
  {
    const uint16_t* qp = q + ((qrow0 + r_c) * hq + h) * kD + L.g * 8;
#pragma unroll
    for (int db = 0; db < QB; ++db) qr[db] = as_bf16x8(ld_global16(qp + db * 16));
  }
  f32x16 o[OB];
#pragma unroll
  for (int i = 0; i < OB; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.f;
  }
  Softmax st{kNegInf, 0.f};
  f32x16 sa[1], sb[1];

  // This wave's share of a K or V tile: load blocks w*kSIPW .. +kSIPW-1. For a
  // full tile (size 64: every key real, wave-uniform) each lane's byte offset
  // within the tile is fixed, so it is computed once here and those loads take
  // no per-tile vector arithmetic; a partial tile clamps its rows to the last
  // real key.
  uint32_t boff[kSIPW];
  {
    const int piece = lane % G::kLanesPerRow;  // a pad piece re-reads the row's last real one
    const uint32_t pc = (uint32_t)(piece < G::kRowPieces ? piece : G::kRowPieces - 1) * 16u;
#pragma unroll
    for (int t = 0; t < kSIPW; ++t) {
      boff[t] = G::block_row_key((uint32_t)(w * kSIPW + t), (uint32_t)(lane / G::kLanesPerRow)) * stride_bytes + pc;
    }
  }
  auto issue = [&](const uint16_t* plane, const Entry& t, uint32_t stage_lds) {
    const uint16_t* tb = plane + (long)t.tile * kBN * kv_stride;
    if (t.size >= kBN) {
#pragma unroll
      for (int i = 0; i < kSIPW; ++i) load_lds16(tb, boff[i], stage_lds + (w * kSIPW + i) * kBlockBytes);
    } else {
      issue_tile<kD, kSIPW>(tb, stride_bytes, t.size, stage_lds, w * kSIPW, lane);
    }
  };
  auto issue_k = [&](const Entry& t, int stage) { issue(kbatch, t, ring + stage * kTileBytes); };
  auto issue_v = [&](const Entry& t, int stage) { issue(vbatch, t, ring + (2 + stage) * kTileBytes); };

  // The kept-tile list goes to LDS first: a list word read from memory inside
  // the loop would need a wait for its load there, and that wait also holds
  // for the ring loads issued earlier in the step (a vector load: vmcnt; a
  // scalar one: lgkmcnt, which every LDS wait also drains). Staged in LDS, a
  // refill waits only for LDS. (The launcher only sends tile counts up to
  // kListCap here.)
  for (int i = tid; i < count; i += 64 * kSW) lst[i] = list[i];
  __syncthreads();
  // A 64-entry window of the list sits in one VGPR (lane i holds entry
  // win_base + i) and entries are taken with v_readlane: one LDS read per 64
  // kept tiles instead of one per step, whose wait would otherwise sit in
  // every step right before the MFMA slots. Entries are asked for in
  // increasing order, so the window only moves forward.
  int win_base = 0;
  int32_t win = lst[lane];
  auto entry = [&](int j) -> int32_t {
    if (j >= win_base + 64) {
      win_base += 64;
      win = lst[win_base + lane];  // win_base + 63 < kListCap since j < count <= kListCap
    }
    return __builtin_amdgcn_readlane(win, j - win_base);
  };
  // entry of tile j (unpacked) and raw entries of tiles j+1, j+2: each list
  // word is read one step before its first use
  Entry cur{0, 1};
  int32_t n1 = 0, n2 = 0;
  if (count > 0) cur = unpack(entry(0), num_tiles);
  if (count > 1) n1 = entry(1);
  if (count > 2) n2 = entry(2);

  if (count > 0) {
    issue_k(cur, 0);
    if (count > 1) {
      issue_k(unpack(n1, num_tiles), 1);
      wait_loads_barrier<kSIPW>();  // K of tile 0 has landed
    } else {
      wait_loads_barrier<0>();
    }
    if (wave_live) qk<kD, 1>(smem, L, qr, sa);
  }
  settle_q(qr);

  // Pipelined step j: the softmax of tile j runs under the S^T MFMAs of tile
  // j+1 and the PV MFMAs of tile j-1. On entry K of tile j+1 and V of tile j-1
  // (issued one step earlier) must have landed, and every wave is done with K
  // of tile j (its S^T ran one step earlier) and V of tile j-2 (its PV ran one
  // step earlier): their stages (j & 1) receive K of tile j+2 and V of tile j.
  bf16x8 pa[2], pb[2];
  auto step = [&](int j, auto pv_tag, f32x16 (&s)[1], f32x16 (&sn)[1], bf16x8 (&pp)[2], bf16x8 (&pc)[2]) {
    constexpr bool HAS_PV = decltype(pv_tag)::value;
    wait_loads_barrier<0>();
    if (j + 2 < count) issue_k(unpack(n2, num_tiles), j & 1);
    issue_v(cur, j & 1);
    const int size = cur.size;
    cur = unpack(n1, num_tiles);
    n1 = n2;
    if (j + 3 < count) n2 = entry(j + 3);
    if (wave_live) {
      // after the last tile the "next" K stage holds stale data; its S^T is unused
      const char* nk = smem + ((j + 1) & 1) * kTileBytes;
      const uint32_t vt_prev = ring + (2 + ((j + 1) & 1)) * kTileBytes;  // V of tile j-1
      tile_step_pp1<D, HAS_PV>(s, sn, nk, vt_prev, L, qr, pp, pc, o, st, c, size < 32 * kh + 32, 32 * kh, size,
                               0x7fffffff);
    }
  };
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;
  if (count > 0) {
    // the loop runs at issue priority 1, its MFMA slots at 2 (tile_step_pp1);
    // prologue, merge and store stay at 0
    __builtin_amdgcn_s_setprio(1);
    step(0, no{}, sa, sb, pb, pa);
    for (int j = 1; j < count; j += 2) {
      step(j, yes{}, sb, sa, pa, pb);
      if (j + 1 < count) step(j + 1, yes{}, sa, sb, pb, pa);
    }
    // PV of the last tile (P of tile j sits in pa for even j, pb for odd j);
    // its V was issued in the last step
    wait_loads_barrier<0>();
    if (wave_live) {
      const uint32_t vt = ring + (2 + ((count - 1) & 1)) * kTileBytes;
      if ((count - 1) & 1) {
        pv<kD, 1>(vt, L, pb, o);
      } else {
        pv<kD, 1>(vt, L, pa, o);
      }
    }
  }

  __builtin_amdgcn_s_setprio(0);
  // merge the two key halves of each row: wave (rh, 1) hands its O^T block,
  // reference maximum and lane-partial sum to wave (rh, 0) through LDS
  wait_loads_barrier<0>();
  f32x4* mo = reinterpret_cast<f32x4*>(smem + rh * kMergeOBytes) + lane;
  float2* mml = reinterpret_cast<float2*>(smem + 2 * kMergeOBytes + rh * 512) + lane;
  if (kh == 1) {
#pragma unroll
    for (int i = 0; i < OB; ++i) {
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        f32x4 t;
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = o[i][4 * grp + e];
        mo[(4 * i + grp) * 64] = t;
      }
    }
    *mml = make_float2(st.m, st.l);
  }
  __syncthreads();
  if (kh == 1) return;
  const float2 ml = *mml;
  const float mm = fmaxf(st.m, ml.x);
  const float a0 = st.m == kNegInf ? 0.f : hw_exp2((st.m - mm) * c);
  const float a1 = ml.x == kNegInf ? 0.f : hw_exp2((ml.x - mm) * c);
#pragma unroll
  for (int i = 0; i < OB; ++i) {
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const f32x4 t = mo[(4 * i + grp) * 64];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[i][4 * grp + e] = o[i][4 * grp + e] * a0 + t[e] * a1;
    }
  }
  st.m = mm;
  st.l = r < qsize ? st.l * a0 + ml.y * a1 : 0.f;  // padding rows: zeros, LSE = -inf
  store_rows<OB>(o, st, L, c, true, out + ((qrow0 + r) * hq + h) * kD,
             lse != nullptr ? lse + ((long)b * hq + h) * seq + (long)a * kBN + r : nullptr);
}

}  // namespace

bool sparse_pipe_supported(int head_dim, int num_tiles) {
  return (head_dim == 96 || head_dim == 128 || head_dim == 192 || head_dim == 256) && num_tiles <= kSparsePipeMaxTiles;
}

template <int D>
static void launch_block_sparse_pipe_d(const SparseArgs& a, long n_items, long per_xcd, hipStream_t stream) {
  hipLaunchKernelGGL((block_sparse_pipe_kernel<D>), dim3((unsigned)(per_xcd * 8)), dim3(64 * kSW), 0, stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.tile_sizes, a.idx, a.num,
                     a.order, a.num_tiles, a.num_heads, a.num_kv_heads, (int)n_items, (int)per_xcd, a.scale * kLog2e,
                     (uint16_t*)a.out, a.lse);
}

hipError_t launch_block_sparse_pipe(const SparseArgs& a, hipStream_t stream) {
  const long n_items = (long)a.batch * a.num_heads * a.num_tiles;
  const long per_xcd = (n_items + 7) / 8;
  hipLaunchKernelGGL(order_items_kernel, dim3(8), dim3(kOrderThreads), 0, stream, a.num, (int)n_items, (int)per_xcd,
                     a.order);
  switch (a.head_dim) {
    case 96:
      launch_block_sparse_pipe_d<96>(a, n_items, per_xcd, stream);
      break;
    case 128:
      launch_block_sparse_pipe_d<128>(a, n_items, per_xcd, stream);
      break;
    case 192:
      launch_block_sparse_pipe_d<192>(a, n_items, per_xcd, stream);
      break;
    case 256:
      launch_block_sparse_pipe_d<256>(a, n_items, per_xcd, stream);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace attn
