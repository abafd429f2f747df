// Pipelined varlen prefill for head_dim 128 on gfx950.
//
// Work unit: one workgroup of NW waves owns NW*32 query rows of one document
// and one query head; wave w owns rows [32w, 32w+32). K/V tiles of 64 keys
// stream through an NS-stage LDS ring:
//   * global -> LDS with direct-to-LDS 16-byte loads (no VGPR staging, no
//     transpose on the way in). Load block b (16 per tile) is one contiguous
//     1 KB holding the four keys κ(b) + {0, 16, 32, 48}; blocks sit 1040 bytes
//     apart (16 bytes = 4 banks of pad). Key k%16 = (b3 b2 b1 b0) lives in
//     block (b1 b0 b3 b2). A 16-lane slice of a K read then covers the 16
//     blocks (all 64 banks once), and a 32-lane slice of a transposing V read
//     (4 keys x 64 bytes) puts its 4 rows 16 banks apart: both conflict-free on
//     gfx950's 64-bank LDS, as measured. Every LDS address is a per-lane base
//     plus a compile-time offset.
//   * K is read row-wise (ds_read_b128) as the A operand of S^T = K Q^T.
//   * V stays row-major and is read with the transposing ds_read_b64_tr_b16,
//     which hands each lane four keys of one column: exactly the k-slot layout
//     of the A operand of O^T += V^T P^T.
// Per tile a wave issues the S^T MFMAs of the next tile interleaved with the
// softmax of the current one (the scheduler is asked for that interleave), so
// the VALU/transcendental work runs while the matrix unit is busy; then it
// issues the PV MFMAs of the current tile. One barrier per tile guards the
// ring. The output accumulator is only rescaled when some row maximum grows by
// more than 2^8 (in exp2 units); until then the stale maximum keeps every exp2
// argument <= 8, exact up to rounding.
#include "attn_common.hpp"
#include "launch.hpp"

namespace attn {
namespace {

constexpr int kD = 128;
constexpr int kBN = 64;
constexpr int kRowBytes = kD * 2;             // 256 B per K/V row
constexpr int kBlockBytes = 1040;             // one 1 KB load block + 16 B pad
constexpr int kTileBytes = 16 * kBlockBytes;  // 16 blocks of 4 rows per K (or V) tile
constexpr int kStageBytes = 2 * kTileBytes;   // K tile, then V tile
constexpr float kRescaleThreshold = 8.f;      // log2 units

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// LDS block of key k (0..15 within its group of 16): bits (b3 b2 b1 b0) -> (b1 b0 b3 b2).
__device__ __forceinline__ uint32_t key_block(uint32_t k) { return ((k & 3u) << 2) | ((k >> 2) & 3u); }
// The key held by LDS block b (the same 2-bit rotation undoes itself).
__device__ __forceinline__ uint32_t block_key(uint32_t b) { return ((b & 3u) << 2) | ((b >> 2) & 3u); }
// Byte offset of 16-byte chunk `ch` of key `key` inside a K or V tile.
__device__ __forceinline__ uint32_t tile_off(uint32_t key, uint32_t ch) {
  return key_block(key & 15u) * kBlockBytes + (key >> 4) * kRowBytes + ch * 16u;
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One 16-byte-per-lane direct-to-LDS load: lane l's bytes land at lds + 16*l.
__device__ __forceinline__ void load_lds16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}

// Wait until at most N of this wave's direct-to-LDS loads are in flight, drain
// its LDS reads, and meet the other waves.
template <int N>
__device__ __forceinline__ void wait_loads_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

// max / sum of a lane's value and lane (l ^ 32)'s, via one lane swap.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int NW>
struct Ring {
  static constexpr int IPW = 16 / NW;    // load blocks per wave per K (or V) tile
  static constexpr int LOADS = 2 * IPW;  // per wave per tile (K and V)
  static_assert(IPW * NW == 16, "waves must split the 16 load blocks evenly");

  // Issue this wave's share of one K/V tile. kbase/vbase: first key row of the
  // tile (this kv head); rows >= nvalid re-read row nvalid-1.
  __device__ __forceinline__ static void issue(const uint16_t* kbase, const uint16_t* vbase, uint32_t stride_bytes,
                                               int nvalid, uint32_t stage_lds, int w, int lane) {
#pragma unroll
    for (int t = 0; t < IPW; ++t) {
      const int blk = w * IPW + t;
      const int key = (int)block_key((uint32_t)blk) + 16 * (lane >> 4);
      const int kc = key < nvalid ? key : nvalid - 1;
      const uint32_t voff = (uint32_t)kc * stride_bytes + (uint32_t)(lane & 15) * 16u;
      const uint32_t lds = __builtin_amdgcn_readfirstlane(stage_lds + blk * kBlockBytes);
      load_lds16(kbase, voff, lds);
      load_lds16(vbase, voff, lds + kTileBytes);
    }
  }
};

// Per-lane LDS read bases.
struct Lane {
  uint32_t k_base;  // K A operand for key 32kb + n, d = 16db + 8g: k_base + 512kb + 32db
  uint32_t v_base;  // transposing read (c, h, b): v_base + 2080h + 256c + 64b
  int n, g;
};

__device__ __forceinline__ Lane make_lane(int lane) {
  Lane L;
  L.n = lane & 31;
  L.g = lane >> 5;
  L.k_base = tile_off((uint32_t)L.n, (uint32_t)L.g);
  // source lane (G, s) of a transposing read points at key 16c + 8h + 4(G/2) + s/4,
  // columns 32b + 16(G%2) + 4(s%4) .. +3
  const uint32_t G = (uint32_t)lane >> 4, s = (uint32_t)lane & 15u;
  L.v_base = tile_off(4u * (G >> 1) + (s >> 2), 2u * (G & 1u) + ((s & 3u) >> 1)) + (s & 1u) * 8u;
  return L;
}

// O^T (128 d x 32 queries) += V^T P^T for one tile. P chunk c holds keys
// 16c + 8*(i/4) + 4g + i%4 in k-slot (g, i); the transposing reads deliver the
// matching V columns (key + 8 sits two LDS blocks further: + 2080 bytes).
__device__ __forceinline__ void pv(uint32_t vt, const Lane& L, const bf16x8 (&p)[4], f32x16 (&o)[4]) {
  const lds_bf16x4* base = (const lds_bf16x4*)(vt + L.v_base);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      // byte offsets 2080h + 256c + 64b, in 8-byte units
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + 32 * c + 8 * b));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + 260 + 32 * c + 8 * b));
      const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      o[b] = mfma32x32x16(a, p[c], o[b]);
    }
  }
}

// S^T for one tile: s[kb] = keys 32kb..32kb+31 x the wave's 32 queries.
__device__ __forceinline__ void qk(const char* kt, const Lane& L, const bf16x8 (&q)[8], f32x16 (&s)[2]) {
  const char* base = kt + L.k_base;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
  }
#pragma unroll
  for (int db = 0; db < 8; ++db) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 a = ld_lds16(base, kb * 2 * kRowBytes + db * 32);
      s[kb] = mfma32x32x16(a, q[db], s[kb]);
    }
  }
}

struct Softmax {
  float m;  // reference maximum of the raw scores (the exp2 shift is m * c)
  float l;  // lane-partial sum of the unrounded probabilities
};

// One tile: masking of `s` when some key of the tile is hidden from some row
// of the wave (a wave-uniform branch), the row maximum, then 16 steps that
// each issue one S^T MFMA of the next tile (K operand prefetched four steps
// ahead; after the last tile the result is not used) next to two exp2 of this
// tile, so the transcendental/VALU work runs under the matrix unit; a
// scheduling fence between steps keeps that order. Then O += V^T P^T.
__device__ __forceinline__ void tile_step(f32x16 (&s)[2], f32x16 (&sn)[2], const char* nk, uint32_t vt,
                                          const Lane& L, const bf16x8 (&q)[8], f32x16 (&o)[4], Softmax& st,
                                          float c, bool mask, int key0, int len_k, int lim) {
  if (mask) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * L.g + (r & 3);
        if (key >= len_k || key > lim) s[kb][r] = kNegInf;
      }
    }
  }
  // row maximum over the lane's 32 keys, four independent chains
  float mx4[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) mx4[t] = fmaxf(s[t >> 1][8 * (t & 1)], s[t >> 1][8 * (t & 1) + 1]);
#pragma unroll
  for (int i = 2; i < 8; ++i) {
#pragma unroll
    for (int t = 0; t < 4; ++t) mx4[t] = fmaxf(mx4[t], s[t >> 1][8 * (t & 1) + i]);
  }
  const float mx = pair_max(fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3])));
  const float m_new = fmaxf(st.m, mx);
  const bool need = (m_new - st.m) * c > kRescaleThreshold;  // true on the first finite maximum
  const float alpha = need ? hw_exp2((st.m - m_new) * c) : 1.f;
  const float m_ref = need ? m_new : st.m;
  const float ms = (m_ref == kNegInf ? 0.f : m_ref) * c;

  // step i: MFMA (db = i/2, kb = i%2) of the next tile, and elements 2i, 2i+1
  // of this tile (P chunk t = i/4 collects 8 of them)
  const char* kbase = nk + L.k_base;
  bf16x8 kr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) kr[i] = ld_lds16(kbase, (i & 1) * 2 * kRowBytes + (i >> 1) * 32);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sn[kb][r] = 0.f;
  }
  bf16x8 p[4];
  f32x8 e;
  float rs0 = 0.f, rs1 = 0.f;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int db = i >> 1, kb = i & 1;
    sn[kb] = mfma32x32x16(kr[i & 3], q[db], sn[kb]);
    if (i + 4 < 16) kr[i & 3] = ld_lds16(kbase, ((i + 4) & 1) * 2 * kRowBytes + ((i + 4) >> 1) * 32);
    const int t = i >> 2, u = 2 * (i & 3);
    e[u] = hw_exp2(__builtin_fmaf(s[t >> 1][8 * (t & 1) + u], c, -ms));
    e[u + 1] = hw_exp2(__builtin_fmaf(s[t >> 1][8 * (t & 1) + u + 1], c, -ms));
    rs0 += e[u];
    rs1 += e[u + 1];
    if ((i & 3) == 3) p[t] = to_bf16x8(e);
    __builtin_amdgcn_sched_barrier(0);
  }
  const float rs = rs0 + rs1;
  st.l = st.l * alpha + rs;
  st.m = m_ref;
  // Rare rescale of O. The row sum takes part in the condition (it is never
  // NaN for finite inputs) so that the exp2 above stay interleaved with the
  // MFMAs instead of being sunk past the branch.
  if (__builtin_amdgcn_ballot_w64(need || rs != rs) != 0ull) {
#pragma unroll
    for (int b = 0; b < 4; ++b) o[b] *= alpha;
  }
  pv(vt, L, p, o);
}

template <bool CAUSAL, int NW, int NS>
__global__ __launch_bounds__(64 * NW) void prefill_d128_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch, int total_q, int total_k,
    int tiles_per_doc, int hq, int hkv, int n_items, int per_xcd, float c, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  using R = Ring<NW>;
  constexpr int BM = 32 * NW;
  static_assert(NS == 3 || NS == 4, "the load-count waits below cover 3- and 4-stage rings");
  __shared__ __attribute__((aligned(1024))) char smem[NS * kStageBytes];

  // XCD-aware order: the hardware deals workgroups round-robin over 8 XCDs, so
  // XCD x receives logical items [x*per_xcd, (x+1)*per_xcd), laid out
  // kv-head-major so that one XCD's L2 serves the K/V of its kv heads, and
  // every XCD gets the same mix of documents.
  const int hw = blockIdx.x;
  const int item = (hw & 7) * per_xcd + (hw >> 3);
  if (item >= n_items) return;
  const int group = hq / hkv;
  int rest = item;
  const int qh = rest % group;
  rest /= group;
  const int tile = tiles_per_doc - 1 - rest % tiles_per_doc;  // heaviest (last) tiles first
  rest /= tiles_per_doc;
  const int doc = rest % batch;
  const int hk = rest / batch;
  const int h = hk * group + qh;

  const int q0 = clampi(cu_q[doc], 0, total_q);
  const int q1 = clampi(cu_q[doc + 1], q0, total_q);
  const int k0 = clampi(cu_k[doc], 0, total_k);
  const int k1 = clampi(cu_k[doc + 1], k0, total_k);
  const int len_q = q1 - q0, len_k = k1 - k0;
  const int m0 = tile * BM;
  if (m0 >= len_q) return;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const Lane L = make_lane(lane);
  const int diag = len_k - len_q;
  const int row = m0 + w * 32 + L.n;
  const int row_c = row < len_q ? row : len_q - 1;
  const int wrow0 = m0 + w * 32;
  const bool wave_live = wrow0 < len_q;

  // key tiles the workgroup streams; the last one this wave needs; and how
  // many of them are visible to every row of this wave (no mask needed)
  int n_end = len_k, n_end_w = len_k, n_full_w = len_k;
  if (CAUSAL) {
    const int lim = m0 + BM + diag;
    n_end = lim < n_end ? lim : n_end;
    const int limw = wrow0 + 32 + diag;
    n_end_w = limw < n_end_w ? limw : n_end_w;
    const int full = wrow0 + diag + 1;  // keys < full are visible to every row of the wave
    n_full_w = full < n_full_w ? full : n_full_w;
  }
  n_end = n_end < 0 ? 0 : n_end;
  n_end_w = (n_end_w < 0 || !wave_live) ? 0 : n_end_w;
  const int ntiles = (n_end + kBN - 1) / kBN;
  const int ntiles_w = (n_end_w + kBN - 1) / kBN;
  const int nomask_w = n_full_w < 0 ? 0 : n_full_w / kBN;

  const uint32_t stride_bytes = (uint32_t)hkv * kD * 2u;
  const uint16_t* kb0 = k + ((long)k0 * hkv + hk) * kD;
  const uint16_t* vb0 = v + ((long)k0 * hkv + hk) * kD;
  const uint32_t ring = lds_u32(smem);

  // Q into registers first (the compiler's wait for these also covers the
  // ring loads issued after them, which the first tile needs anyway)
  bf16x8 qr[8];
  {
    const uint16_t* qp = q + ((long)(q0 + row_c) * hq + h) * kD + L.g * 8;
#pragma unroll
    for (int b = 0; b < 8; ++b) qr[b] = as_bf16x8(ld_global16(qp + b * 16));
  }
  // prologue: the first NS-1 tiles in flight
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) {
    if (s < ntiles) {
      const long off = (long)s * kBN * hkv * kD;
      R::issue(kb0 + off, vb0 + off, stride_bytes, len_k - s * kBN, ring + s * kStageBytes, w, lane);
    }
  }
  f32x16 o[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
#pragma unroll
    for (int r = 0; r < 16; ++r) o[b][r] = 0.f;
  }
  Softmax st{kNegInf, 0.f};
  f32x16 sa[2], sb[2];

  if (ntiles > 0) {
    // tile 0 has landed once at most the later prologue tiles are in flight
    const int later = (ntiles < NS - 1 ? ntiles : NS - 1) - 1;
    if (later >= 2) {
      wait_loads_barrier<2 * R::LOADS>();
    } else if (later == 1) {
      wait_loads_barrier<R::LOADS>();
    } else {
      wait_loads_barrier<0>();
    }
    if (ntiles_w > 0) qk(smem, L, qr, sa);
  }

  // one iteration of the ring: refill, then this wave's compute for tile j
  auto iteration = [&](int j, f32x16 (&s)[2], f32x16 (&sn)[2]) {
    if (j + 1 < ntiles) {
      if (NS >= 4 && j + 2 < ntiles) {
        wait_loads_barrier<(NS - 3) * R::LOADS>();
      } else {
        wait_loads_barrier<0>();
      }
      const int jn = j + NS - 1;
      if (jn < ntiles) {
        const long off = (long)jn * kBN * hkv * kD;
        R::issue(kb0 + off, vb0 + off, stride_bytes, len_k - jn * kBN, ring + (jn % NS) * kStageBytes, w, lane);
      }
    }
    if (j >= ntiles_w) return;
    // the next tile's K (after this wave's last tile: any resident stage; the
    // result is not used)
    const char* nk = smem + ((j + 1 < ntiles ? j + 1 : j) % NS) * kStageBytes;
    const uint32_t vt = ring + (j % NS) * kStageBytes + kTileBytes;
    const int key0 = j * kBN;
    const bool mask = !(j < nomask_w && key0 + kBN <= len_k);
    tile_step(s, sn, nk, vt, L, qr, o, st, c, mask, key0, len_k, CAUSAL ? row + diag : 0x7fffffff);
  };
  for (int j = 0; j < ntiles; j += 2) {
    iteration(j, sa, sb);
    if (j + 1 < ntiles) iteration(j + 1, sb, sa);
  }

  const float lt = pair_sum(st.l);
  if (row < len_q) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* orow = out + ((long)(q0 + row) * hq + h) * kD;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        f32x4 t;
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] = o[b][4 * grp + i] * inv;
        *reinterpret_cast<bf16x4*>(orow + b * 32 + 8 * grp + 4 * L.g) = to_bf16x4(t);
      }
    }
    if (lse != nullptr && L.g == 0) {
      lse[(long)h * total_q + q0 + row] = lt > 0.f ? (st.m * c + hw_log2(lt)) * kLn2 : kNegInf;
    }
  }
}

}  // namespace

constexpr int kPrefillWaves = 8;
constexpr int kPrefillStages = 3;

bool prefill_d128_supported(const VarlenArgs& a) { return a.head_dim == 128; }

hipError_t launch_prefill_d128(const VarlenArgs& a, hipStream_t stream) {
  constexpr int BM = 32 * kPrefillWaves;
  const int tiles = (a.max_seqlen_q + BM - 1) / BM;
  const long n_items = (long)tiles * a.batch * a.num_heads;
  const long per_xcd = (n_items + 7) / 8;
  const float c = a.scale * kLog2e;
  const dim3 grid((unsigned)(per_xcd * 8)), block(64 * kPrefillWaves);
  if (a.causal) {
    hipLaunchKernelGGL((prefill_d128_kernel<true, kPrefillWaves, kPrefillStages>), grid, block, 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.cu_q, a.cu_k, a.batch,
                       a.total_q, a.total_k, tiles, a.num_heads, a.num_kv_heads, (int)n_items, (int)per_xcd, c,
                       (uint16_t*)a.out, a.lse);
  } else {
    hipLaunchKernelGGL((prefill_d128_kernel<false, kPrefillWaves, kPrefillStages>), grid, block, 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.cu_q, a.cu_k, a.batch,
                       a.total_q, a.total_k, tiles, a.num_heads, a.num_kv_heads, (int)n_items, (int)per_xcd, c,
                       (uint16_t*)a.out, a.lse);
  }
  return hipGetLastError();
}

}  // namespace attn
