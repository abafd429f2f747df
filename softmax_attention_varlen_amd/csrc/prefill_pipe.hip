// Pipelined varlen prefill for head dims 64 (non-causal), 96, 128, 192 and 256
// on gfx950.
//
// Work unit: one workgroup of NW waves owns NW*32 query rows of one document
// and one query head; wave w owns rows [32w, 32w+32). K/V tiles of 64 keys
// stream through a 4-stage LDS ring filled by direct-to-LDS loads (no VGPR
// staging, no transpose on the way in), in the bank-conflict-free layout of
// pipe.hpp. The loop is software-pipelined: it runs the softmax of tile j
// under the S^T MFMAs of tile j+1 and the PV MFMAs of tile j-1. One barrier
// per tile guards the ring. SPLIT replaces the ring by separate two-stage K
// and V rings (at step j, K of tile j+2 and V of tile j are in flight while K
// of tile j+1 and V of tile j-1 are read), which fit two 4-wave workgroups
// per CU at head_dims 64 to 128 (64 and 96 pad their rows to 256 bytes in
// LDS), and raises the issue priority of the loop (1) and of its MFMA slots
// (2) above the prologue and store (0). At head_dims 192 and 256 a tile takes
// twice the LDS (512-byte rows), so the split rings (130 KB) fit one 4-wave
// workgroup per CU, whose O (up to 8 accumulator blocks) and Q fragments (up
// to 16) take the whole register file of one wave per SIMD.
#include <type_traits>

#include "key_rows.hpp"
#include "launch.hpp"
#include "pipe.hpp"

namespace attn {
namespace {

using namespace pipe;

template <int D, int NW>
struct Ring {
  static constexpr int kTileBytes = Geom<D>::kTileBytes;
  static constexpr int kStageBytes = 2 * kTileBytes;     // K tile, then V tile
  static constexpr int IPW = Geom<D>::kBlocks / NW;      // load blocks per wave per K (or V) tile
  static constexpr int LOADS = 2 * IPW;                  // per wave per tile (K and V)
  static_assert(IPW * NW == Geom<D>::kBlocks, "waves must split the load blocks evenly");

  // Issue this wave's share of one K/V tile. kbase/vbase: first key row of the
  // tile (this kv head); rows >= nvalid re-read row nvalid-1.
  __device__ __forceinline__ static void issue(const uint16_t* kbase, const uint16_t* vbase, uint32_t stride_bytes,
                                               int nvalid, uint32_t stage_lds, int w, int lane) {
    issue_tile<D, IPW>(kbase, stride_bytes, nvalid, stage_lds, w * IPW, lane);
    issue_tile<D, IPW>(vbase, stride_bytes, nvalid, stage_lds + kTileBytes, w * IPW, lane);
  }
};

// Workgroups per CU: two at head_dims 96 and 128 on the split rings, else one.
template <int D, bool SPLIT>
constexpr int kWgPerCu = (SPLIT && D <= 128) ? 2 : 1;

// PAGED: keys come from a paged cache (k, v = its K and V planes) through
// block_tables, with context_lens[doc] (clamped to max_len_k) keys per
// document; otherwise from contiguous rows delimited by cu_k. q_used / k_used
// (nullable) cut each document to a valid prefix of its rows.
template <int D, bool CAUSAL, bool PAGED, int NW, bool SPLIT>
__global__ __launch_bounds__(64 * NW, (kWgPerCu<D, SPLIT>)) void prefill_pipe_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch, int total_q, int total_k,
    int tiles_per_doc, int hq, int hkv, int n_items, int per_xcd, float c, uint16_t* __restrict__ out,
    float* __restrict__ lse, const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    int max_blocks_per_seq, int num_blocks, int max_len_k, const int32_t* __restrict__ q_used,
    const int32_t* __restrict__ k_used) {
  using R = Ring<D, NW>;
  constexpr int kTileBytes = R::kTileBytes, kStageBytes = R::kStageBytes;
  constexpr int QB = Geom<D>::kQB, OB = Geom<D>::kOB;
  constexpr int BM = 32 * NW;
  // the pipelined loop keeps tile j-1's V while tile j+2 loads: 4 stages of K
  // and V; SPLIT: separate two-stage K and V rings (K stages 0, 1, then V
  // stages 0, 1)
  __shared__ __attribute__((aligned(1024))) char smem[SPLIT ? 4 * kTileBytes : 4 * kStageBytes];

  // XCD-aware order: the hardware deals workgroups round-robin over 8 XCDs, so
  // XCD x receives logical items [x*per_xcd, (x+1)*per_xcd), laid out
  // kv-head-major so that one XCD's L2 serves the K/V of its kv heads.
  const int hw = blockIdx.x;
  const int item = (hw & 7) * per_xcd + (hw >> 3);
  if (item >= n_items) return;
  const int group = hq / hkv;
  int rest = item;
  const int qh = rest % group;
  rest /= group;
  // within a kv head, documents one after the other (the workgroups running at
  // once on an XCD then share one document's K/V in its L2), and in each
  // document the query tiles from the last (heaviest under a causal mask) to
  // the first
  const int tile = tiles_per_doc - 1 - rest % tiles_per_doc;
  rest /= tiles_per_doc;
  const int doc = rest % batch;
  const int hk = rest / batch;
  const int h = hk * group + qh;

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
  const int m0 = tile * BM;
  if (m0 >= len_q) return;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const Lane L = make_lane<D>(lane);
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

  const uint32_t stride_bytes = (uint32_t)hkv * D * 2u;
  const uint16_t* kb0 = k + ((long)k0 * hkv + hk) * D;
  const uint16_t* vb0 = v + ((long)k0 * hkv + hk) * D;
  const KeyRows<PAGED> rows{(long)hkv * D, PAGED ? block_tables + (long)doc * max_blocks_per_seq : nullptr,
                            num_blocks};
  const uint32_t ring = lds_u32(smem);
  constexpr bool kLateLoads = SPLIT && D > 128;

  // Q into registers first (the compiler's wait for these also covers the
  // ring loads issued after them, which the first tile needs anyway)
  bf16x8 qr[QB];
  {
    const uint16_t* qp = q + ((long)(q0 + row_c) * hq + h) * D + L.g * 8;
#pragma unroll
    for (int b = 0; b < QB; ++b) qr[b] = as_bf16x8(ld_global16(qp + b * 16));
  }
  // prologue: the first two tiles in flight
  constexpr int PRE = 2;
#pragma unroll
  for (int s = 0; s < PRE; ++s) {
    if (SPLIT) {
      if (s < ntiles) {
        const long off = rows.row(s * kBN);
        issue_tile<D, R::IPW>(kb0 + off, stride_bytes, len_k - s * kBN, ring + s * kTileBytes, w * R::IPW, lane);
      }
    } else if (s < ntiles) {
      const long off = rows.row(s * kBN);
      R::issue(kb0 + off, vb0 + off, stride_bytes, len_k - s * kBN, ring + s * kStageBytes, w, lane);
    }
  }
  f32x16 o[OB];
#pragma unroll
  for (int b = 0; b < OB; ++b) {
#pragma unroll
    for (int r = 0; r < 16; ++r) o[b][r] = 0.f;
  }
  Softmax st{kNegInf, 0.f};
  f32x16 sa[2], sb[2];

  if (ntiles > 0) {
    // tile 0 has landed once at most the later prologue tiles are in flight
    const int later = (ntiles < PRE ? ntiles : PRE) - 1;
    if (SPLIT) {
      if (later >= 1) {
        wait_loads_barrier<R::IPW>();
      } else {
        wait_loads_barrier<0>();
      }
    } else if (later == 1) {
      wait_loads_barrier<R::LOADS>();
    } else {
      wait_loads_barrier<0>();
    }
    if (ntiles_w > 0) qk<D, 2>(smem, L, qr, sa);
  }
  settle_q(qr);

  {
    // Pipelined loop: step j runs the softmax of tile j under the S^T MFMAs of
    // tile j+1 and the PV MFMAs of tile j-1. Tile j+2 is issued at step j into
    // the stage of tile j-2, whose PV every wave finished in step j-1 (the
    // barrier); tile j-1's V stays resident through step j.
    bf16x8 pa[4], pb[4];
    auto step = [&](int j, auto pv_tag, f32x16 (&s)[2], f32x16 (&sn)[2], bf16x8 (&pp)[4], bf16x8 (&pc)[4]) {
      constexpr bool HAS_PV = decltype(pv_tag)::value;
      uint32_t vt_prev;
      const char* nk;
      // SPLIT at head_dims 192/256 (one workgroup per CU): a wave with a tile
      // to process issues its loads from inside the step, in its first slots,
      // under the MFMAs (see below); before the step they had nothing to hide
      // under (+3 % at 192, +8 % at 256)
      const bool late = kLateLoads && j < ntiles_w;
      if (SPLIT) {
        // K of tile j+2 into the K stage of tile j (its S^T ran in step j-1),
        // V of tile j into the V stage of tile j-2 (its PV ran in step j-1)
        wait_loads_barrier<0>();
      }
      if (SPLIT && !late) {
        if (j + 2 < ntiles) {
          const long off = rows.row((j + 2) * kBN);
          issue_tile<D, R::IPW>(kb0 + off, stride_bytes, len_k - (j + 2) * kBN, ring + (j & 1) * kTileBytes,
                                w * R::IPW, lane);
        }
        {
          const long off = rows.row(j * kBN);
          issue_tile<D, R::IPW>(vb0 + off, stride_bytes, len_k - j * kBN, ring + (2 + (j & 1)) * kTileBytes,
                                w * R::IPW, lane);
        }
      }
      if (SPLIT) {
        vt_prev = ring + (2 + ((j + 1) & 1)) * kTileBytes;
        nk = smem + ((j + 1) & 1) * kTileBytes;
      } else {
        if (j + 1 < ntiles) {
          wait_loads_barrier<0>();  // tile j+1 (issued at step j-1) has landed everywhere
          const int jn = j + 2;
          if (jn < ntiles) {
            const long off = rows.row(jn * kBN);
            R::issue(kb0 + off, vb0 + off, stride_bytes, len_k - jn * kBN, ring + (jn % 4) * kStageBytes, w, lane);
          }
        }
        vt_prev = ring + ((j + 3) % 4) * kStageBytes + kTileBytes;  // V of tile j-1
        nk = smem + ((j + 1 < ntiles ? j + 1 : j) % 4) * kStageBytes;
      }
      if (j < ntiles_w) {
        const int key0 = j * kBN;
        const bool mask = !(j < nomask_w && key0 + kBN <= len_k);
        if constexpr (kLateLoads) {
          // past the last tile the K loads re-read tile j into its own stage
          // (free, and read by nothing after), which keeps branches out of
          // the slots
          const int jk = j + 2 < ntiles ? j + 2 : j;
          const uint16_t* kt = uniform_ptr(kb0 + rows.row(jk * kBN));
          const uint16_t* vtile = uniform_ptr(vb0 + rows.row(j * kBN));
          const int k_valid = len_k - jk * kBN, v_valid = len_k - j * kBN;
          const uint32_t k_lds = ring + (j & 1) * kTileBytes, v_lds = ring + (2 + (j & 1)) * kTileBytes;
          // load i (K blocks, then V blocks) in slot i at head_dim 192 and in
          // slot 2i + 1 at 256 (measured against each other and against
          // spreading the loads over the whole step, which left them too
          // little time to land: -5 to -6 %)
          constexpr int kGap = D == 256 ? 2 : 1;
          auto loads = [&](auto slot_c) __attribute__((always_inline)) {
            constexpr int slot = decltype(slot_c)::value;
            constexpr int i = (slot - (kGap - 1)) / kGap;
            if constexpr (slot >= kGap - 1 && (slot - (kGap - 1)) % kGap == 0 && i < 2 * R::IPW) {
              if constexpr (i < R::IPW) {
                issue_block<D>(kt, stride_bytes, k_valid, k_lds, w * R::IPW + i, lane);
              } else {
                issue_block<D>(vtile, stride_bytes, v_valid, v_lds, w * R::IPW + i - R::IPW, lane);
              }
            }
          };
          tile_step_pp<D, HAS_PV, SPLIT>(s, sn, nk, vt_prev, L, qr, pp, pc, o, st, c, mask, key0, len_k,
                                         CAUSAL ? row + diag : 0x7fffffff, loads);
        } else {
          tile_step_pp<D, HAS_PV, SPLIT>(s, sn, nk, vt_prev, L, qr, pp, pc, o, st, c, mask, key0, len_k,
                                         CAUSAL ? row + diag : 0x7fffffff);
        }
      } else if (HAS_PV && j == ntiles_w) {
        pv<D, 2>(vt_prev, L, pp, o);  // this wave's last tile
      }
    };
    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;
    if (ntiles > 0) {
      // SPLIT: the loop runs at issue priority 1 and its MFMA slots at 2, so
      // the other workgroup's prologue and store (at 0) yield to them
      if constexpr (SPLIT) __builtin_amdgcn_s_setprio(1);
      step(0, no{}, sa, sb, pb, pa);
      for (int j = 1; j < ntiles; j += 2) {
        step(j, yes{}, sb, sa, pa, pb);
        if (j + 1 < ntiles) step(j + 1, yes{}, sa, sb, pb, pa);
      }
      if (SPLIT) wait_loads_barrier<0>();  // V of the last tile was issued in the last step
      if (ntiles_w == ntiles) {  // the last tile's PV (its stage is never refilled)
        const uint32_t vt = SPLIT ? ring + (2 + ((ntiles - 1) & 1)) * kTileBytes
                                  : ring + ((ntiles - 1) % 4) * kStageBytes + kTileBytes;
        if ((ntiles - 1) & 1) {
          pv<D, 2>(vt, L, pb, o);
        } else {
          pv<D, 2>(vt, L, pa, o);
        }
      }
    }
    if constexpr (SPLIT) __builtin_amdgcn_s_setprio(0);
    store_rows<OB>(o, st, L, c, row < len_q, out + ((long)(q0 + row_c) * hq + h) * D,
               lse != nullptr ? lse + (long)h * total_q + q0 + row_c : nullptr);
  }
}

}  // namespace

// head_dim 64 only without the causal mask: its 16-slot step measured +10 %
// dense and -6 % causal against the register-staged kernel.
bool prefill_pipe_supported(const VarlenArgs& a) {
  return a.head_dim == 96 || a.head_dim == 128 || a.head_dim == 192 || a.head_dim == 256 ||
         (a.head_dim == 64 && !a.causal);
}

// head_dims 96 and 128, keys from contiguous rows: 4-wave workgroups (128
// query rows) on split two-stage K and V rings (66.5 KB), two workgroups per
// CU out of phase, so one workgroup's prologue and store run under the other's
// loop, with the loop at raised issue priority. Keys from the paged cache:
// 8-wave workgroups (256 rows) on the 4-stage ring, one per CU, which copies
// each K/V tile into LDS for twice as many rows. head_dims 192 and 256: 4-wave
// workgroups on the split rings (130 KB), one per CU, for both.
template <int D, bool CAUSAL, bool PAGED>
static void launch_prefill_pipe_t(const VarlenArgs& a, hipStream_t stream) {
  constexpr bool SPLIT = !PAGED || D > 128;
  constexpr int NW = SPLIT ? 4 : 8;
  constexpr int BM = 32 * NW;
  const int tiles = (a.max_seqlen_q + BM - 1) / BM;
  const long n_items = (long)tiles * a.batch * a.num_heads;
  const long per_xcd = (n_items + 7) / 8;
  const float c = a.scale * kLog2e;
  hipLaunchKernelGGL((prefill_pipe_kernel<D, CAUSAL, PAGED, NW, SPLIT>),
                     dim3((unsigned)(per_xcd * 8)), dim3(64 * NW), 0, stream, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, a.cu_q, a.cu_k, a.batch, a.total_q, a.total_k, tiles,
                     a.num_heads, a.num_kv_heads, (int)n_items, (int)per_xcd, c, (uint16_t*)a.out, a.lse,
                     a.block_tables, a.context_lens, a.max_blocks_per_seq, a.num_blocks, a.max_seqlen_k, a.q_used,
                     PAGED ? nullptr : a.k_used);
}

template <int D>
static void launch_prefill_pipe_d(const VarlenArgs& a, hipStream_t stream) {
  if constexpr (D == 64) {  // non-causal contiguous keys only (prefill_pipe_supported)
    launch_prefill_pipe_t<64, false, false>(a, stream);
    return;
  }
  if (a.paged) {
    if (a.causal) {
      launch_prefill_pipe_t<D, true, true>(a, stream);
    } else {
      launch_prefill_pipe_t<D, false, true>(a, stream);
    }
  } else if (a.causal) {
    launch_prefill_pipe_t<D, true, false>(a, stream);
  } else {
    launch_prefill_pipe_t<D, false, false>(a, stream);
  }
}

hipError_t launch_prefill_pipe(const VarlenArgs& a, hipStream_t stream) {
  switch (a.head_dim) {
    case 64:
      launch_prefill_pipe_d<64>(a, stream);
      break;
    case 96:
      launch_prefill_pipe_d<96>(a, stream);
      break;
    case 128:
      launch_prefill_pipe_d<128>(a, stream);
      break;
    case 192:
      launch_prefill_pipe_d<192>(a, stream);
      break;
    case 256:
      launch_prefill_pipe_d<256>(a, stream);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace attn
