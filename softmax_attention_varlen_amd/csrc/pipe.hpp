// Building blocks of the pipelined attention kernels on gfx950: dense/varlen
// prefill at head dims 64 (without the causal mask), 96, 128, 192 and 256, and
// 64-token block-sparse attention at 96 to 256.
//
// LDS tile layout. A K (or V) tile holds 64 keys and is filled by
// direct-to-LDS 16-byte loads, each writing one contiguous 1 KB load block.
// A key's row takes 256 bytes in LDS at head dims up to 128 and 512 at 192
// and 256 (64, 96 and 192 pad their rows; a pad piece re-reads the row's last
// real 16 bytes), so a block holds 4 or 2 rows. Blocks sit 1040
// bytes apart (16 bytes = 4 banks of pad). Keys go in groups of 16: within a
// group, key k%16 = (b3 b2 b1 b0) lives in block (b1 b0 b3 b2) of a run of 16
// blocks; with 256-byte rows the four groups are the four rows of those 16
// blocks, with 512-byte rows groups 0 and 1 take rows 0 of two runs of 16
// blocks and groups 2 and 3 their rows 1. A 16-lane slice of a K read then covers 16 blocks of
// one run (all 64 banks once), and a 32-lane slice of a transposing V read
// (4 keys x 64 bytes) puts its 4 rows 16 banks apart: both conflict-free on
// gfx950's 64-bank LDS, as measured at head_dim 128. Every LDS address is a
// per-lane base plus a compile-time offset.
//
// Per 32x32 block the orientation is S^T = K Q^T: a lane owns one query (its
// row of S is spread over the lane and lane^32), K is read row-wise
// (ds_read_b128) as the A operand, and V stays row-major and is read with the
// transposing ds_read_b64_tr_b16, which hands each lane four keys of one
// column: exactly the k-slot layout of the A operand of O^T += V^T P^T.
#pragma once
#include <utility>

#include "attn_common.hpp"

namespace attn {
namespace pipe {

// f(std::integral_constant<int, i>) for i = 0 .. N-1, in order, each call a
// compile-time instance.
template <typename F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

constexpr int kBN = 64;                       // keys per LDS tile
constexpr int kBlockBytes = 1040;             // one 1 KB load block + 16 B pad
constexpr int kHalfBytes = 512;               // keys 32..63 of a tile sit 512 B after keys 0..31
constexpr float kRescaleThreshold = 8.f;      // log2 units

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// LDS block of key k (0..15 within its group of 16): bits (b3 b2 b1 b0) -> (b1 b0 b3 b2).
__device__ __forceinline__ constexpr uint32_t key_block(uint32_t k) { return ((k & 3u) << 2) | ((k >> 2) & 3u); }
// The key held by LDS block b (the same 2-bit rotation undoes itself).
__device__ __forceinline__ constexpr uint32_t block_key(uint32_t b) { return ((b & 3u) << 2) | ((b >> 2) & 3u); }
// Tile geometry for head dim D.
template <int D>
struct Geom {
  static_assert(D == 64 || D == 96 || D == 128 || D == 192 || D == 256, "head dims 64 to 256");
  static constexpr int kRowLds = D <= 128 ? 256 : 512;     // LDS bytes of one key row (192 padded to 512)
  static constexpr int kRowsPerBlock = 1024 / kRowLds;      // 4 or 2
  static constexpr int kBlocks = 64 / kRowsPerBlock;        // load blocks per tile: 16 or 32
  static constexpr int kRuns = kBlocks / 16;                // runs of 16 blocks: 1 or 2
  static constexpr int kTileBytes = kBlocks * kBlockBytes;
  static constexpr int kLanesPerRow = kRowLds / 16;         // 16-byte pieces of an LDS row: 16 or 32
  static constexpr int kRowPieces = D / 8;                  // the real ones: 16, 24 or 32
  static constexpr int kQB = D / 16;                        // 16-wide d steps of S^T (Q fragments)
  static constexpr int kOB = D / 32;                        // 32-wide d blocks of O^T
  // Byte offset of 16-byte piece `ch` of key `key` (0..63) inside a K or V tile.
  __device__ __forceinline__ static constexpr uint32_t tile_off(uint32_t key, uint32_t ch) {
    return ((key >> 4) % kRuns * 16u + key_block(key & 15u)) * kBlockBytes + (key >> 4) / kRuns * kRowLds +
           ch * 16u;
  }
  // The key held by row r of load block b (block_key reads b's low 4 bits).
  __device__ __forceinline__ static constexpr uint32_t block_row_key(uint32_t b, uint32_t r) {
    return 16u * ((kRuns == 1 ? 0u : b / 16u) + kRuns * r) + block_key(b);
  }
  // Offset of keys 16c.. from keys 0.., in 8-byte units (transposing V reads).
  __device__ __forceinline__ static constexpr int chunk_units(int c) { return (int)(tile_off(16u * c, 0) / 8u); }
};

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

// This wave's share (blocks [b0, b0 + NB)) of one K or V tile. base: first row
// of the tile (this kv head); rows >= nvalid (nvalid >= 1) re-read row nvalid-1.
// Lane l writes row l / kLanesPerRow of the block, piece l % kLanesPerRow; the
// padding pieces of a head_dim-192 row re-read its last real piece.
template <int D>
__device__ __forceinline__ void issue_block(const uint16_t* base, uint32_t stride_bytes, int nvalid,
                                            uint32_t tile_lds, int blk, int lane) {
  using G = Geom<D>;
  const int piece = lane % G::kLanesPerRow;
  const uint32_t pc = (uint32_t)(piece < G::kRowPieces ? piece : G::kRowPieces - 1) * 16u;
  const int key = (int)G::block_row_key((uint32_t)blk, (uint32_t)(lane / G::kLanesPerRow));
  const int kc = key < nvalid ? key : nvalid - 1;
  const uint32_t voff = (uint32_t)kc * stride_bytes + pc;
  load_lds16(base, voff, __builtin_amdgcn_readfirstlane(tile_lds + blk * kBlockBytes));
}
template <int D, int NB>
__device__ __forceinline__ void issue_tile(const uint16_t* base, uint32_t stride_bytes, int nvalid,
                                           uint32_t tile_lds, int b0, int lane) {
#pragma unroll
  for (int t = 0; t < NB; ++t) issue_block<D>(base, stride_bytes, nvalid, tile_lds, b0 + t, lane);
}

// p, which is the same in every lane, in scalar registers (for load bases the
// compiler cannot prove uniform).
__device__ __forceinline__ const uint16_t* uniform_ptr(const uint16_t* p) {
  const uint64_t b = (uint64_t)(uintptr_t)p;
  return (const uint16_t*)(uintptr_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b));
}

// A per-slot hook of tile_step_pp that does nothing.
struct NoHook {
  template <typename S>
  __device__ __forceinline__ void operator()(S) const {}
};

// Retire the loads of the Q fragments here, on every path. The compiler's
// wait counters do not see the direct-to-LDS loads, so a wait for Q that it
// placed inside the tile loop (where the first use is, on paths that skip the
// prologue's S^T) would also hold back the ring's prefetches in every step.
template <int QB>
__device__ __forceinline__ void settle_q(const bf16x8 (&q)[QB]) {
  if constexpr (QB % 4 == 0) {
#pragma unroll
    for (int b = 0; b < QB; b += 4) asm volatile("" : : "v"(q[b]), "v"(q[b + 1]), "v"(q[b + 2]), "v"(q[b + 3]));
  } else {
#pragma unroll
    for (int b = 0; b < QB; ++b) asm volatile("" : : "v"(q[b]));
  }
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

// Per-lane LDS read bases. key_off selects the first key of the wave's share
// of a tile (0, or 32 for the upper half).
struct Lane {
  uint32_t k_base;  // K A operand for key 32kb + n, d = 16db + 8g: k_base + 512kb + 32db
  uint32_t v_base;  // transposing read (c, h, b): v_base + 2080h + 256c + 64b
  int n, g;
};

template <int D>
__device__ __forceinline__ Lane make_lane(int lane, int key_off = 0) {
  using Gm = Geom<D>;
  Lane L;
  L.n = lane & 31;
  L.g = lane >> 5;
  const uint32_t half = (uint32_t)(key_off >> 5) * kHalfBytes;
  L.k_base = Gm::tile_off((uint32_t)L.n, (uint32_t)L.g) + half;
  // source lane (G, s) of a transposing read points at key 16c + 8h + 4(G/2) + s/4,
  // columns 32b + 16(G%2) + 4(s%4) .. +3
  const uint32_t G = (uint32_t)lane >> 4, s = (uint32_t)lane & 15u;
  L.v_base = Gm::tile_off(4u * (G >> 1) + (s >> 2), 2u * (G & 1u) + ((s & 3u) >> 1)) + (s & 1u) * 8u + half;
  return L;
}

// V^T operand of PV MFMA (chunk c, d-block b) for the transposing reads: key
// + 8 sits two LDS blocks further (+ 2080 bytes), the 32 columns of d-block b
// 64 bytes further per block.
template <int D>
__device__ __forceinline__ bf16x8 read_vt(const lds_bf16x4* base, int c, int b) {
  const int off = Geom<D>::chunk_units(c) + 8 * b;  // in 8-byte units
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + off));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + 260 + off));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// O^T (D d x 32 queries) += V^T P^T over KB blocks of 32 keys. P chunk c
// holds keys 16c + 8*(i/4) + 4g + i%4 in k-slot (g, i); the transposing reads
// deliver the matching V columns.
template <int D, int KB>
__device__ __forceinline__ void pv(uint32_t vt, const Lane& L, const bf16x8 (&p)[2 * KB],
                                   f32x16 (&o)[Geom<D>::kOB]) {
  const lds_bf16x4* base = (const lds_bf16x4*)(vt + L.v_base);
#pragma unroll
  for (int c = 0; c < 2 * KB; ++c) {
#pragma unroll
    for (int b = 0; b < Geom<D>::kOB; ++b) o[b] = mfma32x32x16(read_vt<D>(base, c, b), p[c], o[b]);
  }
}

// S^T for one tile: s[kb] = keys 32kb..32kb+31 of the wave's share x its 32 queries.
template <int D, int KB>
__device__ __forceinline__ void qk(const char* kt, const Lane& L, const bf16x8 (&q)[Geom<D>::kQB],
                                   f32x16 (&s)[KB]) {
  const char* base = kt + L.k_base;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
  }
#pragma unroll
  for (int db = 0; db < Geom<D>::kQB; ++db) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const bf16x8 a = ld_lds16(base, kb * kHalfBytes + db * 32);
      s[kb] = mfma32x32x16(a, q[db], s[kb]);
    }
  }
}

struct Softmax {
  float m;  // reference maximum of the raw scores (the exp2 shift is m * c)
  float l;  // lane-partial sum of the unrounded probabilities
};

// Software-pipelined step for tile j of 64 keys (two 32-key halves per wave):
// the softmax of tile j (s) runs under NS = D/4 MFMAs (32 at head_dim 128), the
// S^T of tile j+1 (sn, K from nk) on even slots and, when PV, the
// O^T += V^T P^T of tile j-1 (P in p_prev, V^T from vt_prev) on odd slots, so
// every MFMA has VALU work beside it. Slots 0-5 carry the row maximum, slot 6
// the reference update, slots 7 on the 32 exp2 (spread over the step). P of
// tile j goes to p_cur. O and the row sum are rescaled at the end (after the
// PV of tile j-1, which still belongs to the old reference). hook(slot) runs
// at the start of every slot (the caller's load issue, say).
template <int D, bool PV, bool PRIO = false, typename Hook = NoHook>
__device__ __forceinline__ void tile_step_pp(f32x16 (&s)[2], f32x16 (&sn)[2], const char* nk, uint32_t vt_prev,
                                             const Lane& L, const bf16x8 (&q)[Geom<D>::kQB],
                                             const bf16x8 (&p_prev)[4], bf16x8 (&p_cur)[4],
                                             f32x16 (&o)[Geom<D>::kOB], Softmax& st, float c, bool mask, int key0,
                                             int len_k, int lim, Hook hook = Hook{}) {
  constexpr int OB = Geom<D>::kOB;
  constexpr int NT = 2 * Geom<D>::kQB;  // S^T MFMAs per step = PV MFMAs per step
  constexpr int NS = 2 * NT;            // MFMA slots
  // slot of element x's exp2: spread over slots 7 .. 7 + 23*NS/32 with 32 or
  // more slots, two per slot over slots 7..22 with the 24 slots of head_dim
  // 96, four per slot over slots 7..14 with the 16 slots of head_dim 64
  auto exp_slot = [](int x) constexpr {
    return NS >= 32 ? 7 + ((3 * x) / 4) * NS / 32 : NS >= 24 ? 7 + x / 2 : 7 + x / 4;
  };
  static_assert(NS >= 16, "the softmax needs 16 MFMA slots per step");
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
  const char* kbase = nk + L.k_base;
  const lds_bf16x4* vbase = (const lds_bf16x4*)(vt_prev + L.v_base);
  // no LDS read is outstanding here (the step's barrier waited for them all);
  // saying so lets the compiler's first MFMA wait for its own K operand only
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt untouched
  // K and V operands are read PF MFMA steps of their kind (2*PF slots) ahead;
  // 3 and 4 measured level with 2 on dense, causal and padded prefill (same
  // box, three alternating rounds), so LDS latency does not hold the loop back
  constexpr int PF = 2;
  bf16x8 kr[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) kr[i] = ld_lds16(kbase, (i % 2) * kHalfBytes + (i / 2) * 32);
  bf16x8 va[PF];
  if (PV) {
#pragma unroll
    for (int i = 0; i < PF; ++i) va[i] = read_vt<D>(vbase, i / OB, i % OB);
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sn[kb][r] = 0.f;
  }
  float mx4[4];
  float alpha = 1.f, ms = 0.f, m_ref = st.m;
  bool need = false;
  f32x8 e;
  float rs0 = 0.f, rs1 = 0.f;
  // PRIO: issue priority 2 for the MFMA slots, back to the caller's loop
  // level 1 after them (kernels that run two workgroups per CU out of phase)
  if constexpr (PRIO) __builtin_amdgcn_s_setprio(2);
  __builtin_amdgcn_sched_barrier(0);
  // one instance per slot (a counted loop this long exceeds the unroller's
  // size limit at head_dims 192 and 256)
  static_for<NS>([&](auto slot_c) __attribute__((always_inline)) {
    constexpr int slot = decltype(slot_c)::value;
    hook(slot_c);
    constexpr int t = slot >> 1;
    if constexpr ((slot & 1) == 0) {  // S^T of tile j+1: step t = (d-block t/2, key half t%2)
      sn[t & 1] = mfma32x32x16(kr[t % PF], q[t >> 1], sn[t & 1]);
      if (t + PF < NT) kr[t % PF] = ld_lds16(kbase, ((t + PF) % 2) * kHalfBytes + ((t + PF) / 2) * 32);
    } else if constexpr (PV) {  // PV of tile j-1: chunk t/OB, d-block t%OB
      const bf16x8 a = va[t % PF];
      if (t + PF < NT) va[t % PF] = read_vt<D>(vbase, (t + PF) / OB, (t + PF) % OB);
      o[t % OB] = mfma32x32x16(a, p_prev[t / OB], o[t % OB]);
    }
    if constexpr (slot < 4) {  // row maximum: chain slot over 8 keys (2 slots per chain pair)
      constexpr int ch = slot;  // chain ch: half ch/2, elements 8(ch%2) .. +7
      float m = fmaxf(s[ch >> 1][8 * (ch & 1)], s[ch >> 1][8 * (ch & 1) + 1]);
#pragma unroll
      for (int i = 2; i < 8; ++i) m = fmaxf(m, s[ch >> 1][8 * (ch & 1) + i]);
      mx4[ch] = m;
    } else if constexpr (slot == 5) {
      const float mx = pair_max(fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3])));
      const float m_new = fmaxf(st.m, mx);
      need = (m_new - st.m) * c > kRescaleThreshold;  // true on the first finite maximum
      alpha = need ? hw_exp2((st.m - m_new) * c) : 1.f;
      m_ref = need ? m_new : st.m;
      ms = (m_ref == kNegInf ? 0.f : m_ref) * c;
    } else if constexpr (slot >= 7) {
      // element x's exp2 runs in slot exp_slot(x) (slots 7..30 at head_dim
      // 128); its row-sum add, and the bf16 packing of a finished chunk, one
      // slot later, so that no VALU op waits on the exp2 issued just before it
#pragma unroll
      for (int x = 0; x < 32; ++x) {
        if (exp_slot(x) + 1 == slot) {
          const int u = x & 7;
          if (u & 1) {
            rs1 += e[u];
          } else {
            rs0 += e[u];
          }
          if (u == 7) {
            p_cur[x >> 3] = to_bf16x8(e);
            // keep the packing in this slot: otherwise it is sunk past the
            // rescale branch below, off the MFMAs and with all 32 exp2
            // results held until the end of the step
            asm volatile("" : : "v"(p_cur[x >> 3]));
          }
        }
      }
#pragma unroll
      for (int x = 0; x < 32; ++x) {
        if (exp_slot(x) == slot) {
          const int ch = x >> 3, u = x & 7;
          e[u] = hw_exp2(__builtin_fmaf(s[ch >> 1][8 * (ch & 1) + u], c, -ms));
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  });
  if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
  const float rs = rs0 + rs1;
  st.l = st.l * alpha + rs;
  st.m = m_ref;
  // Rare rescale of O, after the PV of tile j-1 (old reference). The row sum
  // takes part in the condition so that the exp2 stay in their slots.
  if (__builtin_amdgcn_ballot_w64(need || rs != rs) != 0ull) {
#pragma unroll
    for (int b = 0; b < OB; ++b) o[b] *= alpha;
  }
}

// The same pipeline for a 32-key share per wave (KB = 1): NS = D/8 MFMA slots
// (16 at head_dim 128), the S^T of tile j+1 (D/16 MFMAs, K from nk) on even
// slots and, when PV, the PV of tile j-1 (D/16 MFMAs, P in p_prev, V^T from
// vt_prev) on odd slots. Slots 0-1 carry the two row-maximum chains, slot 2 the
// reference update, slots 3 on the 16 exp2 (each row-sum add and bf16 packing
// one slot after its exp2): slot 3 + 3x/4 for element x at head_dim 128,
// stretched over the step at 192 and 256, two per slot at 96.
template <int D, bool PV>
__device__ __forceinline__ void tile_step_pp1(f32x16 (&s)[1], f32x16 (&sn)[1], const char* nk, uint32_t vt_prev,
                                              const Lane& L, const bf16x8 (&q)[Geom<D>::kQB],
                                              const bf16x8 (&p_prev)[2], bf16x8 (&p_cur)[2],
                                              f32x16 (&o)[Geom<D>::kOB], Softmax& st, float c, bool mask, int key0,
                                              int len_k, int lim) {
  constexpr int OB = Geom<D>::kOB;
  constexpr int NT = Geom<D>::kQB;  // S^T MFMAs per step = PV MFMAs per step (2 chunks x OB)
  constexpr int NS = 2 * NT;        // MFMA slots
  static_assert(NS >= 12, "the softmax needs 12 MFMA slots per step");
  auto exp_slot = [](int x) constexpr { return NS >= 16 ? 3 + ((3 * x) / 4) * (NS - 4) / 12 : 3 + x / 2; };
  if (mask) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + 8 * (r >> 2) + 4 * L.g + (r & 3);
      if (key >= len_k || key > lim) s[0][r] = kNegInf;
    }
  }
  const char* kbase = nk + L.k_base;
  const lds_bf16x4* vbase = (const lds_bf16x4*)(vt_prev + L.v_base);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): as in tile_step_pp
  bf16x8 kr[2];  // K operand two S^T steps ahead
  kr[0] = ld_lds16(kbase, 0);
  kr[1] = ld_lds16(kbase, 32);
  bf16x8 va[2];
  if (PV) {
    va[0] = read_vt<D>(vbase, 0, 0);
    va[1] = read_vt<D>(vbase, 1 / OB, 1 % OB);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) sn[0][r] = 0.f;
  float mx2[2];
  float alpha = 1.f, ms = 0.f, m_ref = st.m;
  bool need = false;
  f32x8 e;
  float rs0 = 0.f, rs1 = 0.f;
  // Issue priority 2 for the MFMA slots, back to 1 (the caller's loop level)
  // after them: the block-sparse kernel runs two workgroups per CU out of
  // phase (head_dims 96 and 128), and the other workgroup's ring refills (1)
  // and prologue, merge and store (0) then yield the issue slot to these steps.
  __builtin_amdgcn_s_setprio(2);
  __builtin_amdgcn_sched_barrier(0);
  static_for<NS>([&](auto slot_c) __attribute__((always_inline)) {
    constexpr int slot = decltype(slot_c)::value;
    constexpr int t = slot >> 1;
    if constexpr ((slot & 1) == 0) {  // S^T of tile j+1, d-block t
      sn[0] = mfma32x32x16(kr[t & 1], q[t], sn[0]);
      if (t + 2 < NT) kr[t & 1] = ld_lds16(kbase, (t + 2) * 32);
    } else if constexpr (PV) {  // PV of tile j-1: chunk t/OB, d-block t%OB
      const bf16x8 a = va[t & 1];
      if (t + 2 < NT) va[t & 1] = read_vt<D>(vbase, (t + 2) / OB, (t + 2) % OB);
      o[t % OB] = mfma32x32x16(a, p_prev[t / OB], o[t % OB]);
    }
    if constexpr (slot < 2) {  // row maximum: chain slot over elements 8*slot .. +7
      float m = fmaxf(s[0][8 * slot], s[0][8 * slot + 1]);
#pragma unroll
      for (int i = 2; i < 8; ++i) m = fmaxf(m, s[0][8 * slot + i]);
      mx2[slot] = m;
    } else if constexpr (slot == 2) {
      const float mx = pair_max(fmaxf(mx2[0], mx2[1]));
      const float m_new = fmaxf(st.m, mx);
      need = (m_new - st.m) * c > kRescaleThreshold;  // true on the first finite maximum
      alpha = need ? hw_exp2((st.m - m_new) * c) : 1.f;
      m_ref = need ? m_new : st.m;
      ms = (m_ref == kNegInf ? 0.f : m_ref) * c;
    } else {
      // element x's exp2 runs in slot exp_slot(x); its row-sum add, and the
      // packing of a finished chunk, one slot later
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        if (exp_slot(x) + 1 == slot) {
          const int u = x & 7;
          if (u & 1) {
            rs1 += e[u];
          } else {
            rs0 += e[u];
          }
          if (u == 7) {
            p_cur[x >> 3] = to_bf16x8(e);
            asm volatile("" : : "v"(p_cur[x >> 3]));  // keep the packing in this slot
          }
        }
      }
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        if (exp_slot(x) == slot) e[x & 7] = hw_exp2(__builtin_fmaf(s[0][x], c, -ms));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  });
  __builtin_amdgcn_s_setprio(1);
  const float rs = rs0 + rs1;
  st.l = st.l * alpha + rs;
  st.m = m_ref;
  if (__builtin_amdgcn_ballot_w64(need || rs != rs) != 0ull) {
#pragma unroll
    for (int b = 0; b < OB; ++b) o[b] *= alpha;
  }
}

// Write the wave's 32 normalised output rows (bf16) and their LSE. o holds
// O^T (d = 32b + 8*grp + 4g + i for element 4*grp + i of block b); st.l is
// lane-partial.
template <int OB>
__device__ __forceinline__ void store_rows(const f32x16 (&o)[OB], const Softmax& st, const Lane& L, float c,
                                           bool live, uint16_t* orow, float* lse_out) {
  const float lt = pair_sum(st.l);
  if (!live) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
  for (int b = 0; b < OB; ++b) {
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      f32x4 t;
#pragma unroll
      for (int i = 0; i < 4; ++i) t[i] = o[b][4 * grp + i] * inv;
      *reinterpret_cast<bf16x4*>(orow + b * 32 + 8 * grp + 4 * L.g) = to_bf16x4(t);
    }
  }
  if (lse_out != nullptr && L.g == 0) *lse_out = lt > 0.f ? (st.m * c + hw_log2(lt)) * kLn2 : kNegInf;
}

}  // namespace pipe
}  // namespace attn
