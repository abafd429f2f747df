// Device helpers shared by the gfx950 attention kernels: vector types, MFMA
// wrappers, 16-byte loads, exp2/log2, and the LDS staging of one K/V tile.
//
// MFMA lane layouts used throughout (CDNA3/CDNA4 ISA, wave64):
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     A: lane l holds row m = l%32, k-slots 8*(l/32) .. +7
//     B: lane l holds col n = l%32, k-slots 8*(l/32) .. +7
//     D: lane l, element r holds (m = 8*(r/4) + 4*(l/32) + r%4, n = l%32)
//   v_mfma_f32_16x16x32_bf16  D[16x16] += A[16x32] * B[32x16]
//     A: lane l holds row m = l%16, k-slots 8*(l/16) .. +7
//     B: lane l holds col n = l%16, k-slots 8*(l/16) .. +7
//     D: lane l, element r holds (m = 4*(l/16) + r, n = l%16)
// Only the D layout matters for correctness: A and B are always filled with
// the same k-slot convention, and a contraction does not care how k is
// permuted as long as both operands agree.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 2^x and log2(x) on the hardware transcendental unit (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ u32x4 ld_global16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return (bf16x8)x; }

__device__ __forceinline__ bf16x8 ld_lds16(const char* base, int byte_off) {
  return (bf16x8)(*reinterpret_cast<const u32x4*>(base + byte_off));
}

// fp32 -> bf16, round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16x8 to_bf16x8(f32x8 x) { return __builtin_convertvector(x, bf16x8); }
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) { return __builtin_convertvector(x, bf16x4); }

__device__ __forceinline__ float wave_xor_max(float x, int mask) { return fmaxf(x, __shfl_xor(x, mask, 64)); }
__device__ __forceinline__ float wave_xor_sum(float x, int mask) { return x + __shfl_xor(x, mask, 64); }

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Position of key t (0 <= t < 64) inside a transposed V row of the LDS tile.
// Within every 16 keys, bits 2 and 3 of the key index are swapped, so that the
// 8 keys one lane feeds into a PV MFMA (keys 16c+4g+{0..3} and 16c+8+4g+{0..3},
// which is where the S^T accumulator leaves them) sit in 8 consecutive slots.
__device__ __forceinline__ int vt_pos32(int t) {
  return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1);
}

// ---------------------------------------------------------------------------
// One K/V tile of BN keys staged through LDS, loaded by NT threads.
//   K is stored as rows  [key][D]  with a 16-byte pad per row.
//   V is stored transposed [d][BN] with a 16-byte pad per row and the vt_pos32
//   key permutation, so each lane reads its PV MFMA operand with one 16-byte
//   LDS read.
// Rows at or past n_valid are loaded from row n_valid-1 (finite data; the
// caller masks those keys).
// ---------------------------------------------------------------------------
template <int D, int BN, int NT>
struct KVTile {
  static_assert(BN == 64, "tile loader assumes 64 keys");
  static constexpr int KCH = D / 8;                      // 16-byte chunks per row
  static constexpr int K_STRIDE = D * 2 + 16;            // bytes per K row in LDS
  static constexpr int V_STRIDE = BN * 2 + 16;           // bytes per V^T row in LDS
  static constexpr int K_BYTES = BN * K_STRIDE;
  static constexpr int V_BYTES = D * V_STRIDE;
  static constexpr int BYTES = K_BYTES + V_BYTES;
  static constexpr int K_UNITS = BN * KCH;
  static constexpr int K_PER_T = (K_UNITS + NT - 1) / NT;
  static constexpr int V_UNITS = (BN / 4) * KCH;         // (4 keys x 8 d) units
  static constexpr int V_PER_T = (V_UNITS + NT - 1) / NT;

  u32x4 kr[K_PER_T];
  u32x4 vr[V_PER_T][4];

  // kbase/vbase point at key row 0 of this tile for the right kv head;
  // row_stride is the element distance between consecutive keys.
  __device__ __forceinline__ void load(const uint16_t* kbase, const uint16_t* vbase, long row_stride,
                                       int n_valid, int tid) {
    const int last = n_valid - 1;
#pragma unroll
    for (int j = 0; j < K_PER_T; ++j) {
      const int u = tid + j * NT;
      if (K_UNITS % NT == 0 || u < K_UNITS) {
        const int row = u / KCH, ch = u % KCH;
        const int r = row < last ? row : last;
        kr[j] = ld_global16(kbase + (long)r * row_stride + ch * 8);
      }
    }
#pragma unroll
    for (int j = 0; j < V_PER_T; ++j) {
      const int u = tid + j * NT;
      if (V_UNITS % NT == 0 || u < V_UNITS) {
        const int kq = u % (BN / 4), ch = u / (BN / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int row = kq * 4 + r;
          row = row < last ? row : last;
          vr[j][r] = ld_global16(vbase + (long)row * row_stride + ch * 8);
        }
      }
    }
  }

  __device__ __forceinline__ void store(char* smem, int tid) const {
#pragma unroll
    for (int j = 0; j < K_PER_T; ++j) {
      const int u = tid + j * NT;
      if (K_UNITS % NT == 0 || u < K_UNITS) {
        const int row = u / KCH, ch = u % KCH;
        *reinterpret_cast<u32x4*>(smem + row * K_STRIDE + ch * 16) = kr[j];
      }
    }
    char* vt = smem + K_BYTES;
#pragma unroll
    for (int j = 0; j < V_PER_T; ++j) {
      const int u = tid + j * NT;
      if (V_UNITS % NT == 0 || u < V_UNITS) {
        const int kq = u % (BN / 4), ch = u / (BN / 4);
        const int pos = vt_pos32(kq * 4);  // 4 consecutive keys stay consecutive
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // word w of each row holds d = ch*8 + 2w (low half) and d+1 (high half)
          const uint32_t a0 = vr[j][0][w], a1 = vr[j][1][w], a2 = vr[j][2][w], a3 = vr[j][3][w];
          u32x2 lo, hi;
          lo[0] = (a0 & 0xffffu) | (a1 << 16);
          lo[1] = (a2 & 0xffffu) | (a3 << 16);
          hi[0] = (a0 >> 16) | (a1 & 0xffff0000u);
          hi[1] = (a2 >> 16) | (a3 & 0xffff0000u);
          const int d = ch * 8 + 2 * w;
          *reinterpret_cast<u32x2*>(vt + d * V_STRIDE + pos * 2) = lo;
          *reinterpret_cast<u32x2*>(vt + (d + 1) * V_STRIDE + pos * 2) = hi;
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Per-wave online-softmax state for 32 query rows, computing S^T = K Q^T so that
// each lane owns one query (l%32) and the row reductions stay inside the lane
// plus one exchange with lane l^32.
// ---------------------------------------------------------------------------
template <int D>
struct WaveRows32 {
  static constexpr int QB = D / 16;  // 16-wide d blocks (QK^T k-steps)
  static constexpr int OB = D / 32;  // 32-wide d blocks (PV output tiles)
  bf16x8 q[QB];
  f32x16 o[OB];
  float m;  // running max of raw scores q.k (scale applied later), -inf = none yet
  float l;  // lane-partial running sum of exp2((s - m) * c)

  __device__ __forceinline__ void init(const uint16_t* qrow, int g) {
#pragma unroll
    for (int b = 0; b < QB; ++b) q[b] = as_bf16x8(ld_global16(qrow + b * 16 + g * 8));
#pragma unroll
    for (int b = 0; b < OB; ++b) {
#pragma unroll
      for (int r = 0; r < 16; ++r) o[b][r] = 0.f;
    }
    m = kNegInf;
    l = 0.f;
  }

  // S^T for a 64-key tile: s[kb] covers keys 32*kb .. 32*kb+31.
  template <int K_STRIDE>
  __device__ __forceinline__ void scores(const char* ksm, int lane, f32x16 (&s)[2]) const {
    const int g = lane >> 5, n = lane & 31;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        const bf16x8 a = ld_lds16(ksm, (kb * 32 + n) * K_STRIDE + (b * 16 + g * 8) * 2);
        s[kb] = mfma32x32x16(a, q[b], s[kb]);
      }
    }
  }

  // Online-softmax update with the (masked) scores of one tile, then O += P V.
  // c = softmax_scale * log2(e).
  template <int V_STRIDE>
  __device__ __forceinline__ void update(const char* vsm, int lane, f32x16 (&s)[2], float c) {
    const int g = lane >> 5, n = lane & 31;
    float mx = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    mx = wave_xor_max(mx, 32);
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = hw_exp2((m - m_use) * c);  // m = -inf -> 0
    const float ms = m_use * c;
    float rs = 0.f;
    bf16x8 p[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x8 t;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float e = hw_exp2(__builtin_fmaf(s[kb][8 * h + i], c, -ms));
          t[i] = e;
          rs += e;
        }
        p[2 * kb + h] = to_bf16x8(t);
      }
    }
    l = l * alpha + rs;
    m = m_new;
#pragma unroll
    for (int b = 0; b < OB; ++b) {
#pragma unroll
      for (int r = 0; r < 16; ++r) o[b][r] *= alpha;
    }
#pragma unroll
    for (int ck = 0; ck < 4; ++ck) {
#pragma unroll
      for (int b = 0; b < OB; ++b) {
        const bf16x8 a = ld_lds16(vsm, (b * 32 + n) * V_STRIDE + (ck * 16 + g * 8) * 2);
        o[b] = mfma32x32x16(a, p[ck], o[b]);
      }
    }
    (void)g;
  }

  // Normalise and write this lane's query row. orow points at d = 0 of the
  // output row; lse_out (nullable) at its LSE slot. Only lanes with g == 0 write
  // the LSE.
  __device__ __forceinline__ void finish(uint16_t* orow, float* lse_out, int lane, float c) {
    const int g = lane >> 5;
    const float lt = wave_xor_sum(l, 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
    for (int b = 0; b < OB; ++b) {
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        f32x4 t;
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] = o[b][4 * grp + i] * inv;
        const int d = b * 32 + 8 * grp + 4 * g;
        *reinterpret_cast<bf16x4*>(orow + d) = to_bf16x4(t);
      }
    }
    if (lse_out != nullptr && g == 0) {
      *lse_out = lt > 0.f ? (m * c + hw_log2(lt)) * kLn2 : kNegInf;
    }
  }
};

}  // namespace attn
