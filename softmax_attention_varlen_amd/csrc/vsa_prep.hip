// Video tile geometry and the pooled-score top-k block map, on the GPU.
//
// Geometry (fastvideo_vsa.py page: _get_tile_partition_indices,
// _construct_variable_block_sizes, _get_non_pad_index, _get_tile_metadata):
// a raster (T, H, W) latent is cut into boxes of (tt, th, tw) tokens, boxes
// enumerated t-box slowest, then h, then w; tokens inside a box in raster
// order; edge boxes clipped. Box c owns rows [64c, 64c + 64) of the tile-order
// layout, the first size(c) of them real, the rest zero padding.
//   tile_gather : raster rows -> padded tile-order rows (+ tile sizes)
//   untile      : tile-order rows -> raster rows
// Both map one destination row per wave and move 16 bytes per lane; the index
// arithmetic is integer and exact.
//
// Block map (FastVideoVSAImpl._forward_h3, _pool_h3_tiles, _build_h3_block_map):
//   pool   : per (batch, tile, head) fp32 mean of the tile's real rows
//   scores : per (batch, head) fp32 scale * qbar kbar^T, an LDS-tiled batched
//            GEMM over [tiles x head_dim] operands
//   select : per map row keep the top-k key tiles (ties: lower tile index wins;
//            every tile when k reaches the tile count) as uint8
// Compressed branch (FastVideoVSAImpl.forward's coarse path): softmax of the
// same scores over all key tiles, times the value means (a second batched
// GEMM), gated and added to every row of the query tile.
#include "attn_common.hpp"
#include "launch.hpp"

namespace attn {

struct BoxGeom {
  int T, H, W, tt, th, tw, nbt, nbh, nbw;
  __device__ __forceinline__ void box_extent(int c, int& bt, int& bh, int& bw, int& et, int& eh, int& ew) const {
    bw = c % nbw;
    bh = (c / nbw) % nbh;
    bt = c / (nbw * nbh);
    et = min(tt, T - bt * tt);
    eh = min(th, H - bh * th);
    ew = min(tw, W - bw * tw);
  }
};

// H3 prefix rows ([VSA] _get_h3_tile_metadata): segment s covers raster rows
// [start[s], start[s + 1]) (start[n_seg] = len) and tiles [tile0[s],
// tile0[s + 1]), 64 rows each, its last tile holding the remainder. Segments
// are non-empty; n_seg = 0 is the plain video layout.
struct PrefixLayout {
  int n_seg, n_tiles, len;
  int start[kMaxPrefixSegments + 1];
  int tile0[kMaxPrefixSegments + 1];
};

// Raster row (batch-local) that fills padded row r of tile c, or -1 for a
// padding row; *size = the tile's real row count.
__device__ __forceinline__ int tile_source(const BoxGeom& gm, const PrefixLayout& pl, int c, int r, int* size) {
  if (c < pl.n_tiles) {
    int s = 0;
    while (s + 1 < pl.n_seg && pl.tile0[s + 1] <= c) ++s;
    const int first = pl.start[s] + (c - pl.tile0[s]) * 64;
    const int sz = min(64, pl.start[s + 1] - first);
    *size = sz;
    return r < sz ? first + r : -1;
  }
  int bt, bh, bw, et, eh, ew;
  gm.box_extent(c - pl.n_tiles, bt, bh, bw, et, eh, ew);
  *size = et * eh * ew;
  if (r >= *size) return -1;
  const int it = r / (eh * ew), ih = (r / ew) % eh, iw = r % ew;
  return pl.len + ((bt * gm.tt + it) * gm.H + (bh * gm.th + ih)) * gm.W + (bw * gm.tw + iw);
}

// One wave per tile-order destination row.
__global__ __launch_bounds__(256) void tile_gather_kernel(const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
                                                          int32_t* __restrict__ sizes, BoxGeom gm, PrefixLayout pl,
                                                          int n_tiles, int batch, int row_elems) {
  const int lane = threadIdx.x & 63;
  const long dst = (long)blockIdx.x * 4 + (threadIdx.x >> 6);  // over batch * n_tiles * 64
  const long rows_per_batch = (long)n_tiles * 64;
  if (dst >= batch * rows_per_batch) return;
  const int b = (int)(dst / rows_per_batch);
  const int p = (int)(dst % rows_per_batch);
  const int c = p >> 6, r = p & 63;
  int size;
  const int src = tile_source(gm, pl, c, r, &size);
  if (sizes != nullptr && b == 0 && r == 0 && lane == 0) sizes[c] = size;
  uint16_t* yrow = y + dst * row_elems;
  const int chunks = row_elems / 8;
  if (src < 0) {
    for (int j = lane; j < chunks; j += 64) *reinterpret_cast<u32x4*>(yrow + j * 8) = u32x4{0u, 0u, 0u, 0u};
    return;
  }
  const long n_rows = (long)pl.len + (long)gm.T * gm.H * gm.W;
  const uint16_t* xrow = x + ((long)b * n_rows + src) * row_elems;
  for (int j = lane; j < chunks; j += 64) *reinterpret_cast<u32x4*>(yrow + j * 8) = ld_global16(xrow + j * 8);
}

// One wave per raster destination row.
__global__ __launch_bounds__(256) void untile_kernel(const uint16_t* __restrict__ y, uint16_t* __restrict__ x,
                                                     BoxGeom gm, PrefixLayout pl, int n_tiles, int batch,
                                                     int row_elems) {
  const int lane = threadIdx.x & 63;
  const long n_rows = (long)pl.len + (long)gm.T * gm.H * gm.W;
  const long dst = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (dst >= batch * n_rows) return;
  const int b = (int)(dst / n_rows);
  const long n = dst % n_rows;
  int c, r;
  if (n < pl.len) {
    int s = 0;
    while (s + 1 < pl.n_seg && pl.start[s + 1] <= n) ++s;
    const int off = (int)n - pl.start[s];
    c = pl.tile0[s] + off / 64;
    r = off % 64;
  } else {
    const long tok = n - pl.len;
    const int w = (int)(tok % gm.W), h = (int)((tok / gm.W) % gm.H), t = (int)(tok / ((long)gm.W * gm.H));
    const int cv = ((t / gm.tt) * gm.nbh + h / gm.th) * gm.nbw + w / gm.tw;
    int bt, bh, bw, et, eh, ew;
    gm.box_extent(cv, bt, bh, bw, et, eh, ew);
    r = ((t - bt * gm.tt) * eh + (h - bh * gm.th)) * ew + (w - bw * gm.tw);
    c = pl.n_tiles + cv;
  }
  const uint16_t* yrow = y + ((long)b * n_tiles * 64 + (long)c * 64 + r) * row_elems;
  uint16_t* xrow = x + dst * row_elems;
  const int chunks = row_elems / 8;
  for (int j = lane; j < chunks; j += 64) *reinterpret_cast<u32x4*>(xrow + j * 8) = ld_global16(yrow + j * 8);
}

// Tile means: pooled[b][h][c][d] = (sum of the size(c) real rows) / max(size, 1),
// fp32. One workgroup per (batch, tile, source tensor); the tensors of one
// launch (q, k, v) may differ in head count. Wave g sums rows 16g .. 16g + 15
// (rows at or past the size count as zero) of 64 consecutive 16-byte chunks,
// all 16 loads in flight at once; the four wave partials are then added in
// ascending wave order through LDS.
struct PoolSrc {
  const uint16_t* x;
  float* pooled;
  int heads;
};
struct PoolArgs {
  PoolSrc s[3];
};

__global__ __launch_bounds__(256) void tile_pool_kernel(PoolArgs pa, const int32_t* __restrict__ sizes, int n_tiles,
                                                       int head_dim) {
  __shared__ f32x4 part[4][64][2];
  const PoolSrc src = pa.s[blockIdx.y];
  const int c = (int)(blockIdx.x % n_tiles);
  const long b = blockIdx.x / n_tiles;
  const int size = clampi(sizes[c], 0, 64);
  const float inv = 1.f / (float)(size > 1 ? size : 1);
  const long row_elems = (long)src.heads * head_dim;
  const uint16_t* base = src.x + (b * n_tiles + c) * 64 * row_elems;
  const int chunks = (int)(row_elems / 8);
  const int tid = threadIdx.x, g = tid >> 6, jl = tid & 63;
  for (int j0 = 0; j0 < chunks; j0 += 64) {
    const int j = j0 + jl;
    f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
    if (j < chunks) {
      u32x4 v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = ld_global16(base + (long)(16 * g + i) * row_elems + j * 8);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (16 * g + i < size) {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            lo[2 * e] += __uint_as_float(v[i][e] << 16);
            lo[2 * e + 1] += __uint_as_float(v[i][e] & 0xffff0000u);
            hi[2 * e] += __uint_as_float(v[i][2 + e] << 16);
            hi[2 * e + 1] += __uint_as_float(v[i][2 + e] & 0xffff0000u);
          }
        }
      }
    }
    part[g][jl][0] = lo;
    part[g][jl][1] = hi;
    __syncthreads();
    if (tid < 128) {
      const int jj = j0 + (tid >> 1), half = tid & 1;
      if (jj < chunks) {
        f32x4 t = part[0][tid >> 1][half];
#pragma unroll
        for (int w = 1; w < 4; ++w) t += part[w][tid >> 1][half];
        const int h = (jj * 8) / head_dim, d = (jj * 8) % head_dim + 4 * half;
        float* prow = src.pooled + ((b * src.heads + h) * n_tiles + c) * (long)head_dim + d;
        *reinterpret_cast<f32x4*>(prow) = t * inv;
      }
    }
    __syncthreads();
  }
}

// Tile gather and tile means in one pass (q and k of the block map): one
// workgroup per (batch, tile, tensor, group of 64 16-byte column chunks)
// copies those columns of the tile's 64 rows from raster to tile order, as
// tile_gather_kernel does (padding rows written as zeros), and sums them
// exactly as tile_pool_kernel does (wave g adds rows 16g .. 16g + 15 in order,
// the four wave partials are added in ascending wave order), so the means, and
// the map built from them, are bit-identical to the two-pass form while the
// tile-order copies are not read back.
struct GatherPoolSrc {
  const uint16_t* x;  // raster [batch][n_rows][heads * head_dim]
  uint16_t* y;        // tile order [batch][n_tiles * 64][heads * head_dim]
  float* pooled;      // [batch][heads][n_tiles][head_dim]
  int heads;
};
struct GatherPoolArgs {
  GatherPoolSrc s[2];
};

__global__ __launch_bounds__(256) void tile_gather_pool_kernel(GatherPoolArgs pa, BoxGeom gm, PrefixLayout pl,
                                                               int n_tiles, long n_rows, int head_dim,
                                                               int32_t* __restrict__ sizes) {
  __shared__ f32x4 part[4][64][2];
  const GatherPoolSrc src = pa.s[blockIdx.y];
  const int c = (int)(blockIdx.x % n_tiles);
  const long b = blockIdx.x / n_tiles;
  const int tid = threadIdx.x, g = tid >> 6, jl = tid & 63;
  int size = 0;
  int srow[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) srow[i] = tile_source(gm, pl, c, 16 * g + i, &size);
  if (sizes != nullptr && b == 0 && blockIdx.y == 0 && blockIdx.z == 0 && tid == 0) sizes[c] = size;
  const float inv = 1.f / (float)(size > 1 ? size : 1);
  const long row_elems = (long)src.heads * head_dim;
  const uint16_t* xb = src.x + b * n_rows * row_elems;
  uint16_t* yb = src.y + (b * n_tiles + c) * 64 * row_elems;
  const int chunks = (int)(row_elems / 8);
  const int j0 = (int)blockIdx.z * 64;  // this workgroup's 64 chunk columns
  if (j0 >= chunks) return;             // whole workgroup (k may have fewer heads than q)
  {
    const int j = j0 + jl;
    f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
    if (j < chunks) {
      u32x4 v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        v[i] = srow[i] >= 0 ? ld_global16(xb + (long)srow[i] * row_elems + j * 8) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) *reinterpret_cast<u32x4*>(yb + (long)(16 * g + i) * row_elems + j * 8) = v[i];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (16 * g + i < size) {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            lo[2 * e] += __uint_as_float(v[i][e] << 16);
            lo[2 * e + 1] += __uint_as_float(v[i][e] & 0xffff0000u);
            hi[2 * e] += __uint_as_float(v[i][2 + e] << 16);
            hi[2 * e + 1] += __uint_as_float(v[i][2 + e] & 0xffff0000u);
          }
        }
      }
    }
    part[g][jl][0] = lo;
    part[g][jl][1] = hi;
    __syncthreads();
    if (tid < 128) {
      const int jj = j0 + (tid >> 1), half = tid & 1;
      if (jj < chunks) {
        f32x4 t = part[0][tid >> 1][half];
#pragma unroll
        for (int w = 1; w < 4; ++w) t += part[w][tid >> 1][half];
        const int h = (jj * 8) / head_dim, d = (jj * 8) % head_dim + 4 * half;
        float* prow = src.pooled + ((b * src.heads + h) * n_tiles + c) * (long)head_dim + d;
        *reinterpret_cast<f32x4*>(prow) = t * inv;
      }
    }
    __syncthreads();
  }
}

// Batched fp32 GEMM for the pooled scores and the compressed rows:
// C[z] = alpha * A[z] B'[z], A [M][K] (row stride lda); B' = B^T with B stored
// [N][K] (TRANS_B), else B' = B stored [K][N]; C row stride ldc. The launch
// covers batch entries z0 + z = b * heads + h; A and C are indexed by z (the
// caller offsets them), B by b * kv_heads + h / (heads / kv_heads) (grouped
// heads). lda and ldb are multiples of 4 and cover K (resp. N) rounded up to 4.
//
// A workgroup of 4 waves owns a 32 x 32 tile of C. K runs in chunks of kKC:
// each chunk of A and B is loaded whole (every thread's loads in flight at
// once, the next chunk's issued before this one is consumed) and staged in
// LDS; wave w multiplies the w-th quarter of the chunk, so each wave keeps a
// partial 32 x 32 tile (lane (tx, ty): rows ty + 8i, columns tx + 8j, or
// 4 tx + j for a row-major B), and the four partials are added in wave order.
// k past K reads as zero.
constexpr int kKC = 128;

template <bool TRANS_B>
struct GemmStage {
  f32x4 a[4], b[4];
};

template <bool TRANS_B>
__device__ __forceinline__ GemmStage<TRANS_B> gemm_fetch(const float* Az, const float* Bz, int m0, int n0, int M,
                                                         int N, int K, int lda, int ldb, int kc, int tid) {
  GemmStage<TRANS_B> g;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int idx = p * 256 + tid;  // 32 rows x 32 four-wide k groups
    const int r = idx >> 5, k = kc + (idx & 31) * 4;
    const int m = min(m0 + r, M - 1);
    const int kk = min(k, ((K - 1) & ~3));
    f32x4 t = *reinterpret_cast<const f32x4*>(Az + (long)m * lda + kk);
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = (k + e < K) ? t[e] : 0.f;
    g.a[p] = t;
  }
  if (TRANS_B) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int idx = p * 256 + tid;
      const int r = idx >> 5, k = kc + (idx & 31) * 4;
      const int n = min(n0 + r, N - 1);
      const int kk = min(k, ((K - 1) & ~3));
      f32x4 t = *reinterpret_cast<const f32x4*>(Bz + (long)n * ldb + kk);
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = (k + e < K) ? t[e] : 0.f;
      g.b[p] = t;
    }
  } else {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int idx = p * 256 + tid;  // kKC rows x 8 four-wide column groups
      const int k = kc + (idx >> 3), c = n0 + (idx & 7) * 4;
      const int kr = min(k, K - 1);
      const int cc = min(c, (N - 1) & ~3);
      f32x4 t = *reinterpret_cast<const f32x4*>(Bz + (long)kr * ldb + cc);
      g.b[p] = k < K ? t : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  return g;
}

template <bool TRANS_B>
__global__ __launch_bounds__(256) void sgemm_kernel(const float* __restrict__ A, const float* __restrict__ B,
                                                    float* __restrict__ C, int M, int N, int K, int lda, int ldb,
                                                    int ldc, int z0, int heads, int kv_heads, float alpha) {
  __shared__ __attribute__((aligned(16))) float As[32][kKC + 4];
  __shared__ __attribute__((aligned(16))) float Bs[TRANS_B ? 32 : kKC][TRANS_B ? kKC + 4 : 36];
  __shared__ f32x4 red[3][4][64];
  const int tiles_n = (N + 31) / 32;
  const int m0 = (int)(blockIdx.x / tiles_n) * 32, n0 = (int)(blockIdx.x % tiles_n) * 32;
  const long z = blockIdx.y, za = z0 + z;
  const long zb = (za / heads) * kv_heads + (za % heads) / (heads / kv_heads);
  const float* Az = A + z * (long)M * lda;
  const float* Bz = B + zb * (TRANS_B ? (long)N * ldb : (long)K * ldb);
  float* Cz = C + z * (long)M * ldc;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int tx = lane & 7, ty = lane >> 3;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  }
  GemmStage<TRANS_B> g = gemm_fetch<TRANS_B>(Az, Bz, m0, n0, M, N, K, lda, ldb, 0, tid);
  for (int kc = 0; kc < K; kc += kKC) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int idx = p * 256 + tid;
      *reinterpret_cast<f32x4*>(&As[idx >> 5][(idx & 31) * 4]) = g.a[p];
      if (TRANS_B) {
        *reinterpret_cast<f32x4*>(&Bs[idx >> 5][(idx & 31) * 4]) = g.b[p];
      } else {
        *reinterpret_cast<f32x4*>(&Bs[idx >> 3][(idx & 7) * 4]) = g.b[p];
      }
    }
    __syncthreads();
    if (kc + kKC < K) g = gemm_fetch<TRANS_B>(Az, Bz, m0, n0, M, N, K, lda, ldb, kc + kKC, tid);
#pragma unroll 2
    for (int k = w * (kKC / 4); k < (w + 1) * (kKC / 4); k += 4) {
      f32x4 av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = *reinterpret_cast<const f32x4*>(&As[ty + 8 * i][k]);
      if (TRANS_B) {
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[j] = *reinterpret_cast<const f32x4*>(&Bs[tx + 8 * j][k]);
      } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) bv[kk] = *reinterpret_cast<const f32x4*>(&Bs[k + kk][4 * tx]);
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float bb = TRANS_B ? bv[j][kk] : bv[kk][j];
            acc[i][j] = __builtin_fmaf(av[i][kk], bb, acc[i][j]);
          }
        }
      }
    }
    __syncthreads();
  }
  if (w > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[w - 1][i][lane] = f32x4{acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
  }
  __syncthreads();
  if (w > 0) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f32x4 t = f32x4{acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
#pragma unroll
    for (int p = 0; p < 3; ++p) t += red[p][i][lane];
    const int m = m0 + ty + 8 * i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = TRANS_B ? n0 + tx + 8 * j : n0 + 4 * tx + j;
      if (n < N) Cz[(long)m * ldc + n] = t[j] * alpha;
    }
  }
}

// Block reductions over a 256-thread workgroup (4 waves).
__device__ __forceinline__ float block_max(float x, float* red) {
  for (int m = 32; m > 0; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  x = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return x;
}
__device__ __forceinline__ float block_sum(float x, float* red) {
  for (int m = 32; m > 0; m >>= 1) x += __shfl_xor(x, m, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  x = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return x;
}

// One map row per workgroup: the row's scores go to LDS, then tile c is kept
// when fewer than k tiles beat it (a higher score, or an equal score at a
// lower index), or when k reaches the tile count. With an H3 prefix
// (n_prefix tiles), prefix rows and prefix columns are kept and only the video
// columns are ranked.
__global__ __launch_bounds__(256) void topk_map_kernel(const float* __restrict__ scores, uint8_t* __restrict__ map,
                                                       int n_tiles, int ld, int keep, int n_prefix) {
  extern __shared__ float srow[];  // [stride]
  const int stride = (n_tiles + 3) & ~3;
  const long row = blockIdx.x;
  const bool dense_row = keep >= n_tiles - n_prefix || (int)(row % n_tiles) < n_prefix;
  const float* in = scores + row * ld;
  // prefix columns sit out the ranking (kept anyway): below every score
  for (int c = threadIdx.x; c < stride; c += blockDim.x) srow[c] = c < n_tiles && c >= n_prefix ? in[c] : kNegInf;
  __syncthreads();
  uint8_t* mrow = map + row * n_tiles;
  for (int c = threadIdx.x; c < n_tiles; c += blockDim.x) {
    uint8_t kept = 1;
    if (!dense_row && c >= n_prefix) {
      const float v = srow[c];
      int r0 = 0, r1 = 0, r2 = 0, r3 = 0;
      for (int j = 0; j < stride; j += 4) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(srow + j);
        r0 += (t[0] > v) || (t[0] == v && j < c);
        r1 += (t[1] > v) || (t[1] == v && j + 1 < c);
        r2 += (t[2] > v) || (t[2] == v && j + 2 < c);
        r3 += (t[3] > v) || (t[3] == v && j + 3 < c);
      }
      kept = (r0 + r1 + r2 + r3) < keep;
    }
    mrow[c] = kept;
  }
}

// Order-preserving map of a float to an unsigned key (larger float, larger
// key; -0 sorts just below +0). Key 0 is below every finite score.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One map row per wave, for rows of at most 64 R tiles (lane l holds tiles
// l, l + 64, ...). The keep-th largest key T is found bit by bit from the top
// (the largest T with at least keep keys >= T, counted with wave ballots);
// then every key above T is kept, and of the keys equal to T the lowest-index
// ones until keep is reached. With an H3 prefix, prefix rows keep everything
// and prefix columns are kept outside the ranking (keep < video tiles here).
template <int R>
__global__ __launch_bounds__(256) void topk_wave_kernel(const float* __restrict__ scores, uint8_t* __restrict__ map,
                                                        int n_tiles, int ld, int keep, long rows, int n_prefix) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  uint8_t* mrow = map + row * n_tiles;
  if ((int)(row % n_tiles) < n_prefix) {  // a prefix query tile keeps every key tile
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r * 64 + lane < n_tiles) mrow[r * 64 + lane] = 1;
    }
    return;
  }
  const float* in = scores + row * ld;
  uint32_t key[R];  // prefix columns get key 0: below every score, never counted
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int idx = r * 64 + lane;
    key[r] = idx < n_tiles && idx >= n_prefix ? order_key(in[idx]) : 0u;
  }
  uint32_t t = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = t | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) cnt += __popcll(__ballot(key[r] >= cand));
    if (cnt >= keep) t = cand;
  }
  int above = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) above += __popcll(__ballot(key[r] > t));
  const int quota = keep - above;
  int eq_before = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int idx = r * 64 + lane;
    const unsigned long long eq = __ballot(idx < n_tiles && idx >= n_prefix && key[r] == t);
    const int rank = eq_before + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(eq >> 32),
                                                                __builtin_amdgcn_mbcnt_lo((uint32_t)eq, 0u));
    eq_before += __popcll(eq);
    if (idx < n_tiles) {
      mrow[idx] = (uint8_t)(idx < n_prefix || key[r] > t || (key[r] == t && idx >= n_prefix && rank < quota));
    }
  }
}

// Row softmax in place (fp32, exp2 of (s - max) * log2 e) over the first n
// entries of rows ld apart: one row per workgroup.
__global__ __launch_bounds__(256) void softmax_rows_kernel(float* __restrict__ x, int n, int ld) {
  __shared__ float red[4];
  float* row = x + (long)blockIdx.x * ld;
  float mx = kNegInf;
  for (int c = threadIdx.x; c < n; c += blockDim.x) mx = fmaxf(mx, row[c]);
  mx = block_max(mx, red);
  float sum = 0.f;
  for (int c = threadIdx.x; c < n; c += blockDim.x) {
    const float e = hw_exp2((row[c] - mx) * kLog2e);
    row[c] = e;
    sum += e;
  }
  const float inv = 1.f / block_sum(sum, red);
  for (int c = threadIdx.x; c < n; c += blockDim.x) row[c] *= inv;
}

template <bool TRANS_B>
static hipError_t launch_sgemm(const float* A, const float* B, float* C, int M, int N, int K, int lda, int ldb,
                               int ldc, int z0, int nz, int heads, int kv_heads, float alpha, hipStream_t stream) {
  const dim3 grid((unsigned)(((M + 31) / 32) * ((N + 31) / 32)), (unsigned)nz);
  hipLaunchKernelGGL((sgemm_kernel<TRANS_B>), grid, dim3(256), 0, stream, A, B, C, M, N, K, lda, ldb, ldc, z0, heads,
                     kv_heads, alpha);
  return hipGetLastError();
}

// The score matrices [n_tiles][n_tiles] are built for a chunk of (batch, head)
// pairs at a time, so the workspace stays within kScoreChunkBytes (or one
// pair's matrix, when that is larger).
constexpr size_t kScoreChunkBytes = (size_t)64 << 20;

static int score_ld(int n_tiles) { return (n_tiles + 3) & ~3; }

static int score_chunk(int batch, int heads, int n_tiles) {
  const size_t one = (size_t)n_tiles * score_ld(n_tiles) * sizeof(float);
  size_t c = kScoreChunkBytes / (one > 0 ? one : 1);
  const size_t total = (size_t)batch * heads;
  c = c < 1 ? 1 : (c > total ? total : c);
  c = c > 65535 ? 65535 : c;  // the launch grid's y extent
  return (int)c;
}

static size_t score_bytes(int batch, int heads, int n_tiles) {
  return (size_t)score_chunk(batch, heads, n_tiles) * n_tiles * score_ld(n_tiles) * sizeof(float);
}

static hipError_t launch_pool(const PoolArgs& pa, int n_src, const int32_t* sizes, int batch, int n_tiles,
                              int head_dim, hipStream_t stream) {
  hipLaunchKernelGGL(tile_pool_kernel, dim3((unsigned)((long)batch * n_tiles), (unsigned)n_src), dim3(256), 0, stream,
                     pa, sizes, n_tiles, head_dim);
  return hipGetLastError();
}

// out[b][64a + r][h][:] += c[b][h][a][:] * gate[b][64a + r][h][:] for every row of
// every tile, in fp32, rounded to bf16 once. One wave per tile-order row; a lane
// owns 8 consecutive elements of the row (all heads).
__global__ __launch_bounds__(256) void compressed_add_kernel(const float* __restrict__ comp,
                                                             const uint16_t* __restrict__ gate,
                                                             uint16_t* __restrict__ out, int n_tiles, int heads,
                                                             int head_dim, long rows) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);  // over batch * n_tiles * 64
  if (row >= rows) return;
  const long per_batch = (long)n_tiles * 64;
  const long b = row / per_batch;
  const int a = (int)((row % per_batch) >> 6);
  const int row_elems = heads * head_dim;
  const uint16_t* grow = gate + row * row_elems;
  uint16_t* orow = out + row * row_elems;
  for (int j = lane * 8; j < row_elems; j += 64 * 8) {
    const int h = j / head_dim, d = j % head_dim;
    const float* crow = comp + ((b * heads + h) * n_tiles + a) * (long)head_dim + d;
    const u32x4 gv = ld_global16(grow + j);
    const u32x4 ov = ld_global16(orow + j);
    const f32x4 c0 = *reinterpret_cast<const f32x4*>(crow);
    const f32x4 c1 = *reinterpret_cast<const f32x4*>(crow + 4);
    f32x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float g0 = __uint_as_float(gv[i] << 16), g1 = __uint_as_float(gv[i] & 0xffff0000u);
      const float o0 = __uint_as_float(ov[i] << 16), o1 = __uint_as_float(ov[i] & 0xffff0000u);
      const float cc0 = i < 2 ? c0[2 * i] : c1[2 * i - 4];
      const float cc1 = i < 2 ? c0[2 * i + 1] : c1[2 * i - 3];
      r[2 * i] = __builtin_fmaf(cc0, g0, o0);
      r[2 * i + 1] = __builtin_fmaf(cc1, g1, o1);
    }
    *reinterpret_cast<bf16x8*>(orow + j) = to_bf16x8(r);
  }
}

static BoxGeom make_geom(const VsaGeometry& g) {
  BoxGeom b;
  b.T = g.t; b.H = g.h; b.W = g.w;
  b.tt = g.tile_t; b.th = g.tile_h; b.tw = g.tile_w;
  b.nbt = (g.t + g.tile_t - 1) / g.tile_t;
  b.nbh = (g.h + g.tile_h - 1) / g.tile_h;
  b.nbw = (g.w + g.tile_w - 1) / g.tile_w;
  return b;
}

// Non-empty segments only; the host has checked num_segments <= kMaxPrefixSegments.
static PrefixLayout make_prefix(const VsaGeometry& g) {
  PrefixLayout p{};
  for (int i = 0; i < g.num_segments; ++i) {
    const int len = g.prefix_segments[i];
    if (len <= 0) continue;
    p.start[p.n_seg] = p.len;
    p.tile0[p.n_seg] = p.n_tiles;
    p.len += len;
    p.n_tiles += (len + 63) / 64;
    ++p.n_seg;
  }
  p.start[p.n_seg] = p.len;
  p.tile0[p.n_seg] = p.n_tiles;
  return p;
}

int vsa_prefix_tiles(const VsaGeometry& g) { return make_prefix(g).n_tiles; }

int vsa_num_tiles(const VsaGeometry& g) {
  const BoxGeom b = make_geom(g);
  return vsa_prefix_tiles(g) + b.nbt * b.nbh * b.nbw;
}

hipError_t launch_tile_gather(const void* x, const VsaGeometry& g, int batch, int row_elems, void* y,
                              int32_t* sizes, hipStream_t stream) {
  const BoxGeom gm = make_geom(g);
  const PrefixLayout pl = make_prefix(g);
  const int nt = pl.n_tiles + gm.nbt * gm.nbh * gm.nbw;
  const long rows = (long)batch * nt * 64;
  hipLaunchKernelGGL(tile_gather_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream,
                     (const uint16_t*)x, (uint16_t*)y, sizes, gm, pl, nt, batch, row_elems);
  return hipGetLastError();
}

hipError_t launch_untile(const void* y, const VsaGeometry& g, int batch, int row_elems, void* x, hipStream_t stream) {
  const BoxGeom gm = make_geom(g);
  const PrefixLayout pl = make_prefix(g);
  const int nt = pl.n_tiles + gm.nbt * gm.nbh * gm.nbw;
  const long rows = (long)batch * (pl.len + (long)g.t * g.h * g.w);
  hipLaunchKernelGGL(untile_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, (const uint16_t*)y,
                     (uint16_t*)x, gm, pl, nt, batch, row_elems);
  return hipGetLastError();
}

template <int R>
static void launch_topk_wave(const float* scores, uint8_t* map, int n_tiles, int ld, int keep, long rows,
                             int n_prefix, hipStream_t stream) {
  hipLaunchKernelGGL(topk_wave_kernel<R>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, scores, map,
                     n_tiles, ld, keep, rows, n_prefix);
}

// Rows of up to 1024 tiles take the one-wave radix select; longer rows (and
// k covering every video tile) the workgroup-per-row ranking.
static hipError_t launch_topk(const float* scores, uint8_t* map, int n_tiles, int ld, int keep, long rows, size_t lds,
                              int n_prefix, hipStream_t stream) {
  if (keep >= n_tiles - n_prefix || n_tiles > 1024) {
    hipLaunchKernelGGL(topk_map_kernel, dim3((unsigned)rows), dim3(256), lds, stream, scores, map, n_tiles, ld, keep,
                       n_prefix);
  } else if (n_tiles <= 64) {
    launch_topk_wave<1>(scores, map, n_tiles, ld, keep, rows, n_prefix, stream);
  } else if (n_tiles <= 128) {
    launch_topk_wave<2>(scores, map, n_tiles, ld, keep, rows, n_prefix, stream);
  } else if (n_tiles <= 256) {
    launch_topk_wave<4>(scores, map, n_tiles, ld, keep, rows, n_prefix, stream);
  } else if (n_tiles <= 512) {
    launch_topk_wave<8>(scores, map, n_tiles, ld, keep, rows, n_prefix, stream);
  } else {
    launch_topk_wave<16>(scores, map, n_tiles, ld, keep, rows, n_prefix, stream);
  }
  return hipGetLastError();
}

size_t vsa_map_workspace_bytes(int batch, int heads, int kv_heads, int n_tiles, int head_dim) {
  return ((size_t)batch * heads * n_tiles * head_dim + (size_t)batch * kv_heads * n_tiles * head_dim) * sizeof(float) +
         score_bytes(batch, heads, n_tiles);
}

static hipError_t map_from_means(const float* qpool, const float* kpool, float* scores, int batch, int n_tiles,
                                 int heads, int kv_heads, int head_dim, float scale, int topk, uint8_t* map,
                                 hipStream_t stream, int n_prefix);

hipError_t launch_vsa_block_map(const void* q_tiled, const void* k_tiled, const int32_t* sizes, int batch,
                                int n_tiles, int heads, int kv_heads, int head_dim, float scale, int topk,
                                uint8_t* map, void* workspace, hipStream_t stream, int n_prefix) {
  float* qpool = (float*)workspace;
  float* kpool = qpool + (size_t)batch * heads * n_tiles * head_dim;
  float* scores = kpool + (size_t)batch * kv_heads * n_tiles * head_dim;
  PoolArgs pa{};
  pa.s[0] = PoolSrc{(const uint16_t*)q_tiled, qpool, heads};
  pa.s[1] = PoolSrc{(const uint16_t*)k_tiled, kpool, kv_heads};
  const hipError_t e = launch_pool(pa, 2, sizes, batch, n_tiles, head_dim, stream);
  if (e != hipSuccess) return e;
  return map_from_means(qpool, kpool, scores, batch, n_tiles, heads, kv_heads, head_dim, scale, topk, map, stream,
                        n_prefix);
}

hipError_t launch_vsa_gather_block_map(const void* q, const void* k, const VsaGeometry& g, int batch, int heads,
                                       int kv_heads, int head_dim, float scale, int topk, void* q_tiled,
                                       void* k_tiled, int32_t* sizes, uint8_t* map, void* workspace,
                                       hipStream_t stream) {
  const BoxGeom gm = make_geom(g);
  const PrefixLayout pl = make_prefix(g);
  const int n_tiles = pl.n_tiles + gm.nbt * gm.nbh * gm.nbw;
  const long n_rows = (long)pl.len + (long)gm.T * gm.H * gm.W;
  float* qpool = (float*)workspace;
  float* kpool = qpool + (size_t)batch * heads * n_tiles * head_dim;
  float* scores = kpool + (size_t)batch * kv_heads * n_tiles * head_dim;
  GatherPoolArgs pa{};
  pa.s[0] = GatherPoolSrc{(const uint16_t*)q, (uint16_t*)q_tiled, qpool, heads};
  pa.s[1] = GatherPoolSrc{(const uint16_t*)k, (uint16_t*)k_tiled, kpool, kv_heads};
  const int col_groups = (heads * head_dim / 8 + 63) / 64;  // q has at least as many heads as k
  hipLaunchKernelGGL(tile_gather_pool_kernel, dim3((unsigned)((long)batch * n_tiles), 2u, (unsigned)col_groups),
                     dim3(256), 0, stream, pa, gm, pl, n_tiles, n_rows, head_dim, sizes);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return map_from_means(qpool, kpool, scores, batch, n_tiles, heads, kv_heads, head_dim, scale, topk, map, stream,
                        pl.n_tiles);
}

// Pooled scores (batched fp32 GEMM of the tile means) and the per-row top-k,
// in chunks of (batch, head) pairs sized to the score buffer.
static hipError_t map_from_means(const float* qpool, const float* kpool, float* scores, int batch, int n_tiles,
                                 int heads, int kv_heads, int head_dim, float scale, int topk, uint8_t* map,
                                 hipStream_t stream, int n_prefix) {
  hipError_t e = hipSuccess;
  const int n_video = n_tiles - n_prefix;
  const int keep = topk < n_video ? topk : n_video;
  const int total = batch * heads, chunk = score_chunk(batch, heads, n_tiles), ld = score_ld(n_tiles);
  const size_t lds = (size_t)((n_tiles + 3) & ~3) * sizeof(float);
  const size_t mat = (size_t)n_tiles * head_dim;
  for (int z0 = 0; z0 < total; z0 += chunk) {
    const int nz = total - z0 < chunk ? total - z0 : chunk;
    e = launch_sgemm<true>(qpool + z0 * mat, kpool, scores, n_tiles, n_tiles, head_dim, head_dim, head_dim, ld, z0,
                           nz, heads, kv_heads, scale, stream);
    if (e != hipSuccess) return e;
    e = launch_topk(scores, map + (size_t)z0 * n_tiles * n_tiles, n_tiles, ld, keep, (long)nz * n_tiles, lds,
                    n_prefix, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

size_t vsa_compressed_workspace_bytes(int batch, int heads, int kv_heads, int n_tiles, int head_dim) {
  return ((size_t)2 * batch * heads * n_tiles * head_dim + (size_t)2 * batch * kv_heads * n_tiles * head_dim) *
             sizeof(float) +
         score_bytes(batch, heads, n_tiles);
}

// Compressed branch: pooled q, k, v per tile; per (batch, head) the scores
// scale * qbar kbar^T, their row softmax over all key tiles, and the weighted
// sum of the value means (one fp32 row per query tile); then every row of a
// query tile adds its tile's row, times the gate, into the output.
hipError_t launch_vsa_compressed_add(const void* q_tiled, const void* k_tiled, const void* v_tiled,
                                     const int32_t* sizes, const void* gate, int batch, int n_tiles, int heads,
                                     int kv_heads, int head_dim, float scale, void* out, void* workspace,
                                     hipStream_t stream) {
  float* qpool = (float*)workspace;
  float* comp = qpool + (size_t)batch * heads * n_tiles * head_dim;
  float* kpool = comp + (size_t)batch * heads * n_tiles * head_dim;
  float* vpool = kpool + (size_t)batch * kv_heads * n_tiles * head_dim;
  float* scores = vpool + (size_t)batch * kv_heads * n_tiles * head_dim;
  PoolArgs pa{};
  pa.s[0] = PoolSrc{(const uint16_t*)q_tiled, qpool, heads};
  pa.s[1] = PoolSrc{(const uint16_t*)k_tiled, kpool, kv_heads};
  pa.s[2] = PoolSrc{(const uint16_t*)v_tiled, vpool, kv_heads};
  hipError_t e = launch_pool(pa, 3, sizes, batch, n_tiles, head_dim, stream);
  if (e != hipSuccess) return e;
  const int total = batch * heads, chunk = score_chunk(batch, heads, n_tiles), ld = score_ld(n_tiles);
  const size_t mat = (size_t)n_tiles * head_dim;
  for (int z0 = 0; z0 < total; z0 += chunk) {
    const int nz = total - z0 < chunk ? total - z0 : chunk;
    e = launch_sgemm<true>(qpool + z0 * mat, kpool, scores, n_tiles, n_tiles, head_dim, head_dim, head_dim, ld, z0,
                           nz, heads, kv_heads, scale, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(softmax_rows_kernel, dim3((unsigned)((long)nz * n_tiles)), dim3(256), 0, stream, scores,
                       n_tiles, ld);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_sgemm<false>(scores, vpool, comp + z0 * mat, n_tiles, head_dim, n_tiles, ld, head_dim, head_dim, z0, nz,
                            heads, kv_heads, 1.f, stream);
    if (e != hipSuccess) return e;
  }
  const long rows = (long)batch * n_tiles * 64;
  hipLaunchKernelGGL(compressed_add_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, comp,
                     (const uint16_t*)gate, (uint16_t*)out, n_tiles, heads, head_dim, rows);
  return hipGetLastError();
}


}  // namespace attn
