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

// One wave per tile-order destination row.
__global__ __launch_bounds__(256) void tile_gather_kernel(const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
                                                          int32_t* __restrict__ sizes, BoxGeom gm, int n_tiles,
                                                          int batch, int row_elems) {
  const int lane = threadIdx.x & 63;
  const long dst = (long)blockIdx.x * 4 + (threadIdx.x >> 6);  // over batch * n_tiles * 64
  const long rows_per_batch = (long)n_tiles * 64;
  if (dst >= batch * rows_per_batch) return;
  const int b = (int)(dst / rows_per_batch);
  const int p = (int)(dst % rows_per_batch);
  const int c = p >> 6, r = p & 63;
  int bt, bh, bw, et, eh, ew;
  gm.box_extent(c, bt, bh, bw, et, eh, ew);
  const int size = et * eh * ew;
  if (sizes != nullptr && b == 0 && r == 0 && lane == 0) sizes[c] = size;
  uint16_t* yrow = y + dst * row_elems;
  const int chunks = row_elems / 8;
  if (r >= size) {
    for (int j = lane; j < chunks; j += 64) *reinterpret_cast<u32x4*>(yrow + j * 8) = u32x4{0u, 0u, 0u, 0u};
    return;
  }
  const int it = r / (eh * ew), ih = (r / ew) % eh, iw = r % ew;
  const long tok = ((long)(bt * gm.tt + it) * gm.H + (bh * gm.th + ih)) * gm.W + (bw * gm.tw + iw);
  const uint16_t* xrow = x + ((long)b * gm.T * gm.H * gm.W + tok) * row_elems;
  for (int j = lane; j < chunks; j += 64) *reinterpret_cast<u32x4*>(yrow + j * 8) = ld_global16(xrow + j * 8);
}

// One wave per raster destination row.
__global__ __launch_bounds__(256) void untile_kernel(const uint16_t* __restrict__ y, uint16_t* __restrict__ x,
                                                     BoxGeom gm, int n_tiles, int batch, int row_elems) {
  const int lane = threadIdx.x & 63;
  const long n_tok = (long)gm.T * gm.H * gm.W;
  const long dst = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (dst >= batch * n_tok) return;
  const int b = (int)(dst / n_tok);
  const long tok = dst % n_tok;
  const int w = (int)(tok % gm.W), h = (int)((tok / gm.W) % gm.H), t = (int)(tok / ((long)gm.W * gm.H));
  const int c = ((t / gm.tt) * gm.nbh + h / gm.th) * gm.nbw + w / gm.tw;
  int bt, bh, bw, et, eh, ew;
  gm.box_extent(c, bt, bh, bw, et, eh, ew);
  const int r = ((t - bt * gm.tt) * eh + (h - bh * gm.th)) * ew + (w - bw * gm.tw);
  const uint16_t* yrow = y + ((long)b * n_tiles * 64 + (long)c * 64 + r) * row_elems;
  uint16_t* xrow = x + dst * row_elems;
  const int chunks = row_elems / 8;
  for (int j = lane; j < chunks; j += 64) *reinterpret_cast<u32x4*>(xrow + j * 8) = ld_global16(yrow + j * 8);
}

// Tile means: pooled[b][h][c][d] = (sum of the size(c) real rows) / max(size, 1),
// fp32, rows summed in ascending order. One workgroup per (batch, tile); a
// thread owns one 16-byte chunk (8 columns of one head) of the tile's rows, so
// a row is read by consecutive threads.
__global__ __launch_bounds__(256) void tile_pool_kernel(const uint16_t* __restrict__ x,
                                                       const int32_t* __restrict__ sizes, float* __restrict__ pooled,
                                                       int n_tiles, int heads, int head_dim) {
  const int c = (int)(blockIdx.x % n_tiles);
  const long b = blockIdx.x / n_tiles;
  const int size = clampi(sizes[c], 0, 64);
  const float inv = 1.f / (float)(size > 1 ? size : 1);
  const long row_elems = (long)heads * head_dim;
  const uint16_t* base = x + (b * n_tiles + c) * 64 * row_elems;
  const int chunks = (int)(row_elems / 8);
  for (int j = threadIdx.x; j < chunks; j += blockDim.x) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll 8
    for (int r = 0; r < size; ++r) {
      const u32x4 v = ld_global16(base + (long)r * row_elems + j * 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += __uint_as_float(v[i] << 16);
        acc[2 * i + 1] += __uint_as_float(v[i] & 0xffff0000u);
      }
    }
    const int h = (j * 8) / head_dim, d = (j * 8) % head_dim;
    float* prow = pooled + ((b * heads + h) * n_tiles + c) * (long)head_dim + d;
    *reinterpret_cast<f32x4*>(prow) = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    *reinterpret_cast<f32x4*>(prow + 4) = f32x4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
  }
}

// Batched fp32 GEMM for the pooled scores and the compressed rows:
// C[z] = alpha * A[z] B'[z], A [M][K] row-major; B' = B^T with B stored [N][K]
// (TRANS_B), else B' = B stored [K][N]. The launch covers batch entries
// z0 + z = b * heads + h; A and C are indexed by z (the caller offsets them),
// B by b * kv_heads + h / (heads / kv_heads) (grouped heads). A
// 256-thread workgroup owns a 64 x 64 tile of C, each thread 4 x 4 of it;
// K advances 16 at a time through LDS. Sums run over k in ascending order.
template <bool TRANS_B>
__global__ __launch_bounds__(256) void sgemm_kernel(const float* __restrict__ A, const float* __restrict__ B,
                                                    float* __restrict__ C, int M, int N, int K, int z0,
                                                    int heads, int kv_heads, float alpha) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const int tiles_n = (N + 63) / 64;
  const int m0 = (int)(blockIdx.x / tiles_n) * 64, n0 = (int)(blockIdx.x % tiles_n) * 64;
  const long z = blockIdx.y, za = z0 + z;
  const long zb = (za / heads) * kv_heads + (za % heads) / (heads / kv_heads);
  const float* Az = A + z * (long)M * K;
  const float* Bz = B + zb * (long)N * K;
  float* Cz = C + z * (long)M * N;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    {  // A tile [64 rows][16 k] -> As[k][row]
      const int r = tid >> 2, c = (tid & 3) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + r, k = k0 + c + i;
        As[c + i][r] = (m < M && k < K) ? Az[(long)m * K + k] : 0.f;
      }
    }
    if (TRANS_B) {  // B stored [N][K]: tile [64 n][16 k] -> Bs[k][n]
      const int r = tid >> 2, c = (tid & 3) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n0 + r, k = k0 + c + i;
        Bs[c + i][r] = (n < N && k < K) ? Bz[(long)n * K + k] : 0.f;
      }
    } else {  // B stored [K][N]: tile [16 k][64 n] -> Bs[k][n]
      const int r = tid >> 4, c = (tid & 15) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = k0 + r, n = n0 + c + i;
        Bs[r][c + i] = (n < N && k < K) ? Bz[(long)k * N + n] : 0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < N) Cz[(long)m * N + n] = acc[i][j] * alpha;
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
// lower index), or when k reaches the tile count.
__global__ __launch_bounds__(256) void topk_map_kernel(const float* __restrict__ scores, uint8_t* __restrict__ map,
                                                       int n_tiles, int keep) {
  extern __shared__ float srow[];  // [stride]
  const int stride = (n_tiles + 3) & ~3;
  const long row = blockIdx.x;
  const float* in = scores + row * n_tiles;
  for (int c = threadIdx.x; c < stride; c += blockDim.x) srow[c] = c < n_tiles ? in[c] : kNegInf;
  __syncthreads();
  uint8_t* mrow = map + row * n_tiles;
  for (int c = threadIdx.x; c < n_tiles; c += blockDim.x) {
    uint8_t kept = 1;
    if (keep < n_tiles) {
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

// Row softmax in place (fp32, exp2 of (s - max) * log2 e): one row per workgroup.
__global__ __launch_bounds__(256) void softmax_rows_kernel(float* __restrict__ x, int n) {
  __shared__ float red[4];
  float* row = x + (long)blockIdx.x * n;
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
static hipError_t launch_sgemm(const float* A, const float* B, float* C, int M, int N, int K, int z0, int nz,
                               int heads, int kv_heads, float alpha, hipStream_t stream) {
  const dim3 grid((unsigned)(((M + 63) / 64) * ((N + 63) / 64)), (unsigned)nz);
  hipLaunchKernelGGL((sgemm_kernel<TRANS_B>), grid, dim3(256), 0, stream, A, B, C, M, N, K, z0, heads, kv_heads,
                     alpha);
  return hipGetLastError();
}

// The score matrices [n_tiles][n_tiles] are built for a chunk of (batch, head)
// pairs at a time, so the workspace stays within kScoreChunkBytes (or one
// pair's matrix, when that is larger).
constexpr size_t kScoreChunkBytes = (size_t)64 << 20;

static int score_chunk(int batch, int heads, int n_tiles) {
  const size_t one = (size_t)n_tiles * n_tiles * sizeof(float);
  size_t c = kScoreChunkBytes / (one > 0 ? one : 1);
  const size_t total = (size_t)batch * heads;
  c = c < 1 ? 1 : (c > total ? total : c);
  c = c > 65535 ? 65535 : c;  // the launch grid's y extent
  return (int)c;
}

static size_t score_bytes(int batch, int heads, int n_tiles) {
  return (size_t)score_chunk(batch, heads, n_tiles) * n_tiles * n_tiles * sizeof(float);
}

static hipError_t launch_pool(const void* x, const int32_t* sizes, float* pooled, int batch, int n_tiles, int heads,
                              int head_dim, hipStream_t stream) {
  hipLaunchKernelGGL(tile_pool_kernel, dim3((unsigned)((long)batch * n_tiles)), dim3(256), 0, stream,
                     (const uint16_t*)x, sizes, pooled, n_tiles, heads, head_dim);
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

int vsa_num_tiles(const VsaGeometry& g) {
  const BoxGeom b = make_geom(g);
  return b.nbt * b.nbh * b.nbw;
}

hipError_t launch_tile_gather(const void* x, const VsaGeometry& g, int batch, int row_elems, void* y,
                              int32_t* sizes, hipStream_t stream) {
  const BoxGeom gm = make_geom(g);
  const int nt = gm.nbt * gm.nbh * gm.nbw;
  const long rows = (long)batch * nt * 64;
  hipLaunchKernelGGL(tile_gather_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream,
                     (const uint16_t*)x, (uint16_t*)y, sizes, gm, nt, batch, row_elems);
  return hipGetLastError();
}

hipError_t launch_untile(const void* y, const VsaGeometry& g, int batch, int row_elems, void* x, hipStream_t stream) {
  const BoxGeom gm = make_geom(g);
  const int nt = gm.nbt * gm.nbh * gm.nbw;
  const long rows = (long)batch * g.t * g.h * g.w;
  hipLaunchKernelGGL(untile_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, (const uint16_t*)y,
                     (uint16_t*)x, gm, nt, batch, row_elems);
  return hipGetLastError();
}

size_t vsa_map_workspace_bytes(int batch, int heads, int kv_heads, int n_tiles, int head_dim) {
  return ((size_t)batch * heads * n_tiles * head_dim + (size_t)batch * kv_heads * n_tiles * head_dim) * sizeof(float) +
         score_bytes(batch, heads, n_tiles);
}

hipError_t launch_vsa_block_map(const void* q_tiled, const void* k_tiled, const int32_t* sizes, int batch,
                                int n_tiles, int heads, int kv_heads, int head_dim, float scale, int topk,
                                uint8_t* map, void* workspace, hipStream_t stream) {
  float* qpool = (float*)workspace;
  float* kpool = qpool + (size_t)batch * heads * n_tiles * head_dim;
  float* scores = kpool + (size_t)batch * kv_heads * n_tiles * head_dim;
  hipError_t e = launch_pool(q_tiled, sizes, qpool, batch, n_tiles, heads, head_dim, stream);
  if (e == hipSuccess) e = launch_pool(k_tiled, sizes, kpool, batch, n_tiles, kv_heads, head_dim, stream);
  if (e != hipSuccess) return e;
  const int keep = topk < n_tiles ? topk : n_tiles;
  const int total = batch * heads, chunk = score_chunk(batch, heads, n_tiles);
  const size_t lds = (size_t)((n_tiles + 3) & ~3) * sizeof(float);
  const size_t mat = (size_t)n_tiles * head_dim;
  for (int z0 = 0; z0 < total; z0 += chunk) {
    const int nz = total - z0 < chunk ? total - z0 : chunk;
    e = launch_sgemm<true>(qpool + z0 * mat, kpool, scores, n_tiles, n_tiles, head_dim, z0, nz, heads, kv_heads,
                           scale, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_map_kernel, dim3((unsigned)((long)nz * n_tiles)), dim3(256), lds, stream, scores,
                       map + (size_t)z0 * n_tiles * n_tiles, n_tiles, keep);
    e = hipGetLastError();
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
  hipError_t e = launch_pool(q_tiled, sizes, qpool, batch, n_tiles, heads, head_dim, stream);
  if (e == hipSuccess) e = launch_pool(k_tiled, sizes, kpool, batch, n_tiles, kv_heads, head_dim, stream);
  if (e == hipSuccess) e = launch_pool(v_tiled, sizes, vpool, batch, n_tiles, kv_heads, head_dim, stream);
  if (e != hipSuccess) return e;
  const int total = batch * heads, chunk = score_chunk(batch, heads, n_tiles);
  const size_t mat = (size_t)n_tiles * head_dim;
  for (int z0 = 0; z0 < total; z0 += chunk) {
    const int nz = total - z0 < chunk ? total - z0 : chunk;
    e = launch_sgemm<true>(qpool + z0 * mat, kpool, scores, n_tiles, n_tiles, head_dim, z0, nz, heads, kv_heads,
                           scale, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(softmax_rows_kernel, dim3((unsigned)((long)nz * n_tiles)), dim3(256), 0, stream, scores,
                       n_tiles);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_sgemm<false>(scores, vpool, comp + z0 * mat, n_tiles, head_dim, n_tiles, z0, nz, heads, kv_heads, 1.f,
                            stream);
    if (e != hipSuccess) return e;
  }
  const long rows = (long)batch * n_tiles * 64;
  hipLaunchKernelGGL(compressed_add_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, comp,
                     (const uint16_t*)gate, (uint16_t*)out, n_tiles, heads, head_dim, rows);
  return hipGetLastError();
}


}  // namespace attn
