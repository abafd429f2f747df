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
//   select : per (batch, head, query tile) fp32 scores scale * qbar . kbar over
//            all key tiles, then keep the top-k (ties: lower tile index wins;
//            every tile when k reaches the tile count) as a uint8 map row.
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

constexpr int kMapRows = 4;  // query tiles per workgroup of the top-k kernel (at most)

// Scores of up to qg query tiles of one (batch, head) against every key tile,
// then a top-k mask per query tile. LDS holds the qg query means and the
// qg x n_tiles scores. Thread c computes key tile c's scores (one pass over
// its mean); a score is fp32 scale * sum_d qbar[d] kbar[d], d ascending.
// Selection: tile c is kept when fewer than k tiles beat it (a higher score,
// or an equal score at a lower index), or when k reaches the tile count.
__global__ __launch_bounds__(256) void topk_map_kernel(const float* __restrict__ qpool,
                                                       const float* __restrict__ kpool, uint8_t* __restrict__ map,
                                                       int n_tiles, int heads, int kv_heads, int head_dim, float scale,
                                                       int keep, int qg) {
  extern __shared__ float sh[];  // [qg][head_dim] query means, then [qg][stride] scores
  const int stride = (n_tiles + 3) & ~3;  // score rows padded to whole 16-byte groups
  float* qs = sh;
  float* sc = sh + qg * head_dim;
  const int groups = (n_tiles + qg - 1) / qg;
  const int a0 = (int)(blockIdx.x % groups) * qg;
  const long bh = blockIdx.x / groups;
  const int h = (int)(bh % heads), b = (int)(bh / heads);
  const int hk = h / (heads / kv_heads);
  const int nq = n_tiles - a0 < qg ? n_tiles - a0 : qg;
  const float* kbase = kpool + ((long)b * kv_heads + hk) * n_tiles * (long)head_dim;
  for (int i = threadIdx.x; i < nq * head_dim; i += blockDim.x) qs[i] = qpool[(bh * n_tiles + a0) * (long)head_dim + i];
  __syncthreads();
  for (int c = threadIdx.x; c < stride; c += blockDim.x) {
    if (c >= n_tiles) {  // padding: never beats a real score
#pragma unroll
      for (int qi = 0; qi < kMapRows; ++qi) {
        if (qi < nq) sc[qi * stride + c] = kNegInf;
      }
      continue;
    }
    const f32x4* krow = reinterpret_cast<const f32x4*>(kbase + (long)c * head_dim);
    float s[kMapRows];
#pragma unroll
    for (int qi = 0; qi < kMapRows; ++qi) s[qi] = 0.f;
    for (int d4 = 0; d4 < head_dim / 4; ++d4) {
      const f32x4 kv = krow[d4];
#pragma unroll
      for (int qi = 0; qi < kMapRows; ++qi) {
        if (qi < nq) {
          const float* qrow = qs + qi * head_dim + 4 * d4;
          s[qi] = __builtin_fmaf(qrow[0], kv[0], s[qi]);
          s[qi] = __builtin_fmaf(qrow[1], kv[1], s[qi]);
          s[qi] = __builtin_fmaf(qrow[2], kv[2], s[qi]);
          s[qi] = __builtin_fmaf(qrow[3], kv[3], s[qi]);
        }
      }
    }
#pragma unroll
    for (int qi = 0; qi < kMapRows; ++qi) {
      if (qi < nq) sc[qi * stride + c] = s[qi] * scale;
    }
  }
  __syncthreads();
  for (int qi = 0; qi < nq; ++qi) {
    const float* srow = sc + qi * stride;
    uint8_t* mrow = map + (bh * n_tiles + a0 + qi) * n_tiles;
    for (int c = threadIdx.x; c < n_tiles; c += blockDim.x) {
      uint8_t kept = 1;
      if (keep < n_tiles) {
        const float v = srow[c];
        // tiles beating c: a higher score, or an equal one at a lower index
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
  return ((size_t)batch * heads * n_tiles * head_dim + (size_t)batch * kv_heads * n_tiles * head_dim) * sizeof(float);
}

hipError_t launch_vsa_block_map(const void* q_tiled, const void* k_tiled, const int32_t* sizes, int batch,
                                int n_tiles, int heads, int kv_heads, int head_dim, float scale, int topk,
                                uint8_t* map, void* workspace, hipStream_t stream) {
  float* qpool = (float*)workspace;
  float* kpool = qpool + (size_t)batch * heads * n_tiles * head_dim;
  hipLaunchKernelGGL(tile_pool_kernel, dim3((unsigned)((long)batch * n_tiles)), dim3(256), 0, stream,
                     (const uint16_t*)q_tiled, sizes, qpool, n_tiles, heads, head_dim);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(tile_pool_kernel, dim3((unsigned)((long)batch * n_tiles)), dim3(256), 0, stream,
                     (const uint16_t*)k_tiled, sizes, kpool, n_tiles, kv_heads, head_dim);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int keep = topk < n_tiles ? topk : n_tiles;
  // as many query tiles per workgroup as keep the scores within 64 KB of LDS
  const int stride = (n_tiles + 3) & ~3;
  int qg = (int)((64 * 1024 / sizeof(float) - (size_t)kMapRows * head_dim) / (size_t)stride);
  qg = qg < 1 ? 1 : (qg > kMapRows ? kMapRows : qg);
  const size_t lds = (size_t)qg * (head_dim + stride) * sizeof(float);
  const long groups = (n_tiles + qg - 1) / qg;
  hipLaunchKernelGGL(topk_map_kernel, dim3((unsigned)((long)batch * heads * groups)), dim3(256), lds, stream,
                     qpool, kpool, map, n_tiles, heads, kv_heads, head_dim, scale, keep, qg);
  return hipGetLastError();
}

}  // namespace attn
