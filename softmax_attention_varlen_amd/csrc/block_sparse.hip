// 64-token-tile block-sparse attention for gfx950, driven by a boolean block map.
//
// Step 1 (map -> index): each map row (batch, head, query tile) becomes the
// ascending list of kept key tiles plus a count, built with a wave ballot and
// a prefix popcount (bit-exact, no atomics).
// Step 2 (attention at head_dim 64, and beyond 3072 tiles; head_dims 96 to
// 256 otherwise take the pipelined kernel of block_sparse_pipe.hip): one
// workgroup of 2 waves owns one (batch, head, query
// tile); each wave owns 32 query rows. It walks only the kept key tiles, each
// staged through LDS exactly as in the varlen prefill (K row-major, V
// transposed), with the same S^T = K Q^T MFMA / online softmax / O^T += V^T P^T
// inner step. Rows at or past a tile's size are padding: padding keys are
// masked, padding query rows are written as zeros with LSE = -inf.
#include "attn_common.hpp"
#include "launch.hpp"

namespace attn {

constexpr int kSparseTile = 64;
constexpr int kSparseThreads = 128;

// With `sizes` (the launch of the pipelined kernel) tiles of size 0 are
// dropped and each entry is packed as (size << 24) | tile, so the attention
// loop reads one word per kept tile.
__global__ __launch_bounds__(256) void map_to_index_kernel(const uint8_t* __restrict__ map, int rows, int n_cols,
                                                           const int32_t* __restrict__ sizes,
                                                           int32_t* __restrict__ idx, int32_t* __restrict__ num) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint8_t* mrow = map + row * n_cols;
  int32_t* irow = idx + row * n_cols;
  const unsigned long long below = (1ull << lane) - 1ull;
  int base = 0;
  for (int c0 = 0; c0 < n_cols; c0 += 64) {
    const int col = c0 + lane;
    bool keep = col < n_cols && mrow[col] != 0;
    int32_t val = col;
    if (sizes != nullptr && keep) {
      const int sz = clampi(sizes[col], 0, kSparseTile);
      keep = sz > 0;
      val = (sz << 24) | col;
    }
    const unsigned long long bits = __ballot(keep);
    if (keep) irow[base + __popcll(bits & below)] = val;
    base += __popcll(bits);
  }
  if (lane == 0) num[row] = base;
}

hipError_t launch_map_to_index(const uint8_t* map, int rows, int n_cols, const int32_t* sizes, int32_t* idx,
                               int32_t* num, hipStream_t stream) {
  hipLaunchKernelGGL(map_to_index_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, map, rows,
                     n_cols, sizes, idx, num);
  return hipGetLastError();
}

template <int D>
__global__ __launch_bounds__(kSparseThreads, (D <= 128 ? 2 : 1)) void block_sparse_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ tile_sizes, const int32_t* __restrict__ kidx, const int32_t* __restrict__ knum,
    int num_tiles, int hq, int hkv, float c, uint16_t* __restrict__ out, float* __restrict__ lse) {
  using Tile = KVTile<D, kSparseTile, kSparseThreads>;
  __shared__ __attribute__((aligned(16))) char smem[Tile::BYTES];

  // query tiles fastest, then heads, then batch
  const long id = blockIdx.x;
  const int a = (int)(id % num_tiles);
  const long bh = id / num_tiles;
  const int h = (int)(bh % hq);
  const int b = (int)(bh / hq);
  const int seq = num_tiles * kSparseTile;
  const int hk = h / (hq / hkv);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, n = lane & 31;
  const int qsize = clampi(tile_sizes[a], 0, kSparseTile);
  const int r = w * 32 + n;  // row inside the query tile
  const int r_c = r < qsize ? r : (qsize > 0 ? qsize - 1 : 0);
  const long qrow = (long)b * seq + (long)a * kSparseTile;

  WaveRows32<D> st;
  st.init(q + ((qrow + r_c) * hq + h) * D, g);

  const int32_t* list = kidx + id * (long)num_tiles;
  const int count = qsize > 0 ? clampi(knum[id], 0, num_tiles) : 0;
  const bool wave_live = w * 32 < qsize;
  const long kv_stride = (long)hkv * D;
  const uint16_t* kbatch = k + (long)b * seq * kv_stride + hk * D;
  const uint16_t* vbatch = v + (long)b * seq * kv_stride + hk * D;

  // skip empty key tiles up front so every loaded tile has a real row
  int j = 0;
  int ct = 0, csize = 0;
  auto next_tile = [&](int from, int& tile, int& size) -> int {
    for (int jj = from; jj < count; ++jj) {
      const int t = clampi(list[jj], 0, num_tiles - 1);
      const int sz = clampi(tile_sizes[t], 0, kSparseTile);
      if (sz > 0) {
        tile = t;
        size = sz;
        return jj;
      }
    }
    return count;
  };

  Tile tl;
  j = next_tile(0, ct, csize);
  if (j < count) {
    tl.load(kbatch + (long)ct * kSparseTile * kv_stride, vbatch + (long)ct * kSparseTile * kv_stride, kv_stride,
            csize, tid);
  }
  while (j < count) {
    const int cur_size = csize;
    __syncthreads();
    tl.store(smem, tid);
    __syncthreads();
    int nt = 0, nsize = 0;
    const int jn = next_tile(j + 1, nt, nsize);
    if (jn < count) {
      tl.load(kbatch + (long)nt * kSparseTile * kv_stride, vbatch + (long)nt * kSparseTile * kv_stride,
              kv_stride, nsize, tid);
    }
    if (wave_live) {
      f32x16 s[2];
      st.template scores<Tile::K_STRIDE>(smem, lane, s);
      if (cur_size < kSparseTile) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kb * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
            if (key >= cur_size) s[kb][e] = kNegInf;
          }
        }
      }
      st.template update<Tile::V_STRIDE>(smem + Tile::K_BYTES, lane, s, c);
    }
    j = jn;
    ct = nt;
    csize = nsize;
  }

  if (r >= qsize) {  // padding query row: zeros and LSE = -inf
    st.l = 0.f;
    st.m = kNegInf;
  }
  float* lp = lse != nullptr ? lse + ((long)b * hq + h) * seq + (long)a * kSparseTile + r : nullptr;
  st.finish(out + ((qrow + r) * hq + h) * D, lp, lane, c);
}

size_t sparse_workspace_bytes(int batch, int num_heads, int num_tiles) {
  const size_t rows = (size_t)batch * num_heads * num_tiles;
  return rows * (size_t)num_tiles * sizeof(int32_t) + 2 * rows * sizeof(int32_t);
}

template <int D>
static hipError_t launch_sparse_d(const SparseArgs& a, hipStream_t stream) {
  const long grid = (long)a.batch * a.num_heads * a.num_tiles;
  hipLaunchKernelGGL((block_sparse_fwd_kernel<D>), dim3((unsigned)grid), dim3(kSparseThreads), 0, stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.tile_sizes, a.idx, a.num,
                     a.num_tiles, a.num_heads, a.num_kv_heads, a.scale * kLog2e, (uint16_t*)a.out, a.lse);
  return hipGetLastError();
}

hipError_t launch_block_sparse_fwd(const SparseArgs& a, hipStream_t stream) {
  const int rows = a.batch * a.num_heads * a.num_tiles;
  const bool pipe = sparse_pipe_supported(a.head_dim, a.num_tiles);
  hipError_t e = launch_map_to_index(a.block_map, rows, a.num_tiles, pipe ? a.tile_sizes : nullptr, a.idx, a.num,
                                     stream);
  if (e != hipSuccess) return e;
  if (pipe) return launch_block_sparse_pipe(a, stream);
  switch (a.head_dim) {  // head_dim 64, and more than kSparsePipeMaxTiles tiles
    case 64: return launch_sparse_d<64>(a, stream);
    case 96: return launch_sparse_d<96>(a, stream);
    case 128: return launch_sparse_d<128>(a, stream);
    case 192: return launch_sparse_d<192>(a, stream);
    case 256: return launch_sparse_d<256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
