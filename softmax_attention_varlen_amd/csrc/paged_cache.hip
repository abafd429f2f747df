// Paged KV cache write: new tokens' K and V rows scattered to their cache
// slots. With 128-token blocks, slot s = block * 128 + offset is also the
// cache row index, so a token's whole row (all kv heads, Hkv * D elements)
// lands at row s of the K plane and of the V plane. One wave per token moves
// 16 bytes per lane; a negative or out-of-range slot is skipped.
#include "attn_common.hpp"
#include "launch.hpp"

namespace attn {

__global__ __launch_bounds__(256) void paged_kv_write_kernel(const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v,
                                                            const int32_t* __restrict__ slots, int num_tokens,
                                                            int row_elems, long num_slots,
                                                            uint16_t* __restrict__ cache) {
  const int lane = threadIdx.x & 63;
  const long t = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= num_tokens) return;
  const long slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const long v_plane = num_slots * row_elems;
  const uint16_t* ks = k + t * row_elems;
  const uint16_t* vs = v + t * row_elems;
  uint16_t* kd = cache + slot * row_elems;
  uint16_t* vd = kd + v_plane;
  for (int j = lane * 8; j < row_elems; j += 64 * 8) {
    *reinterpret_cast<u32x4*>(kd + j) = ld_global16(ks + j);
    *reinterpret_cast<u32x4*>(vd + j) = ld_global16(vs + j);
  }
}

hipError_t launch_paged_kv_write(const void* k, const void* v, const int32_t* slots, int num_tokens, int row_elems,
                                 int num_blocks, void* kv_cache, hipStream_t stream) {
  const long num_slots = (long)num_blocks * 128;
  hipLaunchKernelGGL(paged_kv_write_kernel, dim3((unsigned)((num_tokens + 3) / 4)), dim3(256), 0, stream,
                     (const uint16_t*)k, (const uint16_t*)v, slots, num_tokens, row_elems, num_slots,
                     (uint16_t*)kv_cache);
  return hipGetLastError();
}

}  // namespace attn
