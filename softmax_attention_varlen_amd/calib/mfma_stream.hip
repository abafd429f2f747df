// Calibration kernel for the MFMA roofline (not part of the attention
// library): a stream of v_mfma_f32_32x32x16_bf16, the instruction the
// prefill and block-sparse kernels run, on operands held in registers.
//
// Each wave loads 8 A and 8 B fragments (one bf16x8 per lane each) from
// `operands` and then issues iters x 8 MFMAs into 4 accumulators, taking a
// different A and B fragment for every MFMA, so the operand values change
// from one MFMA to the next as K, V and P do in the attention step. Two
// 4-wave workgroups per CU, as in the attention kernels. The accumulators'
// sum goes to `sink` (one float per thread) so that nothing is removed.
//
// Under a power cap the rate depends on the operand values: bench.py runs it
// on seeded N(0,1) operands (the attention workloads' distribution) and on
// constant ones, and reports both beside the attention roofline.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 calib_bf16x8 __attribute__((ext_vector_type(8)));
typedef float calib_f32x16 __attribute__((ext_vector_type(16)));

// operands: [16][threads] bf16x8 (fragment slot s of thread t at s * threads + t);
// sink: [threads] fp32; threads = gridDim.x * 256; iters a multiple of 8.
__global__ __launch_bounds__(256, 2) void mfma_stream_kernel(const calib_bf16x8* __restrict__ operands,
                                                             float* __restrict__ sink, int iters) {
  const long threads = (long)gridDim.x * blockDim.x;
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  calib_bf16x8 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = operands[(2 * i) * threads + t];
    b[i] = operands[(2 * i + 1) * threads + t];
  }
  calib_f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  }
  for (int it = 0; it < iters; it += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[(i + u) & 7], acc[i & 3], 0, 0, 0);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  }
  sink[t] = s;
}

// workgroups >= 1 (256 threads each); iters > 0, rounded down to a multiple of
// 8; operands and sink sized as above for threads = workgroups * 256.
// Returns 0, or the HIP error of the launch (1 for bad arguments).
extern "C" int attn_calib_mfma_stream(const void* operands, float* sink, int workgroups, int iters, void* stream) {
  if (operands == nullptr || sink == nullptr || workgroups < 1 || iters < 8) return 1;
  hipLaunchKernelGGL(mfma_stream_kernel, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream,
                     (const calib_bf16x8*)operands, sink, iters - iters % 8);
  return (int)hipGetLastError();
}
