// Device-resident scratch of the allocation-free decode entry point.
//
// The array lives in the code object: every GPU the library runs on holds its
// own copy, at its own address, from module load until the process ends. In
// host code `scratch` names only a host-side stand-in for the symbol, never a
// device address, so it is resolved once per device with hipGetSymbolAddress
// (with that device current) and only the resolved address is handed to
// kernels.
#include <mutex>

#include "launch.hpp"

namespace attn {

static __device__ __align__(256) char scratch[kDecodeScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

}  // namespace

hipError_t decode_scratch_address(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *ptr = g_scratch_addr[dev];
  return hipSuccess;
}

}  // namespace attn
