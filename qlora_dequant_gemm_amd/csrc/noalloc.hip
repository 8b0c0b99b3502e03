// Scratch memory of the allocation-free forward entry point: one file-scope
// device array per GPU, held until the process ends. Host code never passes
// the array's name to a kernel or a copy (on the host it is only a stand-in
// for the symbol): it uses the device address that hipGetSymbolAddress gives
// for the current device, looked up once per device.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "kernels.hpp"

namespace qnf4 {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Zero the arrival counters at the start of the scratch (a kernel rather than
// a memset, so that a call recorded into a graph clears them on every replay).
__global__ __launch_bounds__(256) void k_zero_counters(uint4* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = uint4{0u, 0u, 0u, 0u};
}

}  // namespace

hipError_t noalloc_scratch(void** ptr, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev];
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev] = p;
    }
  }
  constexpr int n = static_cast<int>(kWsCounterBytes / 16);
  hipLaunchKernelGGL(k_zero_counters, dim3((n + 255) / 256), dim3(256), 0, stream, static_cast<uint4*>(p), n);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  *ptr = p;
  return hipSuccess;
}

}  // namespace qnf4
