// Static scratch memory of uaii_decode_step_noalloc: the split partials and
// the arrival counters of the one-call decode step live in a file-scope
// device array instead of caller buffers, for callers that cannot allocate.
//
// Every GPU the library runs on holds its own copy of the array until the
// process ends.  In host code the array's name is only a stand-in for the
// symbol; its device address on the current GPU comes from
// hipGetSymbolAddress, taken once per device and kept, and only that address
// is handed to kernels.
#include <mutex>

#include "launch.h"

namespace uaii {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

__global__ void zero_words(int32_t* p, int n) {
  const int i = static_cast<int>(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < n) p[i] = 0;
}

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_base[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void** base, hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_base[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    // The arrival counters must start at zero; every completed step leaves
    // them at zero again, so they are cleared once, on the first caller's
    // stream, ahead of its first step (a kernel, not a memset node).
    constexpr int kThreads = 256;
    hipLaunchKernelGGL(zero_words, dim3((kNoAllocCounterWords + kThreads - 1) / kThreads), dim3(kThreads),
                       0, stream, static_cast<int32_t*>(p), kNoAllocCounterWords);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_base[dev] = p;
  }
  *base = g_base[dev];
  return hipSuccess;
}

}  // namespace uaii
