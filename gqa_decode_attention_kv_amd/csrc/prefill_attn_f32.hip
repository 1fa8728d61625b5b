// Chunk (prefill) attention over f32 key and value caches, head dims 64 and 128:
// instantiations of the kernel in prefill_kernel.h (f32 tiles, f32 matrix products).
#include "prefill_kernel.h"

namespace uaii {

hipError_t launch_prefill_f32(int D, int G, int B, const PrefillArgs& a, hipStream_t stream) {
  switch (D) {
    case 64: return launch_d<64, kF32, kF32>(G, B, a, stream);
    case 128: return launch_d<128, kF32, kF32>(G, B, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace uaii
