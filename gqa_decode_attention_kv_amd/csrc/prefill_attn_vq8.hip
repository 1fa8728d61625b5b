// Chunk (prefill) attention over vq8 (bf16 keys, int8 values with one f32 scale per token)
// caches: instantiations of the kernel in prefill_kernel.h.
#include "prefill_kernel.h"

namespace uaii {

hipError_t launch_prefill_vq8(int D, int G, int B, const PrefillArgs& a, hipStream_t stream) {
  return launch_prefill_typed<kBF16, kI8>(D, G, B, a, stream);
}

}  // namespace uaii
