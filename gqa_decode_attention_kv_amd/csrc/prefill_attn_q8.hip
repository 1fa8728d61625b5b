// Chunk (prefill) attention over q8 (int8 keys and values, each with one f32 scale per token)
// caches: instantiations of the kernel in prefill_kernel.h.
#include "prefill_kernel.h"

namespace uaii {

hipError_t launch_prefill_q8(int D, int G, int B, const PrefillArgs& a, hipStream_t stream) {
  return launch_prefill_typed<kI8, kI8>(D, G, B, a, stream);
}

}  // namespace uaii
