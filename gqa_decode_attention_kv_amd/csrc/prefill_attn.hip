// Chunk (prefill) attention over bf16 key and value caches: instantiations of the kernel
// in prefill_kernel.h, and the dispatch over cache types.
#include "prefill_kernel.h"

namespace uaii {

hipError_t launch_prefill_bf16(int D, int G, int B, const PrefillArgs& a, hipStream_t stream) {
  return launch_prefill_typed<kBF16, kBF16>(D, G, B, a, stream);
}

hipError_t launch_prefill_attn(int D, int G, int B, int k_dtype, int v_dtype, const PrefillArgs& a,
                               hipStream_t stream) {
  if (k_dtype == kBF16 && v_dtype == kBF16) return launch_prefill_bf16(D, G, B, a, stream);
  if (k_dtype == kBF16 && v_dtype == kI8) return launch_prefill_vq8(D, G, B, a, stream);
  if (k_dtype == kI8 && v_dtype == kI8) return launch_prefill_q8(D, G, B, a, stream);
  if (k_dtype == kF32 && v_dtype == kF32) return launch_prefill_f32(D, G, B, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace uaii
