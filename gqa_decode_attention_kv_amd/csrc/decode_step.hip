// The fused single-launch decode step over contiguous caches
// [B][Hkv][capacity][d]: producer, split-K partials and combine in one
// kernel (decode_partial_kernel.h, FUSED = true).
#include "decode_partial_kernel.h"

namespace uaii {

hipError_t launch_decode_step(int D, int G, int k_dtype, int v_dtype, const StepArgs& s, hipStream_t stream) {
  return dispatch<false, true>(D, G, k_dtype, v_dtype, s, stream);
}

}  // namespace uaii
