// The fused single-launch decode step over a paged cache (block table):
// producer, split-K partials and combine in one kernel
// (decode_partial_kernel.h, FUSED = true, paged addressing).
#include "decode_partial_kernel.h"

namespace uaii {

hipError_t launch_decode_step_paged(int D, int G, int k_dtype, int v_dtype, const StepArgs& s,
                                    hipStream_t stream) {
  return dispatch<true, true>(D, G, k_dtype, v_dtype, s, stream);
}

}  // namespace uaii
