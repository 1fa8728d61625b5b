// Split-K decode partials over contiguous per-sequence caches
// [B][Hkv][capacity][d]; the kernel itself is in decode_partial_kernel.h.
#include "decode_partial_kernel.h"

namespace uaii {

hipError_t launch_decode_partial(int D, int G, int k_dtype, int v_dtype, const AttnArgs& a,
                                 hipStream_t stream) {
  return dispatch<false, false>(D, G, k_dtype, v_dtype, a, stream);
}

}  // namespace uaii
