// Split-K decode partials over a paged cache: pools [num_blocks][Hkv]
// [block_size][d] addressed through a per-sequence block table.  The kernel
// is in decode_partial_kernel.h.
#include "decode_partial_kernel.h"

namespace uaii {

hipError_t launch_decode_partial_paged(int D, int G, int k_dtype, int v_dtype, const AttnArgs& a,
                                       hipStream_t stream) {
  return dispatch<true, false>(D, G, k_dtype, v_dtype, a, stream);
}

}  // namespace uaii
