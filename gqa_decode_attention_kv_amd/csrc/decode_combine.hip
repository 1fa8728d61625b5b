// Log-sum-exp combine of split-K decode partials: for each (sequence, query
// head), M = max over valid splits of lse, out = sum e^(lse - M) o / sum
// e^(lse - M).  Source: "Algenta - Model support matrix" (Conformance CLI:
// decode_attn=splitk_flash_decoding; Kernel path capabilities: split-K decode
// partials).  One wave per (b, h); only the splits that hold visible keys
// are read, so the partial buffer needs no initialisation.
//
// With an attention sink ("llamay - Models and formats", Architectures:
// gpt-oss), the head's sink logit joins the denominator as a term
// e^(sink - M) that carries no value (combine_math.h).
#include "combine_math.h"
#include "launch.h"

namespace uaii {
namespace {

template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(CombineArgs a) {
  const int lane = threadIdx.x;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int s0 = a.t.first_split[b];
  const int ns = a.t.work_prefix[b + 1] - a.t.work_prefix[b];
  const int64_t row0 = (static_cast<int64_t>(b) * a.H + h) * a.max_splits + s0;
  const bool has_sink = a.sinks != nullptr;
  combine_row<D>(a.part_lse + row0, a.part_o + row0 * D + lane, ns, has_sink, has_sink ? a.sinks[h] : 0.0f,
                 a.out + (static_cast<int64_t>(b) * a.H + h) * D, lane);
}

}  // namespace

hipError_t launch_decode_combine(int D, int B, const CombineArgs& a, hipStream_t stream) {
  const dim3 grid(a.H, B);
  switch (D) {
    case 64: hipLaunchKernelGGL(decode_combine_kernel<64>, grid, dim3(64), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(decode_combine_kernel<128>, grid, dim3(64), 0, stream, a); break;
    case 256: hipLaunchKernelGGL(decode_combine_kernel<256>, grid, dim3(64), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace uaii
