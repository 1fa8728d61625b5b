// Log-sum-exp combine of split-K decode partials: for each (sequence, query
// head), M = max over valid splits of lse, out = sum e^(lse - M) o / sum
// e^(lse - M).  Source: "Algenta - Model support matrix" (Conformance CLI:
// decode_attn=splitk_flash_decoding; Kernel path capabilities: split-K decode
// partials).  One wave per (b, h); only the splits that hold visible keys
// are read, so the partial buffer needs no initialisation.
//
// With an attention sink ("llamay - Models and formats", Architectures:
// gpt-oss), the head's sink logit joins the denominator as a term
// e^(sink - M) that carries no value: the running max starts at the sink
// with a denominator of 1 and no numerator.
#include "launch.h"

#include <math.h>

namespace uaii {
namespace {

template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(CombineArgs a) {
  constexpr int EPL = D / 64;  // output elements per lane
  constexpr int U = 8;         // splits whose partial rows are loaded together
  const int lane = threadIdx.x;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int s0 = a.t.first_split[b];
  const int ns = a.t.work_prefix[b + 1] - a.t.work_prefix[b];
  const int64_t row0 = (static_cast<int64_t>(b) * a.H + h) * a.max_splits + s0;
  const float* lse = a.part_lse + row0;
  const float* po = a.part_o + row0 * D + lane;

  // One pass with a running max: the loads of U splits are issued together,
  // and for up to U splits no cross-lane reduction is needed at all.
  float M = -INFINITY, den = 0.0f;
  if (a.sinks != nullptr) {
    M = a.sinks[h];
    den = 1.0f;
  }
  float num[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) num[e] = 0.0f;
  for (int s = 0; s < ns; s += U) {
    float w[U], v[U][EPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int su = min(s + u, ns - 1);
      w[u] = lse[su];
#pragma unroll
      for (int e = 0; e < EPL; ++e) v[u][e] = po[static_cast<int64_t>(su) * D + 64 * e];
    }
    float bm = w[0];
#pragma unroll
    for (int u = 1; u < U; ++u) bm = fmaxf(bm, w[u]);  // clamped duplicates do not change it
    const float m_new = fmaxf(M, bm);
    const float alpha = (M == -INFINITY) ? 0.0f : expf(M - m_new);
    den *= alpha;
#pragma unroll
    for (int e = 0; e < EPL; ++e) num[e] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float wu = (s + u < ns) ? expf(w[u] - m_new) : 0.0f;
      den += wu;
#pragma unroll
      for (int e = 0; e < EPL; ++e) num[e] = fmaf(wu, v[u][e], num[e]);
    }
    M = m_new;
  }
  float* out = a.out + (static_cast<int64_t>(b) * a.H + h) * D;
#pragma unroll
  for (int e = 0; e < EPL; ++e) out[lane + 64 * e] = num[e] / den;
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
