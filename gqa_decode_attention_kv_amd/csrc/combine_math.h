// Log-sum-exp combine of the split partials of one (sequence, query head),
// shared by the standalone combine (decode_combine.hip) and the fused step
// (decode_partial_kernel.h).  Source: "Algenta - Model support matrix"
// (Conformance CLI: decode_attn=splitk_flash_decoding); the optional sink
// follows "llamay - Models and formats" (Architectures: gpt-oss puts a
// per-head sink in the softmax denominator).
#pragma once

#include <math.h>

#include "launch.h"

namespace uaii {

// One wave: lse points at the row's ns split log-sum-exps, po at its first
// partial row plus this lane (lane + 64 e is output element e).  out[e] =
// sum e^(lse - M) o / (sum e^(lse - M) [+ e^(sink - M)]).  One pass with a
// running max: the loads of U splits are issued together, and for up to U
// splits no cross-lane reduction is needed at all.  With a sink the running
// max starts at the sink with a denominator of 1 and no numerator.
template <int D>
__device__ inline void combine_row(const float* lse, const float* po, int ns, bool has_sink, float sink,
                                   float* out, int lane) {
  constexpr int EPL = D / 64;  // output elements per lane
  constexpr int U = 8;         // splits whose partial rows are loaded together
  float M = -INFINITY, den = 0.0f;
  if (has_sink) {
    M = sink;
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
#pragma unroll
  for (int e = 0; e < EPL; ++e) out[lane + 64 * e] = num[e] / den;
}

}  // namespace uaii
