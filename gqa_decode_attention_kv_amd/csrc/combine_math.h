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

// combine_row for the NH consecutive query heads of one kv-head group, with
// the loads of all NH heads issued together (one wave): head j's split
// log-sum-exps start at lse + j * lse_stride, its partial rows at
// po + j * po_stride (plus this lane), its output at out + j * D.  sinks is
// nullptr or points at the NH heads' sink logits.  U splits per head are in
// flight at once, with NH * U * D/64 registers of partial rows.
template <int D, int NH>
__device__ inline void combine_group(const float* lse, int64_t lse_stride, const float* po, int64_t po_stride,
                                     int ns, const float* sinks, float* out, int lane) {
  constexpr int EPL = D / 64;
  constexpr int U0 = 64 / (NH * EPL);
  constexpr int U = U0 < 1 ? 1 : (U0 > 8 ? 8 : U0);
  float M[NH], den[NH], num[NH][EPL];
#pragma unroll
  for (int j = 0; j < NH; ++j) {
    M[j] = sinks != nullptr ? sinks[j] : -INFINITY;
    den[j] = sinks != nullptr ? 1.0f : 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) num[j][e] = 0.0f;
  }
  for (int s = 0; s < ns; s += U) {
    float w[NH][U], v[NH][U][EPL];
#pragma unroll
    for (int j = 0; j < NH; ++j)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int su = min(s + u, ns - 1);
        w[j][u] = lse[j * lse_stride + su];
#pragma unroll
        for (int e = 0; e < EPL; ++e) v[j][u][e] = po[j * po_stride + static_cast<int64_t>(su) * D + 64 * e];
      }
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      float bm = w[j][0];
#pragma unroll
      for (int u = 1; u < U; ++u) bm = fmaxf(bm, w[j][u]);  // clamped duplicates do not change it
      const float m_new = fmaxf(M[j], bm);
      const float alpha = (M[j] == -INFINITY) ? 0.0f : expf(M[j] - m_new);
      den[j] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) num[j][e] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float wu = (s + u < ns) ? expf(w[j][u] - m_new) : 0.0f;
        den[j] += wu;
#pragma unroll
        for (int e = 0; e < EPL; ++e) num[j][e] = fmaf(wu, v[j][u][e], num[j][e]);
      }
      M[j] = m_new;
    }
  }
#pragma unroll
  for (int j = 0; j < NH; ++j)
#pragma unroll
    for (int e = 0; e < EPL; ++e) out[j * D + lane + 64 * e] = num[j][e] / den[j];
}

}  // namespace uaii
