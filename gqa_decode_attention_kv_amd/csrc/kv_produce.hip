// KV producer for one decode step: per-head QK-RMSNorm, RoPE at the new
// token's absolute position, append of K and V to the cache.
//
// Sources: "Universal AI Inference - Hugging Face decoder completeness"
// (P0.2 RoPE scaling, P1.1 RMSNorm gain (1+w), P1.2 QK-norm before RoPE,
// P1.3 absolute positions); "llamay - Models and formats" (Architectures:
// interleaved vs NeoX rotary, gpt-oss YaRN; The KV cache, in three
// precisions: vq8 and q8); "Algenta - Model support matrix" (Decoder
// families: linear scaling); "FreeToken PR #722" (Changes: Llama-3 scaling
// constants).
//
// The work is O(B * T * (H + Hkv) * d): one 64-lane wave per hpw head vectors
// of one of the T tokens of a sequence (T = 1 and hpw = 1 for a decode step).  The
// per-vector math lives in producer_math.h (shared with the fused step): the
// norm and the rotation run in double precision and round once to the
// stored format, so the stored key matches a double-precision definition to
// the last bit in all but astronomically rare ties.  The int8 quantiser
// (vq8 values, q8 keys and values) is defined in f32 (IEEE division,
// rounding half away from zero).
#include "launch.h"
#include "producer_math.h"

namespace uaii {
namespace {

template <int D>
__global__ __launch_bounds__(64) void kv_produce_kernel(ProduceArgs a) {
  constexpr int EPL = pm::Shape<D>::EPL;
  constexpr int NP = pm::Shape<D>::NP;
  __shared__ double sx[D];
  const int lane = threadIdx.x;
  const int b = blockIdx.y;
  const int t = blockIdx.z;  // token of the chunk
  const int pos = a.pos[b] + t;
  const int64_t bt = static_cast<int64_t>(b) * a.T + t;
  // Head vectors [x0, x1) of this token: q heads 0..H-1, then kv heads.
  const int x0 = blockIdx.x * a.hpw;
  const int x1 = min(x0 + a.hpw, a.H + a.Hkv);

  // Input rows of head vector x (and, for a kv head, its value row).
  auto load = [&](int x, float (&xin)[EPL], float (&v)[EPL]) {
    const bool is_q = x < a.H;
    const int u = x - a.H;
    const float* src = is_q ? a.q_in + (bt * a.H + x) * D : a.k_in + (bt * a.Hkv + u) * D;
#pragma unroll
    for (int e = 0; e < EPL; ++e) xin[e] = src[lane + 64 * e];
    if (!is_q) {
      const float* vsrc = a.v_in + (bt * a.Hkv + u) * D;
#pragma unroll
      for (int e = 0; e < EPL; ++e) v[e] = vsrc[lane + 64 * e];
    }
  };

  // The first loads overlap with the angles, which depend only on the
  // position; each later head's loads overlap with the previous head.
  float xin[EPL] = {}, v[EPL] = {};
  load(x0, xin, v);
  pm::Angles<D> an;
  pm::rope_angles<D>(a, pos, lane, an);
  for (int x = x0; x < x1; ++x) {
    float nx[EPL] = {}, nv[EPL] = {};
    if (x + 1 < x1) load(x + 1, nx, nv);
    const bool is_q = x < a.H;
    const int u = x - a.H;
    pm::Rotated<D> r;
    pm::norm_rope<D>(a, xin, is_q ? a.w_q : a.w_k, an, sx, lane, r);
    if (is_q) {
      float* q = a.q_out + (bt * a.H + x) * D;
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        if (!r.ok[j]) continue;
        q[r.ia[j]] = static_cast<float>(r.ya[j]);
        q[r.ib[j]] = static_cast<float>(r.yb[j]);
      }
    } else {
      const int64_t slot = pm::cache_slot<D>(a, b, u, pos);
      float kst[2 * NP], vst[EPL];
      pm::store_key<D>(a, r, slot, lane, kst);
      pm::store_value<D>(a, v, slot, lane, vst);
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      xin[e] = nx[e];
      v[e] = nv[e];
    }
  }
}

}  // namespace

hipError_t launch_kv_produce(const ProduceArgs& a, hipStream_t stream) {
  const dim3 grid((a.H + a.Hkv + a.hpw - 1) / a.hpw, a.B, a.T);
  switch (a.D) {
    case 64: hipLaunchKernelGGL(kv_produce_kernel<64>, grid, dim3(64), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(kv_produce_kernel<128>, grid, dim3(64), 0, stream, a); break;
    case 256: hipLaunchKernelGGL(kv_produce_kernel<256>, grid, dim3(64), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace uaii
