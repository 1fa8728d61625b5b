// Split-K flash-decoding partials for grouped-query attention, one query
// token per sequence, over B <= 32 ragged sequences.
//
// Sources: "Algenta - Model support matrix" (Kernel path capabilities:
// split-K decode partials, batched decode partial with B <= 32; Structural
// fact requirements: GQA ratio, attention scale 1/sqrt(head_dim));
// "Universal AI Inference - Hugging Face decoder completeness" (P1.4:
// sliding window and attention-logit softcap as a tanh clip); "llamay -
// Models and formats" (The KV cache, in three precisions: vq8 values).
//
// Design (gfx950, bandwidth bound, no MFMA: one query row per kv head is a
// GEMV; arithmetic intensity is 2-5 flop per KV byte, far below the ridge):
//   * one 256-thread work-group (4 wave64) per (sequence, kv head, split),
//     taken from a flattened per-sequence work table, so ragged batches and
//     windows only launch work-groups that hold visible keys;
//   * the G query heads that share the kv head are held in registers, so
//     every K and V byte is read from HBM exactly once per group;
//   * each wave owns a contiguous block of up to 128 rows of the split and
//     runs two passes over it: K (16-byte coalesced loads, a row spread over
//     d*sizeof(K)/16 lanes, scores reduced across those lanes with DPP),
//     scores parked in LDS, then V with the softmax weights broadcast from
//     LDS; the two passes need no rescaling inside the block;
//   * scores live in the log2 domain (q pre-multiplied by scale*log2 e) so the
//     exponential is a single exp2; with a softcap the tanh clip is applied
//     to the natural-scale score first;
//   * vq8: int8 codes are widened in registers and the per-token scale is
//     folded into the softmax weight, so dequantisation costs no extra pass;
//   * the four waves' (max, sum, accumulator) triples are merged through LDS
//     and the work-group writes one normalised partial and its log-sum-exp
//     per query head.
// Rows outside the visible range are never loaded; masked lanes use
// selects, never multiplications by zero, so poisoned memory cannot leak.
#include "launch.h"

#include <math.h>

namespace uaii {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 128;  // rows of one wave per chunk (chunk = 512 rows)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int CTRL>
__device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N in {4, 8, 16, 32, 64}); every lane of
// a group receives the group's sum.
template <int N>
__device__ inline float group_sum(float x) {
  x += dpp<0xB1>(x);                        // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp<0x4E>(x);                        // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (N >= 8) x += dpp<0x141>(x);   // row_half_mirror: pairs the quads of 8
  if constexpr (N >= 16) x += dpp<0x140>(x);  // row_mirror: pairs the halves of 16
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

__device__ inline float wave_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ inline float wave_sum(float x) { return group_sum<64>(x); }

__device__ inline u32x4 load16(const void* p) { return *static_cast<const u32x4*>(p); }

// Widen the 16 bytes of one lane to E floats.
template <int DT, int E>
__device__ inline void widen(const u32x4& w, float (&out)[E]) {
  if constexpr (DT == kF32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = __uint_as_float(w[e]);
  } else if constexpr (DT == kBF16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      out[2 * e] = __uint_as_float(w[e] << 16);
      out[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e)
      out[e] = static_cast<float>(static_cast<int8_t>(static_cast<uint8_t>(w[e >> 2] >> (8 * (e & 3)))));
  }
}

template <int DT>
struct Elem {
  static constexpr int bytes = DT == kF32 ? 4 : (DT == kBF16 ? 2 : 1);
};

template <int D, int G, int KT, int VT>
__global__ __launch_bounds__(kThreads) void decode_partial_kernel(AttnArgs a) {
  constexpr int KB = Elem<KT>::bytes, VB = Elem<VT>::bytes;
  constexpr int KLPR = D * KB / 16;  // lanes per K row
  constexpr int KRPL = 64 / KLPR;    // K rows per wave load
  constexpr int KE = 16 / KB;        // K elements per lane
  constexpr int VLPR = D * VB / 16;
  constexpr int VRPL = 64 / VLPR;
  constexpr int VE = 16 / VB;
  constexpr int UK = (8 * KRPL <= kRowsPerWave) ? 8 : kRowsPerWave / KRPL;  // loads in flight
  constexpr int UV = (8 * VRPL <= kRowsPerWave) ? 8 : kRowsPerWave / VRPL;
  static_assert(kRowsPerWave % (UK * KRPL) == 0 && kRowsPerWave % (UV * VRPL) == 0, "tiling");
  static_assert(KLPR >= 4 && VLPR >= 4, "row must span at least a quad");

  constexpr int kScoreFloats = kWaves * kRowsPerWave * G;
  constexpr int kCombFloats = kWaves * G * (D + 2);
  __shared__ __attribute__((aligned(16))) float smem[kScoreFloats > kCombFloats ? kScoreFloats : kCombFloats];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kvh = blockIdx.y;

  // Which sequence and split this work-group owns.
  const int w = blockIdx.x;
  int b = 0;
  for (int i = 1; i < a.t.n_seq; ++i) b += (w >= a.t.work_prefix[i]) ? 1 : 0;
  const int sigma = a.t.first_split[b] + (w - a.t.work_prefix[b]);
  const int L = a.t.len[b];
  const int r0 = max(sigma * a.split_size, a.t.lo[b]);
  const int r1 = min((sigma + 1) * a.split_size, L);

  const int64_t slab = (static_cast<int64_t>(b) * a.Hkv + kvh) * a.cap;  // first row of (b, kvh)
  const char* kbase = static_cast<const char*>(a.k) + slab * (D * KB);
  const char* vbase = static_cast<const char*>(a.v) + slab * (D * VB);
  const float* sbase = (VT == kI8) ? a.v_scale + slab : nullptr;

  // Query group in registers: lane holds q[h][kc*KE .. kc*KE + KE) for its K segment.
  const int kr = lane / KLPR, kc = lane % KLPR;
  float q[G][KE];
  {
    const float* qb = a.q + (static_cast<int64_t>(b) * a.H + kvh * G) * D + kc * KE;
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < KE; e += 4) {
        const float4 v = *reinterpret_cast<const float4*>(qb + g * D + e);
        q[g][e] = v.x * a.q_mul;
        q[g][e + 1] = v.y * a.q_mul;
        q[g][e + 2] = v.z * a.q_mul;
        q[g][e + 3] = v.w * a.q_mul;
      }
    }
  }
  const bool capped = a.softcap > 0.0f;
  const float cap_c = a.softcap, cap_inv = capped ? 1.0f / a.softcap : 0.0f;

  const int vr = lane / VLPR, vc = lane % VLPR;
  float acc[G][VE];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[g][e] = 0.0f;
  float m_run[G], l_run[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.0f;
  }

  float* sc = smem + wave * (kRowsPerWave * G);  // this wave's [row][G] scores

  for (int c0 = r0; c0 < r1; c0 += kWaves * kRowsPerWave) {
    const int chunk = min(kWaves * kRowsPerWave, r1 - c0);
    // Even share per wave, rounded to 16 rows (the largest rows-per-load).
    const int per = min(kRowsPerWave, ((chunk + kWaves - 1) / kWaves + 15) & ~15);
    const int a0 = c0 + wave * per;
    const int nrows = max(0, min(per, r1 - a0));  // rows [a0, a0 + nrows)

    // ---- pass 1: scores of this wave's rows -------------------------------
    float mloc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) mloc[g] = -INFINITY;
    for (int t0 = 0; t0 < nrows; t0 += UK * KRPL) {
      u32x4 kd[UK];
#pragma unroll
      for (int u = 0; u < UK; ++u) {
        const int r = t0 + u * KRPL + kr;
        kd[u] = (r < nrows) ? load16(kbase + static_cast<int64_t>(a0 + r) * (D * KB) + kc * 16)
                            : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < UK; ++u) {
        const int r = t0 + u * KRPL + kr;
        float kf[KE];
        widen<KT, KE>(kd[u], kf);
        float s[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float p = 0.0f;
#pragma unroll
          for (int e = 0; e < KE; ++e) p = fmaf(q[g][e], kf[e], p);
          s[g] = group_sum<KLPR>(p);
          if (capped) s[g] = cap_c * tanhf(s[g] * cap_inv) * kLog2e;
          s[g] = (r < nrows) ? s[g] : -INFINITY;
          mloc[g] = fmaxf(mloc[g], s[g]);
        }
        if (kc == 0) {
#pragma unroll
          for (int g = 0; g < G; ++g) sc[r * G + g] = s[g];
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- running max and rescale ------------------------------------------
    float m_new[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m_new[g] = fmaxf(m_run[g], wave_max(mloc[g]));
      const float alpha = (m_run[g] == -INFINITY) ? 0.0f : exp2f(m_run[g] - m_new[g]);
      l_run[g] *= alpha;
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[g][e] *= alpha;
      m_run[g] = m_new[g];
    }

    // ---- weights: p = 2^(s - m); vq8 folds the token's scale into p --------
    for (int r = lane; r < nrows; r += 64) {
      const float vs = (VT == kI8) ? sbase[a0 + r] : 1.0f;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = exp2f(sc[r * G + g] - m_run[g]);
        l_run[g] += p;
        sc[r * G + g] = p * vs;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- pass 2: weighted sum of values -------------------------------------
    for (int t0 = 0; t0 < nrows; t0 += UV * VRPL) {
      u32x4 vd[UV];
#pragma unroll
      for (int u = 0; u < UV; ++u) {
        const int r = t0 + u * VRPL + vr;
        vd[u] = (r < nrows) ? load16(vbase + static_cast<int64_t>(a0 + r) * (D * VB) + vc * 16)
                            : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < UV; ++u) {
        const int r = t0 + u * VRPL + vr;
        float p[G];
#pragma unroll
        for (int g = 0; g < G; ++g) p[g] = (r < nrows) ? sc[r * G + g] : 0.0f;
        float vf[VE];
        widen<VT, VE>(vd[u], vf);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < VE; ++e) acc[g][e] = fmaf(p[g], vf[e], acc[g][e]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge the row groups of the wave, then the waves --------------------
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l_run[g] = wave_sum(l_run[g]);
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      float x = acc[g][e];
#pragma unroll
      for (int m = VLPR; m < 64; m <<= 1) x += __shfl_xor(x, m);
      acc[g][e] = x;
    }
  }
  __syncthreads();  // every wave is done with its scores
  float* comb = smem;                          // [wave][G][D]
  float* ml = smem + kWaves * G * D;           // [wave][G][2]
  if (vr == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < VE; ++e) comb[(wave * G + g) * D + vc * VE + e] = acc[g][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      ml[(wave * G + g) * 2] = m_run[g];
      ml[(wave * G + g) * 2 + 1] = l_run[g];
    }
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int g = idx / D, dd = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) M = fmaxf(M, ml[(wv * G + g) * 2]);
    float den = 0.0f, num = 0.0f;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) {
      const float mw = ml[(wv * G + g) * 2];
      const float aw = (mw == -INFINITY) ? 0.0f : exp2f(mw - M);
      den = fmaf(aw, ml[(wv * G + g) * 2 + 1], den);
      num = fmaf(aw, comb[(wv * G + g) * D + dd], num);
    }
    const int64_t row = (static_cast<int64_t>(b) * a.H + kvh * G + g) * a.max_splits + sigma;
    a.part_o[row * D + dd] = num / den;
    if (dd == 0) a.part_lse[row] = (M + log2f(den)) * kLn2;
  }
}

template <int D, int G, int KT, int VT>
hipError_t launch_one(const AttnArgs& a, hipStream_t stream) {
  const dim3 grid(a.t.work_prefix[a.t.n_seq], a.Hkv);
  hipLaunchKernelGGL((decode_partial_kernel<D, G, KT, VT>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D, int G>
hipError_t by_dtype(int kt, int vt, const AttnArgs& a, hipStream_t s) {
  if (kt == kF32 && vt == kF32) return launch_one<D, G, kF32, kF32>(a, s);
  if (kt == kF32 && vt == kBF16) return launch_one<D, G, kF32, kBF16>(a, s);
  if (kt == kF32 && vt == kI8) return launch_one<D, G, kF32, kI8>(a, s);
  if (kt == kBF16 && vt == kF32) return launch_one<D, G, kBF16, kF32>(a, s);
  if (kt == kBF16 && vt == kBF16) return launch_one<D, G, kBF16, kBF16>(a, s);
  if (kt == kBF16 && vt == kI8) return launch_one<D, G, kBF16, kI8>(a, s);
  return hipErrorInvalidValue;
}

template <int D>
hipError_t by_group(int G, int kt, int vt, const AttnArgs& a, hipStream_t s) {
  switch (G) {
    case 1: return by_dtype<D, 1>(kt, vt, a, s);
    case 2: return by_dtype<D, 2>(kt, vt, a, s);
    case 4: return by_dtype<D, 4>(kt, vt, a, s);
    case 8: return by_dtype<D, 8>(kt, vt, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_partial(int D, int G, int k_dtype, int v_dtype, const AttnArgs& a,
                                 hipStream_t stream) {
  switch (D) {
    case 64: return by_group<64>(G, k_dtype, v_dtype, a, stream);
    case 128: return by_group<128>(G, k_dtype, v_dtype, a, stream);
    case 256: return by_group<256>(G, k_dtype, v_dtype, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace uaii
