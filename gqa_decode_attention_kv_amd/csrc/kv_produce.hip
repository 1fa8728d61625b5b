// KV producer for one decode step: per-head QK-RMSNorm, RoPE at the new
// token's absolute position, append of K and V to the cache.
//
// Sources: "Universal AI Inference - Hugging Face decoder completeness"
// (P0.2 RoPE scaling, P1.1 RMSNorm gain (1+w), P1.2 QK-norm before RoPE,
// P1.3 absolute positions); "llamay - Models and formats" (Architectures:
// interleaved vs NeoX rotary, gpt-oss YaRN; The KV cache, in three
// precisions: vq8 and q8); "Algenta - Model support matrix" (Decoder
// families: linear scaling);
// "FreeToken PR #722" (Changes: Llama-3 scaling constants).
//
// The work is O(B * (H + Hkv) * d): one 64-lane wave per head vector.  The
// norm and the rotation run in double precision and round once to the
// stored format, so the stored key matches a double-precision definition
// to the last bit in all but astronomically rare ties.  The int8 quantiser
// (vq8 values, q8 keys and values) is defined in f32 (IEEE division,
// rounding half away from zero).
#include "launch.h"

#include <math.h>

namespace uaii {
namespace {

#pragma clang fp contract(off)

constexpr double kTwoPi = 6.283185307179586476925286766559;

__device__ inline double wave_sum(double x) {
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

__device__ inline float wave_max(float x) {
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

// Round a double to the nearest bf16 (ties to even) straight from its bits:
// in the normal range, round the 52-bit fraction to 7 bits on the integer
// magnitude (a carry into the exponent is the correct result), then rebias
// the exponent from 1023 to 127; below 2^-126 round on the fixed subnormal
// grid 2^-133.  Overflow gives infinity.  Inputs here are finite.
__device__ inline uint16_t bf16_from_double(double x) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const uint32_t sign = static_cast<uint32_t>(u >> 48) & 0x8000u;
  const uint64_t mag = u & 0x7FFFFFFFFFFFFFFFull;
  const int exp = static_cast<int>(mag >> 52) - 1023;
  if (exp >= -126) {
    const uint64_t rounded = (mag + 0x00000FFFFFFFFFFFull + ((mag >> 45) & 1ull)) >> 45;
    uint64_t bits = rounded - (static_cast<uint64_t>(1023 - 127) << 7);
    if (bits >= 0x7F80ull) bits = 0x7F80ull;
    return static_cast<uint16_t>(sign | static_cast<uint32_t>(bits));
  }
  const double r = rint(fabs(x) * 0x1p133);  // 0..128, exact scaling
  return static_cast<uint16_t>(sign | static_cast<uint32_t>(r));
}

// Rotary frequency of pair i (full head): plain, Llama-3, linear or YaRN.
// YaRN's blend band [c_lo, c_hi] in pair indices comes from the host.
__device__ inline double rope_freq(const ProduceArgs& a, int i) {
  const double f = pow(a.theta, -2.0 * static_cast<double>(i) / static_cast<double>(a.D));
  if (a.scaling == kLinear) return f / a.factor;
  if (a.scaling == kYarn) {
    const double t = fmin(fmax((static_cast<double>(i) - a.c_lo) / (a.c_hi - a.c_lo), 0.0), 1.0);
    return t * f / a.factor + (1.0 - t) * f;
  }
  if (a.scaling != kLlama3) return f;
  const double wavelen = kTwoPi / f;
  if (wavelen < a.orig / a.high) return f;
  if (wavelen > a.orig / a.low) return f / a.factor;
  const double mu = (a.orig / wavelen - a.low) / (a.high - a.low);
  return (1.0 - mu) * f / a.factor + mu * f;
}

// Symmetric int8 quantiser of one row held across the wave, E values per
// lane at element indices idx[e] (valid[e] false for padding): scale =
// max|x| / 127 in f32, code = clamp(round_half_away(x / scale), -127, 127);
// an all-zero row gives scale 0 and codes 0.  Used for vq8 values and q8 keys.
template <int E>
__device__ inline void quantize_row(const float (&x)[E], const int (&idx)[E], const bool (&valid)[E],
                                    int8_t* dst, float* scale_out, int lane) {
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (valid[e]) amax = fmaxf(amax, fabsf(x[e]));
  amax = wave_max(amax);
  const float scale = amax == 0.0f ? 0.0f : __fdiv_rn(amax, 127.0f);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (!valid[e]) continue;
    float r = 0.0f;
    if (amax != 0.0f) {
      r = roundf(__fdiv_rn(x[e], scale));
      r = fminf(fmaxf(r, -127.0f), 127.0f);
    }
    dst[idx[e]] = static_cast<int8_t>(static_cast<int>(r));
  }
  if (lane == 0) *scale_out = scale;
}

template <int D>
__global__ __launch_bounds__(64) void kv_produce_kernel(ProduceArgs a) {
  constexpr int EPL = D / 64;                     // elements per lane
  constexpr int NP = (D / 2 + 63) / 64;           // rotation pairs per lane
  __shared__ double sx[D];
  const int lane = threadIdx.x;
  const int x = blockIdx.x;
  const int b = blockIdx.y;
  const int pos = a.pos[b];
  const bool is_q = x < a.H;
  const int u = x - a.H;

  // Loads first; the data-independent angles below overlap with them.
  const float* src = is_q ? a.q_in + (static_cast<int64_t>(b) * a.H + x) * D
                          : a.k_in + (static_cast<int64_t>(b) * a.Hkv + u) * D;
  float xin[EPL], v[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) xin[e] = src[lane + 64 * e];
  if (!is_q) {
    const float* vsrc = a.v_in + (static_cast<int64_t>(b) * a.Hkv + u) * D;
#pragma unroll
    for (int e = 0; e < EPL; ++e) v[e] = vsrc[lane + 64 * e];
  }

  // cos/sin of pos * g_i for this lane's pairs i = lane + 64 j.
  double cs[NP], sn[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int i = lane + 64 * j;
    cs[j] = 1.0;
    sn[j] = 0.0;
    if (i < D / 2) sincos(static_cast<double>(pos) * rope_freq(a, i), &sn[j], &cs[j]);
  }

  double xv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) xv[e] = static_cast<double>(xin[e]);
  if (a.norm_enabled) {
    const float* w = is_q ? a.w_q : a.w_k;
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) ss += xv[e] * xv[e];
    ss = wave_sum(ss);
    const double r = 1.0 / sqrt(ss / static_cast<double>(D) + static_cast<double>(a.norm_eps));
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      xv[e] = xv[e] * r * (static_cast<double>(w[lane + 64 * e]) + static_cast<double>(a.norm_offset));
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) sx[lane + 64 * e] = xv[e];
  __syncthreads();

  // Element offset of the new token's row: contiguous [B][Hkv][cap][D], or
  // paged [num_blocks][Hkv][bs][D] through the block table (ids outside the
  // pool are clamped, so a bad table cannot write outside it).
  int64_t slot = 0;
  if (!is_q) {
    if (a.block_table != nullptr) {
      int pid = a.block_table[static_cast<int64_t>(b) * a.max_blocks + pos / a.block_size];
      pid = min(max(pid, 0), a.num_blocks - 1);
      slot = ((static_cast<int64_t>(pid) * a.Hkv + u) * a.block_size + pos % a.block_size) * D;
    } else {
      slot = ((static_cast<int64_t>(b) * a.Hkv + u) * a.cap + pos) * D;
    }
  }
  // q8 keys: the rotated key rounded to f32, quantised after the loop.
  float kq[2 * NP];
  int kidx[2 * NP];
  bool kok[2 * NP];
#pragma unroll
  for (int e = 0; e < 2 * NP; ++e) {
    kq[e] = 0.0f;
    kidx[e] = 0;
    kok[e] = false;
  }
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int i = lane + 64 * j;
    if (i >= D / 2) continue;
    const int ia = (a.pairing == kNeox) ? i : 2 * i;
    const int ib = (a.pairing == kNeox) ? i + D / 2 : 2 * i + 1;
    const double c = cs[j], sv = sn[j];
    const double xa = sx[ia], xb = sx[ib];
    double ya = xa * c - xb * sv;
    double yb = xa * sv + xb * c;
    if (a.attn_factor != 1.0) {  // YaRN scales the rotated q and k
      ya *= a.attn_factor;
      yb *= a.attn_factor;
    }
    if (is_q) {
      float* q = a.q_out + (static_cast<int64_t>(b) * a.H + x) * D;
      q[ia] = static_cast<float>(ya);
      q[ib] = static_cast<float>(yb);
    } else if (a.k_dtype == kF32) {
      float* k = static_cast<float*>(a.k) + slot;
      k[ia] = static_cast<float>(ya);
      k[ib] = static_cast<float>(yb);
    } else if (a.k_dtype == kBF16) {
      uint16_t* k = static_cast<uint16_t*>(a.k) + slot;
      k[ia] = bf16_from_double(ya);
      k[ib] = bf16_from_double(yb);
    } else {
      kq[2 * j] = static_cast<float>(ya);
      kq[2 * j + 1] = static_cast<float>(yb);
      kidx[2 * j] = ia;
      kidx[2 * j + 1] = ib;
      kok[2 * j] = kok[2 * j + 1] = true;
    }
  }
  if (is_q) return;
  if (a.k_dtype == kI8)
    quantize_row<2 * NP>(kq, kidx, kok, static_cast<int8_t*>(a.k) + slot, a.k_scale + slot / D, lane);

  // Value of (b, u): stored as given (f32), rounded to bf16, or quantised.
  if (a.v_dtype == kF32) {
    float* dst = static_cast<float*>(a.v) + slot;
#pragma unroll
    for (int e = 0; e < EPL; ++e) dst[lane + 64 * e] = v[e];
  } else if (a.v_dtype == kBF16) {
    uint16_t* dst = static_cast<uint16_t*>(a.v) + slot;
#pragma unroll
    for (int e = 0; e < EPL; ++e) dst[lane + 64 * e] = bf16_from_double(static_cast<double>(v[e]));
  } else {
    int idx[EPL];
    bool ok[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      idx[e] = lane + 64 * e;
      ok[e] = true;
    }
    quantize_row<EPL>(v, idx, ok, static_cast<int8_t*>(a.v) + slot, a.v_scale + slot / D, lane);
  }
}

}  // namespace

hipError_t launch_kv_produce(const ProduceArgs& a, hipStream_t stream) {
  const dim3 grid(a.H + a.Hkv, a.B);
  switch (a.D) {
    case 64: hipLaunchKernelGGL(kv_produce_kernel<64>, grid, dim3(64), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(kv_produce_kernel<128>, grid, dim3(64), 0, stream, a); break;
    case 256: hipLaunchKernelGGL(kv_produce_kernel<256>, grid, dim3(64), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace uaii
