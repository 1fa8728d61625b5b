/*
 * Reference oracle for one decode step of a grouped-query attention layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct CPU
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it; the
 * product path never calls it and shares no code, header or table with it.
 *
 * Everything is scalar C in double precision, except where a storage format
 * fixes the precision (f32 / bf16 cache entries, the vq8 quantiser, which is
 * defined as a sequence of IEEE f32 operations).  No blocking, fusion or
 * reordering: each function is the definition written out.
 *
 * Sources (page title, then section):
 *   [UAII]     "Universal AI Inference - Hugging Face decoder completeness"
 *   [ALGENTA]  "Algenta - Model support matrix"
 *   [FREETOKEN]"FreeToken PR #722 - serve Llama and Mistral llama-arch GGUF"
 *   [LLAMAY]   "llamay - Models and formats"
 *
 * Parity pins: every function below is pinned by a CPU test against closed
 * forms, invariants, special cases or brute force (see the oracle tests).
 * The rotation sign (x_a cos - x_b sin) is a convention the pages do not fix;
 * it is pinned by construction only.
 *
 * Build: gcc -O2 -std=c99 -fPIC -shared -ffp-contract=off oracle.c -lm
 * (x86-64 SSE arithmetic: float and double operations round once, to
 * nearest-even).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_I8 2

#define OR_NEOX 0
#define OR_INTERLEAVED 1

#define OR_PLAIN 0
#define OR_LLAMA3 1
#define OR_LINEAR 2
#define OR_YARN 3

static const double OR_PI = 3.14159265358979323846264338327950288;

/* ------------------------------------------------------------------------ */
/* Storage codecs                                                            */
/* ------------------------------------------------------------------------ */

/* bf16: 1 sign bit, the 8 exponent bits of f32, 7 stored significand bits.
 * A bf16 value is an f32 whose low 16 bits are zero.  Decoding widens it;
 * the bits are never reinterpreted as an f32 buffer
 * ([UAII] P0.1 BF16 ingest: never memcpy BF16 bits into an f32 buffer). */
double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16 value, ties to even.  Normal bf16
 * numbers carry 8 significant bits, so the rounding quantum of x = m*2^e
 * (0.5 <= |m| < 1) is 2^(e-8); below the smallest normal (2^-126) the
 * quantum stays 2^-133 (subnormals).  Results beyond the largest finite bf16
 * become infinities. */
uint16_t oracle_bf16_from_double(double x)
{
    if (isnan(x))
        return (uint16_t)(signbit(x) ? 0xFFC0u : 0x7FC0u);
    if (isinf(x) || x == 0.0) {
        float f = (float)x;
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        return (uint16_t)(u >> 16);
    }
    int e;
    (void)frexp(x, &e);
    if (e < -125)
        e = -125;
    double quantum = ldexp(1.0, e - 8);
    double r = nearbyint(x / quantum) * quantum; /* exact scaling, RNE */
    const double bf16_max = ldexp(255.0, 120);   /* (2 - 2^-7) * 2^127 */
    if (fabs(r) > bf16_max)
        r = (r > 0) ? INFINITY : -INFINITY;
    float f = (float)r; /* exact: r is a bf16 value, so also an f32 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* vq8 value quantiser: one f32 scale per token per kv head, symmetric int8
 * codes ([LLAMAY] The KV cache, in three precisions: vq8 quantises values
 * only, keys stay exact).  Defined as IEEE f32 operations in this order:
 *   a = max_i |v_i|;  a == 0 -> scale 0 and all codes 0;
 *   scale = a / 127;  code_i = clamp(round_half_away(v_i / scale), -127, 127).
 * Dequantised value: code * scale. */
void oracle_quantize_v(const float *v, int d, int8_t *codes, float *scale_out)
{
    float a = 0.0f;
    for (int i = 0; i < d; ++i) {
        float t = fabsf(v[i]);
        if (t > a)
            a = t;
    }
    if (a == 0.0f) {
        *scale_out = 0.0f;
        for (int i = 0; i < d; ++i)
            codes[i] = 0;
        return;
    }
    float scale = a / 127.0f;
    *scale_out = scale;
    for (int i = 0; i < d; ++i) {
        float t = v[i] / scale;
        float r = roundf(t); /* halfway cases away from zero */
        if (r > 127.0f)
            r = 127.0f;
        if (r < -127.0f)
            r = -127.0f;
        codes[i] = (int8_t)r;
    }
}

/* Widen cache element (row, i) of a K or V slab to double. */
static double load_elem(int dtype, const void *base, int64_t row, int d, int i,
                        const float *scale)
{
    int64_t idx = row * (int64_t)d + i;
    switch (dtype) {
    case OR_F32:
        return (double)((const float *)base)[idx];
    case OR_BF16:
        return oracle_bf16_to_double(((const uint16_t *)base)[idx]);
    default: /* OR_I8 (vq8 values, q8 keys and values): code * scale, the
              * double product of the stored values */
        return (double)((const int8_t *)base)[idx] * (double)scale[row];
    }
}

/* ------------------------------------------------------------------------ */
/* KV producer: QK-RMSNorm, RoPE, append                                     */
/* ------------------------------------------------------------------------ */

/* RMSNorm over one head vector: y_i = x_i * (mean(x^2) + eps)^-1/2 * (w_i + offset).
 * offset 0 multiplies by w, offset 1 by (1 + w) (Gemma stores the delta)
 * ([UAII] P1.1 Gemma RMSNorm (1+w); P1.2 QK-norm on the per-head last axis). */
void oracle_rms_norm(const double *x, int d, const float *w, int offset,
                     double eps, double *y)
{
    double ss = 0.0;
    for (int i = 0; i < d; ++i)
        ss += x[i] * x[i];
    double r = 1.0 / sqrt(ss / (double)d + eps);
    for (int i = 0; i < d; ++i)
        y[i] = x[i] * r * ((double)w[i] + (double)offset);
}

/* Rotary frequencies g_i, i in [0, d/2), over the full head
 * ([ALGENTA] Structural fact requirements: rotary coverage is the full head).
 * Plain: g_i = theta^(-2i/d).  Linear scaling divides every frequency by
 * factor, i.e. positions are divided by factor ([ALGENTA] Decoder families:
 * linear global scaling; [UAII] P0.2).  Llama-3 scaling ([UAII] P0.2 RoPE scaling,
 * matching Hugging Face's Llama-3 rotary embedding; [FREETOKEN] Changes:
 * factor, low 1, high 4, original 8192): with wavelength lambda = 2*pi/f,
 *   lambda < orig/high           -> keep f
 *   lambda > orig/low            -> f / factor
 *   otherwise, mu = (orig/lambda - low)/(high - low),
 *                                   (1 - mu) * f / factor + mu * f.
 * YaRN ([UAII] P0.2 names YaRN beside Llama-3 scaling; [LLAMAY]
 * Architectures: gpt-oss uses YaRN), as Hugging Face computes it (the
 * reading the Llama-3 resolution sets): low and high are beta_slow and
 * beta_fast, the rotation counts over the original context that bound the
 * blend.  The pair index at which a frequency makes n turns over orig is
 * c(n) = d ln(orig / (2 pi n)) / (2 ln theta); the blend runs over pair
 * indices from c(beta_fast) to c(beta_slow) (rounded outwards to whole
 * indices when truncate is set, then clamped to [0, d - 1]), with weight
 * t_i = clamp((i - c_lo) / (c_hi - c_lo), 0, 1) on the divided frequency:
 *   g_i = t_i * f / factor + (1 - t_i) * f. */
void oracle_rope_freqs(int d, int scaling, double theta, double factor,
                       double low, double high, double orig, int truncate,
                       double *g)
{
    double c_lo = 0.0, c_hi = 1.0;
    if (scaling == OR_YARN) {
        c_lo = (double)d * log(orig / (2.0 * OR_PI * high)) / (2.0 * log(theta));
        c_hi = (double)d * log(orig / (2.0 * OR_PI * low)) / (2.0 * log(theta));
        if (truncate) {
            c_lo = floor(c_lo);
            c_hi = ceil(c_hi);
        }
        if (c_lo < 0.0)
            c_lo = 0.0;
        if (c_hi > (double)(d - 1))
            c_hi = (double)(d - 1);
        if (c_hi == c_lo)
            c_hi += 0.001; /* a zero-width band still ramps */
    }
    for (int i = 0; i < d / 2; ++i) {
        double f = pow(theta, -2.0 * (double)i / (double)d);
        if (scaling == OR_LLAMA3) {
            double lambda = 2.0 * OR_PI / f;
            if (lambda < orig / high) {
                g[i] = f;
            } else if (lambda > orig / low) {
                g[i] = f / factor;
            } else {
                double mu = (orig / lambda - low) / (high - low);
                g[i] = (1.0 - mu) * f / factor + mu * f;
            }
        } else if (scaling == OR_LINEAR) {
            g[i] = f / factor;
        } else if (scaling == OR_YARN) {
            double t = ((double)i - c_lo) / (c_hi - c_lo);
            if (t < 0.0)
                t = 0.0;
            if (t > 1.0)
                t = 1.0;
            g[i] = t * f / factor + (1.0 - t) * f;
        } else {
            g[i] = f;
        }
    }
}

/* Rotate x in place at absolute position pos.  Pair (a, b) is (i, i + d/2)
 * for NeoX and (2i, 2i + 1) for interleaved ([UAII] P0.2; [LLAMAY]
 * Architectures; [FREETOKEN] Changes).  With angle t = pos * g_i:
 *   (x_a, x_b) <- (x_a cos t - x_b sin t, x_a sin t + x_b cos t). */
void oracle_rope_apply(double *x, int d, int pairing, const double *g, int64_t pos)
{
    for (int i = 0; i < d / 2; ++i) {
        int a = (pairing == OR_NEOX) ? i : 2 * i;
        int b = (pairing == OR_NEOX) ? i + d / 2 : 2 * i + 1;
        double t = (double)pos * g[i];
        double c = cos(t), s = sin(t);
        double xa = x[a], xb = x[b];
        x[a] = xa * c - xb * s;
        x[b] = xa * s + xb * c;
    }
}

/* One head vector through the producer: optional RMSNorm, then RoPE
 * ([UAII] P1.2: the norm sits before RoPE), then the rotary attention factor
 * (1 except for YaRN, whose cos and sin carry it, so q and k both scale). */
static void norm_rope(const float *in, int d, int norm_enabled, const float *w,
                      int offset, double eps, int pairing, const double *g,
                      int64_t pos, double attn_factor, double *out)
{
    double x[256];
    for (int i = 0; i < d; ++i)
        x[i] = (double)in[i];
    if (norm_enabled)
        oracle_rms_norm(x, d, w, offset, eps, out);
    else
        memcpy(out, x, sizeof(double) * (size_t)d);
    oracle_rope_apply(out, d, pairing, g, pos);
    if (attn_factor != 1.0)
        for (int i = 0; i < d; ++i)
            out[i] *= attn_factor;
}

/* YaRN's attention factor: 0.1 ln(factor) + 1 for factor > 1, else 1
 * (Hugging Face's default when the config gives none). */
double oracle_yarn_attn_factor(double factor)
{
    return factor <= 1.0 ? 1.0 : 0.1 * log(factor) + 1.0;
}

/* Store one row (double values) in the cache's storage format. */
static void store_row_double(int dtype, void *base, int64_t row, int d,
                             const double *x)
{
    for (int i = 0; i < d; ++i) {
        int64_t idx = row * (int64_t)d + i;
        if (dtype == OR_F32)
            ((float *)base)[idx] = (float)x[i]; /* RNE */
        else
            ((uint16_t *)base)[idx] = oracle_bf16_from_double(x[i]);
    }
}

/* The producer for a batch.  Position of sequence b is positions[b]; the
 * same absolute position rotates q and k ([UAII] P1.3: positions follow the
 * absolute KV index, same as RoPE).  Writes q_out (double, [B][H][d]) and
 * slot positions[b] of the caches ([B][Hkv][cap][d]; k_scale and v_scale
 * [B][Hkv][cap] for int8 keys and values).
 * Returns 0, or -1 for an argument outside what the oracle handles. */
int oracle_kv_produce(int B, int H, int Hkv, int d,
                      int pairing, int scaling, double theta, double factor,
                      double low, double high, double orig, int truncate,
                      double attn_factor,
                      int norm_enabled, double eps, int offset,
                      const float *w_q, const float *w_k,
                      const float *q_in, const float *k_in, const float *v_in,
                      const int32_t *positions,
                      int k_dtype, int v_dtype, int cap,
                      void *cache_k, void *cache_v, float *k_scale,
                      float *v_scale, double *q_out)
{
    if (d > 256 || d < 2 || (d & 1) || H % Hkv != 0)
        return -1;
    double g[128];
    oracle_rope_freqs(d, scaling, theta, factor, low, high, orig, truncate, g);
    if (scaling != OR_YARN)
        attn_factor = 1.0;
    double tmp[256];
    for (int b = 0; b < B; ++b) {
        int64_t pos = positions[b];
        if (pos < 0 || pos >= cap)
            return -1;
        for (int h = 0; h < H; ++h) {
            const float *src = q_in + ((int64_t)b * H + h) * d;
            norm_rope(src, d, norm_enabled, w_q, offset, eps, pairing, g, pos,
                      attn_factor, q_out + ((int64_t)b * H + h) * d);
        }
        for (int u = 0; u < Hkv; ++u) {
            int64_t slab = (int64_t)b * Hkv + u;
            int64_t row = slab * cap + pos;
            norm_rope(k_in + slab * d, d, norm_enabled, w_k, offset, eps, pairing,
                      g, pos, attn_factor, tmp);
            if (k_dtype == OR_I8) {
                /* q8 keys: the rotated key rounded to f32, then the same
                 * quantiser as the values ([LLAMAY] The KV cache, in three
                 * precisions: q8 quantises both keys and values). */
                float kf[256];
                for (int i = 0; i < d; ++i)
                    kf[i] = (float)tmp[i];
                oracle_quantize_v(kf, d, (int8_t *)cache_k + row * d, &k_scale[row]);
            } else {
                store_row_double(k_dtype, cache_k, row, d, tmp);
            }
            const float *v = v_in + slab * d;
            if (v_dtype == OR_I8) {
                oracle_quantize_v(v, d, (int8_t *)cache_v + row * d, &v_scale[row]);
            } else {
                for (int i = 0; i < d; ++i)
                    tmp[i] = (double)v[i];
                store_row_double(v_dtype, cache_v, row, d, tmp);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Attention                                                                 */
/* ------------------------------------------------------------------------ */

/* First visible key for a sequence of L keys (the new one included) under a
 * sliding window of W keys that counts the current key; W = 0 is no window
 * ([UAII] P1.4 sliding window). */
static int64_t visible_lo(int64_t L, int64_t W)
{
    return (W > 0 && L > W) ? L - W : 0;
}

/* Score of q head h against key j: scale * <q_h, K[u][j]> with u = h / G
 * (consecutive groups of G query heads share a kv head; [ALGENTA] Structural
 * fact requirements: n_heads is an exact multiple of n_kv_heads; attention
 * scale is 1/sqrt(head_dim)), then the logit softcap c * tanh(s / c) when
 * c > 0 ([UAII] P1.4: logit softcapping as a tanh clip). */
static double score(int d, int k_dtype, const void *cache_k, const float *k_scale,
                    int64_t krow, const double *q, double scale, double softcap)
{
    double acc = 0.0;
    for (int i = 0; i < d; ++i)
        acc += q[i] * load_elem(k_dtype, cache_k, krow, d, i, k_scale);
    double s = scale * acc;
    if (softcap > 0.0)
        s = softcap * tanh(s / softcap);
    return s;
}

/* Scores of one (b, h) over all L keys: visible keys get their (capped)
 * score, the rest -inf.  s_out has L entries. */
void oracle_scores(int H, int Hkv, int d, int k_dtype, int cap,
                   const void *cache_k, const float *k_scale, const double *q /* [d] */,
                   int b, int h, int64_t L, int64_t W, double softcap,
                   double *s_out)
{
    int G = H / Hkv;
    int u = h / G;
    int64_t slab = (int64_t)b * Hkv + u;
    int64_t lo = visible_lo(L, W);
    double scale = 1.0 / sqrt((double)d);
    for (int64_t j = 0; j < L; ++j)
        s_out[j] = (j >= lo)
                       ? score(d, k_dtype, cache_k, k_scale, slab * cap + j, q, scale, softcap)
                       : -INFINITY;
}

/* Softmax attention of one (b, h) over the keys [j0, j1) intersected with
 * the visible range.  out = sum_j e^(s_j - m) v_j / sum_j e^(s_j - m),
 * m = max s_j.  With an attention sink (a per-head logit sink that enters
 * the softmax denominator only; [LLAMAY] Architectures: gpt-oss) the
 * denominator gains e^(sink - m); has_sink = 0 means no sink.  Returns the
 * number of keys used; when it is > 0 and lse is not NULL,
 * *lse = m + ln(sum_j e^(s_j - m)) (over the keys only). */
static int64_t attend_range(int H, int Hkv, int d, int k_dtype, int v_dtype,
                            int cap, const void *cache_k, const void *cache_v,
                            const float *k_scale, const float *v_scale,
                            const double *q, int b, int h,
                            int64_t L, int64_t W, double softcap, int64_t j0,
                            int64_t j1, int has_sink, double sink, double *out,
                            double *lse)
{
    int G = H / Hkv;
    int u = h / G;
    int64_t slab = (int64_t)b * Hkv + u;
    int64_t lo = visible_lo(L, W);
    if (j0 < lo)
        j0 = lo;
    if (j1 > L)
        j1 = L;
    for (int i = 0; i < d; ++i)
        out[i] = 0.0;
    if (j1 <= j0)
        return 0;
    double scale = 1.0 / sqrt((double)d);
    double m = -INFINITY;
    for (int64_t j = j0; j < j1; ++j) {
        double s = score(d, k_dtype, cache_k, k_scale, slab * cap + j, q, scale, softcap);
        if (s > m)
            m = s;
    }
    double l = 0.0;
    for (int64_t j = j0; j < j1; ++j) {
        int64_t row = slab * cap + j;
        double w = exp(score(d, k_dtype, cache_k, k_scale, row, q, scale, softcap) - m);
        l += w;
        for (int i = 0; i < d; ++i)
            out[i] += w * load_elem(v_dtype, cache_v, row, d, i, v_scale);
    }
    double z = l + (has_sink ? exp(sink - m) : 0.0);
    for (int i = 0; i < d; ++i)
        out[i] /= z;
    if (lse)
        *lse = m + log(l);
    return j1 - j0;
}

/* Single-pass attention for a list of (b, h) pairs.  q is [B][H][d] double,
 * seq_lens[b] = keys attended by sequence b (the new one included), out is
 * [n_pairs][d] double.  pairs holds 2*n_pairs ints (b, h). */
int oracle_decode_pairs(int B, int H, int Hkv, int d, int k_dtype, int v_dtype,
                        int cap, const void *cache_k, const void *cache_v,
                        const float *k_scale, const float *v_scale, const double *q,
                        const int32_t *seq_lens, int32_t window, double softcap,
                        const double *sinks /* [H] or NULL */,
                        const int32_t *pairs, int n_pairs, double *out)
{
    if (H % Hkv != 0 || d > 256)
        return -1;
    for (int n = 0; n < n_pairs; ++n) {
        int b = pairs[2 * n], h = pairs[2 * n + 1];
        if (b < 0 || b >= B || h < 0 || h >= H)
            return -1;
        int64_t L = seq_lens[b];
        if (L < 1 || L > cap)
            return -1;
        attend_range(H, Hkv, d, k_dtype, v_dtype, cap, cache_k, cache_v, k_scale,
                     v_scale, q + ((int64_t)b * H + h) * d, b, h, L, window, softcap, 0, L,
                     sinks != NULL, sinks ? sinks[h] : 0.0, out + (int64_t)n * d, NULL);
    }
    return 0;
}

/* Split partial of one (b, h): split sigma covers keys
 * [sigma*S, (sigma+1)*S) intersected with the visible range.  Writes the
 * normalised partial output o[d] and its log-sum-exp; an empty split has
 * lse = -inf and o = 0 and is excluded from the combine.  Returns the
 * number of keys in the split.  Split-K flash decoding: per-split partials,
 * then a combine ([ALGENTA] Kernel path capabilities: split-K decode
 * partials; Conformance CLI: decode_attn=splitk_flash_decoding). */
int64_t oracle_split_partial(int H, int Hkv, int d, int k_dtype, int v_dtype,
                             int cap, const void *cache_k, const void *cache_v,
                             const float *k_scale, const float *v_scale,
                             const double *q /* [d] */,
                             int b, int h, int64_t L, int64_t W, double softcap,
                             int64_t S, int64_t sigma, double *o, double *lse)
{
    int64_t n = attend_range(H, Hkv, d, k_dtype, v_dtype, cap, cache_k, cache_v,
                             k_scale, v_scale, q, b, h, L, W, softcap, sigma * S,
                             (sigma + 1) * S, 0, 0.0, o, lse);
    if (n == 0)
        *lse = -INFINITY;
    return n;
}

/* Log-sum-exp combine of n partials: M = max lse_s over non-empty splits,
 * out = sum_s e^(lse_s - M) o_s / sum_s e^(lse_s - M).  Splits whose lse is
 * -inf are skipped.  With an attention sink the denominator gains
 * e^(sink - M) (the sink belongs to no split).
 * Returns the number of splits used. */
int oracle_combine(int n, int d, const double *o /* [n][d] */,
                   const double *lse /* [n] */, int has_sink, double sink,
                   double *out)
{
    double M = -INFINITY;
    for (int s = 0; s < n; ++s)
        if (lse[s] > M)
            M = lse[s];

    for (int i = 0; i < d; ++i)
        out[i] = 0.0;
    if (M == -INFINITY)
        return 0;
    double den = has_sink ? exp(sink - M) : 0.0;
    int used = 0;
    for (int s = 0; s < n; ++s) {
        if (lse[s] == -INFINITY)
            continue;
        double w = exp(lse[s] - M);
        den += w;
        for (int i = 0; i < d; ++i)
            out[i] += w * o[(int64_t)s * d + i];
        ++used;
    }
    for (int i = 0; i < d; ++i)
        out[i] /= den;
    return used;
}
