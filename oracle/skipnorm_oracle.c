/*
 * skipnorm_oracle.c -- plain, slow, single-threaded CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the product library.  It shares no
 * code with the HIP path.  Build: C99, no fast-math, -ffp-contract=off, so
 * every float operation below is one IEEE-754 operation in the precision
 * written.
 *
 * Every step follows the operator definitions on the kernels-hub READMEs
 * "com.microsoft.SkipSimplifiedLayerNormalization", "com.microsoft.GatedRMSNorm"
 * and "com.microsoft.SkipGroupNorm"; each function names its passage.
 *
 * Readings taken where the pages leave a step open (all listed in the design
 * notes of the repository):
 *   - The residual sum is formed in float32 as (X + skip) + bias, in that order,
 *     then rounded once to T; with no bias there is no third addition at all.
 *     SkipSimplifiedLayerNormalization's statistic sees this T-valued sum, as
 *     SkipGroupNorm's Description states for its own sum.
 *   - Group variance is the population variance (divide by the element count).
 *   - SiLU(v) = v / (1 + exp(-v)).
 *   - epsilon is the float32 attribute value, widened exactly to double.
 */
#include "skipnorm_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------------- */
/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Normal numbers: (1 + f/1024) * 2^(e-15), e in 1..30.  Subnormals (e = 0):
 * f * 2^-24.  e = 31: infinity (f = 0) or NaN.                             */

float oracle_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    if (e == 31) {
        /* Infinity or NaN: keep sign and fraction (NaN payload moves to the
         * top fraction bits of binary32). */
        uint32_t bits = ((uint32_t)sign << 31) | 0x7f800000u | ((uint32_t)f << 13);
        float out;
        memcpy(&out, &bits, sizeof out);
        return out;
    }
    double mag = (e == 0) ? ldexp((double)f, -24)
                          : ldexp(1.0 + (double)f / 1024.0, e - 15);
    return (float)(sign ? -mag : mag); /* exact: binary16 is a subset */
}

/* Round half to even of a non-negative double that has at most 53
 * significant bits (every value passed here is exact). */
static double round_half_even(double v)
{
    double fl = floor(v);
    double frac = v - fl;
    if (frac > 0.5) return fl + 1.0;
    if (frac < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* Nearest binary16 value to v, ties to the even significand, with gradual
 * underflow and overflow to infinity.  v is rounded directly (one rounding). */
uint16_t oracle_f64_to_f16(double v)
{
    if (isnan(v)) {
        /* Quiet NaN with the sign; binary16 NaN payloads are not compared. */
        return (uint16_t)((signbit(v) ? 0x8000u : 0u) | 0x7e00u);
    }
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    /* 65520 is the midpoint between the largest finite value 65504 and 2^16;
     * a tie there goes to the even neighbour 2^16, which overflows. */
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00u);
    if (a < ldexp(1.0, -14)) {
        /* Subnormal range: quantum 2^-24.  n == 1024 encodes the smallest
         * normal 2^-14 with the same bits, so no special case is needed. */
        double n = round_half_even(a * ldexp(1.0, 24));
        return (uint16_t)(sign | (uint16_t)n);
    }
    int ex;
    (void)frexp(a, &ex);      /* a = m * 2^ex, m in [0.5, 1) */
    int e = ex - 1;           /* a in [2^e, 2^(e+1)) */
    double n = round_half_even(ldexp(a, 10 - e)); /* in [1024, 2048] */
    /* n == 2048 carries into the exponent field, which the sum below does. */
    uint32_t bits = ((uint32_t)(e + 15) << 10) + (uint32_t)(n - 1024.0);
    return (uint16_t)(sign | bits);
}

uint16_t oracle_f32_to_f16(float v)
{
    return oracle_f64_to_f16((double)v); /* widening is exact */
}

void oracle_f16_to_f32_array(const uint16_t* h, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f32(h[i]);
}

void oracle_f32_to_f16_array(const float* f, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_f16(f[i]);
}

/* ---------------------------------------------------------------------- */
/* Typed element access.                                                    */

static float load_f32(int type, const void* p, int64_t i)
{
    if (type == ORACLE_F32) return ((const float*)p)[i];
    return oracle_f16_to_f32(((const uint16_t*)p)[i]);
}

/* Round a float32 value to T and return the T value widened to float32. */
static float round_f32_to_type(int type, float v)
{
    if (type == ORACLE_F32) return v;
    return oracle_f16_to_f32(oracle_f32_to_f16(v));
}

/* Store a float64 result rounded once to T. */
static void store_f64(int type, void* p, int64_t i, double v)
{
    if (type == ORACLE_F32) ((float*)p)[i] = (float)v;
    else ((uint16_t*)p)[i] = oracle_f64_to_f16(v);
}

/* Store a value that is already representable in T. */
static void store_exact(int type, void* p, int64_t i, float v)
{
    if (type == ORACLE_F32) ((float*)p)[i] = v;
    else ((uint16_t*)p)[i] = oracle_f32_to_f16(v);
}

static int valid_type(int t) { return t == ORACLE_F32 || t == ORACLE_F16; }

/* Residual sum of one element: float32 (x + skip), then + bias when a bias
 * is given, then one rounding to T.  SkipGroupNorm, Description ("rounded to
 * the tensor type before the statistics see it"); SkipSimplifiedLayer-
 * Normalization, Inputs (bias "added to the input + skip sum") and Outputs
 * (input_skip_bias_sum). */
static float residual_sum(int T, float x, float skip, int has_bias, float bias)
{
    float s = x + skip;
    if (has_bias) s = s + bias;
    return round_f32_to_type(T, s);
}

/* ---------------------------------------------------------------------- */
/* com.microsoft.SkipSimplifiedLayerNormalization, Description: S = input +
 * skip (+ bias); output = S * 1/sqrt(mean(S^2) + epsilon) * gamma over the
 * last axis.  Outputs: mean is zero for the simplified form; inv_std_var is
 * the inverse RMS; input_skip_bias_sum is S.                               */
int oracle_skip_rms_norm(int T, int64_t rows, int64_t hidden,
                         const void* input, const void* skip,
                         const void* gamma, const void* bias, float epsilon,
                         void* output, float* mean, float* inv_std_var,
                         void* input_skip_bias_sum)
{
    if (!valid_type(T) || hidden <= 0 || rows < 0) return -1;
    double* s = (double*)malloc((size_t)hidden * sizeof(double));
    if (!s) return -2;
    const double eps = (double)epsilon;
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t base = r * hidden;
        double sum_sq = 0.0;
        for (int64_t j = 0; j < hidden; ++j) {
            float sv = residual_sum(T, load_f32(T, input, base + j),
                                    load_f32(T, skip, base + j), bias != NULL,
                                    bias ? load_f32(T, bias, j) : 0.0f);
            if (input_skip_bias_sum) store_exact(T, input_skip_bias_sum, base + j, sv);
            s[j] = (double)sv;
            sum_sq += s[j] * s[j];
        }
        const double mean_sq = sum_sq / (double)hidden;
        const double inv_rms = 1.0 / sqrt(mean_sq + eps);
        for (int64_t j = 0; j < hidden; ++j)
            store_f64(T, output, base + j,
                      s[j] * inv_rms * (double)load_f32(T, gamma, j));
        if (mean) mean[r] = 0.0f;
        if (inv_std_var) inv_std_var[r] = (float)inv_rms;
    }
    free(s);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Skip layer normalization with the mean removed: the operator whose
 * simplified form is SkipSimplifiedLayerNormalization.  The SSLN page's
 * Outputs section describes its `mean` output as the per-row mean (zero only
 * for the simplified form) and `inv_std_var` as the per-row inverse standard
 * deviation (the inverse RMS only for the simplified form); this is that
 * non-simplified form: S as for SSLN, mean = sum(S)/hidden,
 * var = sum((S - mean)^2)/hidden (population), inv = 1/sqrt(var + eps),
 * output = (S - mean) * inv * gamma (+ beta when beta is given).          */
int oracle_skip_layer_norm(int T, int64_t rows, int64_t hidden,
                           const void* input, const void* skip,
                           const void* gamma, const void* beta, const void* bias,
                           float epsilon, void* output, float* mean,
                           float* inv_std_var, void* input_skip_bias_sum)
{
    if (!valid_type(T) || hidden <= 0 || rows < 0) return -1;
    double* s = (double*)malloc((size_t)hidden * sizeof(double));
    if (!s) return -2;
    const double eps = (double)epsilon;
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t base = r * hidden;
        double sum = 0.0;
        for (int64_t j = 0; j < hidden; ++j) {
            float sv = residual_sum(T, load_f32(T, input, base + j),
                                    load_f32(T, skip, base + j), bias != NULL,
                                    bias ? load_f32(T, bias, j) : 0.0f);
            if (input_skip_bias_sum) store_exact(T, input_skip_bias_sum, base + j, sv);
            s[j] = (double)sv;
            sum += s[j];
        }
        const double mu = sum / (double)hidden;
        double ssd = 0.0;
        for (int64_t j = 0; j < hidden; ++j) ssd += (s[j] - mu) * (s[j] - mu);
        const double inv = 1.0 / sqrt(ssd / (double)hidden + eps);
        for (int64_t j = 0; j < hidden; ++j) {
            double y = (s[j] - mu) * inv * (double)load_f32(T, gamma, j);
            if (beta) y += (double)load_f32(T, beta, j);
            store_f64(T, output, base + j, y);
        }
        if (mean) mean[r] = (float)mu;
        if (inv_std_var) inv_std_var[r] = (float)inv;
    }
    free(s);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* com.microsoft.GatedRMSNorm, Description: Y = X * rsqrt(mean(X^2) + eps) *
 * scale * SiLU(gate), the mean taken over each contiguous run of C elements,
 * C = element count of scale, rows counted flat as numel / C.             */
static double silu(double v) { return v / (1.0 + exp(-v)); }

int oracle_gated_rms_norm(int T, int64_t numel, int64_t C,
                          const void* X, const void* scale, const void* gate,
                          float epsilon, void* Y)
{
    if (!valid_type(T) || C <= 0 || numel < 0 || numel % C != 0) return -1;
    const double eps = (double)epsilon;
    const int64_t rows = numel / C;
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t base = r * C;
        double sum_sq = 0.0;
        for (int64_t j = 0; j < C; ++j) {
            double x = (double)load_f32(T, X, base + j);
            sum_sq += x * x;
        }
        const double inv_rms = 1.0 / sqrt(sum_sq / (double)C + eps);
        for (int64_t j = 0; j < C; ++j) {
            double x = (double)load_f32(T, X, base + j);
            double g = (double)load_f32(T, gate, base + j);
            double sc = (double)load_f32(T, scale, j);
            store_f64(T, Y, base + j, x * inv_rms * sc * silu(g));
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------- */
/* com.microsoft.SkipGroupNorm, Description and Inputs/Attributes:
 *   S = X + skip + bias, rounded to T;
 *   per batch item n and group g of C/groups channels, over every spatial
 *   position: mean and (population) variance of S;
 *   Y = gamma_c * (S - mean) / sqrt(variance + epsilon) + beta_c;
 *   activation 1 applies SiLU after the affine step.
 * Layout (channels_last attribute): NHWC when non-zero, NCHW otherwise.    */
static int64_t x_index(int channels_last, int64_t C, int64_t H, int64_t W,
                       int64_t n, int64_t c, int64_t h, int64_t w)
{
    if (channels_last) return ((n * H + h) * W + w) * C + c;
    return ((n * C + c) * H + h) * W + w;
}

int oracle_skip_group_norm(int T, int M, int64_t N, int64_t C, int64_t H,
                           int64_t W, int channels_last,
                           const void* X, const void* gamma, const void* beta,
                           const void* skip, int skip_broadcast,
                           const void* bias, float epsilon, int64_t groups,
                           int activation, void* Y, void* S)
{
    if (!valid_type(T) || !valid_type(M)) return -1;
    if (N < 0 || C <= 0 || H < 0 || W < 0 || groups <= 0 || C % groups != 0) return -1;
    if (activation != 0 && activation != 1) return -1;
    const int64_t total = N * C * H * W;
    double* s = (double*)malloc((size_t)(total > 0 ? total : 1) * sizeof(double));
    if (!s) return -2;

    /* Pass 1: the residual sum S, stored as T when requested. */
    for (int64_t n = 0; n < N; ++n)
        for (int64_t c = 0; c < C; ++c)
            for (int64_t h = 0; h < H; ++h)
                for (int64_t w = 0; w < W; ++w) {
                    const int64_t i = x_index(channels_last, C, H, W, n, c, h, w);
                    const int64_t k = skip_broadcast ? n * C + c : i;
                    float sv = residual_sum(T, load_f32(T, X, i), load_f32(T, skip, k),
                                            bias != NULL,
                                            bias ? load_f32(T, bias, c) : 0.0f);
                    if (S) store_exact(T, S, i, sv);
                    s[i] = (double)sv;
                }

    /* Pass 2: two-pass statistics per (n, group), then the affine step. */
    const int64_t cpg = C / groups;
    const double count = (double)(cpg * H * W);
    const double eps = (double)epsilon;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t g = 0; g < groups; ++g) {
            double sum = 0.0;
            for (int64_t c = g * cpg; c < (g + 1) * cpg; ++c)
                for (int64_t h = 0; h < H; ++h)
                    for (int64_t w = 0; w < W; ++w)
                        sum += s[x_index(channels_last, C, H, W, n, c, h, w)];
            const double mean = sum / count;
            double sq = 0.0;
            for (int64_t c = g * cpg; c < (g + 1) * cpg; ++c)
                for (int64_t h = 0; h < H; ++h)
                    for (int64_t w = 0; w < W; ++w) {
                        double d = s[x_index(channels_last, C, H, W, n, c, h, w)] - mean;
                        sq += d * d;
                    }
            const double var = sq / count;
            const double rstd = 1.0 / sqrt(var + eps);
            for (int64_t c = g * cpg; c < (g + 1) * cpg; ++c) {
                const double gm = (double)load_f32(M, gamma, c);
                const double bt = (double)load_f32(M, beta, c);
                for (int64_t h = 0; h < H; ++h)
                    for (int64_t w = 0; w < W; ++w) {
                        const int64_t i = x_index(channels_last, C, H, W, n, c, h, w);
                        double y = gm * (s[i] - mean) * rstd + bt;
                        if (activation == 1) y = silu(y);
                        store_f64(T, Y, i, y);
                    }
            }
        }
    free(s);
    return 0;
}
