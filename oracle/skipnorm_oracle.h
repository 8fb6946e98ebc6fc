/*
 * skipnorm_oracle.h -- plain, slow, single-threaded CPU oracle for the fused
 * skip-add + normalize operators.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this code; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no source with the HIP path.
 *
 * Sources (the kernels-hub READMEs of the three ONNX Runtime contrib ops):
 *   - "com.microsoft.SkipSimplifiedLayerNormalization": Description, Inputs,
 *     Outputs, Attributes, Type constraints.
 *   - "com.microsoft.GatedRMSNorm": Description, Inputs, Outputs, Attributes.
 *   - "com.microsoft.SkipGroupNorm": Description, Inputs, Outputs, Attributes,
 *     Type constraints.
 *
 * Precision: the residual sum S is formed exactly as the operator defines it
 * (float32 additions, then one rounding to the tensor type T); every statistic
 * and every normalized value is then computed in float64 from the T-valued S
 * and rounded once to T at the end.
 *
 * Element types: 0 = float32, 1 = float16 (IEEE-754 binary16 bit patterns in
 * uint16_t storage).  All arrays are host memory, dense and row-major.
 * Every function returns 0 on success and a negative value on an argument it
 * cannot evaluate (unknown type code, zero span, groups not dividing C).
 */
#ifndef SKIPNORM_ORACLE_H
#define SKIPNORM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_F16 = 1 };

/* IEEE-754 binary16 conversions written from the format's definition. */
float    oracle_f16_to_f32(uint16_t h);
uint16_t oracle_f64_to_f16(double v);
uint16_t oracle_f32_to_f16(float v);
void     oracle_f16_to_f32_array(const uint16_t* h, float* out, int64_t n);
void     oracle_f32_to_f16_array(const float* f, uint16_t* out, int64_t n);

/* SkipSimplifiedLayerNormalization over `rows` rows of `hidden` elements.
 * bias, mean, inv_std_var and input_skip_bias_sum may be NULL. */
int oracle_skip_rms_norm(int T, int64_t rows, int64_t hidden,
                         const void* input, const void* skip,
                         const void* gamma, const void* bias, float epsilon,
                         void* output, float* mean, float* inv_std_var,
                         void* input_skip_bias_sum);

/* Skip layer normalization with the mean removed (the non-simplified form
 * of SkipSimplifiedLayerNormalization): mean = sum(S)/hidden, population
 * variance, output = (S - mean) / sqrt(var + eps) * gamma (+ beta).
 * beta, bias, mean, inv_std_var and input_skip_bias_sum may be NULL. */
int oracle_skip_layer_norm(int T, int64_t rows, int64_t hidden,
                           const void* input, const void* skip,
                           const void* gamma, const void* beta, const void* bias,
                           float epsilon, void* output, float* mean,
                           float* inv_std_var, void* input_skip_bias_sum);

/* GatedRMSNorm: numel elements, normalization span C = element count of
 * scale; rows = numel / C, counted flat. */
int oracle_gated_rms_norm(int T, int64_t numel, int64_t C,
                          const void* X, const void* scale, const void* gate,
                          float epsilon, void* Y);

/* SkipGroupNorm on X of logical shape (N, C, H, W); the memory order is
 * (N, H, W, C) when channels_last != 0 and (N, C, H, W) otherwise.
 * skip_broadcast != 0 means skip holds one value per (n, c) at skip[n*C + c];
 * otherwise skip has X's shape and layout.  bias and S may be NULL. */
int oracle_skip_group_norm(int T, int M, int64_t N, int64_t C, int64_t H,
                           int64_t W, int channels_last,
                           const void* X, const void* gamma, const void* beta,
                           const void* skip, int skip_broadcast,
                           const void* bias, float epsilon, int64_t groups,
                           int activation, void* Y, void* S);

#ifdef __cplusplus
}
#endif
#endif
