/*
 * skipnorm.h -- C ABI of libskipnorm: fused skip-add + normalize operators on
 * AMD Instinct MI355X (gfx950).
 *
 * Three operators, each defined on its ONNX Runtime contrib-op kernels-hub
 * README, and the non-simplified form of the first:
 *   skip_rms_norm   "com.microsoft.SkipSimplifiedLayerNormalization"
 *   skip_layer_norm its form with the row mean removed (see below)
 *   gated_rms_norm  "com.microsoft.GatedRMSNorm"
 *   skip_group_norm "com.microsoft.SkipGroupNorm"
 * Every entry point keeps the page's input and output names, order,
 * optionality and attributes; allocation moves to the caller (the pages'
 * loader allocates outputs; here the caller passes them).
 *
 * Conventions shared by every entry point:
 *   - Tensors are passed as descriptors (sn_tensor_in / sn_tensor_out):
 *     a DEVICE pointer on the current HIP device, the element type, the rank
 *     and the shape.  Data is dense and row-major (C-contiguous).  A NULL
 *     descriptor means an optional input or output is absent; a required one
 *     may not be NULL.  The descriptors themselves are read during the call
 *     only (they may live on the caller's stack).
 *   - The caller owns every buffer; the library never allocates, frees or
 *     synchronizes device memory.
 *   - Work is enqueued on `stream` (0 = the null stream) and returns
 *     immediately, like a kernel launch.
 *   - Arithmetic: the residual sum is formed in float32 and rounded once to
 *     the tensor type T; statistics and normalization are float32; every
 *     output is rounded once to its type.
 *   - Validation happens on the host before anything is enqueued: ranks,
 *     shapes and element types of every tensor against the operator's
 *     contract, attributes, pointers, aliasing and sizes.  On any status
 *     other than SN_OK and SN_ERR_HIP nothing was launched and no output was
 *     written.  SN_ERR_HIP reports a failed launch.  The message for the
 *     last non-OK status of the calling thread is returned by
 *     skipnorm_last_error().
 *   - Outputs may not overlap inputs or each other (SN_ERR_ALIAS).
 *   - Pointers need no particular alignment (beyond their element type's):
 *     each call reads and writes in the widest of 16-, 8- and 4-byte vectors
 *     that divides a row (pixel, image plane) and every base address, else
 *     element by element -- except where aligned 16-byte vectors are read
 *     across the boundaries of rows, spans or groups instead:
 *     skip_rms_norm / skip_layer_norm rows that would be read with accesses
 *     narrower than 16 bytes, when input, skip, output and S share their
 *     offset from a 16-byte boundary (short rows read as one stream take
 *     gamma, beta and bias at any alignment; longer rows need them 16-byte
 *     aligned); gated_rms_norm spans likewise when X, gate and Y share their
 *     offset (longer spans need scale 16-byte aligned); skip_group_norm NCHW groups
 *     when X, skip, Y and S share their offset and H*W holds a 16-byte
 *     vector; and NHWC pixels that are not a whole number of 16-byte
 *     vectors, read as runs of pixels that are, when X, Y, S and a full
 *     skip are 16-byte aligned.  Results are the same up to float32
 *     summation order.  Such reads touch at most the 15 bytes beside a
 *     tensor's first and last element that lie in the same aligned 16-byte
 *     block (GPU memory is allocated and protected in far larger units, so
 *     they never fault); nothing outside a tensor is written.
 *   - Zero-sized leading dimensions are valid and launch nothing.  A row
 *     (hidden, span) or one SkipGroupNorm image (C*H*W) may hold at most
 *     2^30 elements.
 *   - Results are deterministic: no floating-point atomics; every reduction
 *     runs in a fixed order, and requesting an optional output never changes
 *     the others.  No kernel waits on another workgroup without a bound.
 * Route-selection and measurement hooks for tests are declared separately,
 * in skipnorm_testing.h.
 */
#ifndef SKIPNORM_H
#define SKIPNORM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SKIPNORM_ABI_VERSION 3

/* Element types.  T (tensor data) and M (SkipGroupNorm gamma/beta) take
 * float32 or float16 ("Type constraints" on each page); statistics outputs
 * are always float32 (U).  bfloat16 is listed only to be rejected: the pages
 * state that it is not implemented. */
typedef enum sn_dtype {
    SN_F32 = 0,
    SN_F16 = 1,
    SN_BF16 = 2
} sn_dtype;

typedef enum sn_status {
    SN_OK = 0,
    SN_ERR_NULL = 1,      /* a required tensor or pointer is NULL             */
    SN_ERR_DTYPE = 2,     /* unsupported or mismatched element type           */
    SN_ERR_SHAPE = 3,     /* rank or shape against the contract, or too large */
    SN_ERR_ATTR = 4,      /* attribute out of range (epsilon, groups, ...)    */
    SN_ERR_ALIAS = 5,     /* an output overlaps an input or another output    */
    SN_ERR_WORKSPACE = 6, /* workspace missing or smaller than required       */
    SN_ERR_HIP = 7        /* a HIP launch failed                              */
} sn_status;

#define SN_MAX_RANK 8

/* A tensor argument: device data, element type, rank (0..SN_MAX_RANK) and
 * shape (shape[0 .. rank-1], every extent >= 0; the rest is ignored). */
typedef struct sn_tensor_in {
    const void* data;
    sn_dtype dtype;
    int32_t rank;
    int64_t shape[SN_MAX_RANK];
} sn_tensor_in;

typedef struct sn_tensor_out {
    void* data;
    sn_dtype dtype;
    int32_t rank;
    int64_t shape[SN_MAX_RANK];
} sn_tensor_out;

/* ------------------------------------------------------------------------
 * SkipSimplifiedLayerNormalization ("com.microsoft.SkipSimplifiedLayer-
 * Normalization": Description, Inputs, Outputs, Attributes, Type
 * constraints).
 *
 * Over the last axis (hidden) of every row:
 *   S[j]  = round_T((input[j] + skip[j]) + bias[j])   (bias term only if given)
 *   r     = 1 / sqrt(sum_j S[j]^2 / hidden + epsilon)
 *   output[j] = round_T(S[j] * r * gamma[j])
 * Inputs (T = float32 or float16, the same for all of them):
 *   input        rank 2 (token_count, hidden) or rank 3 (batch, sequence,
 *                hidden); hidden >= 1, leading extents >= 0.
 *   skip         input's shape.
 *   gamma        (hidden).
 *   bias         (hidden) or NULL.
 *   epsilon      >= 0 and finite (the page's default is 9.999999960041972e-13).
 * Outputs:
 *   output       input's shape, T.
 *   mean         input's shape with the last extent 1, float32, or NULL;
 *                written as 0 (the simplified form has no mean).
 *   inv_std_var  as mean, or NULL; receives r.
 *   input_skip_bias_sum  input's shape, T, or NULL; receives S.
 * ------------------------------------------------------------------------ */
sn_status skip_rms_norm(const sn_tensor_in* input, const sn_tensor_in* skip,
                        const sn_tensor_in* gamma, const sn_tensor_in* bias,
                        float epsilon, const sn_tensor_out* output,
                        const sn_tensor_out* mean, const sn_tensor_out* inv_std_var,
                        const sn_tensor_out* input_skip_bias_sum, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Skip layer normalization with the row mean removed: the non-simplified
 * form of SkipSimplifiedLayerNormalization, whose page describes the `mean`
 * output as the per-row mean (zero only for the simplified form) and
 * `inv_std_var` as the inverse standard deviation (the inverse RMS only for
 * the simplified form); the optional `beta` is added after the scaling
 * (layer normalization's affine form).
 *   S[j]  = round_T((input[j] + skip[j]) + bias[j])   (bias term only if given)
 *   mu    = sum_j S[j] / hidden
 *   r     = 1 / sqrt(sum_j (S[j] - mu)^2 / hidden + epsilon)
 *   output[j] = round_T((S[j] - mu) * r * gamma[j] + beta[j])   (beta only if given)
 * Arguments as for skip_rms_norm, plus:
 *   beta         (hidden) T or NULL.
 *   mean         receives mu.   inv_std_var: receives r.
 * ------------------------------------------------------------------------ */
sn_status skip_layer_norm(const sn_tensor_in* input, const sn_tensor_in* skip,
                          const sn_tensor_in* gamma, const sn_tensor_in* beta,
                          const sn_tensor_in* bias, float epsilon,
                          const sn_tensor_out* output, const sn_tensor_out* mean,
                          const sn_tensor_out* inv_std_var,
                          const sn_tensor_out* input_skip_bias_sum, hipStream_t stream);

/* ------------------------------------------------------------------------
 * GatedRMSNorm ("com.microsoft.GatedRMSNorm": Description, Inputs, Outputs,
 * Attributes).
 *
 * C = element count of scale.  X is read as numel(X) / C flat rows of C
 * contiguous elements, whatever its rank:
 *   r    = 1 / sqrt(sum_j X[j]^2 / C + epsilon)
 *   Y[j] = round_T(X[j] * r * scale[j] * SiLU(gate[j])),  SiLU(g) = g / (1 + e^-g)
 * with every intermediate in float32.
 * Inputs (T = float32 or float16 for all):
 *   X        rank >= 1; numel(X) a multiple of C.
 *   scale    a vector of C >= 1 elements in any spelling: (C), (1, C),
 *            (C, 1), ... (at most one extent differs from 1).
 *   gate     X's shape.
 *   epsilon  >= 0 and finite (the page's default is 1e-5).
 * Output:
 *   Y        X's shape, T.
 * ------------------------------------------------------------------------ */
sn_status gated_rms_norm(const sn_tensor_in* X, const sn_tensor_in* scale,
                         const sn_tensor_in* gate, float epsilon,
                         const sn_tensor_out* Y, hipStream_t stream);

/* ------------------------------------------------------------------------
 * SkipGroupNorm ("com.microsoft.SkipGroupNorm": Description, Inputs,
 * Outputs, Attributes, Type constraints).
 *
 * X has rank 4: (N, H, W, C) when channels_last != 0 (any non-zero value
 * selects it) and (N, C, H, W) when channels_last == 0.
 *   S = round_T((X + skip) + bias)        (bias term only if given)
 *   per (n, group g of C/groups channels), over all H*W positions:
 *     mean, var = population mean and variance of S
 *   Y = round_T(act(gamma[c] * (S - mean) / sqrt(var + epsilon) + beta[c]))
 *   act = identity (activation 0) or SiLU (activation 1).
 * Inputs:
 *   X              T = float32 or float16; C >= 1, N, H, W >= 0.
 *   gamma, beta    (C), M = float32 or float16 (both the same; independent
 *                  of T).
 *   skip           T; X's exact shape (checked first), or (N, C) or
 *                  (N, 1, 1, C): one value per batch item and channel.
 *   bias           (C) T, or NULL.
 *   epsilon        >= 0 and finite (the page's default is 1e-5).
 *   groups         >= 1 and divides C.
 *   activation     0 (none) or 1 (SiLU).
 * Outputs:
 *   Y              X's shape, T.   S: X's shape, T, or NULL.
 *   workspace      device memory of at least the size that
 *                  skip_group_norm_workspace_size returns for the same X,
 *                  groups and channels_last (may be NULL when that size is
 *                  0), 16-byte aligned.  Its contents on entry do not
 *                  matter.  Calls that share a workspace must be ordered
 *                  (same stream).
 * The single-launch routes tell a call's exchanged partial moments from
 * earlier ones by a per-call value.  On a stream that is being captured into
 * a HIP graph (whose replays repeat every argument) the call records, ahead
 * of such a launch, a small kernel that clears those values in the
 * workspace, so that every replay is correct.
 * ------------------------------------------------------------------------ */

/* Workspace bytes skip_group_norm needs for X (only X's dtype, rank and
 * shape are read; its data pointer may be NULL), into *bytes. */
sn_status skip_group_norm_workspace_size(const sn_tensor_in* X, int64_t groups,
                                         int32_t channels_last, size_t* bytes);

sn_status skip_group_norm(const sn_tensor_in* X, const sn_tensor_in* gamma,
                          const sn_tensor_in* beta, const sn_tensor_in* skip,
                          const sn_tensor_in* bias, float epsilon, int64_t groups,
                          int32_t channels_last, int32_t activation,
                          const sn_tensor_out* Y, const sn_tensor_out* S,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * skip_group_norm without a workspace argument, for callers that cannot
 * allocate device memory: code being captured into a HIP graph, tight
 * serving loops, hosts that forbid hipMalloc.  It allocates nothing (no
 * hipMalloc, hipFree or allocating library call); its partial moments live
 * in a static device array of SKIPNORM_NOALLOC_SCRATCH_BYTES inside the
 * library, one copy on each device it runs on, held until the process ends.
 * Arguments, results and routes are skip_group_norm's (the caller still
 * passes every input and output).  Errors as skip_group_norm, plus
 * SN_ERR_WORKSPACE when the shape needs more scratch than the array holds
 * (skip_group_norm_workspace_size tells how much it needs) and SN_ERR_HIP
 * when the array's device address cannot be obtained.
 * Every call on one device shares that device's array and leaves its
 * contents behind (no call depends on them): calls that overlap in time on
 * one device -- on different streams, or from host threads without
 * ordering -- race on it and must not be issued.
 * ------------------------------------------------------------------------ */
#define SKIPNORM_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

sn_status skip_group_norm_noalloc(const sn_tensor_in* X, const sn_tensor_in* gamma,
                                  const sn_tensor_in* beta, const sn_tensor_in* skip,
                                  const sn_tensor_in* bias, float epsilon, int64_t groups,
                                  int32_t channels_last, int32_t activation,
                                  const sn_tensor_out* Y, const sn_tensor_out* S,
                                  hipStream_t stream);

/* ------------------------------------------------------------------------
 * Library information.
 * ------------------------------------------------------------------------ */

/* Message for the calling thread's last non-OK status ("" if none).  The
 * string stays valid until that thread's next call into the library. */
const char* skipnorm_last_error(void);

/* SKIPNORM_ABI_VERSION of the built library. */
int skipnorm_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SKIPNORM_H */
