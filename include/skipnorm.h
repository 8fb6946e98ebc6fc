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
 *
 * Conventions shared by every entry point:
 *   - Tensor arguments are DEVICE pointers on the current HIP device, dense
 *     and row-major (C-contiguous) in the layout stated per argument.  The
 *     caller owns every buffer; the library never allocates, frees or
 *     synchronizes device memory.
 *   - Work is enqueued on `stream` (0 = the null stream) and returns
 *     immediately, like a kernel launch.
 *   - Optional inputs and outputs are passed as NULL when absent.
 *   - Arithmetic: the residual sum is formed in float32 and rounded once to
 *     the tensor type T; statistics and normalization are float32; every
 *     output is rounded once to its type.
 *   - Validation happens on the host before anything is enqueued: on any
 *     status other than SN_OK and SN_ERR_HIP nothing was launched and no
 *     output was written.  SN_ERR_HIP reports a failed launch.  The message
 *     for the last non-OK status of the calling thread is returned by
 *     skipnorm_last_error().
 *   - Outputs may not overlap inputs or each other (SN_ERR_ALIAS).
 *   - Pointers need no particular alignment (beyond their element type's):
 *     each call reads and writes in the widest of 16-, 8- and 4-byte vectors
 *     that divides a row (pixel, image plane) and every base address, else
 *     element by element -- except that skip_rms_norm / skip_layer_norm rows
 *     left with element-by-element accesses read aligned 16-byte vectors
 *     across row boundaries when input, skip, output and S share their
 *     offset from a 16-byte boundary and gamma, beta and bias are 16-byte
 *     aligned, and skip_group_norm NCHW groups likewise across group
 *     boundaries when X, skip, Y and S share their offset and H*W holds a
 *     16-byte vector (reads then touch the up to 15 bytes beside a tensor's
 *     first and last element that share their 16-byte block; nothing
 *     outside a tensor is written) -- with the same results up to float32
 *     summation order.
 *   - Zero-sized leading dimensions are valid and launch nothing.  A row
 *     (hidden, span) or one SkipGroupNorm image (C*H*W) may hold at most
 *     2^30 elements.
 *   - Results are deterministic: no floating-point atomics; every reduction
 *     runs in a fixed order, and requesting an optional output never changes
 *     the others.  No kernel waits on another workgroup without a bound.
 */
#ifndef SKIPNORM_H
#define SKIPNORM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SKIPNORM_ABI_VERSION 2

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
    SN_ERR_NULL = 1,      /* a required pointer is NULL                       */
    SN_ERR_DTYPE = 2,     /* unsupported element type                         */
    SN_ERR_SHAPE = 3,     /* sizes inconsistent or out of range               */
    SN_ERR_ATTR = 4,      /* attribute out of range (epsilon, groups, ...)    */
    SN_ERR_ALIAS = 5,     /* an output overlaps an input or another output    */
    SN_ERR_WORKSPACE = 6, /* workspace missing or smaller than required       */
    SN_ERR_HIP = 7        /* a HIP launch failed                              */
} sn_status;

/* ------------------------------------------------------------------------
 * SkipSimplifiedLayerNormalization ("com.microsoft.SkipSimplifiedLayer-
 * Normalization": Description, Inputs, Outputs, Attributes).
 *
 * For each of `rows` rows of `hidden` elements (the input's leading axes
 * folded; the page allows (token_count, hidden_size) and (batch, sequence,
 * hidden_size)):
 *   S[j]  = round_T((input[j] + skip[j]) + bias[j])   (bias term only if given)
 *   r     = 1 / sqrt(sum_j S[j]^2 / hidden + epsilon)
 *   output[j] = round_T(S[j] * r * gamma[j])
 * Arguments:
 *   T            SN_F32 or SN_F16, the type of every tensor except the stats.
 *   rows         >= 0.   hidden: >= 1.
 *   input, skip  [rows, hidden] T.        gamma: [hidden] T.
 *   bias         [hidden] T or NULL.
 *   epsilon      >= 0 and finite (the page's default is 9.999999960041972e-13).
 *   output       [rows, hidden] T.
 *   mean         [rows] float32 or NULL; written as 0 (the simplified form has
 *                no mean).
 *   inv_std_var  [rows] float32 or NULL; receives r.
 *   input_skip_bias_sum  [rows, hidden] T or NULL; receives S.
 * ------------------------------------------------------------------------ */
sn_status skip_rms_norm(sn_dtype T, int64_t rows, int64_t hidden,
                        const void* input, const void* skip, const void* gamma,
                        const void* bias, float epsilon,
                        void* output, float* mean, float* inv_std_var,
                        void* input_skip_bias_sum, hipStream_t stream);

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
 *   beta         [hidden] T or NULL.
 *   mean         [rows] float32 or NULL; receives mu.
 *   inv_std_var  [rows] float32 or NULL; receives r.
 * ------------------------------------------------------------------------ */
sn_status skip_layer_norm(sn_dtype T, int64_t rows, int64_t hidden,
                          const void* input, const void* skip, const void* gamma,
                          const void* beta, const void* bias, float epsilon,
                          void* output, float* mean, float* inv_std_var,
                          void* input_skip_bias_sum, hipStream_t stream);

/* ------------------------------------------------------------------------
 * GatedRMSNorm ("com.microsoft.GatedRMSNorm": Description, Inputs, Outputs,
 * Attributes).
 *
 * C = `span` = element count of scale.  X is read as numel / C flat rows of
 * C contiguous elements (any rank >= 1 folds to this):
 *   r    = 1 / sqrt(sum_j X[j]^2 / C + epsilon)
 *   Y[j] = round_T(X[j] * r * scale[j] * SiLU(gate[j])),  SiLU(g) = g / (1 + e^-g)
 * with every intermediate in float32.
 * Arguments:
 *   T        SN_F32 or SN_F16.
 *   numel    >= 0, a multiple of span.   span: >= 1.
 *   X, gate  [numel] T.   scale: [span] T.   Y: [numel] T.
 *   epsilon  >= 0 and finite (the page's default is 1e-5).
 * ------------------------------------------------------------------------ */
sn_status gated_rms_norm(sn_dtype T, int64_t numel, int64_t span,
                         const void* X, const void* scale, const void* gate,
                         float epsilon, void* Y, hipStream_t stream);

/* ------------------------------------------------------------------------
 * SkipGroupNorm ("com.microsoft.SkipGroupNorm": Description, Inputs,
 * Outputs, Attributes, Type constraints).
 *
 * X has logical shape (N, C, H, W), stored NHWC when channels_last != 0 and
 * NCHW when channels_last == 0 (any non-zero value selects NHWC).
 *   S = round_T((X + skip) + bias)        (bias term only if given)
 *   per (n, group g of C/groups channels), over all H*W positions:
 *     mean, var = population mean and variance of S
 *   Y = round_T(act(gamma[c] * (S - mean) / sqrt(var + epsilon) + beta[c]))
 *   act = identity (activation 0) or SiLU (activation 1).
 * Arguments:
 *   T              SN_F32 or SN_F16 for X, skip, bias, Y, S.
 *   M              SN_F32 or SN_F16 for gamma, beta (independent of T).
 *   N, H, W        >= 0.   C: >= 1.
 *   X              X's layout as above, T.
 *   gamma, beta    [C] M.
 *   skip           T; X's shape and layout when skip_broadcast == 0, else
 *                  [N, C] (one value per batch item and channel; the page's
 *                  (N, C) and (N, 1, 1, C) spellings).
 *   bias           [C] T or NULL.
 *   epsilon        >= 0 and finite (the page's default is 1e-5).
 *   groups         >= 1 and divides C.
 *   activation     0 or 1.
 *   Y              X's shape and layout, T.   S: same, or NULL.
 *   workspace      device memory of at least the size that
 *                  skip_group_norm_workspace_size returns for the same
 *                  arguments (may be NULL when that size is 0).  Its
 *                  contents on entry do not matter.  Calls that share a
 *                  workspace must be ordered (same stream).
 * The single-launch routes tell a call's exchanged partial moments from
 * earlier ones by a per-call value.  On a stream that is being captured into
 * a HIP graph (whose replays repeat every argument) the call records, ahead
 * of such a launch, a small kernel that clears those values in the
 * workspace, so that every replay is correct.
 * ------------------------------------------------------------------------ */
sn_status skip_group_norm_workspace_size(sn_dtype T, int64_t N, int64_t C,
                                         int64_t H, int64_t W, int64_t groups,
                                         int32_t channels_last, size_t* bytes);

sn_status skip_group_norm(sn_dtype T, sn_dtype M, int64_t N, int64_t C,
                          int64_t H, int64_t W,
                          const void* X, const void* gamma, const void* beta,
                          const void* skip, int32_t skip_broadcast,
                          const void* bias, float epsilon, int64_t groups,
                          int32_t channels_last, int32_t activation,
                          void* Y, void* S, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

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

sn_status skip_group_norm_noalloc(sn_dtype T, sn_dtype M, int64_t N, int64_t C,
                                  int64_t H, int64_t W,
                                  const void* X, const void* gamma, const void* beta,
                                  const void* skip, int32_t skip_broadcast,
                                  const void* bias, float epsilon, int64_t groups,
                                  int32_t channels_last, int32_t activation,
                                  void* Y, void* S, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Library information and test hooks.
 * ------------------------------------------------------------------------ */

/* Message for the calling thread's last non-OK status ("" if none).  The
 * string stays valid until that thread's next call into the library. */
const char* skipnorm_last_error(void);

/* SKIPNORM_ABI_VERSION of the built library. */
int skipnorm_abi_version(void);

/* Route selection for every later call in the process, so that tests can
 * cover each kernel family on the same shapes:
 *   0 = automatic (the default);
 *   1 = element-by-element accesses (vectors off);
 *   2 = vectorized where the preconditions hold (same as automatic, except
 *       that gated_rms_norm keeps one power-of-two lane group per row for
 *       every row length, where automatic packs rows that are not a power
 *       of two of vectors back to back);
 *   3 = skip_rms_norm / skip_layer_norm / gated_rms_norm: one workgroup per
 *       row, two passes, element by element;
 *       skip_group_norm: the three-launch split route with scalar accesses;
 *   4 = skip_group_norm: the three-launch split route (vectorized where the
 *       preconditions hold) even where a single-launch route would apply;
 *       others: automatic.
 *   5 = gated_rms_norm: the flat route (rows read as one stream of aligned
 *       16-byte vectors) wherever it applies -- rows of at most 1016
 *       (float16) or 1020 (float32) elements, X, gate and Y at one offset
 *       from a 16-byte boundary --
 *       where automatic takes it only for the row lengths it measured
 *       faster on; others: automatic.
 * Returns the previous value; an unknown value leaves the setting unchanged
 * and returns the current one. */
int skipnorm_force_route(int route);

/* SkipGroupNorm's single-launch routes spread each (n, group) over several
 * workgroups (NCHW: up to 8; NHWC: up to 64 pixel slices of an image) that
 * exchange partial moments; a workgroup waits at most this long for
 * another's moments and otherwise recomputes them itself with the same
 * arithmetic (results are identical either way).  Sets the wait for
 * later calls in the process (negative: the default, 100 us) and returns the
 * previous value.  A test hook: 0 forces every recomputation path. */
int skipnorm_set_exchange_timeout_us(int microseconds);

/* Name of the route the calling thread's last successful op call took
 * (e.g. "ssln.wave2.vec16", "ssln.segment.vec8", "gated.tile.vec8",
 * "sgn.cluster.nhwc.vec16", "sgn.split.nchw.scalar"). */
const char* skipnorm_last_route(void);

/* Measurement helper: copies `bytes` bytes from src to dst with one kernel
 * of 16-byte loads and stores (both 16-byte aligned, bytes a multiple of
 * 16).  Serves as the copy-bandwidth reference and as the calibration
 * kernel of known traffic for hardware counters. */
sn_status skipnorm_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SKIPNORM_H */
