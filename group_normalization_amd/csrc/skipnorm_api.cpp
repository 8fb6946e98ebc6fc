// skipnorm_api.cpp -- C-ABI front end of libskipnorm: validation of every
// tensor descriptor and attribute against the operators' contracts (host
// only, before anything is enqueued), route selection hooks, error
// reporting, and the calls into the kernel launchers.
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/skipnorm.h"
#include "../../include/skipnorm_testing.h"
#include "skipnorm_internal.h"

namespace {

thread_local std::string g_error;
thread_local const char* g_route = "";
std::atomic<int> g_force_route{0};

// Wall-clock ticks (100 MHz device clock) a SkipGroupNorm workgroup waits for
// another workgroup's published moments before recomputing them itself.
constexpr long long kDefaultExchangeTimeoutUs = 100;
std::atomic<long long> g_exchange_timeout_us{kDefaultExchangeTimeoutUs};

// Per-call publication tags: a process-unique 64-bit sequence, so tags left
// in a reused workspace by earlier calls (or other processes) never match.
uint64_t initial_tag() {
    const uint64_t now = uint64_t(std::chrono::steady_clock::now().time_since_epoch().count());
    uint64_t x = now ^ (uint64_t(reinterpret_cast<uintptr_t>(&g_force_route)) << 17);
    x ^= x >> 33;
    x *= 0xff51afd7ed558ccdULL;  // a 64-bit finalizer mix
    x ^= x >> 33;
    return x | 1;
}
std::atomic<uint64_t> g_tag{initial_tag()};

sn_status fail(sn_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return st;
}

sn_status ok() {
    g_error.clear();
    return SN_OK;
}

#define SN_TRY(expr)                     \
    do {                                 \
        sn_status st_ = (expr);          \
        if (st_ != SN_OK) return st_;    \
    } while (0)

constexpr int64_t kMaxRowElems = int64_t(1) << 30;   // hidden / span / image size
constexpr int64_t kMaxElems = int64_t(1) << 46;      // whole tensor
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1; // rows; blocks of one launch
static_assert(sn::kStaticScratchBytes == SKIPNORM_NOALLOC_SCRATCH_BYTES,
              "the header states the static scratch size");

size_t elem_size(sn_dtype t) { return t == SN_F32 ? 4 : 2; }
int kernel_dtype(sn_dtype t) { return t == SN_F32 ? 0 : 1; }

sn_status check_dtype(sn_dtype t, const char* op, const char* what) {
    if (t == SN_F32 || t == SN_F16) return SN_OK;
    if (t == SN_BF16) return fail(SN_ERR_DTYPE, "%s: %s: bfloat16 is not implemented", op, what);
    return fail(SN_ERR_DTYPE, "%s: %s: unknown dtype code %d", op, what, int(t));
}

sn_status check_epsilon(const char* op, float eps) {
    if (!std::isfinite(eps) || eps < 0.0f)
        return fail(SN_ERR_ATTR, "%s: epsilon must be finite and non-negative (got %g)", op,
                    double(eps));
    return SN_OK;
}

bool mul_overflows(int64_t a, int64_t b, int64_t* out) { return __builtin_mul_overflow(a, b, out); }

// ---------------------------------------------------------------- descriptors
// A descriptor read and checked for internal consistency: rank within
// 0..SN_MAX_RANK, every extent >= 0, element count without overflow.
struct Tensor {
    const char* name = "";
    bool present = false;
    void* data = nullptr;
    sn_dtype dtype = SN_F32;
    int rank = 0;
    int64_t shape[SN_MAX_RANK] = {};
    int64_t numel = 0;
};

template <typename D>
sn_status read_tensor(const char* op, const char* name, const D* d, bool required, Tensor* out) {
    out->name = name;
    if (!d) {
        if (required) return fail(SN_ERR_NULL, "%s: %s is required", op, name);
        return SN_OK;
    }
    out->present = true;
    out->data = const_cast<void*>(static_cast<const void*>(d->data));
    out->dtype = d->dtype;
    if (d->rank < 0 || d->rank > SN_MAX_RANK)
        return fail(SN_ERR_SHAPE, "%s: %s: rank %d outside 0..%d", op, name, int(d->rank), SN_MAX_RANK);
    out->rank = d->rank;
    int64_t n = 1;
    for (int i = 0; i < d->rank; ++i) {
        if (d->shape[i] < 0)
            return fail(SN_ERR_SHAPE, "%s: %s: negative extent %lld", op, name, (long long)d->shape[i]);
        out->shape[i] = d->shape[i];
        if (mul_overflows(n, d->shape[i], &n) || n > kMaxElems)
            return fail(SN_ERR_SHAPE, "%s: %s: more than 2^46 elements", op, name);
    }
    out->numel = n;
    return SN_OK;
}

std::string shape_str(const int64_t* shape, int rank) {
    std::string s = "(";
    for (int i = 0; i < rank; ++i) {
        if (i) s += ", ";
        s += std::to_string(shape[i]);
    }
    if (rank == 1) s += ",";
    return s + ")";
}
std::string shape_str(const Tensor& t) { return shape_str(t.shape, t.rank); }

bool same_shape(const Tensor& a, const int64_t* shape, int rank) {
    if (a.rank != rank) return false;
    for (int i = 0; i < rank; ++i)
        if (a.shape[i] != shape[i]) return false;
    return true;
}

// t (if present) has exactly this shape.
sn_status expect_shape(const char* op, const Tensor& t, const int64_t* shape, int rank,
                       const char* what) {
    if (!t.present || same_shape(t, shape, rank)) return SN_OK;
    return fail(SN_ERR_SHAPE, "%s: %s must have shape %s (%s), got %s", op, t.name,
                shape_str(shape, rank).c_str(), what, shape_str(t).c_str());
}

// t (if present) has element type `want`.
sn_status expect_dtype(const char* op, const Tensor& t, sn_dtype want, const char* what) {
    if (!t.present || t.dtype == want) return SN_OK;
    if (t.dtype != SN_F32 && t.dtype != SN_F16) SN_TRY(check_dtype(t.dtype, op, t.name));
    return fail(SN_ERR_DTYPE, "%s: %s must be %s (%s)", op, t.name,
                want == SN_F32 ? "float32" : "float16", what);
}

// Present tensors holding elements need a data pointer.
sn_status expect_data(const char* op, const Tensor& t) {
    if (t.present && t.numel > 0 && !t.data)
        return fail(SN_ERR_NULL, "%s: %s has %lld elements and a NULL data pointer", op, t.name,
                    (long long)t.numel);
    return SN_OK;
}

// A byte range of a tensor; empty when absent, NULL or without elements.
struct Span {
    const char* name;
    uintptr_t lo, hi;
    bool empty() const { return lo == hi; }
};

Span span_of(const char* name, const void* p, size_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Span{name, lo, p ? lo + bytes : lo};
}
Span span_of(const Tensor& t) {
    if (!t.present) return Span{t.name, 0, 0};
    return span_of(t.name, t.data, size_t(t.numel) * elem_size(t.dtype));
}

bool overlap(const Span& a, const Span& b) {
    return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi;
}

// Every output against every input and every other output.
sn_status check_alias(const Span* outs, int n_out, const Span* ins, int n_in) {
    for (int i = 0; i < n_out; ++i) {
        for (int j = 0; j < n_in; ++j)
            if (overlap(outs[i], ins[j]))
                return fail(SN_ERR_ALIAS, "output %s overlaps input %s", outs[i].name, ins[j].name);
        for (int j = i + 1; j < n_out; ++j)
            if (overlap(outs[i], outs[j]))
                return fail(SN_ERR_ALIAS, "output %s overlaps output %s", outs[i].name, outs[j].name);
    }
    return SN_OK;
}

sn::Route current_route() { return static_cast<sn::Route>(g_force_route.load(std::memory_order_relaxed)); }
// The flat route is the row norms'; SkipGroupNorm runs it as automatic.
sn::Route current_route_not_flat() {
    const sn::Route r = current_route();
    return r == sn::Route::Flat ? sn::Route::Auto : r;
}

sn_status finish_launch(hipError_t err, const char* route, const char* op) {
    if (err != hipSuccess)
        return fail(SN_ERR_HIP, "%s: launch failed: %s", op, hipGetErrorString(err));
    g_route = route;
    return ok();
}

// ---------------------------------------------------------------- row norms
// SkipSimplifiedLayerNormalization and its mean-removing form share
// validation and kernels; `center` removes the row mean (skip_layer_norm).
sn_status row_norm(const char* op, bool center, const sn_tensor_in* input_d,
                   const sn_tensor_in* skip_d, const sn_tensor_in* gamma_d,
                   const sn_tensor_in* beta_d, const sn_tensor_in* bias_d, float epsilon,
                   const sn_tensor_out* output_d, const sn_tensor_out* mean_d,
                   const sn_tensor_out* inv_d, const sn_tensor_out* sum_d, hipStream_t stream) {
    Tensor input, skip, gamma, beta, bias, output, mean, inv, sum;
    SN_TRY(read_tensor(op, "input", input_d, true, &input));
    SN_TRY(read_tensor(op, "skip", skip_d, true, &skip));
    SN_TRY(read_tensor(op, "gamma", gamma_d, true, &gamma));
    SN_TRY(read_tensor(op, "beta", beta_d, false, &beta));
    SN_TRY(read_tensor(op, "bias", bias_d, false, &bias));
    SN_TRY(read_tensor(op, "output", output_d, true, &output));
    SN_TRY(read_tensor(op, "mean", mean_d, false, &mean));
    SN_TRY(read_tensor(op, "inv_std_var", inv_d, false, &inv));
    SN_TRY(read_tensor(op, "input_skip_bias_sum", sum_d, false, &sum));

    // Element types: one T for every tensor but the statistics (float32).
    const sn_dtype T = input.dtype;
    SN_TRY(check_dtype(T, op, "input"));
    for (const Tensor* t : {&skip, &gamma, &beta, &bias, &output, &sum})
        SN_TRY(expect_dtype(op, *t, T, "the input's type"));
    for (const Tensor* t : {&mean, &inv}) SN_TRY(expect_dtype(op, *t, SN_F32, "statistics"));

    // Shapes: input (token_count, hidden) or (batch, sequence, hidden).
    if (input.rank != 2 && input.rank != 3)
        return fail(SN_ERR_SHAPE,
                    "%s: input must have rank 2 (token_count, hidden) or 3 (batch, sequence, hidden), "
                    "got %s", op, shape_str(input).c_str());
    const int64_t hidden = input.shape[input.rank - 1];
    if (hidden < 1 || hidden > kMaxRowElems)
        return fail(SN_ERR_SHAPE, "%s: hidden (the last extent) must be in 1..2^30, got %lld", op,
                    (long long)hidden);
    const int64_t rows = input.numel / hidden;
    if (rows > kMaxRows) return fail(SN_ERR_SHAPE, "%s: more than 2^31 - 1 rows", op);
    int64_t stat_shape[SN_MAX_RANK];
    for (int i = 0; i < input.rank; ++i) stat_shape[i] = input.shape[i];
    stat_shape[input.rank - 1] = 1;
    SN_TRY(expect_shape(op, skip, input.shape, input.rank, "the input's shape"));
    for (const Tensor* t : {&gamma, &beta, &bias}) SN_TRY(expect_shape(op, *t, &hidden, 1, "hidden"));
    for (const Tensor* t : {&output, &sum})
        SN_TRY(expect_shape(op, *t, input.shape, input.rank, "the input's shape"));
    for (const Tensor* t : {&mean, &inv})
        SN_TRY(expect_shape(op, *t, stat_shape, input.rank, "the input's shape, last extent 1"));

    SN_TRY(check_epsilon(op, epsilon));
    for (const Tensor* t : {&input, &skip, &gamma, &beta, &bias, &output, &mean, &inv, &sum})
        SN_TRY(expect_data(op, *t));

    const Span ins[] = {span_of(input), span_of(skip), span_of(gamma), span_of(bias), span_of(beta)};
    const Span outs[] = {span_of(output), span_of(mean), span_of(inv), span_of(sum)};
    SN_TRY(check_alias(outs, 4, ins, 5));

    sn::SslnArgs a{kernel_dtype(T), rows, hidden, input.data, skip.data, gamma.data,
                   beta.present ? beta.data : nullptr, bias.present ? bias.data : nullptr, epsilon,
                   output.data, static_cast<float*>(mean.present ? mean.data : nullptr),
                   static_cast<float*>(inv.present ? inv.data : nullptr),
                   sum.present ? sum.data : nullptr, center};
    const char* route = "";
    return finish_launch(sn::launch_ssln(a, current_route(), stream, &route), route, op);
}

// ---------------------------------------------------------------- SkipGroupNorm
sn_status check_sgn_geometry(const char* op, sn_dtype T, int64_t N, int64_t C, int64_t H,
                             int64_t W, int64_t groups) {
    if (C < 1) return fail(SN_ERR_SHAPE, "%s: X must have C >= 1 channels", op);
    int64_t hw, image;
    if (mul_overflows(H, W, &hw) || mul_overflows(hw, C, &image) || image > kMaxRowElems)
        return fail(SN_ERR_SHAPE, "%s: C * H * W must not exceed 2^30", op);
    if (groups < 1 || C % groups != 0)
        return fail(SN_ERR_ATTR, "%s: groups (%lld) must be >= 1 and divide C (%lld)", op,
                    (long long)groups, (long long)C);
    // Launch grids: N * groups * B blocks, B blocks per (n, group) partial row.
    const int64_t B = sn::sgn_partials_per_group(kernel_dtype(T), N, C, H, W, groups, true);
    const int64_t B2 = sn::sgn_partials_per_group(kernel_dtype(T), N, C, H, W, groups, false);
    int64_t blocks;
    if (mul_overflows(N * groups, B > B2 ? B : B2, &blocks) || blocks > kMaxRows)
        return fail(SN_ERR_SHAPE, "%s: too many (n, group) pairs for one launch", op);
    return SN_OK;
}

// X's logical (N, C, H, W) from its rank-4 shape and layout.
struct Nchw {
    int64_t N, C, H, W;
};
sn_status sgn_dims(const char* op, const Tensor& X, int32_t channels_last, Nchw* d) {
    if (X.rank != 4)
        return fail(SN_ERR_SHAPE, "%s: X must have rank 4 (%s), got %s", op,
                    channels_last ? "N, H, W, C" : "N, C, H, W", shape_str(X).c_str());
    d->N = X.shape[0];
    if (channels_last) {
        d->H = X.shape[1];
        d->W = X.shape[2];
        d->C = X.shape[3];
    } else {
        d->C = X.shape[1];
        d->H = X.shape[2];
        d->W = X.shape[3];
    }
    return SN_OK;
}

// skip_group_norm with the caller's workspace, or (noalloc) with the
// library's static scratch on the current device.
sn_status group_norm(const char* op, const sn_tensor_in* X_d, const sn_tensor_in* gamma_d,
                     const sn_tensor_in* beta_d, const sn_tensor_in* skip_d,
                     const sn_tensor_in* bias_d, float epsilon, int64_t groups,
                     int32_t channels_last, int32_t activation, const sn_tensor_out* Y_d,
                     const sn_tensor_out* S_d, void* workspace, size_t workspace_bytes,
                     bool noalloc, hipStream_t stream) {
    Tensor X, gamma, beta, skip, bias, Y, S;
    SN_TRY(read_tensor(op, "X", X_d, true, &X));
    SN_TRY(read_tensor(op, "gamma", gamma_d, true, &gamma));
    SN_TRY(read_tensor(op, "beta", beta_d, true, &beta));
    SN_TRY(read_tensor(op, "skip", skip_d, true, &skip));
    SN_TRY(read_tensor(op, "bias", bias_d, false, &bias));
    SN_TRY(read_tensor(op, "Y", Y_d, true, &Y));
    SN_TRY(read_tensor(op, "S", S_d, false, &S));

    // Element types: T for X, skip, bias, Y, S; M for gamma and beta.
    const sn_dtype T = X.dtype, M = gamma.dtype;
    SN_TRY(check_dtype(T, op, "X"));
    SN_TRY(check_dtype(M, op, "gamma"));
    for (const Tensor* t : {&skip, &bias, &Y, &S}) SN_TRY(expect_dtype(op, *t, T, "X's type"));
    SN_TRY(expect_dtype(op, beta, M, "gamma's type"));

    // Shapes.
    Nchw d;
    SN_TRY(sgn_dims(op, X, channels_last, &d));
    SN_TRY(check_sgn_geometry(op, T, d.N, d.C, d.H, d.W, groups));
    for (const Tensor* t : {&gamma, &beta, &bias}) SN_TRY(expect_shape(op, *t, &d.C, 1, "C"));
    for (const Tensor* t : {&Y, &S}) SN_TRY(expect_shape(op, *t, X.shape, 4, "X's shape"));
    // skip: X's exact shape first, then the broadcast spellings (N, C) and
    // (N, 1, 1, C).
    bool broadcast = false;
    if (!same_shape(skip, X.shape, 4)) {
        const int64_t nc[2] = {d.N, d.C}, n11c[4] = {d.N, 1, 1, d.C};
        if (!same_shape(skip, nc, 2) && !same_shape(skip, n11c, 4))
            return fail(SN_ERR_SHAPE, "%s: skip must have X's shape %s, or %s or %s; got %s", op,
                        shape_str(X).c_str(), shape_str(nc, 2).c_str(), shape_str(n11c, 4).c_str(),
                        shape_str(skip).c_str());
        broadcast = true;
    }

    SN_TRY(check_epsilon(op, epsilon));
    if (activation != 0 && activation != 1)
        return fail(SN_ERR_ATTR, "%s: activation must be 0 (none) or 1 (SiLU), got %d", op,
                    int(activation));
    for (const Tensor* t : {&X, &gamma, &beta, &skip, &bias, &Y, &S}) SN_TRY(expect_data(op, *t));

    const int64_t numel = X.numel;
    size_t need = 0;
    if (numel > 0)
        need = sn::sgn_workspace_bytes(kernel_dtype(T), d.N, d.C, d.H, d.W, groups, channels_last != 0);
    size_t trace_at = 0;  // offset of the phase-timestamp area (measurement builds)
#ifdef SN_PHASE_TRACE
    if (need > 0 && !noalloc) {
        trace_at = (need + 255) / 256 * 256;
        need = trace_at + sn::kTraceBytes;
    }
#endif
    if (noalloc) {
        if (need > sn::kStaticScratchBytes)
            return fail(SN_ERR_WORKSPACE,
                        "%s: this shape needs %zu bytes of scratch; the static scratch holds %zu "
                        "(use skip_group_norm with a workspace)",
                        op, need, size_t(sn::kStaticScratchBytes));
        workspace = nullptr;  // looked up after validation
        workspace_bytes = 0;
    } else {
        if (need > 0 && (!workspace || workspace_bytes < need))
            return fail(SN_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got %zu%s", op,
                        need, workspace_bytes, workspace ? "" : " (NULL)");
        if (need > 0 && !sn::aligned16(workspace))
            return fail(SN_ERR_WORKSPACE, "%s: workspace must be 16-byte aligned", op);
    }

    const Span ins[] = {span_of(X), span_of(skip), span_of(bias), span_of(gamma), span_of(beta)};
    const Span outs[] = {span_of(Y), span_of(S), span_of("workspace", workspace, need)};
    SN_TRY(check_alias(outs, 3, ins, 5));
    if (noalloc && need > 0) {
        if (hipError_t e = sn::static_scratch(&workspace); e != hipSuccess)
            return fail(SN_ERR_HIP, "%s: static scratch lookup failed: %s", op, hipGetErrorString(e));
        workspace_bytes = sn::kStaticScratchBytes;
    }

    sn::SgnArgs a;
    a.dtype = kernel_dtype(T);
    a.param_dtype = kernel_dtype(M);
    a.N = d.N;
    a.C = d.C;
    a.H = d.H;
    a.W = d.W;
    a.groups = groups;
    a.channels_last = channels_last != 0;
    a.activation = activation;
    a.X = X.data;
    a.gamma = gamma.data;
    a.beta = beta.data;
    a.skip = skip.data;
    a.bias = bias.present ? bias.data : nullptr;
    a.skip_broadcast = broadcast;
    a.epsilon = epsilon;
    a.Y = Y.data;
    a.S = S.present ? S.data : nullptr;
    a.workspace = workspace;
    a.trace = trace_at ? reinterpret_cast<unsigned long long*>(static_cast<char*>(workspace) + trace_at)
                       : nullptr;
    a.tag = g_tag.fetch_add(2) | 1;  // odd, never 0
    a.exchange_timeout_ticks = g_exchange_timeout_us.load() * 100;
    // A captured graph replays its kernels with the arguments of the
    // capture, so a per-call tag would repeat on every replay and a
    // workgroup could take the moments a slice left in the previous replay.
    // Under capture the cluster routes' publication slots are zeroed by a
    // kernel ahead of each cluster launch instead, and the tag is a
    // constant: only this launch's publications can carry it.
    a.clear_tags = false;
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &capture) == hipSuccess && capture != hipStreamCaptureStatusNone) {
        a.clear_tags = true;
        a.tag = 1;
    }
    const char* route = "";
    return finish_launch(sn::launch_sgn(a, current_route_not_flat(), stream, &route), route, op);
}

}  // namespace

extern "C" {

sn_status skip_rms_norm(const sn_tensor_in* input, const sn_tensor_in* skip,
                        const sn_tensor_in* gamma, const sn_tensor_in* bias, float epsilon,
                        const sn_tensor_out* output, const sn_tensor_out* mean,
                        const sn_tensor_out* inv_std_var,
                        const sn_tensor_out* input_skip_bias_sum, hipStream_t stream) {
    return row_norm("skip_rms_norm", false, input, skip, gamma, nullptr, bias, epsilon, output,
                    mean, inv_std_var, input_skip_bias_sum, stream);
}

sn_status skip_layer_norm(const sn_tensor_in* input, const sn_tensor_in* skip,
                          const sn_tensor_in* gamma, const sn_tensor_in* beta,
                          const sn_tensor_in* bias, float epsilon, const sn_tensor_out* output,
                          const sn_tensor_out* mean, const sn_tensor_out* inv_std_var,
                          const sn_tensor_out* input_skip_bias_sum, hipStream_t stream) {
    return row_norm("skip_layer_norm", true, input, skip, gamma, beta, bias, epsilon, output, mean,
                    inv_std_var, input_skip_bias_sum, stream);
}

sn_status gated_rms_norm(const sn_tensor_in* X_d, const sn_tensor_in* scale_d,
                         const sn_tensor_in* gate_d, float epsilon, const sn_tensor_out* Y_d,
                         hipStream_t stream) {
    const char* op = "gated_rms_norm";
    Tensor X, scale, gate, Y;
    SN_TRY(read_tensor(op, "X", X_d, true, &X));
    SN_TRY(read_tensor(op, "scale", scale_d, true, &scale));
    SN_TRY(read_tensor(op, "gate", gate_d, true, &gate));
    SN_TRY(read_tensor(op, "Y", Y_d, true, &Y));

    const sn_dtype T = X.dtype;
    SN_TRY(check_dtype(T, op, "X"));
    for (const Tensor* t : {&scale, &gate, &Y}) SN_TRY(expect_dtype(op, *t, T, "X's type"));

    if (X.rank < 1) return fail(SN_ERR_SHAPE, "%s: X must have rank >= 1", op);
    // scale: a vector in any spelling -- at most one extent differs from 1.
    int non_unit = 0;
    for (int i = 0; i < scale.rank; ++i) non_unit += scale.shape[i] != 1;
    if (scale.rank < 1 || non_unit > 1)
        return fail(SN_ERR_SHAPE, "%s: scale must be a vector ((C), (1, C), (C, 1), ...), got %s", op,
                    shape_str(scale).c_str());
    const int64_t span = scale.numel;
    if (span < 1 || span > kMaxRowElems)
        return fail(SN_ERR_SHAPE, "%s: the span C = numel(scale) must be in 1..2^30, got %lld", op,
                    (long long)span);
    if (X.numel % span != 0)
        return fail(SN_ERR_SHAPE, "%s: numel(X) = %lld is not a multiple of the span C = %lld", op,
                    (long long)X.numel, (long long)span);
    if (X.numel / span > kMaxRows) return fail(SN_ERR_SHAPE, "%s: more than 2^31 - 1 rows", op);
    SN_TRY(expect_shape(op, gate, X.shape, X.rank, "X's shape"));
    SN_TRY(expect_shape(op, Y, X.shape, X.rank, "X's shape"));

    SN_TRY(check_epsilon(op, epsilon));
    for (const Tensor* t : {&X, &scale, &gate, &Y}) SN_TRY(expect_data(op, *t));

    const Span ins[] = {span_of(X), span_of(gate), span_of(scale)};
    const Span outs[] = {span_of(Y)};
    SN_TRY(check_alias(outs, 1, ins, 3));

    sn::GatedArgs a{kernel_dtype(T), X.numel / span, span, X.data, scale.data, gate.data, epsilon, Y.data};
    const char* route = "";
    return finish_launch(sn::launch_gated(a, current_route(), stream, &route), route, op);
}

sn_status skip_group_norm_workspace_size(const sn_tensor_in* X_d, int64_t groups,
                                         int32_t channels_last, size_t* bytes) {
    const char* op = "skip_group_norm_workspace_size";
    if (!bytes) return fail(SN_ERR_NULL, "%s: bytes is NULL", op);
    Tensor X;
    SN_TRY(read_tensor(op, "X", X_d, true, &X));
    SN_TRY(check_dtype(X.dtype, op, "X"));
    Nchw d;
    SN_TRY(sgn_dims(op, X, channels_last, &d));
    SN_TRY(check_sgn_geometry(op, X.dtype, d.N, d.C, d.H, d.W, groups));
    *bytes = X.numel == 0 ? 0
                          : sn::sgn_workspace_bytes(kernel_dtype(X.dtype), d.N, d.C, d.H, d.W, groups,
                                                    channels_last != 0);
#ifdef SN_PHASE_TRACE
    if (*bytes > 0) *bytes = (*bytes + 255) / 256 * 256 + sn::kTraceBytes;
#endif
    return ok();
}

sn_status skip_group_norm(const sn_tensor_in* X, const sn_tensor_in* gamma,
                          const sn_tensor_in* beta, const sn_tensor_in* skip,
                          const sn_tensor_in* bias, float epsilon, int64_t groups,
                          int32_t channels_last, int32_t activation, const sn_tensor_out* Y,
                          const sn_tensor_out* S, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
    return group_norm("skip_group_norm", X, gamma, beta, skip, bias, epsilon, groups,
                      channels_last, activation, Y, S, workspace, workspace_bytes, false, stream);
}

sn_status skip_group_norm_noalloc(const sn_tensor_in* X, const sn_tensor_in* gamma,
                                  const sn_tensor_in* beta, const sn_tensor_in* skip,
                                  const sn_tensor_in* bias, float epsilon, int64_t groups,
                                  int32_t channels_last, int32_t activation,
                                  const sn_tensor_out* Y, const sn_tensor_out* S,
                                  hipStream_t stream) {
    return group_norm("skip_group_norm_noalloc", X, gamma, beta, skip, bias, epsilon, groups,
                      channels_last, activation, Y, S, nullptr, 0, true, stream);
}

const char* skipnorm_last_error(void) { return g_error.c_str(); }

int skipnorm_abi_version(void) { return SKIPNORM_ABI_VERSION; }

int skipnorm_force_route(int route) {
    if (route < 0 || route > 5) return g_force_route.load();
    return g_force_route.exchange(route);
}

const char* skipnorm_last_route(void) { return g_route; }

int skipnorm_set_exchange_timeout_us(int microseconds) {
    const long long prev = g_exchange_timeout_us.load();
    g_exchange_timeout_us.store(microseconds < 0 ? kDefaultExchangeTimeoutUs : microseconds);
    return int(prev);
}

sn_status skipnorm_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
    if (bytes == 0) return ok();
    if (!src || !dst) return fail(SN_ERR_NULL, "skipnorm_copy: NULL pointer");
    if (bytes > (size_t(1) << 40))
        return fail(SN_ERR_SHAPE, "skipnorm_copy: at most 2^40 bytes per call");
    if (!sn::aligned16(src) || !sn::aligned16(dst) || bytes % 16 != 0)
        return fail(SN_ERR_SHAPE, "skipnorm_copy: pointers and size must be multiples of 16 bytes");
    const Span ins[] = {span_of("src", src, bytes)};
    const Span outs[] = {span_of("dst", dst, bytes)};
    SN_TRY(check_alias(outs, 1, ins, 1));
    return finish_launch(sn::launch_copy(src, dst, bytes, stream), "copy.vec16", "skipnorm_copy");
}

}  // extern "C"
