// skipnorm_api.cpp -- C-ABI front end of libskipnorm: argument validation
// (host only, before anything is enqueued), route selection hooks, error
// reporting, and the calls into the kernel launchers.
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/skipnorm.h"
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

size_t elem_size(sn_dtype t) { return t == SN_F32 ? 4 : 2; }

sn_status check_dtype(sn_dtype t, const char* what) {
    if (t == SN_F32 || t == SN_F16) return SN_OK;
    if (t == SN_BF16) return fail(SN_ERR_DTYPE, "%s: bfloat16 is not implemented", what);
    return fail(SN_ERR_DTYPE, "%s: unknown dtype code %d", what, int(t));
}

sn_status check_epsilon(float eps) {
    if (!std::isfinite(eps) || eps < 0.0f)
        return fail(SN_ERR_ATTR, "epsilon must be finite and non-negative (got %g)", double(eps));
    return SN_OK;
}

// A byte range of a tensor; empty when the pointer is NULL or size is 0.
struct Span {
    const char* name;
    uintptr_t lo, hi;
    bool empty() const { return lo == hi; }
};

Span span_of(const char* name, const void* p, size_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Span{name, lo, p ? lo + bytes : lo};
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

bool mul_overflows(int64_t a, int64_t b, int64_t* out) { return __builtin_mul_overflow(a, b, out); }

sn::Route current_route() { return static_cast<sn::Route>(g_force_route.load(std::memory_order_relaxed)); }
// The flat route is GatedRMSNorm's; the other operators run it as automatic.
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

}  // namespace

namespace {

// Both row normalizations share validation and kernels; `center` removes the
// row mean (skip_layer_norm).
sn_status row_norm(const char* op, bool center, sn_dtype T, int64_t rows, int64_t hidden,
                   const void* input, const void* skip, const void* gamma, const void* beta,
                   const void* bias, float epsilon, void* output, float* mean,
                   float* inv_std_var, void* input_skip_bias_sum, hipStream_t stream) {
    SN_TRY(check_dtype(T, op));
    if (rows < 0 || hidden < 1 || hidden > kMaxRowElems)
        return fail(SN_ERR_SHAPE, "%s: need rows >= 0 and 1 <= hidden <= 2^30 (got %lld, %lld)", op,
                    (long long)rows, (long long)hidden);
    int64_t numel;
    if (mul_overflows(rows, hidden, &numel) || numel > kMaxElems || rows > kMaxRows)
        return fail(SN_ERR_SHAPE, "%s: rows * hidden too large (rows < 2^31, elements <= 2^46)", op);
    SN_TRY(check_epsilon(epsilon));
    if (!gamma) return fail(SN_ERR_NULL, "%s: gamma is required", op);
    if (numel > 0 && (!input || !skip || !output))
        return fail(SN_ERR_NULL, "%s: input, skip and output are required", op);

    const size_t es = elem_size(T);
    const size_t tb = size_t(numel) * es;
    const Span ins[] = {span_of("input", input, tb), span_of("skip", skip, tb),
                        span_of("gamma", gamma, size_t(hidden) * es),
                        span_of("bias", bias, size_t(hidden) * es),
                        span_of("beta", beta, size_t(hidden) * es)};
    const Span outs[] = {span_of("output", output, tb),
                         span_of("mean", mean, size_t(rows) * 4),
                         span_of("inv_std_var", inv_std_var, size_t(rows) * 4),
                         span_of("input_skip_bias_sum", input_skip_bias_sum, tb)};
    SN_TRY(check_alias(outs, 4, ins, 5));

    sn::SslnArgs a{T == SN_F32 ? 0 : 1, rows, hidden, input, skip, gamma, beta, bias, epsilon,
                   output, mean, inv_std_var, input_skip_bias_sum, center};
    const char* route = "";
    return finish_launch(sn::launch_ssln(a, current_route_not_flat(), stream, &route), route, op);
}

}  // namespace

extern "C" {

sn_status skip_rms_norm(sn_dtype T, int64_t rows, int64_t hidden, const void* input,
                        const void* skip, const void* gamma, const void* bias, float epsilon,
                        void* output, float* mean, float* inv_std_var,
                        void* input_skip_bias_sum, hipStream_t stream) {
    return row_norm("skip_rms_norm", false, T, rows, hidden, input, skip, gamma, nullptr, bias,
                    epsilon, output, mean, inv_std_var, input_skip_bias_sum, stream);
}

sn_status skip_layer_norm(sn_dtype T, int64_t rows, int64_t hidden, const void* input,
                          const void* skip, const void* gamma, const void* beta, const void* bias,
                          float epsilon, void* output, float* mean, float* inv_std_var,
                          void* input_skip_bias_sum, hipStream_t stream) {
    return row_norm("skip_layer_norm", true, T, rows, hidden, input, skip, gamma, beta, bias,
                    epsilon, output, mean, inv_std_var, input_skip_bias_sum, stream);
}

sn_status gated_rms_norm(sn_dtype T, int64_t numel, int64_t span, const void* X,
                         const void* scale, const void* gate, float epsilon, void* Y,
                         hipStream_t stream) {
    SN_TRY(check_dtype(T, "gated_rms_norm T"));
    if (numel < 0 || span < 1 || span > kMaxRowElems || numel > kMaxElems)
        return fail(SN_ERR_SHAPE, "gated_rms_norm: need numel >= 0 and 1 <= span <= 2^30 (got %lld, %lld)",
                    (long long)numel, (long long)span);
    if (numel / span > kMaxRows)
        return fail(SN_ERR_SHAPE, "gated_rms_norm: more than 2^31 - 1 rows");
    if (numel % span != 0)
        return fail(SN_ERR_SHAPE,
                    "gated_rms_norm: element count %lld is not a multiple of the span C = %lld",
                    (long long)numel, (long long)span);
    SN_TRY(check_epsilon(epsilon));
    if (!scale) return fail(SN_ERR_NULL, "gated_rms_norm: scale is required");
    if (numel > 0 && (!X || !gate || !Y))
        return fail(SN_ERR_NULL, "gated_rms_norm: X, gate and Y are required");

    const size_t es = elem_size(T);
    const size_t tb = size_t(numel) * es;
    const Span ins[] = {span_of("X", X, tb), span_of("gate", gate, tb),
                        span_of("scale", scale, size_t(span) * es)};
    const Span outs[] = {span_of("Y", Y, tb)};
    SN_TRY(check_alias(outs, 1, ins, 3));

    sn::GatedArgs a{T == SN_F32 ? 0 : 1, numel / span, span, X, scale, gate, epsilon, Y};
    const char* route = "";
    return finish_launch(sn::launch_gated(a, current_route(), stream, &route), route, "gated_rms_norm");
}

namespace {

sn_status check_sgn_geometry(sn_dtype T, int64_t N, int64_t C, int64_t H, int64_t W,
                             int64_t groups) {
    SN_TRY(check_dtype(T, "skip_group_norm T"));
    if (N < 0 || H < 0 || W < 0 || C < 1)
        return fail(SN_ERR_SHAPE, "skip_group_norm: need N, H, W >= 0 and C >= 1");
    int64_t hw, image;
    if (mul_overflows(H, W, &hw) || mul_overflows(hw, C, &image) || image > kMaxRowElems)
        return fail(SN_ERR_SHAPE, "skip_group_norm: C * H * W must not exceed 2^30");
    int64_t numel;
    if (mul_overflows(image, N, &numel) || numel > kMaxElems)
        return fail(SN_ERR_SHAPE, "skip_group_norm: tensor too large");
    if (groups < 1 || C % groups != 0)
        return fail(SN_ERR_ATTR, "skip_group_norm: groups (%lld) must be >= 1 and divide C (%lld)",
                    (long long)groups, (long long)C);
    // Launch grids: N * groups * B blocks, B blocks per (n, group) partial row.
    const int64_t B = sn::sgn_partials_per_group(T == SN_F32 ? 0 : 1, N, C, H, W, groups, true);
    const int64_t B2 = sn::sgn_partials_per_group(T == SN_F32 ? 0 : 1, N, C, H, W, groups, false);
    int64_t blocks;
    if (mul_overflows(N * groups, B > B2 ? B : B2, &blocks) || blocks > kMaxRows)
        return fail(SN_ERR_SHAPE, "skip_group_norm: too many (n, group) pairs for one launch");
    return SN_OK;
}

}  // namespace

sn_status skip_group_norm_workspace_size(sn_dtype T, int64_t N, int64_t C, int64_t H, int64_t W,
                                         int64_t groups, int32_t channels_last, size_t* bytes) {
    if (!bytes) return fail(SN_ERR_NULL, "skip_group_norm_workspace_size: bytes is NULL");
    SN_TRY(check_sgn_geometry(T, N, C, H, W, groups));
    *bytes = (N == 0 || H * W == 0)
                 ? 0
                 : sn::sgn_workspace_bytes(T == SN_F32 ? 0 : 1, N, C, H, W, groups, channels_last != 0);
    return ok();
}

}  // extern "C"

namespace {

// skip_group_norm with the caller's workspace, or (noalloc) with the
// library's static scratch on the current device.
sn_status group_norm(const char* op, sn_dtype T, sn_dtype M, int64_t N, int64_t C, int64_t H,
                     int64_t W, const void* X, const void* gamma, const void* beta,
                     const void* skip, int32_t skip_broadcast, const void* bias, float epsilon,
                     int64_t groups, int32_t channels_last, int32_t activation, void* Y, void* S,
                     void* workspace, size_t workspace_bytes, bool noalloc, hipStream_t stream) {
    SN_TRY(check_sgn_geometry(T, N, C, H, W, groups));
    SN_TRY(check_dtype(M, "skip_group_norm M (gamma/beta)"));
    SN_TRY(check_epsilon(epsilon));
    if (activation != 0 && activation != 1)
        return fail(SN_ERR_ATTR, "skip_group_norm: activation must be 0 (none) or 1 (SiLU), got %d",
                    int(activation));
    const int64_t numel = N * C * H * W;
    if (!gamma || !beta) return fail(SN_ERR_NULL, "skip_group_norm: gamma and beta are required");
    if (numel > 0 && (!X || !skip || !Y))
        return fail(SN_ERR_NULL, "skip_group_norm: X, skip and Y are required");
    size_t need = 0;
    if (numel > 0)
        need = sn::sgn_workspace_bytes(T == SN_F32 ? 0 : 1, N, C, H, W, groups, channels_last != 0);
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

    const size_t es = elem_size(T), ms = elem_size(M);
    const size_t tb = size_t(numel) * es;
    const size_t skip_bytes = skip_broadcast ? size_t(N * C) * es : tb;
    const Span ins[] = {span_of("X", X, tb), span_of("skip", skip, skip_bytes),
                        span_of("bias", bias, size_t(C) * es),
                        span_of("gamma", gamma, size_t(C) * ms), span_of("beta", beta, size_t(C) * ms)};
    const Span outs[] = {span_of("Y", Y, tb), span_of("S", S, tb),
                         span_of("workspace", workspace, need)};
    SN_TRY(check_alias(outs, 3, ins, 5));
    if (noalloc && need > 0) {
        if (hipError_t e = sn::static_scratch(&workspace); e != hipSuccess)
            return fail(SN_ERR_HIP, "%s: static scratch lookup failed: %s", op, hipGetErrorString(e));
        workspace_bytes = sn::kStaticScratchBytes;
    }

    sn::SgnArgs a;
    a.dtype = T == SN_F32 ? 0 : 1;
    a.param_dtype = M == SN_F32 ? 0 : 1;
    a.N = N;
    a.C = C;
    a.H = H;
    a.W = W;
    a.groups = groups;
    a.channels_last = channels_last != 0;
    a.activation = activation;
    a.X = X;
    a.gamma = gamma;
    a.beta = beta;
    a.skip = skip;
    a.bias = bias;
    a.skip_broadcast = skip_broadcast != 0;
    a.epsilon = epsilon;
    a.Y = Y;
    a.S = S;
    a.workspace = workspace;
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

sn_status skip_group_norm(sn_dtype T, sn_dtype M, int64_t N, int64_t C, int64_t H, int64_t W,
                          const void* X, const void* gamma, const void* beta, const void* skip,
                          int32_t skip_broadcast, const void* bias, float epsilon, int64_t groups,
                          int32_t channels_last, int32_t activation, void* Y, void* S,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return group_norm("skip_group_norm", T, M, N, C, H, W, X, gamma, beta, skip, skip_broadcast,
                      bias, epsilon, groups, channels_last, activation, Y, S, workspace,
                      workspace_bytes, false, stream);
}

sn_status skip_group_norm_noalloc(sn_dtype T, sn_dtype M, int64_t N, int64_t C, int64_t H,
                                  int64_t W, const void* X, const void* gamma, const void* beta,
                                  const void* skip, int32_t skip_broadcast, const void* bias,
                                  float epsilon, int64_t groups, int32_t channels_last,
                                  int32_t activation, void* Y, void* S, hipStream_t stream) {
    return group_norm("skip_group_norm_noalloc", T, M, N, C, H, W, X, gamma, beta, skip,
                      skip_broadcast, bias, epsilon, groups, channels_last, activation, Y, S,
                      nullptr, 0, true, stream);
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
