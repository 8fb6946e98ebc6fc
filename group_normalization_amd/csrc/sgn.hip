// sgn.hip -- SkipGroupNorm kernels for gfx950.
//
// Operator ("com.microsoft.SkipGroupNorm", Description, Inputs, Attributes):
// S = X + skip (+ bias) rounded to T; per (n, group of C/groups channels)
// over all H*W positions the mean and population variance of S;
// Y = act(gamma_c * (S - mean) / sqrt(var + epsilon) + beta_c), act = none or
// SiLU; optional output S.  gamma/beta have their own type M.
//
// Split route, three launches on one stream (the pages' "partial group
// statistics / combine / normalize" structure, re-tiled for 256 CUs):
//   1. statistics: every block forms S over its tile, stores S if requested,
//      and writes one partial (count, mean, M2) per (n, group) it covers;
//   2. finalize: one block per (n, group) combines the partials in a fixed
//      order into (mean, 1/sqrt(var + epsilon));
//   3. normalize: re-reads S (or re-forms it from X, skip and bias, bit for
//      bit the same) and writes Y.
// Tilings:
//   nhwc   (NHWC, C a whole number of 16-byte vectors, at most 256 of them):
//          a block covers a run of pixels of one image and all channels.
//          Thread t owns channel vector t % Cv at pixels t / Cv + k * P,
//          P = 256 / Cv, so its channels (and their bias, gamma, beta and
//          group) never change.  Per-channel moments are merged into groups
//          through LDS.
//   group  (NCHW, H*W a whole number of vectors; and the scalar route of
//          both layouts): a block covers a contiguous slice of one
//          (n, group)'s elements; NCHW groups are contiguous in memory.
// Moments: each thread uses the shifted-data sums (shift = its first value)
// and all combinations use the pairwise (Chan et al.) update, in a fixed
// order, so results are deterministic and a constant group has variance 0.
#include "device_common.h"
#include "skipnorm_internal.h"

namespace sn {
namespace {

constexpr int kUnroll = 4;

struct alignas(16) Partial {
    float n, mean, m2, pad;
};

__device__ __forceinline__ Moments as_moments(const Partial& p) { return Moments{p.n, p.mean, p.m2}; }

// Fixed-order tree over the 256 threads of a block; thread 0 gets the result.
__device__ Moments block_merge(Moments m, Moments* sh) {
    const int t = threadIdx.x;
    sh[t] = m;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (t < s) sh[t] = merge(sh[t], sh[t + s]);
        __syncthreads();
    }
    return sh[0];
}

template <typename T, int E>
__device__ __forceinline__ void load_param_vec(const T* p, int64_t vi, float (&out)[E]) {
    const Vec<T, E> v = load_vec<T, E>(p, vi);
#pragma unroll
    for (int e = 0; e < E; ++e) out[e] = to_f32(v.v[e]);
}

// ------------------------------------------------------------------ nhwc
template <typename T, int E>
__global__ void __launch_bounds__(256)
sgn_stats_nhwc_kernel(const T* __restrict__ X, const T* __restrict__ skip,
                      const T* __restrict__ bias, T* __restrict__ S, Partial* __restrict__ part,
                      int64_t HW, int C, int Cv, int P, int cpg, int groups, int B, int64_t ppb,
                      bool skip_bcast) {
    using V = Vec<T, E>;
    __shared__ float sh_n[256 * E], sh_mean[256 * E], sh_m2[256 * E];
    const int n = blockIdx.x / B, b = blockIdx.x % B;
    const int t = threadIdx.x;
    const bool active = t < P * Cv;
    const int cv = active ? t % Cv : 0;
    const int p0 = active ? t / Cv : 0;
    const int64_t pb = int64_t(b) * ppb;
    const int64_t pe = pb + ppb < HW ? pb + ppb : HW;
    const int64_t img = int64_t(n) * HW * Cv;
    const bool has_bias = bias != nullptr;

    float bv[E] = {}, kb[E] = {};
    if (active && has_bias) load_param_vec<T, E>(bias, cv, bv);
    if (active && skip_bcast) load_param_vec<T, E>(skip, int64_t(n) * Cv + cv, kb);

    ShiftedSums acc[E];
    float cnt = 0.0f;
    if (active) {
        for (int64_t p = pb + p0; p < pe; p += kUnroll * P) {
            V xs[kUnroll], ks[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t pp = p + int64_t(u) * P;
                if (pp < pe) {
                    xs[u] = load_vec<T, E>(X, img + pp * Cv + cv);
                    if (!skip_bcast) ks[u] = load_vec<T, E>(skip, img + pp * Cv + cv);
                }
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t pp = p + int64_t(u) * P;
                if (pp < pe) {
                    V sv;
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const float k = skip_bcast ? kb[e] : to_f32(ks[u].v[e]);
                        const float s = residual_sum<T>(to_f32(xs[u].v[e]), k, has_bias, bv[e], sv.v[e]);
                        acc[e].add(s, cnt == 0.0f);
                    }
                    if (S) store_vec<T, E>(S, img + pp * Cv + cv, sv);
                    cnt += 1.0f;
                }
            }
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const Moments m = acc[e].moments(cnt);
            const int slot = p0 * C + cv * E + e;
            sh_n[slot] = m.n;
            sh_mean[slot] = m.mean;
            sh_m2[slot] = m.m2;
        }
    }
    __syncthreads();
    // One thread per group merges its channels' per-thread moments,
    // channel-major then pixel-lane, in a fixed order.
    for (int g = t; g < groups; g += 256) {
        Moments m{0.0f, 0.0f, 0.0f};
        for (int c = g * cpg; c < (g + 1) * cpg; ++c)
            for (int q = 0; q < P; ++q) {
                const int slot = q * C + c;
                m = merge(m, Moments{sh_n[slot], sh_mean[slot], sh_m2[slot]});
            }
        part[(int64_t(n) * groups + g) * B + b] = Partial{m.n, m.mean, m.m2, 0.0f};
    }
}

template <typename T, typename M, int E>
__global__ void __launch_bounds__(256)
sgn_norm_nhwc_kernel(const T* __restrict__ X, const T* __restrict__ skip,
                     const T* __restrict__ bias, const T* __restrict__ S_in,
                     const M* __restrict__ gamma, const M* __restrict__ beta,
                     const float2* __restrict__ stat, T* __restrict__ Y, int64_t HW, int Cv, int P,
                     int cpg, int groups, int B, int64_t ppb, bool skip_bcast, bool silu) {
    using V = Vec<T, E>;
    const int n = blockIdx.x / B, b = blockIdx.x % B;
    const int t = threadIdx.x;
    if (t >= P * Cv) return;  // no barrier below
    const int cv = t % Cv;
    const int p0 = t / Cv;
    const int64_t pb = int64_t(b) * ppb;
    const int64_t pe = pb + ppb < HW ? pb + ppb : HW;
    const int64_t img = int64_t(n) * HW * Cv;
    const bool has_bias = bias != nullptr;

    float mean[E], a[E], beta_c[E], bv[E] = {}, kb[E] = {};
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int c = cv * E + e;
        const float2 st = stat[int64_t(n) * groups + c / cpg];
        mean[e] = st.x;
        a[e] = st.y * to_f32(gamma[c]);
        beta_c[e] = to_f32(beta[c]);
    }
    if (!S_in) {
        if (has_bias) load_param_vec<T, E>(bias, cv, bv);
        if (skip_bcast) load_param_vec<T, E>(skip, int64_t(n) * Cv + cv, kb);
    }

    for (int64_t p = pb + p0; p < pe; p += kUnroll * P) {
        V ss[kUnroll], ks[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t pp = p + int64_t(u) * P;
            if (pp < pe) {
                if (S_in) {
                    ss[u] = load_vec<T, E>(S_in, img + pp * Cv + cv);
                } else {
                    ss[u] = load_vec<T, E>(X, img + pp * Cv + cv);
                    if (!skip_bcast) ks[u] = load_vec<T, E>(skip, img + pp * Cv + cv);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t pp = p + int64_t(u) * P;
            if (pp < pe) {
                V out;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    float s;
                    if (S_in) {
                        s = to_f32(ss[u].v[e]);
                    } else {
                        T rounded;
                        const float k = skip_bcast ? kb[e] : to_f32(ks[u].v[e]);
                        s = residual_sum<T>(to_f32(ss[u].v[e]), k, has_bias, bv[e], rounded);
                    }
                    float y = fmaf_(s - mean[e], a[e], beta_c[e]);
                    if (silu) y = silu_f32(y);
                    out.v[e] = from_f32<T>(y);
                }
                store_vec<T, E>(Y, img + pp * Cv + cv, out);
            }
        }
    }
}

// ------------------------------------------------------------------ group
// Element i of group (n, g): NCHW address (n*C + g*cpg)*HW + i, channel
// g*cpg + i/HW; NHWC address (n*HW + i/cpg)*C + g*cpg + i%cpg.
struct GroupGeom {
    int64_t HW;
    int C, cpg, groups;
    FastDiv div;  // by HW (NCHW) or by cpg (NHWC)
};

template <bool NCHW>
__device__ __forceinline__ void group_element(const GroupGeom& geo, int n, int g, uint32_t i,
                                              int64_t& addr, int& c) {
    if constexpr (NCHW) {
        const uint32_t cl = fastdiv(i, geo.div);
        c = g * geo.cpg + int(cl);
        addr = (int64_t(n) * geo.C + int64_t(g) * geo.cpg) * geo.HW + i;
    } else {
        const uint32_t pix = fastdiv(i, geo.div);
        const int cl = int(i - pix * uint32_t(geo.cpg));
        c = g * geo.cpg + cl;
        addr = (int64_t(n) * geo.HW + pix) * geo.C + c;
    }
}

template <typename T, int E, bool NCHW>
__global__ void __launch_bounds__(256)
sgn_stats_group_kernel(const T* __restrict__ X, const T* __restrict__ skip,
                       const T* __restrict__ bias, T* __restrict__ S, Partial* __restrict__ part,
                       GroupGeom geo, uint32_t Kv, uint32_t vpb, int B, bool skip_bcast) {
    using V = Vec<T, E>;
    __shared__ Moments sh[256];
    const int ng = blockIdx.x / B, b = blockIdx.x % B;
    const int n = ng / geo.groups, g = ng % geo.groups;
    const int t = threadIdx.x;
    const uint32_t vb = uint32_t(b) * vpb;
    const uint32_t ve = vb + vpb < Kv ? vb + vpb : Kv;
    const bool has_bias = bias != nullptr;

    ShiftedSums acc;
    float cnt = 0.0f;
    for (uint32_t iv = vb + t; iv < ve; iv += kUnroll * 256) {
        V xs[kUnroll], ks[kUnroll];
        int64_t addr[kUnroll];
        int ch[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t j = iv + uint32_t(u) * 256;
            if (j < ve) {
                // With E > 1 (NCHW only) a vector never straddles channels.
                group_element<NCHW>(geo, n, g, j * E, addr[u], ch[u]);
                xs[u] = load_vec<T, E>(X, addr[u] / E);
                if (!skip_bcast) ks[u] = load_vec<T, E>(skip, addr[u] / E);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t j = iv + uint32_t(u) * 256;
            if (j < ve) {
                const float bb = has_bias ? to_f32(bias[ch[u]]) : 0.0f;
                const float kb = skip_bcast ? to_f32(skip[int64_t(n) * geo.C + ch[u]]) : 0.0f;
                V sv;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float k = skip_bcast ? kb : to_f32(ks[u].v[e]);
                    const float s = residual_sum<T>(to_f32(xs[u].v[e]), k, has_bias, bb, sv.v[e]);
                    acc.add(s, cnt == 0.0f && e == 0);
                }
                if (S) store_vec<T, E>(S, addr[u] / E, sv);
                cnt += float(E);
            }
        }
    }
    const Moments m = block_merge(acc.moments(cnt), sh);
    if (t == 0) part[int64_t(ng) * B + b] = Partial{m.n, m.mean, m.m2, 0.0f};
}

template <typename T, typename M, int E, bool NCHW>
__global__ void __launch_bounds__(256)
sgn_norm_group_kernel(const T* __restrict__ X, const T* __restrict__ skip,
                      const T* __restrict__ bias, const T* __restrict__ S_in,
                      const M* __restrict__ gamma, const M* __restrict__ beta,
                      const float2* __restrict__ stat, T* __restrict__ Y, GroupGeom geo,
                      uint32_t Kv, uint32_t vpb, int B, bool skip_bcast, bool silu) {
    using V = Vec<T, E>;
    const int ng = blockIdx.x / B, b = blockIdx.x % B;
    const int n = ng / geo.groups, g = ng % geo.groups;
    const int t = threadIdx.x;
    const uint32_t vb = uint32_t(b) * vpb;
    const uint32_t ve = vb + vpb < Kv ? vb + vpb : Kv;
    const bool has_bias = bias != nullptr;
    const float2 st = stat[ng];

    for (uint32_t iv = vb + t; iv < ve; iv += kUnroll * 256) {
        V ss[kUnroll], ks[kUnroll];
        int64_t addr[kUnroll];
        int ch[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t j = iv + uint32_t(u) * 256;
            if (j < ve) {
                group_element<NCHW>(geo, n, g, j * E, addr[u], ch[u]);
                if (S_in) {
                    ss[u] = load_vec<T, E>(S_in, addr[u] / E);
                } else {
                    ss[u] = load_vec<T, E>(X, addr[u] / E);
                    if (!skip_bcast) ks[u] = load_vec<T, E>(skip, addr[u] / E);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t j = iv + uint32_t(u) * 256;
            if (j < ve) {
                const int c = ch[u];
                const float a = st.y * to_f32(gamma[c]);
                const float bt = to_f32(beta[c]);
                float bb = 0.0f, kb = 0.0f;
                if (!S_in) {
                    bb = has_bias ? to_f32(bias[c]) : 0.0f;
                    kb = skip_bcast ? to_f32(skip[int64_t(n) * geo.C + c]) : 0.0f;
                }
                V out;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    float s;
                    if (S_in) {
                        s = to_f32(ss[u].v[e]);
                    } else {
                        T rounded;
                        const float k = skip_bcast ? kb : to_f32(ks[u].v[e]);
                        s = residual_sum<T>(to_f32(ss[u].v[e]), k, has_bias, bb, rounded);
                    }
                    float y = fmaf_(s - st.x, a, bt);
                    if (silu) y = silu_f32(y);
                    out.v[e] = from_f32<T>(y);
                }
                store_vec<T, E>(Y, addr[u] / E, out);
            }
        }
    }
}

// ------------------------------------------------------------------ finalize
__global__ void __launch_bounds__(256)
sgn_finalize_kernel(const Partial* __restrict__ part, float2* __restrict__ stat, int B, float eps) {
    __shared__ Moments sh[256];
    const int64_t ng = blockIdx.x;
    Moments m{0.0f, 0.0f, 0.0f};
    for (int b = threadIdx.x; b < B; b += 256) m = merge(m, as_moments(part[ng * B + b]));
    m = block_merge(m, sh);
    if (threadIdx.x == 0) {
        const float var = m.n > 0.0f ? fmaxf(m.m2 / m.n, 0.0f) : 0.0f;
        stat[ng] = make_float2(m.mean, inv_sqrt(var + eps));
    }
}

// ------------------------------------------------------------------ host side
constexpr int64_t kElemsPerBlockTarget = 256 * kUnroll;  // vectors: one unrolled pass

template <typename T, typename M>
hipError_t launch_sgn_tm(const SgnArgs& a, Route want, hipStream_t stream, const char** route) {
    constexpr int EV = VecWidth<T>::value;
    const int64_t HW = a.H * a.W;
    const int C = int(a.C), groups = int(a.groups), cpg = int(a.C / a.groups);
    const int64_t NG = a.N * a.groups;
    const int B = int(sgn_partials_per_group(a.dtype, a.N, a.C, a.H, a.W, a.groups, a.channels_last));
    Partial* part = static_cast<Partial*>(a.workspace);
    float2* stat = reinterpret_cast<float2*>(part + NG * B);
    const T* X = static_cast<const T*>(a.X);
    const T* skip = static_cast<const T*>(a.skip);
    const T* bias = static_cast<const T*>(a.bias);
    T* Y = static_cast<T*>(a.Y);
    T* S = static_cast<T*>(a.S);
    const M* gamma = static_cast<const M*>(a.gamma);
    const M* beta = static_cast<const M*>(a.beta);
    const bool silu = a.activation == 1;

    // Tensors read or written as 16-byte vectors must be 16-byte aligned.
    // NHWC also reads bias and a broadcast skip per channel vector; NCHW
    // reads them one channel at a time.
    const bool data_ok = aligned16(a.X) && aligned16(a.Y) && (!a.S || aligned16(a.S)) &&
                         (a.skip_broadcast || aligned16(a.skip));
    bool nhwc_vec = a.channels_last && a.C % EV == 0 && a.C / EV <= 256 && data_ok &&
                    aligned16(a.skip) && (!a.bias || aligned16(a.bias));
    bool nchw_vec = !a.channels_last && HW % EV == 0 && data_ok;
    if (want == Route::Scalar || want == Route::Block) nhwc_vec = nchw_vec = false;

    if (nhwc_vec) {
        *route = "sgn.nhwc.vec16";
        const int Cv = C / EV, P = 256 / Cv;
        const int64_t ppb = (HW + B - 1) / B;
        const dim3 grid(unsigned(a.N * B));
        hipLaunchKernelGGL((sgn_stats_nhwc_kernel<T, EV>), grid, dim3(256), 0, stream, X, skip, bias,
                           S, part, HW, C, Cv, P, cpg, groups, B, ppb, a.skip_broadcast);
        hipLaunchKernelGGL(sgn_finalize_kernel, dim3(unsigned(NG)), dim3(256), 0, stream, part, stat,
                           B, a.epsilon);
        hipLaunchKernelGGL((sgn_norm_nhwc_kernel<T, M, EV>), grid, dim3(256), 0, stream, X, skip,
                           bias, static_cast<const T*>(S), gamma, beta, stat, Y, HW, Cv, P, cpg,
                           groups, B, ppb, a.skip_broadcast, silu);
        return hipGetLastError();
    }

    GroupGeom geo;
    geo.HW = HW;
    geo.C = C;
    geo.cpg = cpg;
    geo.groups = groups;
    const uint32_t K = uint32_t(int64_t(cpg) * HW);
    const dim3 grid(unsigned(NG * B));
    if (nchw_vec) {
        *route = "sgn.nchw.vec16";
        geo.div = make_fastdiv(uint32_t(HW));
        const uint32_t Kv = K / EV;
        const uint32_t vpb = uint32_t((Kv + B - 1) / B);
        hipLaunchKernelGGL((sgn_stats_group_kernel<T, EV, true>), grid, dim3(256), 0, stream, X, skip,
                           bias, S, part, geo, Kv, vpb, B, a.skip_broadcast);
        hipLaunchKernelGGL(sgn_finalize_kernel, dim3(unsigned(NG)), dim3(256), 0, stream, part, stat,
                           B, a.epsilon);
        hipLaunchKernelGGL((sgn_norm_group_kernel<T, M, EV, true>), grid, dim3(256), 0, stream, X,
                           skip, bias, static_cast<const T*>(S), gamma, beta, stat, Y, geo, Kv, vpb,
                           B, a.skip_broadcast, silu);
        return hipGetLastError();
    }

    const uint32_t vpb = uint32_t((K + B - 1) / B);
    if (!a.channels_last) {
        *route = "sgn.nchw.scalar";
        geo.div = make_fastdiv(uint32_t(HW));
        hipLaunchKernelGGL((sgn_stats_group_kernel<T, 1, true>), grid, dim3(256), 0, stream, X, skip,
                           bias, S, part, geo, K, vpb, B, a.skip_broadcast);
        hipLaunchKernelGGL(sgn_finalize_kernel, dim3(unsigned(NG)), dim3(256), 0, stream, part, stat,
                           B, a.epsilon);
        hipLaunchKernelGGL((sgn_norm_group_kernel<T, M, 1, true>), grid, dim3(256), 0, stream, X,
                           skip, bias, static_cast<const T*>(S), gamma, beta, stat, Y, geo, K, vpb,
                           B, a.skip_broadcast, silu);
    } else {
        *route = "sgn.nhwc.scalar";
        geo.div = make_fastdiv(uint32_t(cpg));
        hipLaunchKernelGGL((sgn_stats_group_kernel<T, 1, false>), grid, dim3(256), 0, stream, X, skip,
                           bias, S, part, geo, K, vpb, B, a.skip_broadcast);
        hipLaunchKernelGGL(sgn_finalize_kernel, dim3(unsigned(NG)), dim3(256), 0, stream, part, stat,
                           B, a.epsilon);
        hipLaunchKernelGGL((sgn_norm_group_kernel<T, M, 1, false>), grid, dim3(256), 0, stream, X,
                           skip, bias, static_cast<const T*>(S), gamma, beta, stat, Y, geo, K, vpb,
                           B, a.skip_broadcast, silu);
    }
    return hipGetLastError();
}

}  // namespace

int64_t sgn_partials_per_group(int dtype, int64_t N, int64_t C, int64_t H, int64_t W,
                               int64_t groups, bool channels_last) {
    const int64_t ev = dtype == 0 ? 4 : 8;
    const int64_t HW = H * W;
    const int64_t per_unit = channels_last ? HW * C : (C / groups) * HW;  // image / group
    int64_t B = (per_unit + ev * kElemsPerBlockTarget - 1) / (ev * kElemsPerBlockTarget);
    if (channels_last && B > HW) B = HW;  // at least one pixel per block
    if (B < 1) B = 1;
    if (B > 4096) B = 4096;
    (void)N;
    return B;
}

size_t sgn_workspace_bytes(int dtype, int64_t N, int64_t C, int64_t H, int64_t W, int64_t groups,
                           bool channels_last) {
    const int64_t B = sgn_partials_per_group(dtype, N, C, H, W, groups, channels_last);
    const int64_t NG = N * groups;
    return size_t(NG * B) * sizeof(Partial) + size_t(NG) * sizeof(float2);
}

hipError_t launch_sgn(const SgnArgs& a, Route want, hipStream_t stream, const char** route) {
    if (a.N == 0 || a.H * a.W == 0) {
        *route = "sgn.empty";
        return hipSuccess;
    }
    if (a.dtype == 0) {
        if (a.param_dtype == 0) return launch_sgn_tm<float, float>(a, want, stream, route);
        return launch_sgn_tm<float, half_t>(a, want, stream, route);
    }
    if (a.param_dtype == 0) return launch_sgn_tm<half_t, float>(a, want, stream, route);
    return launch_sgn_tm<half_t, half_t>(a, want, stream, route);
}

}  // namespace sn
