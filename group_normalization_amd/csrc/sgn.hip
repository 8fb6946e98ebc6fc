// sgn.hip -- SkipGroupNorm kernels for gfx950.
//
// Operator ("com.microsoft.SkipGroupNorm", Description, Inputs, Attributes):
// S = X + skip (+ bias) rounded to T; per (n, group of C/groups channels)
// over all H*W positions the mean and population variance of S;
// Y = act(gamma_c * (S - mean) / sqrt(var + epsilon) + beta_c), act = none or
// SiLU; optional output S.  gamma/beta have their own type M.
//
// On MI355X a grid-wide barrier inside a kernel costs far more (tens of
// microseconds: cross-XCD atomics) than a kernel boundary on one stream, so
// no kernel here waits for another block.  Two routes:
//
// group-block (NCHW, one (n, group) of at most 8 x 16 KiB, 12 x 16 KiB with
//   a broadcast skip, or 16 Ki elements on the scalar route): a group is
//   contiguous in NCHW, so one 1024-thread
//   workgroup reads it once, keeps S in VGPRs, reduces with wave butterflies
//   and one LDS step, and writes S and Y.  One launch, no workspace, exactly
//   the operator's own traffic.
//
// split (everything else; NHWC always), three launches on one stream: the
//   pages' "partial group statistics / combine / normalize" structure,
//   re-tiled for 256 CUs:
//   1. statistics: every block forms S over its tile, stores S if requested,
//      and writes one partial (count, mean, M2) per (n, group) it covers;
//   2. finalize: one block per (n, group) combines its partials in a fixed
//      order into (mean, 1/sqrt(var + epsilon));
//   3. normalize: re-reads S (or re-forms it from X, skip and bias, bit for
//      bit the same) and writes Y.
//   Tilings of passes 1 and 3:
//   nhwc   (NHWC, C a whole number of 16-byte vectors, at most 256 of them):
//          a block covers a run of pixels of one image and all channels.
//          Thread t owns channel vector t % Cv at pixels t / Cv + k * P,
//          P = 256 / Cv, so its channels (and their bias, gamma, beta and
//          group) never change.  Per-channel moments are merged over the
//          pixel lanes, then over each group's channels, through LDS.
//   group  (NCHW groups too large for one workgroup; the scalar route of
//          both layouts): a block covers a slice of one (n, group)'s
//          elements.
//   Caching: when S is requested, pass 1 streams X and skip (they are not
//   read again) and stores S cached for pass 3; otherwise pass 3 re-forms S
//   from X and skip, which stay cached.  Y is always stored nontemporally.
//
// Moments: each thread uses the shifted-data sums (shift = its first value)
// and every combination uses the pairwise update (Chan et al.) in a fixed
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

// Combines the moments of the 64 lanes of a wave.  Partners always combine
// as merge(lower lane, upper lane), so both compute bitwise the same value
// and every lane ends with the same total.
__device__ __forceinline__ Moments wave_merge(Moments m) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
        Moments o;
        o.n = __shfl_xor(m.n, s, 64);
        o.mean = __shfl_xor(m.mean, s, 64);
        o.m2 = __shfl_xor(m.m2, s, 64);
        m = (lane & s) ? merge(o, m) : merge(m, o);
    }
    return m;
}

// Block of W waves: wave totals through LDS, combined in wave order by every
// thread (all threads return the same value).  `sh` holds W entries.
template <int W>
__device__ __forceinline__ Moments block_merge(Moments m, Moments* sh) {
    m = wave_merge(m);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = m;
    __syncthreads();
    Moments tot = sh[0];
#pragma unroll
    for (int w = 1; w < W; ++w) tot = merge(tot, sh[w]);
    return tot;
}

__device__ __forceinline__ float2 finalize(const Moments& m, float eps) {
    const float var = m.n > 0.0f ? fmaxf(m.m2 / m.n, 0.0f) : 0.0f;
    return make_float2(m.mean, inv_sqrt(var + eps));
}

template <typename T, int E>
__device__ __forceinline__ void load_param_vec(const T* p, int64_t vi, float (&out)[E]) {
    const Vec<T, E> v = load_vec<T, E>(p, vi);
#pragma unroll
    for (int e = 0; e < E; ++e) out[e] = to_f32(v.v[e]);
}

template <typename T, int E>
__device__ __forceinline__ Vec<T, E> load_in(const T* p, int64_t i, bool stream) {
    return stream ? load_vec_stream<T, E>(p, i) : load_vec<T, E>(p, i);
}

// ------------------------------------------------------------------ group-block
template <typename T, typename M>
struct GroupBlockArgs {
    const T *X, *skip, *bias;
    T *S, *Y;
    const M *gamma, *beta;
    int64_t HW;
    int C, cpg, groups;
    uint32_t Kv;  // vectors per group
    FastDiv div;  // by H*W
    bool skip_bcast, silu;
    float eps;
};

constexpr int kGroupBlockThreads = 1024;

template <typename T, typename M, int E, int R, bool BCAST>
__global__ void __launch_bounds__(kGroupBlockThreads)
sgn_group_block_kernel(GroupBlockArgs<T, M> a) {
    using V = Vec<T, E>;
    __shared__ Moments sh[kGroupBlockThreads / 64];
    const int t = threadIdx.x;
    const int ng = blockIdx.x;
    const int n = ng / a.groups, g = ng % a.groups;
    const int64_t base = (int64_t(n) * a.C + int64_t(g) * a.cpg) * a.HW / E;  // in vectors
    const bool has_bias = a.bias != nullptr;
    // Channel of vector j of the group; with E > 1, H*W is a whole number of
    // vectors, so no vector straddles channels.
    auto channel = [&](uint32_t j) { return g * a.cpg + int(fastdiv(j * E, a.div)); };

    V sv[R], xs[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const uint32_t j = uint32_t(t) + uint32_t(k) * kGroupBlockThreads;
        if (j < a.Kv) {
            xs[k] = load_vec_stream<T, E>(a.X, base + j);
            if constexpr (!BCAST) sv[k] = load_vec_stream<T, E>(a.skip, base + j);
        }
    }
    ShiftedSums acc;
    float cnt = 0.0f;
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const uint32_t j = uint32_t(t) + uint32_t(k) * kGroupBlockThreads;
        if (j < a.Kv) {
            const int c = channel(j);
            const float bb = has_bias ? to_f32(a.bias[c]) : 0.0f;
            float kb = 0.0f;
            if constexpr (BCAST) kb = to_f32(a.skip[int64_t(n) * a.C + c]);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                float kk = kb;
                if constexpr (!BCAST) kk = to_f32(sv[k].v[e]);
                const float s = residual_sum<T>(to_f32(xs[k].v[e]), kk, has_bias, bb, sv[k].v[e]);
                acc.add(s, cnt == 0.0f && e == 0);
            }
            if (a.S) store_vec_stream<T, E>(a.S, base + j, sv[k]);
            cnt += float(E);
        }
    }
    const float2 st = finalize(block_merge<kGroupBlockThreads / 64>(acc.moments(cnt), sh), a.eps);
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const uint32_t j = uint32_t(t) + uint32_t(k) * kGroupBlockThreads;
        if (j < a.Kv) {
            const int c = channel(j);
            const float scl = st.y * to_f32(a.gamma[c]);
            const float sft = to_f32(a.beta[c]);
            V out;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                float y = fmaf_(to_f32(sv[k].v[e]) - st.x, scl, sft);
                if (a.silu) y = silu_f32(y);
                out.v[e] = from_f32<T>(y);
            }
            store_vec_stream<T, E>(a.Y, base + j, out);
        }
    }
}

// ------------------------------------------------------------------ split: nhwc
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
    const bool stream_in = S != nullptr;  // pass 3 reads S, not X and skip

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
                    xs[u] = load_in<T, E>(X, img + pp * Cv + cv, stream_in);
                    if (!skip_bcast) ks[u] = load_in<T, E>(skip, img + pp * Cv + cv, stream_in);
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
    // Per channel over the P pixel lanes; the totals go to row 0.
    for (int c = t; c < C; c += 256) {
        Moments m{sh_n[c], sh_mean[c], sh_m2[c]};
        for (int q = 1; q < P; ++q) {
            const int slot = q * C + c;
            m = merge(m, Moments{sh_n[slot], sh_mean[slot], sh_m2[slot]});
        }
        sh_n[c] = m.n;
        sh_mean[c] = m.mean;
        sh_m2[c] = m.m2;
    }
    __syncthreads();
    // Per group over its channels.
    for (int g = t; g < groups; g += 256) {
        const int c0 = g * cpg;
        Moments m{sh_n[c0], sh_mean[c0], sh_m2[c0]};
        for (int c = c0 + 1; c < c0 + cpg; ++c) m = merge(m, Moments{sh_n[c], sh_mean[c], sh_m2[c]});
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

    bool first = true;
    float mean[E], scl[E], sft[E], bv[E] = {}, kb[E] = {};
    for (int64_t p = pb + p0; p < pe; p += kUnroll * P) {
        // The data loads go out before the per-channel constants are read.
        V ss[kUnroll], ks[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t pp = p + int64_t(u) * P;
            if (pp < pe) {
                if (S_in) {
                    ss[u] = load_vec_stream<T, E>(S_in, img + pp * Cv + cv);
                } else {
                    ss[u] = load_vec_stream<T, E>(X, img + pp * Cv + cv);
                    if (!skip_bcast) ks[u] = load_vec_stream<T, E>(skip, img + pp * Cv + cv);
                }
            }
        }
        if (first) {
            first = false;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int c = cv * E + e;
                const float2 st = stat[int64_t(n) * groups + c / cpg];
                mean[e] = st.x;
                scl[e] = st.y * to_f32(gamma[c]);
                sft[e] = to_f32(beta[c]);
            }
            if (!S_in) {
                if (has_bias) load_param_vec<T, E>(bias, cv, bv);
                if (skip_bcast) load_param_vec<T, E>(skip, int64_t(n) * Cv + cv, kb);
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
                    float y = fmaf_(s - mean[e], scl[e], sft[e]);
                    if (silu) y = silu_f32(y);
                    out.v[e] = from_f32<T>(y);
                }
                store_vec_stream<T, E>(Y, img + pp * Cv + cv, out);
            }
        }
    }
}

// ------------------------------------------------------------------ split: group
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
    __shared__ Moments sh[4];
    const int ng = blockIdx.x / B, b = blockIdx.x % B;
    const int n = ng / geo.groups, g = ng % geo.groups;
    const int t = threadIdx.x;
    const uint32_t vb = uint32_t(b) * vpb;
    const uint32_t ve = vb + vpb < Kv ? vb + vpb : Kv;
    const bool has_bias = bias != nullptr;
    const bool stream_in = S != nullptr;

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
                xs[u] = load_in<T, E>(X, addr[u] / E, stream_in);
                if (!skip_bcast) ks[u] = load_in<T, E>(skip, addr[u] / E, stream_in);
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
    const Moments m = block_merge<4>(acc.moments(cnt), sh);
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
                    ss[u] = load_vec_stream<T, E>(S_in, addr[u] / E);
                } else {
                    ss[u] = load_vec_stream<T, E>(X, addr[u] / E);
                    if (!skip_bcast) ks[u] = load_vec_stream<T, E>(skip, addr[u] / E);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t j = iv + uint32_t(u) * 256;
            if (j < ve) {
                const int c = ch[u];
                const float scl = st.y * to_f32(gamma[c]);
                const float sft = to_f32(beta[c]);
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
                    float y = fmaf_(s - st.x, scl, sft);
                    if (silu) y = silu_f32(y);
                    out.v[e] = from_f32<T>(y);
                }
                store_vec_stream<T, E>(Y, addr[u] / E, out);
            }
        }
    }
}

// ------------------------------------------------------------------ split: finalize
// One 256-thread block per (n, group): every thread loads its partials
// (t, t + 256, ...) before combining them, then the block combines the
// threads in a fixed order.
__global__ void __launch_bounds__(256)
sgn_finalize_kernel(const Partial* __restrict__ part, float2* __restrict__ stat, int B, float eps) {
    __shared__ Moments sh[4];
    const int t = threadIdx.x;
    const Partial* p = part + int64_t(blockIdx.x) * B;
    Moments m{0.0f, 0.0f, 0.0f};
    for (int b0 = 0; b0 < B; b0 += 4 * 256) {
        Partial q[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int b = b0 + u * 256 + t;
            if (b < B) q[u] = p[b];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int b = b0 + u * 256 + t;
            if (b < B) m = merge(m, as_moments(q[u]));
        }
    }
    m = block_merge<4>(m, sh);
    if (t == 0) stat[blockIdx.x] = finalize(m, eps);
}

// ------------------------------------------------------------------ host side
constexpr int64_t kVectorsPerBlock = 256 * kUnroll;  // one unrolled pass of a 256-thread block

constexpr int kNhwcRowsPerThread = 2;                // pixel rows per thread in the nhwc tiling

// Blocks per image (nhwc) or per (n, group) (group tiling) of the split
// route.  The nhwc tiling gives each thread kNhwcRowsPerThread pixels, so a
// small image still spreads over many CUs; the group tiling gives each block
// one unrolled pass of vectors.
int64_t split_blocks(int dtype, int64_t C, int64_t HW, int64_t groups, bool channels_last) {
    const int64_t ev = dtype == 0 ? 4 : 8;
    int64_t B;
    if (channels_last && C % ev == 0 && C / ev <= 256) {
        const int64_t P = 256 / (C / ev);
        const int64_t ppb = P * kNhwcRowsPerThread;
        B = (HW + ppb - 1) / ppb;
    } else {
        const int64_t per_unit = channels_last ? HW * C : (C / groups) * HW;  // image / group
        B = (per_unit + ev * kVectorsPerBlock - 1) / (ev * kVectorsPerBlock);
        if (channels_last && B > HW) B = HW;  // at least one pixel per block
    }
    if (B < 1) B = 1;
    if (B > 16384) B = 16384;
    return B;
}

// Vectors per thread the group-block route holds within the 128 registers a
// 1024-thread workgroup leaves each thread: 12 sixteen-byte vectors with a
// broadcast skip, 8 with a full skip in flight beside X; 16 scalars.
constexpr int kGroupBlockMaxVecBcast = 12;
constexpr int kGroupBlockMaxVecFull = 8;
constexpr int kGroupBlockMaxScalar = 16;

int group_block_max_r(int E, bool bcast) {
    if (E > 1) return bcast ? kGroupBlockMaxVecBcast : kGroupBlockMaxVecFull;
    return kGroupBlockMaxScalar;
}

template <typename T, typename M, int E, int R>
hipError_t launch_group_block_r(const GroupBlockArgs<T, M>& ga, int64_t NG, hipStream_t stream) {
    if (ga.skip_bcast) {
        hipLaunchKernelGGL((sgn_group_block_kernel<T, M, E, R, true>), dim3(unsigned(NG)),
                           dim3(kGroupBlockThreads), 0, stream, ga);
    } else {
        if constexpr (R <= (E > 1 ? kGroupBlockMaxVecFull : kGroupBlockMaxScalar))
            hipLaunchKernelGGL((sgn_group_block_kernel<T, M, E, R, false>), dim3(unsigned(NG)),
                               dim3(kGroupBlockThreads), 0, stream, ga);
        else
            return hipErrorInvalidValue;  // callers check the size first
    }
    return hipGetLastError();
}

template <typename T, typename M, int E>
hipError_t launch_group_block(const GroupBlockArgs<T, M>& ga, int64_t NG, hipStream_t stream) {
    const uint32_t r = (ga.Kv + kGroupBlockThreads - 1) / kGroupBlockThreads;
    if constexpr (E > 1) {
        if (r <= 2) return launch_group_block_r<T, M, E, 2>(ga, NG, stream);
        if (r <= 4) return launch_group_block_r<T, M, E, 4>(ga, NG, stream);
        if (r <= 8) return launch_group_block_r<T, M, E, 8>(ga, NG, stream);
        return launch_group_block_r<T, M, E, kGroupBlockMaxVecBcast>(ga, NG, stream);
    } else {
        if (r <= 4) return launch_group_block_r<T, M, E, 4>(ga, NG, stream);
        if (r <= 8) return launch_group_block_r<T, M, E, 8>(ga, NG, stream);
        return launch_group_block_r<T, M, E, kGroupBlockMaxScalar>(ga, NG, stream);
    }
}

template <typename T, typename M>
hipError_t launch_sgn_tm(const SgnArgs& a, Route want, hipStream_t stream, const char** route) {
    constexpr int EV = VecWidth<T>::value;
    const int64_t HW = a.H * a.W;
    const int C = int(a.C), groups = int(a.groups), cpg = int(a.C / a.groups);
    const int64_t NG = a.N * a.groups;
    const int64_t K = int64_t(cpg) * HW;  // elements per group
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
    const bool vec_allowed = want != Route::Scalar && want != Route::Block;
    const bool nhwc_vec = vec_allowed && a.channels_last && a.C % EV == 0 && a.C / EV <= 256 &&
                          data_ok && aligned16(a.skip) && (!a.bias || aligned16(a.bias));
    const bool nchw_vec = vec_allowed && !a.channels_last && HW % EV == 0 && data_ok;

    // ---- group-block route (NCHW)
    const bool block_route = !a.channels_last && want != Route::Split && want != Route::Block;
    if (block_route) {
        GroupBlockArgs<T, M> ga{X, skip, bias, S, Y, gamma, beta, HW, C, cpg, groups, 0,
                                make_fastdiv(uint32_t(HW)), a.skip_broadcast, silu, a.epsilon};
        if (nchw_vec && K / EV <= int64_t(group_block_max_r(EV, a.skip_broadcast)) * kGroupBlockThreads) {
            *route = "sgn.block.nchw.vec16";
            ga.Kv = uint32_t(K / EV);
            return launch_group_block<T, M, EV>(ga, NG, stream);
        }
        if (!nchw_vec && K <= int64_t(group_block_max_r(1, a.skip_broadcast)) * kGroupBlockThreads) {
            *route = "sgn.block.nchw.scalar";
            ga.Kv = uint32_t(K);
            return launch_group_block<T, M, 1>(ga, NG, stream);
        }
    }

    // ---- split route
    const int64_t B_ws = sgn_partials_per_group(a.dtype, a.N, a.C, a.H, a.W, a.groups, a.channels_last);
    const int B = int(split_blocks(a.dtype, a.C, HW, a.groups, a.channels_last));
    Partial* part = static_cast<Partial*>(a.workspace);
    float2* stat = reinterpret_cast<float2*>(part + NG * B_ws);
    const dim3 fin_grid = dim3(unsigned(NG));

    if (nhwc_vec) {
        *route = "sgn.split.nhwc.vec16";
        const int Cv = C / EV, P = 256 / Cv;
        const int64_t ppb = (HW + B - 1) / B;
        const dim3 grid(unsigned(a.N * B));
        hipLaunchKernelGGL((sgn_stats_nhwc_kernel<T, EV>), grid, dim3(256), 0, stream, X, skip, bias,
                           S, part, HW, C, Cv, P, cpg, groups, B, ppb, a.skip_broadcast);
        hipLaunchKernelGGL(sgn_finalize_kernel, fin_grid, dim3(256), 0, stream, part, stat, B,
                           a.epsilon);
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
    const dim3 grid(unsigned(NG * B));
    if (nchw_vec) {
        *route = "sgn.split.nchw.vec16";
        geo.div = make_fastdiv(uint32_t(HW));
        const uint32_t Kv = uint32_t(K / EV);
        const uint32_t vpb = uint32_t((Kv + B - 1) / B);
        hipLaunchKernelGGL((sgn_stats_group_kernel<T, EV, true>), grid, dim3(256), 0, stream, X, skip,
                           bias, S, part, geo, Kv, vpb, B, a.skip_broadcast);
        hipLaunchKernelGGL(sgn_finalize_kernel, fin_grid, dim3(256), 0, stream, part, stat, B,
                           a.epsilon);
        hipLaunchKernelGGL((sgn_norm_group_kernel<T, M, EV, true>), grid, dim3(256), 0, stream, X,
                           skip, bias, static_cast<const T*>(S), gamma, beta, stat, Y, geo, Kv, vpb,
                           B, a.skip_broadcast, silu);
        return hipGetLastError();
    }

    const uint32_t vpb = uint32_t((K + B - 1) / B);
    if (!a.channels_last) {
        *route = "sgn.split.nchw.scalar";
        geo.div = make_fastdiv(uint32_t(HW));
        hipLaunchKernelGGL((sgn_stats_group_kernel<T, 1, true>), grid, dim3(256), 0, stream, X, skip,
                           bias, S, part, geo, uint32_t(K), vpb, B, a.skip_broadcast);
        hipLaunchKernelGGL(sgn_finalize_kernel, fin_grid, dim3(256), 0, stream, part, stat, B,
                           a.epsilon);
        hipLaunchKernelGGL((sgn_norm_group_kernel<T, M, 1, true>), grid, dim3(256), 0, stream, X,
                           skip, bias, static_cast<const T*>(S), gamma, beta, stat, Y, geo,
                           uint32_t(K), vpb, B, a.skip_broadcast, silu);
    } else {
        *route = "sgn.split.nhwc.scalar";
        geo.div = make_fastdiv(uint32_t(cpg));
        hipLaunchKernelGGL((sgn_stats_group_kernel<T, 1, false>), grid, dim3(256), 0, stream, X, skip,
                           bias, S, part, geo, uint32_t(K), vpb, B, a.skip_broadcast);
        hipLaunchKernelGGL(sgn_finalize_kernel, fin_grid, dim3(256), 0, stream, part, stat, B,
                           a.epsilon);
        hipLaunchKernelGGL((sgn_norm_group_kernel<T, M, 1, false>), grid, dim3(256), 0, stream, X,
                           skip, bias, static_cast<const T*>(S), gamma, beta, stat, Y, geo,
                           uint32_t(K), vpb, B, a.skip_broadcast, silu);
    }
    return hipGetLastError();
}

}  // namespace

int64_t sgn_partials_per_group(int dtype, int64_t N, int64_t C, int64_t H, int64_t W,
                               int64_t groups, bool channels_last) {
    (void)N;
    return split_blocks(dtype, C, H * W, groups, channels_last);
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
