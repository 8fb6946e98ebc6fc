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
// no kernel here waits for the whole grid; the cluster routes exchange
// moments among a few workgroups with bounded waits.  Three routes:
//
// group-cluster (NCHW, groups of at most 8 x 256 x 16 sixteen-byte vectors
//   or 8 x 256 x 32 scalars): a group is contiguous in NCHW, so K workgroups
//   (K <= 8) read it once, keep S in VGPRs, exchange their slices' moments
//   with a bounded wait (see sgn_cluster_kernel) and write S and Y.  One
//   launch, exactly the operator's own traffic.  Groups off the 16-byte
//   grid (odd H*W, or data bases sharing an offset from it) read aligned
//   16-byte vectors across group boundaries (sgn_cluster_phase_kernel).
//
// channel-block cluster (NHWC, in sgn_nhwc.hip; pixels a whole number of
//   16-, 8- or 4-byte vectors no wider than a group, images of up to
//   64 x 16 x (256 / vectors per block) pixels, and only while each
//   exchange cluster fits in the workgroups the device holds at once and
//   the grid is at most two rounds of them): workgroups own (image, pixel
//   slice, channel block) tiles, hold S in VGPRs and exchange per-group
//   moments the same way.  One launch, exactly the operator's traffic.
//
// Under HIP graph capture the cluster routes' publication slots are cleared
// by a store kernel ahead of each launch and the tag is constant (a replay
// repeats the arguments of the capture).
//
// split (everything else), three launches on one stream: the
//   pages' "partial group statistics / combine / normalize" structure,
//   re-tiled for 256 CUs:
//   1. statistics: every block forms S over its tile, stores S if requested,
//      and writes one partial (count, mean, M2) per (n, group) it covers;
//   2. finalize: one block per (n, group) combines its partials in a fixed
//      order into (mean, 1/sqrt(var + epsilon));
//   3. normalize: re-reads S (or re-forms it from X, skip and bias, bit for
//      bit the same) and writes Y.
//   Tilings of passes 1 and 3:
//   nhwc   (NHWC, C a whole number of 16-, 8- or 4-byte vectors that
//          splits into equal channel blocks of whole groups, at most 256
//          vectors each):
//          a block covers a run of pixels of one image and one channel
//          block (every thread the same number of pixels: at least two,
//          more where the grid would exceed about 2048 blocks).  Thread t
//          owns the block's channel vector t % CBv at pixels t / CBv + k * P,
//          P = 256 / CBv, so its channels (and their bias, gamma, beta and
//          group) never change.  Per-channel moments are merged over the
//          pixel lanes, then over each group's channels, through LDS, by
//          segments of lanes in a fixed order.
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
#include <atomic>
#include <type_traits>

#include "sgn_common.h"

namespace sn {
namespace {

// ------------------------------------------------------------------ group-cluster
// K workgroups of 256 threads per (n, group) of an NCHW tensor (a group is
// contiguous there), K = 1..8 chosen so that the grid covers the CUs: one CU
// streams only ~20-25 GB/s, so a group must be spread over several CUs to
// approach the chip's bandwidth.  Each workgroup forms S for its slice and
// keeps it in VGPRs, publishes its slice's moments with a per-call tag, reads
// the other slices' moments, combines all K in slice order (every workgroup
// of the group computes bitwise the same statistics) and writes Y from its
// registers.  The waits are bounded: a slice whose moments are not published
// in time is recomputed by the waiting workgroup from X and skip with the
// same arithmetic, so results never depend on scheduling and no workgroup
// can wait forever.
template <typename T, typename M>
struct ClusterArgs {
    const T *X, *skip, *bias;
    T *S, *Y;
    const M *gamma, *beta;
    Partial* part;     // N*groups*K publication slots
    PubTags tags;      // this call's publication tags
    long long timeout_ticks;  // wall-clock ticks a workgroup waits for a slice
    int64_t HW;
    int C, cpg, groups, K;
    uint32_t Kv;   // vectors per group
    uint32_t vps;  // vectors per slice
    FastDiv div;   // by H*W
    bool skip_bcast, silu;
    float eps;
    int phase;     // phased route: elements from the 16-byte boundary below the data bases
    unsigned long long* trace;  // phase timestamps (measurement builds)
};


template <typename T, typename M, int E, int R, bool BCAST>
__global__ void __launch_bounds__(kClusterThreads)
sgn_cluster_kernel(ClusterArgs<T, M> a) {
    using V = Vec<T, E>;
    __shared__ Moments sh[kClusterThreads / 64];
    __shared__ Moments slice_m[kClusterMaxK];
    __shared__ int late[kClusterMaxK];
    const int t = threadIdx.x;
    SN_PHASE(a.trace, 0);
    const int ng = blockIdx.x / a.K, k = blockIdx.x % a.K;
    const int n = ng / a.groups, g = ng % a.groups;
    const int64_t base = (int64_t(n) * a.C + int64_t(g) * a.cpg) * a.HW / E;  // in vectors
    const bool has_bias = a.bias != nullptr;
    // Channel of vector j of the group; with E > 1, H*W is a whole number of
    // vectors, so no vector straddles channels.
    auto channel = [&](uint32_t j) { return g * a.cpg + int(fastdiv(j * E, a.div)); };
    auto vec_of = [&](int slice, int r) {
        return uint32_t(slice) * a.vps + uint32_t(t) + uint32_t(r) * kClusterThreads;
    };
    auto end_of = [&](int slice) {
        const uint32_t e = uint32_t(slice + 1) * a.vps;
        return e < a.Kv ? e : a.Kv;
    };
    // S of one vector, rounded to T, from its channel's bias and broadcast
    // skip; the same arithmetic for the own slice and a recomputed one.
    auto form = [&](const V& x, const V& kv, float bb, float kb, V& s) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float kk = kb;
            if constexpr (!BCAST) kk = to_f32(kv.v[e]);
            residual_sum<T>(to_f32(x.v[e]), kk, has_bias, bb, s.v[e]);
        }
    };
    auto accumulate = [&](ShiftedSums& acc, float& cnt, const V& s) {
#pragma unroll
        for (int e = 0; e < E; ++e) acc.add(to_f32(s.v[e]), cnt == 0.0f && e == 0);
        cnt += float(E);
    };

    // ---- own slice: S into registers, slice moments.  The data loads go out
    // first, then each vector's per-channel constants (all needed later).  No
    // load sits behind a lane-dependent branch (the compiler would wait for
    // each in turn): vectors past the slice's end re-read its first vector.
    const uint32_t end = end_of(k);
    auto clamp = [&](uint32_t j) { return j < end ? j : uint32_t(k) * a.vps; };
    V sv[R], xs[R];
    T bias_r[R], kb_r[R];
    M gam_r[R], bet_r[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t j = clamp(vec_of(k, r));
        xs[r] = load_vec_stream<T, E>(a.X, base + j);
        if constexpr (!BCAST) sv[r] = load_vec_stream<T, E>(a.skip, base + j);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int c = channel(clamp(vec_of(k, r)));
        if (has_bias) bias_r[r] = a.bias[c];
        if constexpr (BCAST) kb_r[r] = a.skip[int64_t(n) * a.C + c];
        gam_r[r] = a.gamma[c];
        bet_r[r] = a.beta[c];
    }
    ShiftedSums acc;
    float cnt = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t j = vec_of(k, r);
        if (j < end) {
            form(xs[r], sv[r], has_bias ? to_f32(bias_r[r]) : 0.0f, BCAST ? to_f32(kb_r[r]) : 0.0f, sv[r]);
            accumulate(acc, cnt, sv[r]);
        }
    }
    SN_PHASE(a.trace, 1);
    const Moments mine = block_merge_rcp(acc.moments(cnt), sh);
    SN_PHASE(a.trace, 2);

    // ---- exchange with the other K-1 slices of the group
    Moments tot = mine;
    if (a.K > 1) {
        // Publication: this slice's (mean, M2) in its self-tagged slot;
        // nothing written with plain stores is exchanged, so no cache-wide
        // fence is needed.
        uint64_t* slots = reinterpret_cast<uint64_t*>(a.part) + 2 * (int64_t(ng) * a.K);
        if (t == 0) publish_moments(&slots[2 * k], mine, a.tags);
        if (a.S) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t j = vec_of(k, r);
                if (j < end) store_vec_stream<T, E>(a.S, base + j, sv[r]);
            }
        }
        SN_PHASE(a.trace, 3);
        if (t < a.K && t != k) {
            const long long t0 = wall_clock64();
            bool ok = false;
            float mean = 0.0f, m2 = 0.0f;
            for (;;) {
                if (read_moments(&slots[2 * t], a.tags, &mean, &m2)) {
                    ok = true;
                    break;
                }
                if (wall_clock64() - t0 > a.timeout_ticks) break;
                __builtin_amdgcn_s_sleep(2);
            }
            late[t] = ok ? 0 : 1;
            if (ok) slice_m[t] = Moments{float((end_of(t) - uint32_t(t) * a.vps) * E), mean, m2};
        }
        __syncthreads();
        tot = Moments{0.0f, 0.0f, 0.0f};
        for (int q = 0; q < a.K; ++q) {  // uniform over the workgroup
            Moments m;
            if (q == k) {
                m = mine;
            } else if (!late[q]) {
                m = slice_m[q];
            } else {
                // Slice q was not published in time: recompute its moments
                // exactly as its own workgroup does.
                const uint32_t qend = end_of(q);
                ShiftedSums qacc;
                float qcnt = 0.0f;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint32_t j = vec_of(q, r);
                    if (j < qend) {
                        const int c = channel(j);
                        V x = load_vec<T, E>(a.X, base + j), kv, sq;
                        if constexpr (!BCAST) kv = load_vec<T, E>(a.skip, base + j);
                        form(x, kv, has_bias ? to_f32(a.bias[c]) : 0.0f,
                             BCAST ? to_f32(a.skip[int64_t(n) * a.C + c]) : 0.0f, sq);
                        accumulate(qacc, qcnt, sq);
                    }
                }
                m = block_merge_rcp(qacc.moments(qcnt), sh);
            }
            tot = merge_rcp(tot, m);
        }
    } else {
        if (a.S) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t j = vec_of(k, r);
                if (j < end) store_vec_stream<T, E>(a.S, base + j, sv[r]);
            }
        }
        SN_PHASE(a.trace, 3);
    }
    SN_PHASE(a.trace, 4);

    // ---- normalize the held S
    const float2 st = finalize(tot, a.eps);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t j = vec_of(k, r);
        if (j < end) {
            const float scl = st.y * to_f32(gam_r[r]);
            const float sft = to_f32(bet_r[r]);
            V out;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                float y = fmaf_(to_f32(sv[r].v[e]) - st.x, scl, sft);
                if (a.silu) y = silu_f32(y);
                out.v[e] = from_f32<T>(y);
            }
            store_vec_stream<T, E>(a.Y, base + j, out);
        }
    }
    SN_PHASE(a.trace, 5);
}

// ------------------------------------------------------------------ group-cluster, phased
// NCHW groups whose span does not start on the 16-byte grid (H*W not a
// whole number of 16-byte vectors; X, skip, S and Y sharing a base off the
// grid): the same cluster, but each workgroup reads the aligned 16-byte
// vectors that cover its part of the group's span [s0, s0 + cpg*H*W)
// (counted from the boundary at or below the data bases; the span's first
// and last vector may hold the neighbouring groups' elements, read and
// masked), writes whole vectors where they lie inside the span and the two
// boundary vectors element by element.  With H*W >= E a vector holds at most
// two channels; their constants (bias, broadcast skip, gamma, beta) come
// from a per-workgroup LDS table of the group's channels.  The slices, the
// exchange and the recomputation of late slices are those of
// sgn_cluster_kernel, with each slice's element count in closed form.
constexpr int kPhaseMaxCpg = 512;  // channels per group the LDS table holds
constexpr int kPhaseMaxR = 8;      // vectors per thread

template <typename T, typename M, int E, int R, bool BCAST>
__global__ void __launch_bounds__(kClusterThreads)
sgn_cluster_phase_kernel(ClusterArgs<T, M> a) {
    using V = Vec<T, E>;
    __shared__ Moments sh[kClusterThreads / 64];
    __shared__ Moments slice_m[kClusterMaxK];
    __shared__ int late[kClusterMaxK];
    __shared__ float4 cst[kPhaseMaxCpg];  // per channel: bias, broadcast skip, gamma, beta
    const int t = threadIdx.x;
    SN_PHASE(a.trace, 0);
    const int ng = blockIdx.x / a.K, k = blockIdx.x % a.K;
    const int n = ng / a.groups, g = ng % a.groups;
    const int64_t span = int64_t(a.cpg) * a.HW;
    const int64_t s0 = (int64_t(n) * a.C + int64_t(g) * a.cpg) * a.HW + a.phase;
    const int64_t v0 = s0 / E;                                     // the span's first vector
    const int p = int(s0 - v0 * E);                                // its first element's place
    const uint32_t nvr = uint32_t((s0 + span + E - 1) / E - v0);   // vectors the span touches
    const T* xa = a.X - a.phase;
    const T* ka = a.skip - a.phase;  // full skip only
    T* sa = a.S ? a.S - a.phase : nullptr;
    T* ya = a.Y - a.phase;
    const bool has_bias = a.bias != nullptr;
    const int64_t HW = a.HW;

    auto slice_begin = [&](int s) { return uint32_t(s) * a.vps; };
    auto slice_end = [&](int s) {
        const uint32_t e = uint32_t(s + 1) * a.vps;
        return e < nvr ? e : nvr;
    };
    auto slice_count = [&](int s) {
        const int64_t lo = int64_t(slice_begin(s)) * E - p, hi = int64_t(slice_end(s)) * E - p;
        const int64_t l = lo > 0 ? lo : 0, h = hi < span ? hi : span;
        return h > l ? float(h - l) : 0.0f;
    };
    auto vec_of = [&](int s, int r) { return slice_begin(s) + uint32_t(t) + uint32_t(r) * kClusterThreads; };
    // Where vector i lies in the span, in 32-bit positions (a span holds at
    // most kClusterMaxK * kPhaseMaxR * 256 vectors): its elements [lo, hi)
    // are the span's, those below nlo belong to channel clo of the group and
    // the rest to chi (a vector holds at most two channels since H*W >= E).
    const int span32 = int(span);
    struct Lay {
        int lo, hi, nlo, clo, chi;
    };
    auto lay_of = [&](uint32_t i) {
        const int j0 = int(i) * E - p;
        Lay l;
        l.lo = j0 < 0 ? -j0 : 0;
        const int rem = span32 - j0;
        l.hi = rem < E ? rem : E;
        const uint32_t c = fastdiv(uint32_t(j0 > 0 ? j0 : 0), a.div);
        l.clo = c < uint32_t(a.cpg) ? int(c) : a.cpg - 1;
        l.chi = l.clo + 1 < a.cpg ? l.clo + 1 : l.clo;
        const int below = int(c + 1) * int(HW) - j0;  // >= 1
        l.nlo = below < E ? below : E;
        return l;
    };
    auto form = [&](const V& x, const V& kv, const Lay& l, V& s) {
        const float4 c0 = cst[l.clo], c1 = cst[l.chi];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const bool up = e >= l.nlo;
            const float bb = up ? c1.x : c0.x;
            const float kk = BCAST ? (up ? c1.y : c0.y) : to_f32(kv.v[e]);
            residual_sum<T>(to_f32(x.v[e]), kk, has_bias, bb, s.v[e]);
        }
    };
    // The span's elements in order, shifted by an element of the thread's
    // first vector: its first, or its last for the span's first vector
    // (which ends inside the span, as the span holds at least E elements).
    // Elements outside the span add zero differences.
    auto accumulate = [&](ShiftedSums& acc, float& cnt, const V& s, const Lay& l) {
        if (cnt == 0.0f) acc.shift = to_f32(l.lo > 0 ? s.v[E - 1] : s.v[0]);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float d = e >= l.lo && e < l.hi ? to_f32(s.v[e]) - acc.shift : 0.0f;
            acc.s1 += d;
            acc.s2 = fmaf_(d, d, acc.s2);
        }
        cnt += float(l.hi - l.lo);
    };
    // Vector i of the span into `dst` (aligned base): whole when it lies
    // inside the span, else the span's elements one by one.
    auto put = [&](T* dst, uint32_t i, const Lay& l, const V& v) {
        if (l.lo == 0 && l.hi == E) {
            store_vec_stream<T, E>(dst, v0 + i, v);
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (e >= l.lo && e < l.hi) dst[(v0 + i) * E + e] = v.v[e];
        }
    };

    // ---- own slice: the group's channel table, then the data loads.
    const uint32_t end = slice_end(k);
    auto clamp = [&](uint32_t j) { return j < end ? j : (slice_begin(k) < nvr ? slice_begin(k) : nvr - 1); };
    V sv[R], xs[R];
    // The table's first entries load before the data (the later rounds of
    // groups wider than a workgroup after it), by every thread (threads past
    // the group's channels re-read its first) and with bias read from X when
    // absent, so that no load sits behind a branch (the data loads would
    // wait for it).
    const T* bias_src = has_bias ? a.bias : a.X;  // X holds at least C elements
    const int ch0 = g * a.cpg + (t < a.cpg ? t : 0);
    const T tb = bias_src[ch0];
    T tk = T(0);
    if constexpr (BCAST) tk = a.skip[int64_t(n) * a.C + ch0];
    const M tg = a.gamma[ch0], te = a.beta[ch0];
    __builtin_amdgcn_sched_barrier(0);  // keep them ahead of the data loads
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t j = clamp(vec_of(k, r));
        xs[r] = load_vec_stream<T, E>(xa, v0 + j);
        if constexpr (!BCAST) sv[r] = load_vec_stream<T, E>(ka, v0 + j);
    }
    if (t < a.cpg)
        cst[t] = make_float4(has_bias ? to_f32(tb) : 0.0f, BCAST ? to_f32(tk) : 0.0f, to_f32(tg), to_f32(te));
    for (int c = t + kClusterThreads; c < a.cpg; c += kClusterThreads) {
        const int ch = g * a.cpg + c;
        cst[c] = make_float4(has_bias ? to_f32(bias_src[ch]) : 0.0f,
                             BCAST ? to_f32(a.skip[int64_t(n) * a.C + ch]) : 0.0f, to_f32(a.gamma[ch]),
                             to_f32(a.beta[ch]));
    }
    __syncthreads();
    ShiftedSums acc;
    float cnt = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t j = vec_of(k, r);
        if (j < end) {
            const Lay l = lay_of(j);
            form(xs[r], sv[r], l, sv[r]);
            accumulate(acc, cnt, sv[r], l);
        }
    }
    SN_PHASE(a.trace, 1);
    const Moments mine = block_merge_rcp(acc.moments(cnt), sh);
    SN_PHASE(a.trace, 2);

    // ---- exchange with the other K-1 slices of the group (as sgn_cluster_kernel)
    Moments tot = mine;
    if (a.K > 1) {
        uint64_t* slots = reinterpret_cast<uint64_t*>(a.part) + 2 * (int64_t(ng) * a.K);
        if (t == 0) publish_moments(&slots[2 * k], mine, a.tags);
        if (sa) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t j = vec_of(k, r);
                if (j < end) put(sa, j, lay_of(j), sv[r]);
            }
        }
        SN_PHASE(a.trace, 3);
        if (t < a.K && t != k) {
            const long long t0 = wall_clock64();
            bool ok = false;
            float mean = 0.0f, m2 = 0.0f;
            for (;;) {
                if (read_moments(&slots[2 * t], a.tags, &mean, &m2)) {
                    ok = true;
                    break;
                }
                if (wall_clock64() - t0 > a.timeout_ticks) break;
                __builtin_amdgcn_s_sleep(2);
            }
            late[t] = ok ? 0 : 1;
            if (ok) slice_m[t] = Moments{slice_count(t), mean, m2};
        }
        __syncthreads();
        tot = Moments{0.0f, 0.0f, 0.0f};
        for (int q = 0; q < a.K; ++q) {  // uniform over the workgroup
            Moments m;
            if (q == k) {
                m = mine;
            } else if (!late[q]) {
                m = slice_m[q];
            } else {
                // Slice q was not published in time: recompute its moments
                // exactly as its own workgroup does.
                const uint32_t qend = slice_end(q);
                ShiftedSums qacc;
                float qcnt = 0.0f;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint32_t j = vec_of(q, r);
                    if (j < qend) {
                        V x = load_vec<T, E>(xa, v0 + j), kv, sq;
                        if constexpr (!BCAST) kv = load_vec<T, E>(ka, v0 + j);
                        const Lay l = lay_of(j);
                        form(x, kv, l, sq);
                        accumulate(qacc, qcnt, sq, l);
                    }
                }
                m = block_merge_rcp(qacc.moments(qcnt), sh);
            }
            tot = merge_rcp(tot, m);
        }
    } else {
        if (sa) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t j = vec_of(k, r);
                if (j < end) put(sa, j, lay_of(j), sv[r]);
            }
        }
        SN_PHASE(a.trace, 3);
    }
    SN_PHASE(a.trace, 4);

    // ---- normalize the held S
    const float2 st = finalize(tot, a.eps);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t j = vec_of(k, r);
        if (j < end) {
            const Lay l = lay_of(j);
            const float4 c0 = cst[l.clo], c1 = cst[l.chi];
            const float scl0 = st.y * c0.z, scl1 = st.y * c1.z;
            V out;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const bool up = e >= l.nlo;
                float y = fmaf_(to_f32(sv[r].v[e]) - st.x, up ? scl1 : scl0, up ? c1.w : c0.w);
                if (a.silu) y = silu_f32(y);
                out.v[e] = from_f32<T>(y);
            }
            put(ya, j, l, out);
        }
    }
    SN_PHASE(a.trace, 5);
}

// ------------------------------------------------------------------ split: nhwc
// Block (n, b, cb) covers pixels [b*ppb, (b+1)*ppb) of image n and channel
// block cb: vectors [cb*CBv, (cb+1)*CBv) of each pixel's Cv, a whole number
// of groups.  Thread t owns vector cb*CBv + t % CBv at pixels t / CBv + k*P,
// P = 256 / CBv.
struct NhwcTile {
    int n, b, cv0, cvl, p0;
    bool active;
};

__device__ __forceinline__ NhwcTile nhwc_tile(int B, int NCB, int CBv, int P) {
    NhwcTile tl;
    const int cb = blockIdx.x % NCB, nb = blockIdx.x / NCB;
    tl.n = nb / B;
    tl.b = nb % B;
    tl.cv0 = cb * CBv;
    const int t = threadIdx.x;
    tl.active = t < P * CBv;
    tl.cvl = tl.active ? t % CBv : 0;
    tl.p0 = tl.active ? t / CBv : 0;
    return tl;
}

// Lanes (a power of two, at most 64) that combine each of `items` runs of
// `len` moments in the block's reductions: as many as keep all items within
// one pass of 256 threads, and no more than a run has values.  Each lane
// merges every w-th value of its run, then the w lanes combine in order
// (segment_merge), a fixed order for a given shape.
__device__ __forceinline__ int merge_lanes(int items, int len) {
    int w = 1;
    while (w < 64 && 2 * w * items <= 256 && w < len) w <<= 1;
    return w;
}

// Normalize blocks that combine their groups' partials themselves (no
// finalize launch): at most this many groups per block.
constexpr int kFoldMaxGroups = 64;

// Packed pixels (kpx > 1): element e of vector cv of a run of kpx pixels is
// channel (cv * E + e) mod C; bias and a broadcast skip row are read one
// channel at a time.
template <typename T, int E>
__device__ __forceinline__ void load_packed_params(const T* bias, bool has_bias, const T* skip,
                                                   bool skip_bcast, int n, int cv, int C, float (&bv)[E],
                                                   float (&kb)[E]) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int c = (cv * E + e) % C;
        if (has_bias) bv[e] = to_f32(bias[c]);
        if (skip_bcast) kb[e] = to_f32(skip[int64_t(n) * C + c]);
    }
}

template <typename T, int E>
__global__ void __launch_bounds__(256)
sgn_stats_nhwc_kernel(const T* __restrict__ X, const T* __restrict__ skip,
                      const T* __restrict__ bias, T* __restrict__ S, Partial* __restrict__ part,
                      int64_t HW, int Cv, int CBv, int NCB, int P, int cpg, int groups, int B,
                      int64_t ppb, bool skip_bcast, int kpx, int C) {
    using V = Vec<T, E>;
    __shared__ float sh_n[256 * E], sh_mean[256 * E], sh_m2[256 * E];
    const NhwcTile tl = nhwc_tile(B, NCB, CBv, P);
    const int n = tl.n, b = tl.b, p0 = tl.p0;
    const int cv = tl.cv0 + tl.cvl;
    const int Cw = CBv * E;  // channels of the block
    const int t = threadIdx.x;
    const bool active = tl.active;
    const int64_t pb = int64_t(b) * ppb;
    const int64_t pe = pb + ppb < HW ? pb + ppb : HW;
    const int64_t img = int64_t(n) * HW * Cv;
    const bool has_bias = bias != nullptr;
    const bool stream_in = S != nullptr;  // pass 3 reads S, not X and skip

    float bv[E] = {}, kb[E] = {};
    if (kpx == 1) {  // uniform
        if (active && has_bias) load_param_vec<T, E>(bias, cv, bv);
        if (active && skip_bcast) load_param_vec<T, E>(skip, int64_t(n) * Cv + cv, kb);
    } else if (active) {
        load_packed_params<T, E>(bias, has_bias, skip, skip_bcast, n, cv, C, bv, kb);
    }

    ShiftedSums acc[E];
    float cnt = 0.0f;
    if (active) {
        for (int64_t p = pb + p0; p < pe; p += kUnroll * P) {
            // Pixels past the block's end re-read pixel p (loads stay out of
            // lane-dependent branches); their values are discarded.
            V xs[kUnroll], ks[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int64_t pp = p + int64_t(u) * P;
                const int64_t pc = pp < pe ? pp : p;
                xs[u] = load_in<T, E>(X, img + pc * Cv + cv, stream_in);
                if (!skip_bcast) ks[u] = load_in<T, E>(skip, img + pc * Cv + cv, stream_in);
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
            const int slot = p0 * Cw + tl.cvl * E + e;
            sh_n[slot] = m.n;
            sh_mean[slot] = m.mean;
            sh_m2[slot] = m.m2;
        }
    }
    __syncthreads();
    // Per channel over the P pixel lanes (slots c, Cw + c, ...); the totals
    // go to row 0.
    {
        const int w = merge_lanes(Cw, P);
        const int lane = t & (w - 1);
        for (int c0 = 0; c0 < Cw; c0 += 256 / w) {
            const int c = c0 + t / w;
            Moments m{0.0f, 0.0f, 0.0f};
            if (c < Cw)
                for (int q = lane; q < P; q += w) {
                    const int slot = q * Cw + c;
                    m = merge(m, Moments{sh_n[slot], sh_mean[slot], sh_m2[slot]});
                }
            m = segment_merge(m, w);
            if (c < Cw && lane == 0) {
                sh_n[c] = m.n;
                sh_mean[c] = m.mean;
                sh_m2[c] = m.m2;
            }
        }
    }
    __syncthreads();
    // Per group of the block over its channels: with packed pixels (kpx > 1,
    // one block holds all C channels of kpx pixels) a group's channels in
    // pixel order, then channel order.
    {
        const int Cp = Cw / kpx;  // channels of the block per pixel
        const int g0 = tl.cv0 * E / cpg, gpb = Cp / cpg, len = kpx * cpg;
        const int w = merge_lanes(gpb, len);
        const int lane = t & (w - 1);
        for (int gl0 = 0; gl0 < gpb; gl0 += 256 / w) {
            const int gl = gl0 + t / w;
            Moments m{0.0f, 0.0f, 0.0f};
            if (gl < gpb)
                for (int i = lane; i < len; i += w) {
                    const int c = (i / cpg) * Cp + gl * cpg + i % cpg;
                    m = merge(m, Moments{sh_n[c], sh_mean[c], sh_m2[c]});
                }
            m = segment_merge(m, w);
            if (gl < gpb && lane == 0)
                part[(int64_t(n) * groups + g0 + gl) * B + b] = Partial{m.n, m.mean, m.m2, 0.0f};
        }
    }
}

template <typename T, typename M, int E>
__global__ void __launch_bounds__(256)
sgn_norm_nhwc_kernel(const T* __restrict__ X, const T* __restrict__ skip,
                     const T* __restrict__ bias, const T* __restrict__ S_in,
                     const M* __restrict__ gamma, const M* __restrict__ beta,
                     const float2* __restrict__ stat, T* __restrict__ Y, int64_t HW, int Cv,
                     int CBv, int NCB, int P, int cpg, int groups, int B, int64_t ppb,
                     bool skip_bcast, bool silu, int kpx, int C, const Partial* __restrict__ fold,
                     float eps) {
    using V = Vec<T, E>;
    const NhwcTile tl = nhwc_tile(B, NCB, CBv, P);
    // fold: no separate finalize pass; this block combines its own groups'
    // B partials (at most kFoldMaxGroups groups): wave w takes groups w,
    // w + 4, ..., lane l partials l, l + 64, ... in order, then a butterfly
    // over the wave.
    __shared__ float2 fold_st[kFoldMaxGroups];
    const int g0 = tl.cv0 * E / cpg;
    if (fold) {  // uniform
        const int gpb = CBv * E / kpx / cpg;
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        for (int gl = wave; gl < gpb; gl += 4) {
            const Partial* q = fold + (int64_t(tl.n) * groups + g0 + gl) * B;
            Moments m{0.0f, 0.0f, 0.0f};
            for (int b0 = 0; b0 < B; b0 += 4 * 64) {
                Partial v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int b = b0 + u * 64 + lane;
                    if (b < B) v[u] = q[b];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (b0 + u * 64 + lane < B) m = merge(m, as_moments(v[u]));
            }
            m = segment_merge(m, 64);
            if (lane == 0) fold_st[gl] = finalize(m, eps);
        }
        __syncthreads();
    }
    if (!tl.active) return;  // no barrier below
    const int n = tl.n, b = tl.b, p0 = tl.p0;
    const int cv = tl.cv0 + tl.cvl;
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
            const int64_t pc = pp < pe ? pp : p;  // discarded past the block's end
            if (S_in) {
                ss[u] = load_vec_stream<T, E>(S_in, img + pc * Cv + cv);
            } else {
                ss[u] = load_vec_stream<T, E>(X, img + pc * Cv + cv);
                if (!skip_bcast) ks[u] = load_vec_stream<T, E>(skip, img + pc * Cv + cv);
            }
        }
        if (first) {
            first = false;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int c = kpx == 1 ? cv * E + e : (cv * E + e) % C;  // packed: channel of the pixel
                const float2 st = fold ? fold_st[c / cpg - g0] : stat[int64_t(n) * groups + c / cpg];
                mean[e] = st.x;
                scl[e] = st.y * to_f32(gamma[c]);
                sft[e] = to_f32(beta[c]);
            }
            if (!S_in) {
                if (kpx == 1) {
                    if (has_bias) load_param_vec<T, E>(bias, cv, bv);
                    if (skip_bcast) load_param_vec<T, E>(skip, int64_t(n) * Cv + cv, kb);
                } else {
                    load_packed_params<T, E>(bias, has_bias, skip, skip_bcast, n, cv, C, bv, kb);
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
        // Vectors past the block's end re-read vector iv (loads stay out of
        // lane-dependent branches); their values are discarded.
        V xs[kUnroll], ks[kUnroll];
        T bias_u[kUnroll], kb_u[kUnroll];
        int64_t addr[kUnroll];
        int ch[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t j = iv + uint32_t(u) * 256;
            // With E > 1 (NCHW only) a vector never straddles channels.
            group_element<NCHW>(geo, n, g, (j < ve ? j : iv) * E, addr[u], ch[u]);
            xs[u] = load_in<T, E>(X, addr[u] / E, stream_in);
            if (!skip_bcast) ks[u] = load_in<T, E>(skip, addr[u] / E, stream_in);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (has_bias) bias_u[u] = bias[ch[u]];
            if (skip_bcast) kb_u[u] = skip[int64_t(n) * geo.C + ch[u]];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t j = iv + uint32_t(u) * 256;
            if (j < ve) {
                const float bb = has_bias ? to_f32(bias_u[u]) : 0.0f;
                const float kb = skip_bcast ? to_f32(kb_u[u]) : 0.0f;
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
        // Vectors past the block's end re-read vector iv (loads stay out of
        // lane-dependent branches); their values are discarded.
        V ss[kUnroll], ks[kUnroll];
        T bias_u[kUnroll], kb_u[kUnroll];
        M gam_u[kUnroll], bet_u[kUnroll];
        int64_t addr[kUnroll];
        int ch[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t j = iv + uint32_t(u) * 256;
            group_element<NCHW>(geo, n, g, (j < ve ? j : iv) * E, addr[u], ch[u]);
            if (S_in) {
                ss[u] = load_vec_stream<T, E>(S_in, addr[u] / E);
            } else {
                ss[u] = load_vec_stream<T, E>(X, addr[u] / E);
                if (!skip_bcast) ks[u] = load_vec_stream<T, E>(skip, addr[u] / E);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            gam_u[u] = gamma[ch[u]];
            bet_u[u] = beta[ch[u]];
            if (!S_in && has_bias) bias_u[u] = bias[ch[u]];
            if (!S_in && skip_bcast) kb_u[u] = skip[int64_t(n) * geo.C + ch[u]];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t j = iv + uint32_t(u) * 256;
            if (j < ve) {
                const float scl = st.y * to_f32(gam_u[u]);
                const float sft = to_f32(bet_u[u]);
                float bb = 0.0f, kb = 0.0f;
                if (!S_in) {
                    bb = has_bias ? to_f32(bias_u[u]) : 0.0f;
                    kb = skip_bcast ? to_f32(kb_u[u]) : 0.0f;
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

}  // namespace

// Channel blocks of the nhwc tiling for pixels of C channels read as vectors
// of E: NCB equal blocks of at most 256 vectors, each a whole number of
// groups and of vectors (so a multiple of lcm(cpg, E) channels).  The fewest
// blocks that keep at least 90 % of a block's threads busy (one block of
// 160 vectors would leave 96 of 256 idle; two of 80 leave 16), else the
// busiest.  False when no such block exists (a group wider than 256 vectors
// that is not a whole number of them, or C not a whole number of vectors).
bool nhwc_split_channel_blocks(int64_t C, int64_t cpg, int E, int* ncb_out) {
    if (E < 1 || C % E != 0 || cpg < 1 || C % cpg != 0) return false;
    int64_t x = cpg, y = E;
    while (y) {
        const int64_t r = x % y;
        x = y;
        y = r;
    }
    const int64_t unit = cpg / x * E;  // lcm(cpg, E) channels
    const int64_t nb0 = C / unit;
    int64_t best = 0, best_busy = -1;
    for (int64_t ncb = (C / E + 255) / 256; ncb <= nb0; ++ncb) {  // from the fewest of <= 256 vectors
        if (nb0 % ncb) continue;
        const int64_t cbv = C / E / ncb;
        if (cbv > 256) continue;
        const int64_t busy = 256 / cbv * cbv;
        if (busy > best_busy) {
            best_busy = busy;
            best = ncb;
        }
        if (busy * 10 >= 256 * 9) break;  // always reached once cbv <= 25
    }
    if (best == 0) return false;
    *ncb_out = int(best);
    return true;
}

namespace {

constexpr int kNhwcRowsPerThread = 2;                // least pixel rows per thread in the nhwc tiling
constexpr int64_t kSplitTargetBlocks = 2048;         // nhwc tiling: about 8 workgroups per CU in all

// The nhwc tiling for vectors of E channels: ncb channel blocks of CBv
// vectors, P = 256 / CBv pixel lanes, and runs of ppb = P * R pixels, so
// that every thread of a full run holds R pixels: at least
// kNhwcRowsPerThread, so that a small image still spreads over many CUs;
// more where the N images would take more than about kSplitTargetBlocks
// blocks (thousands of blocks of two pixels per thread spent their time in
// each block's reduction: 2.4 TB/s on a 256x256x512 float16 image); and,
// beyond one unrolled step, a whole number of them (a ragged last step
// issues loads whose values are discarded).
struct NhwcSplit {
    int ncb, P;
    int64_t ppb, B;
};

bool nhwc_split_plan(int64_t N, int64_t C, int64_t HW, int64_t groups, int E, NhwcSplit* sp) {
    int ncb = 0;
    if (N < 1 || HW < 1 || !nhwc_split_channel_blocks(C, C / groups, E, &ncb)) return false;
    const int64_t P = 256 / (C / E / ncb);
    int64_t R = (N * ncb * HW + P * kSplitTargetBlocks - 1) / (P * kSplitTargetBlocks);
    if (R < kNhwcRowsPerThread) R = kNhwcRowsPerThread;
    if (R > kUnroll) R = (R + kUnroll - 1) / kUnroll * kUnroll;
    sp->ncb = ncb;
    sp->P = int(P);
    sp->ppb = P * R;
    sp->B = (HW + sp->ppb - 1) / sp->ppb;
    return true;
}

// NHWC pixels that are not a whole number of 16-byte vectors: runs of kpx
// pixels that are (kpx = 16 / gcd(C * size, 16)), one channel block of all
// C channels per run, element e of vector v the run's channel (v * E + e)
// mod C.  Applies when H * W holds whole runs and a run is at most 256
// vectors; the tiling over runs is nhwc_split_plan's.
struct NhwcPacked {
    int kpx, SV, P;
    int64_t runs, ppb, B;
};

bool nhwc_packed_plan(int64_t N, int64_t C, int64_t HW, int size, NhwcPacked* pk) {
    int64_t g = C * size, h = 16;
    while (h) {
        const int64_t r = g % h;
        g = h;
        h = r;
    }
    const int64_t kpx = 16 / g, SV = kpx * C * size / 16;
    if (kpx < 2 || N < 1 || HW < 1 || HW % kpx != 0 || SV > 256) return false;
    pk->kpx = int(kpx);
    pk->SV = int(SV);
    pk->P = int(256 / SV);
    pk->runs = HW / kpx;
    int64_t R = (N * pk->runs + pk->P * kSplitTargetBlocks - 1) / (pk->P * kSplitTargetBlocks);
    if (R < kNhwcRowsPerThread) R = kNhwcRowsPerThread;
    if (R > kUnroll) R = (R + kUnroll - 1) / kUnroll * kUnroll;
    pk->ppb = pk->P * R;
    pk->B = (pk->runs + pk->ppb - 1) / pk->ppb;
    return true;
}

// Blocks per image (nhwc: pixel runs) or per (n, group) (group tiling: one
// unrolled pass of vectors each) of the split route, planned for 16-byte
// vectors; the partials per (n, group) the workspace holds.
int64_t split_blocks(int dtype, int64_t N, int64_t C, int64_t HW, int64_t groups, bool channels_last) {
    const int64_t ev = dtype == 0 ? 4 : 8;
    int64_t B;
    NhwcSplit sp;
    NhwcPacked pk;
    if (channels_last && nhwc_split_plan(N, C, HW, groups, int(ev), &sp)) {
        B = sp.B;
    } else if (channels_last && nhwc_packed_plan(N, C, HW, dtype == 0 ? 4 : 2, &pk)) {
        B = pk.B;
    } else {
        const int64_t per_unit = channels_last ? HW * C : (C / groups) * HW;  // image / group
        B = (per_unit + ev * kVectorsPerBlock - 1) / (ev * kVectorsPerBlock);
        if (channels_last && B > HW) B = HW;  // at least one pixel per block
    }
    if (B < 1) B = 1;
    if (B > 16384) B = 16384;
    return B;
}

// Vectors per thread a cluster workgroup holds: 16 sixteen-byte vectors or
// 32 scalars; with K <= 8 workgroups per group that bounds the groups this
// route takes (larger ones use the split route).
constexpr int kClusterMaxVec = 16;
constexpr int kClusterMaxScalar = 32;
constexpr int64_t kClusterTargetBlocks = 512;  // two workgroups per CU

template <typename T, typename M, int E, int R>
hipError_t launch_cluster_r(const ClusterArgs<T, M>& ca, int64_t blocks, hipStream_t stream) {
    if (ca.skip_bcast)
        hipLaunchKernelGGL((sgn_cluster_kernel<T, M, E, R, true>), dim3(unsigned(blocks)),
                           dim3(kClusterThreads), 0, stream, ca);
    else
        hipLaunchKernelGGL((sgn_cluster_kernel<T, M, E, R, false>), dim3(unsigned(blocks)),
                           dim3(kClusterThreads), 0, stream, ca);
    return hipGetLastError();
}

template <typename T, typename M, int E>
hipError_t launch_cluster_phase(const ClusterArgs<T, M>& ca, int64_t blocks, hipStream_t stream) {
    const uint32_t r = (ca.vps + kClusterThreads - 1) / kClusterThreads;
    auto go = [&](auto rt) {
        constexpr int R = decltype(rt)::value;
        if (ca.skip_bcast)
            hipLaunchKernelGGL((sgn_cluster_phase_kernel<T, M, E, R, true>), dim3(unsigned(blocks)),
                               dim3(kClusterThreads), 0, stream, ca);
        else
            hipLaunchKernelGGL((sgn_cluster_phase_kernel<T, M, E, R, false>), dim3(unsigned(blocks)),
                               dim3(kClusterThreads), 0, stream, ca);
        return hipGetLastError();
    };
    if (r <= 1) return go(std::integral_constant<int, 1>());
    if (r <= 2) return go(std::integral_constant<int, 2>());
    if (r <= 4) return go(std::integral_constant<int, 4>());
    return go(std::integral_constant<int, kPhaseMaxR>());
}

template <typename T, typename M, int E>
hipError_t launch_cluster(const ClusterArgs<T, M>& ca, int64_t blocks, hipStream_t stream) {
    const uint32_t r = (ca.vps + kClusterThreads - 1) / kClusterThreads;
    if constexpr (E > 1) {
        if (r <= 1) return launch_cluster_r<T, M, E, 1>(ca, blocks, stream);
        if (r <= 2) return launch_cluster_r<T, M, E, 2>(ca, blocks, stream);
        if (r <= 4) return launch_cluster_r<T, M, E, 4>(ca, blocks, stream);
        if (r <= 8) return launch_cluster_r<T, M, E, 8>(ca, blocks, stream);
        if (r <= 12) return launch_cluster_r<T, M, E, 12>(ca, blocks, stream);
        return launch_cluster_r<T, M, E, kClusterMaxVec>(ca, blocks, stream);
    } else {
        if (r <= 4) return launch_cluster_r<T, M, E, 4>(ca, blocks, stream);
        if (r <= 8) return launch_cluster_r<T, M, E, 8>(ca, blocks, stream);
        if (r <= 16) return launch_cluster_r<T, M, E, 16>(ca, blocks, stream);
        return launch_cluster_r<T, M, E, kClusterMaxScalar>(ca, blocks, stream);
    }
}

// Workgroups per (n, group) of the cluster route for a group of Kv vectors
// (0: the group is too large for it).
int cluster_k(int64_t Kv, int64_t NG, int max_r, int single_max_r = kSingleSliceMaxR) {
    if (Kv <= int64_t(kClusterThreads) * single_max_r) return 1;  // one slice, no exchange
    const int64_t cap = int64_t(kClusterThreads) * max_r;
    const int64_t k_fit = (Kv + cap - 1) / cap;
    if (k_fit > kClusterMaxK) return 0;
    int64_t k = (kClusterTargetBlocks + NG - 1) / NG;
    if (k < k_fit) k = k_fit;
    if (k > kClusterMaxK) k = kClusterMaxK;
    if (k > Kv) k = Kv > 0 ? Kv : 1;  // no empty slices
    return int(k);
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
    // NHWC: the widest access that divides a pixel's channels and every base
    // and splits the pixel into channel blocks of whole groups and vectors.
    int nhwc_e = 1;
    if (vec_allowed && a.channels_last) {
        nhwc_e = widest_vector<T>(a.C, {a.X, a.Y, a.S, a.skip, a.bias});
        int ncb = 0;
        if (nhwc_e > 1 && !nhwc_split_channel_blocks(a.C, cpg, nhwc_e, &ncb)) nhwc_e = 1;
    }
    const bool nchw_vec = vec_allowed && !a.channels_last && HW % EV == 0 && data_ok;
    // NCHW groups off the 16-byte grid (odd H*W, or data bases sharing an
    // offset from it): the phased cluster reads aligned 16-byte vectors
    // across the group boundaries, when H*W holds a vector, the group's
    // channel table fits, and X, skip, S and Y share their offset.
    bool nchw_phase = false;
    int phase = 0;
    if (vec_allowed && !a.channels_last && !nchw_vec && HW >= EV && cpg <= kPhaseMaxCpg) {
        const uintptr_t ph = reinterpret_cast<uintptr_t>(a.X) % 16;
        auto same = [&](const void* q) { return !q || reinterpret_cast<uintptr_t>(q) % 16 == ph; };
        nchw_phase = ph % sizeof(T) == 0 && same(a.Y) && same(a.S) && (a.skip_broadcast || same(a.skip));
        phase = int(ph / sizeof(T));
    }

    // ---- group-cluster route (NCHW)
    const int64_t B_ws = sgn_partials_per_group(a.dtype, a.N, a.C, a.H, a.W, a.groups, a.channels_last);
    Partial* part = static_cast<Partial*>(a.workspace);
    float2* stat = reinterpret_cast<float2*>(part + NG * B_ws);
    const bool cluster_route = !a.channels_last && want != Route::Split && want != Route::Block;
    if (cluster_route) {
        const int E = nchw_vec ? EV : 1;
        const int64_t Kv = nchw_phase ? K / EV + 2 : K / E;  // phased: vectors a group's span can touch
        // The phased route keeps one slice only up to two vectors per thread
        // (2 x 1280 x 15 x 15 float16, 1127 vectors a group: one slice
        // 11.5 us, eight 10.4 us).
        const int Kc = nchw_phase ? cluster_k(Kv, NG, kPhaseMaxR, 2)
                                  : cluster_k(Kv, NG, nchw_vec ? kClusterMaxVec : kClusterMaxScalar);
        if (Kc > 0) {
            ClusterArgs<T, M> ca;
            ca.X = X;
            ca.skip = skip;
            ca.bias = bias;
            ca.S = S;
            ca.Y = Y;
            ca.gamma = gamma;
            ca.beta = beta;
            ca.part = part;
            if (Kc > 1)
                if (hipError_t e = clear_publication_tags(a, part, NG * Kc, stream); e != hipSuccess)
                    return e;
            ca.tags = publication_tags(a.tag);
            ca.timeout_ticks = a.exchange_timeout_ticks;
            ca.HW = HW;
            ca.C = C;
            ca.cpg = cpg;
            ca.groups = groups;
            ca.K = Kc;
            ca.Kv = uint32_t(Kv);
            ca.vps = uint32_t((Kv + Kc - 1) / Kc);
            ca.div = make_fastdiv(uint32_t(HW));
            ca.skip_bcast = a.skip_broadcast;
            ca.silu = silu;
            ca.eps = a.epsilon;
            ca.phase = phase;
            ca.trace = a.trace;
            if (nchw_phase) {
                *route = "sgn.cluster.nchw.phase";
                return launch_cluster_phase<T, M, EV>(ca, NG * Kc, stream);
            }
            if (nchw_vec) {
                *route = "sgn.cluster.nchw.vec16";
                return launch_cluster<T, M, EV>(ca, NG * Kc, stream);
            }
            *route = "sgn.cluster.nchw.scalar";
            return launch_cluster<T, M, 1>(ca, NG * Kc, stream);
        }
    }

    // ---- channel-block cluster route (NHWC)
    hipError_t err = hipSuccess;
    if (launch_sgn_nhwc_cluster(a, want, part, stream, route, &err))
        return err;

    // ---- split route
    const int B = int(split_blocks(a.dtype, a.N, a.C, HW, a.groups, a.channels_last));
    const dim3 fin_grid = dim3(unsigned(NG));

    if (nhwc_e > 1) {
        // The plan for this access width; its pixel runs must fit the B
        // partials per (n, group) the workspace holds (planned for 16-byte
        // vectors), else the runs are stretched to B.
        NhwcSplit sp;
        nhwc_split_plan(a.N, a.C, HW, a.groups, nhwc_e, &sp);  // nhwc_e was checked above
        if (sp.B > B) {
            sp.ppb = ((HW + B - 1) / B + sp.P - 1) / sp.P * sp.P;
            sp.B = (HW + sp.ppb - 1) / sp.ppb;
        }
        const int Bn = int(sp.B), ncb = sp.ncb, P = sp.P;
        const int64_t ppb = sp.ppb;
        const dim3 grid(unsigned(a.N * Bn * ncb));
        auto launch = [&](auto tag, const char* name) {
            constexpr int E = decltype(tag)::value;
            const int Cv = C / E, CBv = Cv / ncb;
            *route = name;
            hipLaunchKernelGGL((sgn_stats_nhwc_kernel<T, E>), grid, dim3(256), 0, stream, X, skip, bias,
                               S, part, HW, Cv, CBv, ncb, P, cpg, groups, Bn, ppb, a.skip_broadcast, 1, C);
            hipLaunchKernelGGL(sgn_finalize_kernel, fin_grid, dim3(256), 0, stream, part, stat, Bn,
                               a.epsilon);
            hipLaunchKernelGGL((sgn_norm_nhwc_kernel<T, M, E>), grid, dim3(256), 0, stream, X, skip,
                               bias, static_cast<const T*>(S), gamma, beta, stat, Y, HW, Cv, CBv, ncb,
                               P, cpg, groups, Bn, ppb, a.skip_broadcast, silu, 1, C, nullptr, 0.0f);
            return hipGetLastError();
        };
        if (nhwc_e == EV) return launch(std::integral_constant<int, EV>(), "sgn.split.nhwc.vec16");
        if (nhwc_e == EV / 2) return launch(std::integral_constant<int, EV / 2>(), "sgn.split.nhwc.vec8");
        if constexpr (EV >= 8)
            if (nhwc_e == EV / 4) return launch(std::integral_constant<int, EV / 4>(), "sgn.split.nhwc.vec4");
    }

    // NHWC pixels that are not a whole number of 16-byte vectors: packed runs
    // of pixels (nhwc_packed_plan), when the data tensors are 16-byte aligned.
    NhwcPacked pk;
    if (a.channels_last && nhwc_e == 1 && vec_allowed && data_ok &&
        nhwc_packed_plan(a.N, C, HW, int(sizeof(T)), &pk)) {
        if (pk.B > B_ws) {  // within the partials the workspace holds
            pk.ppb = ((pk.runs + B_ws - 1) / B_ws + pk.P - 1) / pk.P * pk.P;
            pk.B = (pk.runs + pk.ppb - 1) / pk.ppb;
        }
        const int Bn = int(pk.B);
        const dim3 grid(unsigned(a.N * Bn));
        // Each normalize block combines the partials of all the image's
        // groups itself where they are few (at most 1024, 16 KB), in place
        // of the finalize launch (f16 8 x 128 x 128 x 15, 5 x 61 partials
        // a block: 22.8 -> 21.2 us; 16 x 256 x 256 x 3: 28.9 -> 27.6 us).
        const bool fold = groups <= kFoldMaxGroups && int64_t(groups) * Bn <= 1024;
        *route = fold ? "sgn.split.nhwc.packed.fold.vec16" : "sgn.split.nhwc.packed.vec16";
        hipLaunchKernelGGL((sgn_stats_nhwc_kernel<T, EV>), grid, dim3(256), 0, stream, X, skip, bias, S, part,
                           pk.runs, pk.SV, pk.SV, 1, pk.P, cpg, groups, Bn, pk.ppb, a.skip_broadcast, pk.kpx, C);
        if (!fold)
            hipLaunchKernelGGL(sgn_finalize_kernel, fin_grid, dim3(256), 0, stream, part, stat, Bn, a.epsilon);
        hipLaunchKernelGGL((sgn_norm_nhwc_kernel<T, M, EV>), grid, dim3(256), 0, stream, X, skip, bias,
                           static_cast<const T*>(S), gamma, beta, stat, Y, pk.runs, pk.SV, pk.SV, 1, pk.P, cpg,
                           groups, Bn, pk.ppb, a.skip_broadcast, silu, pk.kpx, C, fold ? part : nullptr,
                           a.epsilon);
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
    const int64_t b = split_blocks(dtype, N, C, H * W, groups, channels_last);
    const int64_t k = channels_last ? kNhwcMaxK : kClusterMaxK;
    return b >= k ? b : k;
}

// Workspace: N*groups*B partials of 16 bytes (the split route's partials, or
// the cluster routes' publication slots: at most 8 (NCHW) or 64 (NHWC) per
// (n, group)), then N*groups (mean, rstd) pairs.
size_t sgn_workspace_bytes(int dtype, int64_t N, int64_t C, int64_t H, int64_t W, int64_t groups,
                           bool channels_last) {
    const int64_t B = sgn_partials_per_group(dtype, N, C, H, W, groups, channels_last);
    const int64_t NG = N * groups;
    return size_t(NG * B) * sizeof(Partial) + size_t(NG) * sizeof(float2);
}

namespace {
__global__ void __launch_bounds__(256) sgn_clear_tags_kernel(uint64_t* __restrict__ words, int64_t n) {
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256)
        words[i] = 0;
}
}  // namespace

hipError_t clear_publication_tags(const SgnArgs& a, void* slots, int64_t n, hipStream_t stream) {
    if (!a.clear_tags || n <= 0) return hipSuccess;
    const int64_t words = 2 * n;
    const int64_t blocks = (words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024;
    hipLaunchKernelGGL(sgn_clear_tags_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream,
                       static_cast<uint64_t*>(slots), words);
    return hipGetLastError();
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

// ---------------------------------------------------------------------------
// Static scratch for skip_group_norm_noalloc: the workspace of callers that
// cannot allocate device memory (code being captured into a HIP graph, tight
// serving loops, hosts that forbid allocation).  Each device that runs the
// library holds its own copy of this array until the process ends.  Host
// code never passes `scratch` itself (on the host that name is a stand-in,
// not a device address): static_scratch() looks up the array's device
// address once per device, with that device current, and every launch takes
// that address.  Every call on one device shares the array; calls that
// overlap in time on one device (different streams, or host threads without
// ordering) race on it.  Its contents on entry never matter: each call writes
// every partial before reading it, and the single-launch routes accept only
// moments that carry the current call's tags (under graph capture the slots
// are cleared by a kernel ahead of the launch, as for a caller's workspace).
static __device__ __align__(256) unsigned char scratch[sn::kStaticScratchBytes];

namespace sn {

hipError_t static_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::atomic<void*> by_device[kMaxDevices];
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = by_device[dev].load(std::memory_order_acquire);
    if (!p) {
        // Idempotent: two threads that race here store the same address.
        if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        by_device[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace sn
