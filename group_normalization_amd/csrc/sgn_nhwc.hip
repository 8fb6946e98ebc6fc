// sgn_nhwc.hip -- SkipGroupNorm, NHWC channel-block cluster route (gfx950).
// The operator and the other routes are described in sgn.hip.
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "sgn_common.h"

namespace sn {
namespace {

// ------------------------------------------------------------------ channel-block cluster (NHWC)
// In NHWC a group's channels are a short run inside every pixel, so a group
// is not contiguous.  The channels are cut into NCB blocks, each a whole
// number of groups and of 16-byte vectors (a multiple of lcm(cpg, E)
// channels), and an image's pixels into K slices; one workgroup of 256
// threads owns one (image, slice, channel block).  Thread t owns channel
// vector v = t % CBv of the block at pixels t / CBv + r * P (P = 256 / CBv
// pixel lanes), so its channels never change, and holds S for those pixels
// in VGPRs.
//
// A slice's per-group moments: each thread keeps shifted sums for the (at
// most two, as cpg >= E) groups its vector touches; the pixel lanes of each
// (vector, group) column are merged in LDS, chunk by chunk and then by an
// ordered DPP butterfly; each group merges its columns in channel order.
// The K slices of an (image, block) exchange these moments as the
// group-cluster route does (per-call tags, bounded waits, a late slice
// recomputed with the same code) and each wave combines its groups over the
// K slices with an ordered butterfly in slice order, so every workgroup of
// the cluster holds bitwise the same statistics.  One launch: X and skip are
// read once, S and Y written once.
//
// Block ids are laid out so that the NCB channel blocks of one (image,
// slice) share the id's residue mod 8: consecutive ids are dispatched
// round-robin over the 8 XCDs, so those workgroups, which touch the same
// pixel rows and share their boundary cache lines, run under one L2.  The
// data accesses are ordinary (cached) ones so that this L2 merges the
// blocks' pieces of a line: with nontemporal stores the partial lines
// reached memory separately (1.3-1.5x the written bytes, measured).  Two
// orders (NhwcLayout): slice-major, where the channel blocks of eight
// (image, slice) units follow one another, so that what starts together
// reads contiguous pixel rows; and cluster-major, where a cluster's slices
// are consecutive ids, for grids whose clusters would otherwise spread
// over more ids than the device holds at once.
template <typename T, typename M>
struct NhwcClusterArgs {
    const T *X, *skip, *bias;
    T *S, *Y;
    const M *gamma, *beta;
    Partial* part;     // N * NCB * K * CBg publication slots
    PubTags tags;      // this call's publication tags
    long long timeout_ticks;
    int64_t HW, pps;   // pixels per image and per slice
    int Cv, cpg;       // vectors per pixel, channels per group
    int CBv, NCB, CBg; // vectors per channel block, blocks per pixel, groups per block
    int P, sw_log;     // pixel lanes per workgroup (256 / CBv); log2 of the chunks per column
    int K;             // slices per image
    int N, Kp, G;      // images; block-id layout (NhwcLayout)
    // Invariant divisors (one multiply-high each instead of a division in
    // the set-up every load address waits for).
    FastDiv div_G, div_NCB, div_K, div_CBv, div_cpg, div_P;
    bool skip_bcast, silu;
    float eps;
    unsigned long long* trace;  // phase timestamps (measurement builds)
    int C;    // channels per pixel (packed runs: element e of vector v is channel (v * E + e) mod C)
    int kpx;  // pixels per unit: 1, or the pixels of a packed run
};

constexpr int kNhwcMaxCBg = 16;   // groups per channel block: four per wave
constexpr int kNhwcMaxR = 16;     // pixels per thread
constexpr int kWaves = kClusterThreads / 64;
constexpr int kGroupsPerWave = kNhwcMaxCBg / kWaves;

// PACKED: a unit is a run of kpx pixels that is a whole number of 16-byte
// vectors (pixels of C channels whose bytes are not), one channel block of
// all kpx * C channels; element e of vector v is channel (v * E + e) mod C,
// so a vector may touch any number of groups.  Each thread then keeps
// shifted sums per element (a column per element instead of per group slot),
// and group g merges its columns in pixel, then channel order.
template <typename T, typename M, int E, int R, bool BCAST, bool PACKED>
__global__ void __launch_bounds__(kClusterThreads)
sgn_nhwc_cluster_kernel(NhwcClusterArgs<T, M> a) {
    using V = Vec<T, E>;
    constexpr int kCols = PACKED ? E : 2;  // columns per vector
    __shared__ Moments lane_m[kCols * kClusterThreads];  // [pixel lane][column = kCols * vector + slot]
    __shared__ Moments col_m[kCols * kClusterThreads];   // column totals
    __shared__ Moments own_m[kNhwcMaxCBg];           // this slice's group moments
    __shared__ Moments slice_m[kNhwcMaxK][kNhwcMaxCBg];  // recomputed slices
    __shared__ float2 stat[kNhwcMaxCBg];
    __shared__ int late[kNhwcMaxK];
    __shared__ int any_late;

    // Block id = ((item / m * NCB + cb) * G + (item % m) * Kp + j), m = G / Kp
    // (see NhwcLayout): an item is an (image, slice) unit when Kp == 1, else
    // an image whose slices j take Kp consecutive ids.
    // Slice-major: G = 8, Kp = 1, item = (image, slice) unit; cluster-major:
    // G = Kp, item = image.
    const uint32_t bid = blockIdx.x;
    const uint32_t rest = fastdiv(bid, a.div_G), r = bid - rest * uint32_t(a.G);
    const uint32_t hi = fastdiv(rest, a.div_NCB);
    const int cb = int(rest - hi * uint32_t(a.NCB));
    int n, q;
    if (a.Kp == 1) {  // uniform
        const uint32_t unit = hi * 8 + r;
        n = int(fastdiv(unit, a.div_K));
        q = int(unit - uint32_t(n) * uint32_t(a.K));
    } else {
        n = int(hi);
        q = int(r);
    }
    if (q >= a.K || n >= a.N) return;  // padding; not part of any cluster
    SN_PHASE(a.trace, 0);
    const int t = threadIdx.x;
    const int wave = t >> 6, lane = t & 63;
    const bool active = t < a.P * a.CBv;
    const int pl = active ? int(fastdiv(uint32_t(t), a.div_CBv)) : 0;
    const int v = active ? t - pl * a.CBv : 0;
    const int cvec = cb * a.CBv + v;  // channel vector within the pixel
    const int glo = int(fastdiv(uint32_t(v * E), a.div_cpg));  // block-local group of the vector's first channel
    const int split = (glo + 1) * a.cpg - v * E;  // channels [0, split) are in glo, the rest in glo + 1
    const int ncol = kCols * a.CBv;
    const int SW = 1 << a.sw_log;
    const int64_t img = int64_t(n) * a.HW;
    const bool has_bias = a.bias != nullptr;
    if (t < kNhwcMaxK) late[t] = 0;
    if (t == 0) any_late = 0;

    // Pixels of slice s this thread holds (they are consecutive in r).
    auto slice_len = [&](int s) {
        const int64_t rem = a.HW - int64_t(s) * a.pps;
        return rem < a.pps ? rem : a.pps;
    };
    auto nvalid = [&](int s) {
        const int64_t len = slice_len(s);
        if (!active || len <= pl) return 0;
        const int64_t nv = fastdiv(uint32_t(len - pl + a.P - 1), a.div_P);  // len <= pps < 2^31
        return nv < R ? int(nv) : R;
    };
    auto vidx = [&](int s, int r) {
        return (img + int64_t(s) * a.pps + pl + int64_t(r) * a.P) * a.Cv + cvec;
    };
    // Per-channel constants: bias and broadcast skip (as T), gamma, beta.
    // Packed: per element, by its channel.
    V bvec, kvec;
    M gam[E], bet[E];
    int ch[PACKED ? E : 1];
    if constexpr (PACKED) {
        int c = (cvec * E) % a.C;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            ch[e] = c;
            c = c + 1 == a.C ? 0 : c + 1;
        }
    }
    auto load_constants = [&]() {
        if constexpr (PACKED) {
            const T* bias_src = has_bias ? a.bias : a.X;  // X holds at least C elements
#pragma unroll
            for (int e = 0; e < E; ++e) {
                bvec.v[e] = bias_src[ch[e]];
                if constexpr (BCAST) kvec.v[e] = a.skip[int64_t(n) * a.C + ch[e]];
                gam[e] = a.gamma[ch[e]];
                bet[e] = a.beta[ch[e]];
            }
        } else {
            bvec = load_vec<T, E>(has_bias ? a.bias : a.X, cvec);  // X holds at least C elements
            if constexpr (BCAST) kvec = load_vec<T, E>(a.skip, int64_t(n) * a.Cv + cvec);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                gam[e] = a.gamma[cvec * E + e];
                bet[e] = a.beta[cvec * E + e];
            }
        }
    };
    auto form = [&](const V& x, const V& kv, V& s) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float kk = BCAST ? to_f32(kvec.v[e]) : to_f32(kv.v[e]);
            const float bb = has_bias ? to_f32(bvec.v[e]) : 0.0f;
            residual_sum<T>(to_f32(x.v[e]), kk, has_bias, bb, s.v[e]);
        }
    };
    // Shifted sums of the thread's two groups over its pixels of a slice, in
    // pixel then channel order; the shifts are the first pixel's first and
    // last channels (the last channel is in the upper group when it exists).
    // Packed: one per element, shifted by its value in the first unit.
    struct SlotSums {
        ShiftedSums lo, hi;
    };
    struct ElemSums {
        ShiftedSums el[E];
    };
    using Acc = typename std::conditional<PACKED, ElemSums, SlotSums>::type;
    auto accumulate = [&](Acc& acc, const V& s, int r) {
        if constexpr (PACKED) {
#pragma unroll
            for (int e = 0; e < E; ++e) acc.el[e].add(to_f32(s.v[e]), r == 0);
        } else {
            if (r == 0) {
                acc.lo.shift = to_f32(s.v[0]);
                acc.hi.shift = to_f32(s.v[E - 1]);
            }
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float x = to_f32(s.v[e]);
                const bool in_lo = e < split;
                const float d = x - (in_lo ? acc.lo.shift : acc.hi.shift);
                const float dl = in_lo ? d : 0.0f, dh = in_lo ? 0.0f : d;
                acc.lo.s1 += dl;
                acc.lo.s2 = fmaf_(dl, dl, acc.lo.s2);
                acc.hi.s1 += dh;
                acc.hi.s2 = fmaf_(dh, dh, acc.hi.s2);
            }
        }
    };
    // Group moments of a slice from every thread's sums over its nv pixels,
    // into dst[0 .. CBg).  The same code and thread mapping run wherever a
    // slice is reduced.  Ends with dst written, by thread g for group g
    // (packed: visible to every thread).
    auto reduce_slice = [&](const Acc& acc, int nv, Moments* dst) {
        if (active) {
            if constexpr (PACKED) {
#pragma unroll
                for (int e = 0; e < E; ++e) lane_m[pl * ncol + E * v + e] = acc.el[e].moments(float(nv));
            } else {
                const int nlo = split < E ? split : E;
                lane_m[pl * ncol + 2 * v] = acc.lo.moments(float(nv * nlo));
                lane_m[pl * ncol + 2 * v + 1] = acc.hi.moments(float(nv * (E - nlo)));
            }
        }
        __syncthreads();
        // Column c, chunk j: pixel lanes j, j + SW, ... in order; then the SW
        // chunks (adjacent lanes of one DPP row) in an ordered butterfly.
        for (int i0 = 0; i0 < ncol * SW; i0 += kClusterThreads) {
            const int i = i0 + t;
            const bool on = i < ncol * SW;
            const int c = i >> a.sw_log, j = i & (SW - 1);
            Moments m{0.0f, 0.0f, 0.0f};
            if (on) {
                // Up to four lanes' loads in flight per step.
                for (int l0 = j; l0 < a.P; l0 += 4 * SW) {
                    Moments x[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int l = l0 + k * SW;
                        x[k] = l < a.P ? lane_m[l * ncol + c] : Moments{0.0f, 0.0f, 0.0f};
                    }
#pragma unroll
                    for (int k = 0; k < 4; ++k) m = merge_rcp(m, x[k]);
                }
            }
            m = segment_merge(m, SW);
            if (on && j == 0) col_m[c] = m;
        }
        __syncthreads();
        if constexpr (PACKED) {
            // Group g over its kpx * cpg columns (pixel, then channel order):
            // w lanes per group, lane l merging columns l, l + w, ... in
            // order, then an ordered butterfly over the w lanes.
            const int len = a.kpx * a.cpg;
            int w = 1;
            while (w < 16 && 2 * w * a.CBg <= kClusterThreads && w < len) w <<= 1;
            const int gi = t / w, li = t - gi * w;
            Moments m{0.0f, 0.0f, 0.0f};
            if (gi < a.CBg)
                for (int i = li; i < len; i += w) {
                    const int p = int(fastdiv(uint32_t(i), a.div_cpg));
                    m = merge_rcp(m, col_m[p * a.C + gi * a.cpg + (i - p * a.cpg)]);
                }
            m = segment_merge(m, w);
            if (gi < a.CBg && li == 0) dst[gi] = m;
            __syncthreads();  // dst[g] is read by thread g (publication), not its writer
        } else if (t < a.CBg) {  // group t over its columns, in channel order
            const int vf = (t * a.cpg) / E, vl = ((t + 1) * a.cpg - 1) / E;
            Moments m{0.0f, 0.0f, 0.0f};
            for (int w = vf; w <= vl; ++w)
                m = merge_rcp(m, col_m[2 * w + (int(fastdiv(uint32_t(w * E), a.div_cpg)) == t ? 0 : 1)]);
            dst[t] = m;
        }
    };

    // ---- own slice: S into registers, slice moments.  With vector accesses
    // the per-channel constants load first: loads retire in order, so each
    // pixel's sums can then start once its own data is in (2 x 64 x 64 x 320
    // float16 2.6 % faster); with element accesses, whose constants are single
    // values, the data go first (constants first measured 2.7 % slower).  No
    // load sits behind a branch (the compiler would wait for each in turn):
    // bias is read from X when absent, and a thread's accesses past its
    // pixels re-read the slice's first pixel and are discarded.
    const int nv_own = nvalid(q);
    const int64_t first_px = (img + int64_t(q) * a.pps) * a.Cv + cvec;
    auto own_idx = [&](int r) { return r < nv_own ? vidx(q, r) : first_px; };
    V sv[R];
    {
        V xs[R];
        if constexpr (E > 1) load_constants();
#pragma unroll
        for (int r = 0; r < R; ++r) {
            xs[r] = load_vec<T, E>(a.X, own_idx(r));
            if constexpr (!BCAST) sv[r] = load_vec<T, E>(a.skip, own_idx(r));
        }
        if constexpr (E == 1) load_constants();
        Acc acc;
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (r < nv_own) {
                form(xs[r], sv[r], sv[r]);
                accumulate(acc, sv[r], r);
            }
        SN_PHASE(a.trace, 1);
        reduce_slice(acc, nv_own, own_m);
        SN_PHASE(a.trace, 2);
    }

    // ---- publication: per group, (mean, M2) in its self-tagged slot.
    const int64_t first = (int64_t(n) * a.NCB + cb) * a.K * a.CBg;  // slice 0 of this (image, block)
    uint64_t* slots = reinterpret_cast<uint64_t*>(a.part) + 2 * first;  // two words per (slice, group)
    auto slot = [&](int s, int g) { return &slots[2 * (s * a.CBg + g)]; };
    if (a.K > 1 && t < a.CBg) publish_moments(slot(q, t), own_m[t], a.tags);
    if (a.S) {
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (r < nv_own) store_vec<T, E>(a.S, vidx(q, r), sv[r]);
    }
    SN_PHASE(a.trace, 3);
    __syncthreads();  // own_m visible to every wave

    // ---- statistics: wave w combines groups w, w + 4, ... over the K slices,
    // lane s holding slice s (butterfly over the smallest power of two >= K
    // lanes; the lanes beyond K hold empty moments).
    int kw = 1;
    while (kw < a.K) kw <<= 1;
    auto slice_count = [&](int s) {
        if constexpr (PACKED) return float(slice_len(s) * a.kpx * a.cpg);
        else return float(slice_len(s) * a.cpg);
    };
    auto combine = [&](const Moments (&m)[kGroupsPerWave]) {
#pragma unroll
        for (int i = 0; i < kGroupsPerWave; ++i) {
            const int g = wave + i * kWaves;
            if (g < a.CBg) {  // uniform over the wave
                const Moments tot = segment_merge(m[i], kw);
                if (lane == 0) stat[g] = finalize(tot, a.eps);
            }
        }
    };
    bool wave_late = false;
    if (wave < a.CBg) {
        Moments m[kGroupsPerWave];
        bool ok = true;
        if (lane == q) {
#pragma unroll
            for (int i = 0; i < kGroupsPerWave; ++i) {
                const int g = wave + i * kWaves;
                m[i] = g < a.CBg ? own_m[g] : Moments{0.0f, 0.0f, 0.0f};
            }
        } else if (lane < a.K) {
            const long long t0 = wall_clock64();
            float mean[kGroupsPerWave], m2[kGroupsPerWave];
            for (;;) {
                bool ready = true;
#pragma unroll
                for (int i = 0; i < kGroupsPerWave; ++i) {
                    const int g = wave + i * kWaves;
                    mean[i] = m2[i] = 0.0f;
                    if (g < a.CBg) ready &= read_moments(slot(lane, g), a.tags, &mean[i], &m2[i]);
                }
                if (ready) break;
                if (wall_clock64() - t0 > a.timeout_ticks) {
                    ok = false;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
#pragma unroll
            for (int i = 0; i < kGroupsPerWave; ++i)
                m[i] = ok ? Moments{slice_count(lane), mean[i], m2[i]} : Moments{0.0f, 0.0f, 0.0f};
            if (!ok) late[lane] = 1;
        } else {
#pragma unroll
            for (int i = 0; i < kGroupsPerWave; ++i) m[i] = Moments{0.0f, 0.0f, 0.0f};
        }
        wave_late = __any(!ok);
        if (!wave_late) combine(m);
        else if (lane == 0) any_late = 1;
    }
    __syncthreads();

    // ---- slow path: some slice was not published in time.  Every slice some
    // wave found late is reduced here with the code its owner runs; the waves
    // that found one combine their groups again.
    if (any_late) {  // uniform: written before the barrier
        for (int s = 0; s < a.K; ++s) {
            if (!late[s]) continue;  // uniform
            const int nv = nvalid(s);
            Acc acc;
#pragma unroll
            for (int r = 0; r < R; ++r)
                if (r < nv) {
                    V xv = load_vec<T, E>(a.X, vidx(s, r)), kv, sr;
                    if constexpr (!BCAST) kv = load_vec<T, E>(a.skip, vidx(s, r));
                    form(xv, kv, sr);
                    accumulate(acc, sr, r);
                }
            reduce_slice(acc, nv, slice_m[s]);
            __syncthreads();
        }
        if (wave_late) {
            Moments m[kGroupsPerWave];
#pragma unroll
            for (int i = 0; i < kGroupsPerWave; ++i) {
                const int g = wave + i * kWaves;
                m[i] = Moments{0.0f, 0.0f, 0.0f};
                if (g < a.CBg) {
                    if (lane == q) m[i] = own_m[g];
                    else if (lane < a.K && late[lane]) m[i] = slice_m[lane][g];
                    else if (lane < a.K) {  // this wave saw its tags: the slot holds this call's values
                        float mean = 0.0f, m2 = 0.0f;
                        read_moments(slot(lane, g), a.tags, &mean, &m2);
                        m[i] = Moments{slice_count(lane), mean, m2};
                    }
                }
            }
            combine(m);
        }
        __syncthreads();
    }

    SN_PHASE(a.trace, 4);

    // ---- normalize the held S
    if (nv_own > 0) {
        float2 slo, shi;  // the (at most two) groups of the vector (not packed)
        if constexpr (!PACKED) {
            slo = stat[glo];
            shi = stat[glo + 1 < a.CBg ? glo + 1 : glo];
        }
        float mean[E], scl[E], sft[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float2 st;
            if constexpr (PACKED) st = stat[fastdiv(uint32_t(ch[e]), a.div_cpg)];
            else st = e < split ? slo : shi;
            mean[e] = st.x;
            scl[e] = st.y * to_f32(gam[e]);
            sft[e] = to_f32(bet[e]);
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (r < nv_own) {
                V out;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    float y = fmaf_(to_f32(sv[r].v[e]) - mean[e], scl[e], sft[e]);
                    if (a.silu) y = silu_f32(y);
                    out.v[e] = from_f32<T>(y);
                }
                store_vec<T, E>(a.Y, vidx(q, r), out);
            }
    }
    SN_PHASE(a.trace, 5);
}

// Channel-block cluster plan.  Channel blocks: the fewest (so the most
// channels per workgroup, for coalescing) with at most one group per wave,
// which keeps each wave's combine to one butterfly; among those, the first
// whose grid reaches kNhwcTargetBlocks workgroups (two per CU: fewer leave
// the loads short of bandwidth, more lengthen the exchange more than they
// shorten the streaming).  Slices are as few as that target allows, no more
// than leave each thread about one vector, and as many as the register
// budget (kNhwcMaxR pixels per thread) needs.
constexpr int64_t kNhwcTargetBlocks = 512;
// Slices per cluster where the register budget allows: every slice's
// moments are polled by every other slice's waves (two words per group),
// and beyond 32 slices that traffic cost more than the added workgroups
// bought (1 x 64 x 64 x 320 float16: 64 slices 13.3 us, 32 slices 10.9 us).
constexpr int64_t kNhwcExchangeK = 32;

struct NhwcPlan {
    int CBv, NCB, CBg, P, sw_log, K, R;
    int64_t pps;
};

bool nhwc_cluster_plan(int E, int64_t N, int64_t C, int64_t HW, int64_t groups, NhwcPlan* out) {
    const int64_t cpg = C / groups;
    if (N < 1 || HW < 1 || C % E != 0 || cpg < E) return false;
    int64_t x = cpg, y = E;
    while (y) {
        const int64_t r = x % y;
        x = y;
        y = r;
    }
    const int64_t nb0 = C / (cpg / x * E);  // blocks of lcm(cpg, E) channels
    // Pass 0: at most one group per wave; pass 1: up to four.  Element
    // accesses (E = 1) start from pass 1: its wider blocks give each wave
    // longer runs of a pixel (f16 8 x 64 x 64 x 320 with a group per channel:
    // 16-channel blocks 2.0 TB/s against 1.6 in 4-channel ones; f32 4 x 128 x
    // 64 x 64: 1.9 against 1.2).
    for (int pass = E == 1 ? 1 : 0; pass < 2; ++pass) {
        bool found = false;
        int64_t best_grid = 0;
        for (int64_t ncb = 1; ncb <= nb0; ++ncb) {
            if (nb0 % ncb) continue;
            const int64_t cbv = C / ncb / E, cbg = C / ncb / cpg;
            if (cbv > kClusterThreads || cbg > (pass == 0 ? kWaves : kNhwcMaxCBg)) continue;
            const int64_t P = kClusterThreads / cbv;
            const int64_t k_fit = (HW + P * kNhwcMaxR - 1) / (P * kNhwcMaxR);
            if (k_fit > kNhwcMaxK) continue;
            int64_t K = (kNhwcTargetBlocks + N * ncb - 1) / (N * ncb);
            const int64_t k_work = HW * cbv / kClusterThreads;  // at least one vector per thread
            if (K > k_work) K = k_work;
            if (K > kNhwcExchangeK) K = kNhwcExchangeK;
            if (K < k_fit) K = k_fit;
            if (K > kNhwcMaxK) K = kNhwcMaxK;
            if (K > HW) K = HW;
            if ((HW + P - 1) / P <= kSingleSliceMaxR) K = 1;  // one slice, no exchange
            const int64_t pps = (HW + K - 1) / K;
            K = (HW + pps - 1) / pps;  // no empty slices
            const int64_t grid = N * ncb * K;
            if (!found || grid > best_grid) {
                found = true;
                best_grid = grid;
                out->CBv = int(cbv);
                out->NCB = int(ncb);
                out->CBg = int(cbg);
                out->P = int(P);
                // Chunks per column in the pixel-lane reduction: a power of
                // two, at most 16 (one DPP row), 2 * cbv columns * chunks <= 256.
                int sw = 16;
                while (sw > 1 && (2 * cbv * sw > kClusterThreads || sw / 2 >= P)) sw >>= 1;
                int sw_log = 0;
                while ((1 << sw_log) < sw) ++sw_log;
                out->sw_log = sw_log;
                out->K = int(K);
                out->pps = pps;
                out->R = int((pps + P - 1) / P);
            }
            if (grid >= kNhwcTargetBlocks) break;
        }
        if (found) return true;
    }
    return false;
}

// When the packed runs are taken over the channel-block form (element or
// narrow accesses), measured on 19 images: a run carries eight times the data
// of an element access, so a small image gets few workgroups, and each thread
// merges per element.  Packed runs won with at least one workgroup per CU
// (8 x 128 x 128 x 15 float32: 15.5 against 20.5 us; 16 x 256 x 256 x 3
// float16: 16.0 against 17.9), with at least 12 runs per thread on at least
// 96 workgroups (4 x 256 x 256 x 15 float32: 20.3 against 32.2 us; 6 x 200
// x 256 x 15 float16: 20.2 against 23.6), and wherever the channel-block
// form has no plan (the split route instead: 2 x 512 x 512 x 3 float16: 17.0
// against 19.7 us); they lost with few runs per thread (4 x 128 x 128 x 15:
// +10 %) or few workgroups (2 x 256 x 256 x 15, 64 workgroups: +14 %;
// 1 x 340 x 256 x 15, 40: +39 %).
constexpr int64_t kNhwcPackedMinBlocks = 256;
constexpr int64_t kNhwcPackedDeepBlocks = 96;  // with at least kNhwcPackedDeepR runs per thread
constexpr int kNhwcPackedDeepR = 12;
bool nhwc_packed_preferred(int64_t N, const NhwcPlan& packed, bool block_fits) {
    const int64_t grid = N * packed.K;
    return !block_fits || grid >= kNhwcPackedMinBlocks ||
           (packed.R >= kNhwcPackedDeepR && grid >= kNhwcPackedDeepBlocks);
}

// Packed-run plan for pixels whose C channels are not a whole number of
// 16-byte vectors: units of kpx = 16 / gcd(C * size, 16) pixels, CBv =
// kpx * C * size / 16 vectors each, read whole by one channel block that
// holds every group; slices as in nhwc_cluster_plan.  Needs H * W a whole
// number of units, a unit of at most 256 vectors and at most kNhwcMaxCBg
// groups.
bool nhwc_packed_cluster_plan(int size, int64_t N, int64_t C, int64_t HW, int64_t groups, NhwcPlan* out,
                              int* kpx_out) {
    int64_t x = C * size, y = 16;
    while (y) {
        const int64_t r = x % y;
        x = y;
        y = r;
    }
    const int64_t kpx = 16 / x;
    if (kpx == 1 || N < 1 || HW < 1 || HW % kpx != 0 || groups > kNhwcMaxCBg) return false;
    const int64_t E = 16 / size;
    const int64_t cbv = kpx * C * size / 16;
    if (cbv > kClusterThreads) return false;
    const int64_t units = HW / kpx;
    const int64_t P = kClusterThreads / cbv;
    const int64_t k_fit = (units + P * kNhwcMaxR - 1) / (P * kNhwcMaxR);
    if (k_fit > kNhwcMaxK) return false;
    int64_t K = (kNhwcTargetBlocks + N - 1) / N;
    const int64_t k_work = units * cbv / kClusterThreads;  // at least one vector per thread
    if (K > k_work) K = k_work;
    if (K > kNhwcExchangeK) K = kNhwcExchangeK;
    if (K < k_fit) K = k_fit;
    if (K > kNhwcMaxK) K = kNhwcMaxK;
    if (K > units) K = units;
    if ((units + P - 1) / P <= kSingleSliceMaxR) K = 1;  // one slice, no exchange
    const int64_t pps = (units + K - 1) / K;
    K = (units + pps - 1) / pps;  // no empty slices
    out->CBv = int(cbv);
    out->NCB = 1;
    out->CBg = int(groups);
    out->P = int(P);
    int sw = 16;  // chunks per column: E columns per vector
    while (sw > 1 && (E * cbv * sw > kClusterThreads || sw / 2 >= P)) sw >>= 1;
    int sw_log = 0;
    while ((1 << sw_log) < sw) ++sw_log;
    out->sw_log = sw_log;
    out->K = int(K);
    out->pps = pps;
    out->R = int((pps + P - 1) / P);
    *kpx_out = int(kpx);
    return true;
}

// Workgroups of `kernel` (256 threads) that the current device holds at once:
// its occupancy per CU times the CUs, queried once per device and kernel.
int resident_workgroups(const void* kernel) {
    static std::mutex mu;
    static std::map<std::pair<int, const void*>, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    const auto key = std::make_pair(dev, kernel);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kClusterThreads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;  // unknown: the caller takes another route
    return cache[key] = per_cu * cus;
}

template <typename T, typename M, int E, int R, bool PACKED = false>
const void* nhwc_kernel_r(bool bcast) {
    return bcast ? reinterpret_cast<const void*>(&sgn_nhwc_cluster_kernel<T, M, E, R, true, PACKED>)
                 : reinterpret_cast<const void*>(&sgn_nhwc_cluster_kernel<T, M, E, R, false, PACKED>);
}

// The kernel launch_nhwc_cluster runs for r pixels (units) per thread.
template <typename T, typename M, int E, bool PACKED = false>
const void* nhwc_kernel(int r, bool bcast) {
    if (r <= 1) return nhwc_kernel_r<T, M, E, 1, PACKED>(bcast);
    if (r <= 2) return nhwc_kernel_r<T, M, E, 2, PACKED>(bcast);
    if (r <= 4) return nhwc_kernel_r<T, M, E, 4, PACKED>(bcast);
    if (r <= 8) return nhwc_kernel_r<T, M, E, 8, PACKED>(bcast);
    return nhwc_kernel_r<T, M, E, kNhwcMaxR, PACKED>(bcast);
}

template <typename T, typename M>
const void* nhwc_kernel_for(int E, int r, bool bcast) {
    constexpr int EV = VecWidth<T>::value;
    if (E == EV) return nhwc_kernel<T, M, EV>(r, bcast);
    if (E == EV / 2) return nhwc_kernel<T, M, EV / 2>(r, bcast);
    if constexpr (EV >= 8)
        if (E == EV / 4) return nhwc_kernel<T, M, EV / 4>(r, bcast);
    if (E == 1) return nhwc_kernel<T, M, 1>(r, bcast);
    return nullptr;
}

// The widest block-id range one exchange cluster (an image's K slices of one
// channel block) occupies under the block-id layout of the kernel.  The
// dispatcher starts workgroups in block-id order, so when every cluster's
// range fits in the workgroups the device holds at once, the lowest
// unfinished cluster can always become wholly resident and the launch never
// waits on a workgroup that cannot start; beyond that, waits run into their
// bound and slices are recomputed (correct, but far slower: one 512 x 512 x
// 256 float16 image took 2.5 ms that way).
// Block-id layout: id = (v / m * NCB + cb) * G + (v % m) * Kp + j with
// m = G / Kp, for items v with Kp ids each.
//   slice-major (Kp = 1, G = 8): the items are the N * K (image, slice)
//     units u = n * K + q; eight units' NCB channel blocks follow one
//     another.  Measured faster wherever it fits (below): the workgroups
//     that start together read contiguous pixel rows (8 x 64 x 64 x 640
//     float16, two rounds of resident workgroups: 45 us, against 53 us
//     cluster-major).  A cluster spans about K * NCB ids.
//   cluster-major (G = Kp = K rounded up to a multiple of 8): the items are
//     images, and a cluster's slices j = q take Kp consecutive ids.  A
//     cluster spans Kp ids.
// In both, slice q of image n sits at the same residue mod 8 in every
// channel block.  Ids with q >= K or n >= N are padding.
struct NhwcLayout {
    int Kp, G;
    int64_t grid, span;
};
NhwcLayout nhwc_layout(int64_t N, const NhwcPlan& p, bool cluster_major) {
    if (!cluster_major) {
        const int64_t units = N * p.K;
        int64_t span = 0;  // widest id range of one cluster
        for (int64_t n = 0; n < N; ++n) {
            const int64_t u0 = n * p.K, u1 = n * p.K + p.K - 1;
            const int64_t lo = ((u0 >> 3) * p.NCB) * 8 + (u0 & 7);
            const int64_t hi = ((u1 >> 3) * p.NCB) * 8 + (u1 & 7);
            if (hi - lo + 1 > span) span = hi - lo + 1;
        }
        return NhwcLayout{1, 8, (units + 7) / 8 * p.NCB * 8, span};
    }
    const int Kp = (p.K + 7) / 8 * 8;
    return NhwcLayout{Kp, Kp, N * p.NCB * Kp, Kp};
}

template <typename T, typename M, int E, int R, bool PACKED>
hipError_t launch_nhwc_cluster_r(const NhwcClusterArgs<T, M>& ca, int64_t blocks, hipStream_t stream) {
    if (ca.skip_bcast)
        hipLaunchKernelGGL((sgn_nhwc_cluster_kernel<T, M, E, R, true, PACKED>), dim3(unsigned(blocks)),
                           dim3(kClusterThreads), 0, stream, ca);
    else
        hipLaunchKernelGGL((sgn_nhwc_cluster_kernel<T, M, E, R, false, PACKED>), dim3(unsigned(blocks)),
                           dim3(kClusterThreads), 0, stream, ca);
    return hipGetLastError();
}

template <typename T, typename M, int E, bool PACKED = false>
hipError_t launch_nhwc_cluster(const NhwcClusterArgs<T, M>& ca, int r, int64_t blocks,
                               hipStream_t stream) {
    if (r <= 1) return launch_nhwc_cluster_r<T, M, E, 1, PACKED>(ca, blocks, stream);
    if (r <= 2) return launch_nhwc_cluster_r<T, M, E, 2, PACKED>(ca, blocks, stream);
    if (r <= 4) return launch_nhwc_cluster_r<T, M, E, 4, PACKED>(ca, blocks, stream);
    if (r <= 8) return launch_nhwc_cluster_r<T, M, E, 8, PACKED>(ca, blocks, stream);
    return launch_nhwc_cluster_r<T, M, E, kNhwcMaxR, PACKED>(ca, blocks, stream);
}

template <typename T, typename M>
hipError_t launch_nhwc_typed(const SgnArgs& a, const NhwcPlan& plan, const NhwcLayout& lay, int E,
                             int kpx, void* part, hipStream_t stream) {
    NhwcClusterArgs<T, M> ca;
    ca.X = static_cast<const T*>(a.X);
    ca.skip = static_cast<const T*>(a.skip);
    ca.bias = static_cast<const T*>(a.bias);
    ca.S = static_cast<T*>(a.S);
    ca.Y = static_cast<T*>(a.Y);
    ca.gamma = static_cast<const M*>(a.gamma);
    ca.beta = static_cast<const M*>(a.beta);
    ca.part = static_cast<Partial*>(part);
    if (plan.K > 1)
        if (hipError_t e = clear_publication_tags(a, part, a.N * a.groups * plan.K, stream); e != hipSuccess)
            return e;
    ca.tags = publication_tags(a.tag);
    ca.timeout_ticks = a.exchange_timeout_ticks;
    ca.HW = a.H * a.W / kpx;  // units
    ca.pps = plan.pps;
    ca.Cv = int(a.C * kpx / E);
    ca.C = int(a.C);
    ca.kpx = kpx;
    ca.cpg = int(a.C / a.groups);
    ca.CBv = plan.CBv;
    ca.NCB = plan.NCB;
    ca.CBg = plan.CBg;
    ca.P = plan.P;
    ca.sw_log = plan.sw_log;
    ca.K = plan.K;
    ca.skip_bcast = a.skip_broadcast;
    ca.silu = a.activation == 1;
    ca.eps = a.epsilon;
    ca.N = int(a.N);
    ca.Kp = lay.Kp;
    ca.G = lay.G;
    ca.div_G = make_fastdiv(uint32_t(lay.G));
    ca.div_NCB = make_fastdiv(uint32_t(plan.NCB));
    ca.div_K = make_fastdiv(uint32_t(plan.K));
    ca.div_CBv = make_fastdiv(uint32_t(plan.CBv));
    ca.div_cpg = make_fastdiv(uint32_t(a.C / a.groups));
    ca.div_P = make_fastdiv(uint32_t(plan.P));
    ca.trace = a.trace;
    const int64_t blocks = lay.grid;
    constexpr int EV = VecWidth<T>::value;
    if (kpx > 1) return E == EV ? launch_nhwc_cluster<T, M, EV, true>(ca, plan.R, blocks, stream)
                                : hipErrorInvalidValue;
    if (E == EV) return launch_nhwc_cluster<T, M, EV>(ca, plan.R, blocks, stream);
    if (E == EV / 2) return launch_nhwc_cluster<T, M, EV / 2>(ca, plan.R, blocks, stream);
    if constexpr (EV >= 8)
        if (E == EV / 4) return launch_nhwc_cluster<T, M, EV / 4>(ca, plan.R, blocks, stream);
    if (E == 1) return launch_nhwc_cluster<T, M, 1>(ca, plan.R, blocks, stream);
    return hipErrorInvalidValue;  // the caller picks E from the same widths
}

}  // namespace

bool launch_sgn_nhwc_cluster(const SgnArgs& a, Route want, void* part, hipStream_t stream,
                             const char** route, hipError_t* err) {
    if (!a.channels_last || want == Route::Scalar || want == Route::Block || want == Route::Split)
        return false;
    const int size = a.dtype == 0 ? 4 : 2;
    const int64_t HW = a.H * a.W;
    // The widest access that divides a pixel's channels and every base (the
    // broadcast skip's rows are C elements apart, like the pixels) and is
    // no wider than a group: groups narrower than a 16-byte vector take
    // 8- or 4-byte vectors here rather than three launches, and odd channel
    // counts or one-channel groups single elements, consecutive threads
    // still reading consecutive bytes of a pixel (f16 8 x 128 x 128 x 15:
    // 0.97 against 0.72 TB/s on the split route over packed runs of pixels;
    // 2 x 64 x 64 x 15: 104 against 55 GB/s).
    int E = a.dtype == 0 ? widest_vector<float>(a.C, {a.X, a.Y, a.S, a.skip, a.bias})
                         : widest_vector<half_t>(a.C, {a.X, a.Y, a.S, a.skip, a.bias});
    while (E > 1 && a.C / a.groups < E) E /= 2;
    NhwcPlan plan;
    const bool block_fits = nhwc_cluster_plan(E, a.N, a.C, HW, a.groups, &plan);
    // Pixels that are not a whole number of 16-byte vectors: packed runs of
    // pixels that are, read with 16-byte accesses (the data tensors 16-byte
    // aligned; bias and a broadcast skip are read per element).
    {
        NhwcPlan pp;
        int kpx = 1;
        const bool aligned = aligned16(a.X) && aligned16(a.Y) && (!a.S || aligned16(a.S)) &&
                             (a.skip_broadcast || aligned16(a.skip));
        if (aligned && nhwc_packed_cluster_plan(size, a.N, a.C, HW, a.groups, &pp, &kpx) &&
            nhwc_packed_preferred(a.N, pp, block_fits)) {
            const void* kernel = a.dtype == 0
                ? (a.param_dtype == 0 ? nhwc_kernel<float, float, 4, true>(pp.R, a.skip_broadcast)
                                      : nhwc_kernel<float, half_t, 4, true>(pp.R, a.skip_broadcast))
                : (a.param_dtype == 0 ? nhwc_kernel<half_t, float, 8, true>(pp.R, a.skip_broadcast)
                                      : nhwc_kernel<half_t, half_t, 8, true>(pp.R, a.skip_broadcast));
            const int64_t resident = resident_workgroups(kernel);
            if (kernel && resident >= 64) {
                NhwcLayout lay = nhwc_layout(a.N, pp, false);
                if (pp.K > 1 && (lay.grid <= resident || lay.span > resident)) lay = nhwc_layout(a.N, pp, true);
                *route = lay.Kp > 1 || pp.K == 1 ? "sgn.cluster.nhwc.packed.vec16"
                                                 : "sgn.cluster.nhwc.smajor.packed.vec16";
                const int ev = 16 / size;  // 16-byte accesses
                if (a.dtype == 0) {
                    if (a.param_dtype == 0) *err = launch_nhwc_typed<float, float>(a, pp, lay, ev, kpx, part, stream);
                    else *err = launch_nhwc_typed<float, half_t>(a, pp, lay, ev, kpx, part, stream);
                } else {
                    if (a.param_dtype == 0) *err = launch_nhwc_typed<half_t, float>(a, pp, lay, ev, kpx, part, stream);
                    else *err = launch_nhwc_typed<half_t, half_t>(a, pp, lay, ev, kpx, part, stream);
                }
                return true;
            }
        }
    }
    if (!block_fits) return false;
    const void* kernel = a.dtype == 0
        ? (a.param_dtype == 0 ? nhwc_kernel_for<float, float>(E, plan.R, a.skip_broadcast)
                              : nhwc_kernel_for<float, half_t>(E, plan.R, a.skip_broadcast))
        : (a.param_dtype == 0 ? nhwc_kernel_for<half_t, float>(E, plan.R, a.skip_broadcast)
                              : nhwc_kernel_for<half_t, half_t>(E, plan.R, a.skip_broadcast));
    // Cluster-major where the grid fits in one round of resident
    // workgroups: when another stream's long-lived workgroups leave only
    // part of the device free, the first free slots then hold whole clusters
    // (2 x 64 x 64 x 320 float16 beside LDS-holding spinners on 230 / 240 of
    // the 256 CUs: 48 / 74 us, against 348 / 951 us slice-major, whose
    // clusters all wait out their bound and recompute), at 1-3 % alone.
    // Larger grids slice-major where each cluster's span fits in the
    // resident workgroups (15 % faster alone), else cluster-major (whose
    // span, at most 64, always fits).
    const int64_t resident = resident_workgroups(kernel);
    if (!kernel || resident < 64) return false;
    NhwcLayout lay = nhwc_layout(a.N, plan, false);
    if (plan.K > 1 && (lay.grid <= resident || lay.span > resident)) lay = nhwc_layout(a.N, plan, true);
    // Beyond two rounds of resident workgroups the split route measured
    // faster (10-30 %, e.g. 8 x 128 x 128 x 320 float16: 86 against 112 us)
    // where its blocks hold whole pixels, in either block order (cluster-major
    // there: 116 us; 4 x 256 x 256 x 256: 158 against 121 us); wider pixels
    // stay here (8 x 64 x 64 x 1280 float32: 148 us, against 162 us split
    // over channel blocks).  Plans of one slice per (image, channel block)
    // exchange nothing, so no workgroup waits and the number of rounds does
    // not matter: they stay here at any grid (float16 256 x 16 x 16 x 320:
    // 38.8 against 73.4 us split, 1024 x 8 x 8 x 320 56 against 106, 512 x 16
    // x 16 x 64 26 against 63, 256 x 20 x 20 x 320 57 against 91; float32
    // 256 x 16 x 16 x 320 78.5 against 97.5, 256 x 20 x 20 x 320 120 against
    // 135), except float16 data beyond 8 pixels per thread, which lost (256 x
    // 24 x 24 x 320 +6 %, 256 x 28 x 28 x 320 +23 %).
    const int split_e = a.dtype == 0 ? widest_vector<float>(a.C, {a.X, a.Y, a.S, a.skip, a.bias})
                                     : widest_vector<half_t>(a.C, {a.X, a.Y, a.S, a.skip, a.bias});
    const bool split_whole_pixels = split_e > 1 && a.C / split_e <= 256;
    const int64_t grid = a.N * plan.NCB * plan.K;  // workgroups that do work
    const bool split_beyond_two_rounds = plan.K > 1 || (plan.R > 8 && size == 2);
    if (split_whole_pixels && grid > 2 * resident && split_beyond_two_rounds) return false;
    static const char* const kNames[2][4] = {
        {"sgn.cluster.nhwc.smajor.scalar", "sgn.cluster.nhwc.smajor.vec4", "sgn.cluster.nhwc.smajor.vec8",
         "sgn.cluster.nhwc.smajor.vec16"},
        {"sgn.cluster.nhwc.scalar", "sgn.cluster.nhwc.vec4", "sgn.cluster.nhwc.vec8", "sgn.cluster.nhwc.vec16"}};
    // Named by layout only where slices exchange (K > 1).
    *route = kNames[lay.Kp > 1 || plan.K == 1 ? 1 : 0][E == 1 ? 0 : E * size == 16 ? 3 : E * size == 8 ? 2 : 1];
    if (a.dtype == 0) {
        if (a.param_dtype == 0) *err = launch_nhwc_typed<float, float>(a, plan, lay, E, 1, part, stream);
        else *err = launch_nhwc_typed<float, half_t>(a, plan, lay, E, 1, part, stream);
    } else {
        if (a.param_dtype == 0) *err = launch_nhwc_typed<half_t, float>(a, plan, lay, E, 1, part, stream);
        else *err = launch_nhwc_typed<half_t, half_t>(a, plan, lay, E, 1, part, stream);
    }
    return true;
}

}  // namespace sn
