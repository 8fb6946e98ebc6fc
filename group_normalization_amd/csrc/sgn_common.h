// sgn_common.h -- device helpers and workspace constants shared by the
// SkipGroupNorm sources (sgn.hip, sgn_nhwc.hip).  Internal to the library.
#pragma once

#include "device_common.h"
#include "skipnorm_internal.h"

namespace sn {

constexpr int kClusterThreads = 256;  // threads per workgroup of the cluster routes
constexpr int kClusterMaxK = 8;       // workgroups per (n, group), NCHW cluster route
constexpr int kNhwcMaxK = 64;         // slices per (image, channel block), NHWC cluster route
// A cluster whose whole tile fits one workgroup at this many accesses per
// thread or fewer takes one slice (no exchange): measured 10-27 % faster on
// groups of 2560-5120 elements than several slices and their exchange.
constexpr int kSingleSliceMaxR = 6;

// Phase k of this workgroup, recorded by its leader in measurement builds:
// 0 start, 1 own data loaded (leader's wave), 2 slice moments reduced,
// 3 moments published and S stores issued, 4 statistics combined,
// 5 Y stores issued.
#ifdef SN_PHASE_TRACE
#define SN_PHASE(trace, k)                                                        \
    do {                                                                          \
        if ((trace) && threadIdx.x == 0 && blockIdx.x < kTraceBlocks)             \
            (trace)[size_t(blockIdx.x) * kTraceStamps + (k)] = wall_clock64();    \
    } while (0)
#else
#define SN_PHASE(trace, k) \
    do {                   \
    } while (0)
#endif

// Launches the NHWC channel-block cluster route when the shapes, alignments
// and `want` allow it (returns false, having launched nothing, otherwise).
// `part` is the workspace's partial area (the publication slots).
bool launch_sgn_nhwc_cluster(const SgnArgs& a, Route want, void* part, hipStream_t stream,
                             const char** route, hipError_t* err);

// Channel blocks (*ncb equal blocks of whole groups, at most 256 vectors of E
// channels each) of the split route's NHWC tiling for pixels of C channels in
// groups of cpg; false when no such blocking exists.
bool nhwc_split_channel_blocks(int64_t C, int64_t cpg, int E, int* ncb);

// Zeroes n publication slots of the cluster routes on `stream` when
// a.clear_tags is set (a kernel of plain stores, not a memset, so that graph
// replays rerun it faithfully); nothing otherwise.
hipError_t clear_publication_tags(const SgnArgs& a, void* slots, int64_t n, hipStream_t stream);

// Publication of one slice's moments in the cluster routes: a 16-byte slot
// of two 64-bit words holding the mean and M2 in their low halves and, in
// their high halves, two 32-bit tags taken from a 64-bit mix of the call's
// tag.  Each word is one 64-bit agent-scope store (single-copy atomic, and
// coherent across the XCDs' separate L2 caches), so a reader that finds
// both words carrying this call's tags has this call's values: no fence,
// no separate flag, and no second round trip to fetch the data after the
// flag.  The count is implied by the slice's size.  A stale slot would have
// to match the tags in 62 bits; zeroed slots (tags are odd) never match.
struct PubTags {
    uint32_t lo, hi;
};

inline PubTags publication_tags(uint64_t tag) {
    uint64_t z = tag;  // MurmurHash3's 64-bit finalizer
    z ^= z >> 33;
    z *= 0xff51afd7ed558ccdULL;
    z ^= z >> 33;
    z *= 0xc4ceb9fe1a85ec53ULL;
    z ^= z >> 33;
    return PubTags{uint32_t(z) | 1u, uint32_t(z >> 32) | 1u};
}

namespace {

constexpr int kUnroll = 4;

struct alignas(16) Partial {
    float n, mean, m2, pad;
};

__device__ __forceinline__ Moments as_moments(const Partial& p) { return Moments{p.n, p.mean, p.m2}; }

// The two words of a publication slot (see publication_tags).
__device__ __forceinline__ void publish_moments(uint64_t* slot, const Moments& m, PubTags tg) {
    __hip_atomic_store(&slot[0], uint64_t(__float_as_uint(m.mean)) | (uint64_t(tg.lo) << 32),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&slot[1], uint64_t(__float_as_uint(m.m2)) | (uint64_t(tg.hi) << 32),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Reads a publication slot: true when both words carry this call's tags,
// and then *mean and *m2 are the published values.
__device__ __forceinline__ bool read_moments(uint64_t* slot, PubTags tg, float* mean, float* m2) {
    const uint64_t w0 = __hip_atomic_load(&slot[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t w1 = __hip_atomic_load(&slot[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *mean = __uint_as_float(uint32_t(w0));
    *m2 = __uint_as_float(uint32_t(w1));
    return uint32_t(w0 >> 32) == tg.lo && uint32_t(w1 >> 32) == tg.hi;
}

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
    __syncthreads();  // `sh` may be reused right away
    return tot;
}

__device__ __forceinline__ float2 finalize(const Moments& m, float eps) {
    // Negative rounding residue clamps to 0; NaN (a group holding an
    // infinity or NaN) stays NaN, so the whole group's output is NaN.
    const float v = m.m2 / m.n;
    const float var = m.n > 0.0f ? (v < 0.0f ? 0.0f : v) : 0.0f;
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

// Pairwise combination without branches, the weight taken from the
// hardware reciprocal (about 1 ulp) rather than an IEEE division: thousands
// of these sit on the cluster route's critical path.  Empty moments are
// (0, 0, 0); merging with one is exact either way (weight 0, or weight 1
// when the other side is empty).  Every workgroup runs the same operations,
// so the results stay bitwise reproducible.
__device__ __forceinline__ Moments merge_rcp(const Moments& a, const Moments& b) {
    const float n = a.n + b.n;
    const float wb = b.n == n ? 1.0f : b.n * __builtin_amdgcn_rcpf(n);
    const float d = b.mean - a.mean;
    Moments r;
    r.n = n;
    r.mean = fmaf_(d, wb, a.mean);
    r.m2 = fmaf_(d * d, a.n * wb, a.m2 + b.m2);
    return r;
}

template <int CTRL>
__device__ __forceinline__ Moments dpp_merge_step(const Moments& m, bool upper) {
    const Moments o{dpp_mov<CTRL>(m.n), dpp_mov<CTRL>(m.mean), dpp_mov<CTRL>(m.m2)};
    return upper ? merge_rcp(o, m) : merge_rcp(m, o);
}

// Ordered butterfly over aligned segments of W lanes (W a power of two, at
// most 64; uniform over the wave): every lane of a segment ends with bitwise
// the same combination of the segment's values in lane order.  After the two
// quad steps each quad is uniform, so mirroring inside 8 and 16 lanes pairs
// the same quads and half-rows as an xor by 4 and by 8 would.
__device__ __forceinline__ Moments segment_merge(Moments m, int W) {
    const int lane = threadIdx.x & 63;
    if (W >= 2) m = dpp_merge_step<kQuadXor1>(m, lane & 1);
    if (W >= 4) m = dpp_merge_step<kQuadXor2>(m, lane & 2);
    if (W >= 8) m = dpp_merge_step<kRowHalfMirror>(m, lane & 4);
    if (W >= 16) m = dpp_merge_step<kRowMirror>(m, lane & 8);
    for (int s = 16; s < W; s <<= 1) {
        const Moments o{__shfl_xor(m.n, s, 64), __shfl_xor(m.mean, s, 64), __shfl_xor(m.m2, s, 64)};
        m = (lane & s) ? merge_rcp(o, m) : merge_rcp(m, o);
    }
    return m;
}

// Block of 256 threads: each wave's ordered butterfly, then the four wave
// totals in wave order through LDS; every thread returns the same value.
// `sh` holds four entries.
__device__ __forceinline__ Moments block_merge_rcp(Moments m, Moments* sh) {
    m = segment_merge(m, 64);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = m;
    __syncthreads();
    Moments tot = sh[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) tot = merge_rcp(tot, sh[w]);
    __syncthreads();  // `sh` may be reused right away
    return tot;
}

}  // namespace
}  // namespace sn
