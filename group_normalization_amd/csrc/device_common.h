// device_common.h -- device helpers shared by the libskipnorm kernels
// (gfx950 / CDNA4, wave64).  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <initializer_list>

namespace sn {

typedef _Float16 half_t;

// ---------------------------------------------------------------------------
// Element vectors.  Vec<T, E> holds E elements of T and is aligned to its
// size: E * sizeof(T) == 16 is the 16-byte vector that becomes one
// global_load/store_dwordx4 per lane, 8 and 4 bytes the narrower vectors of
// rows whose length (or base) is not a whole number of 16-byte vectors, and
// E == 1 the scalar route.
template <typename T, int E> struct Vec { T v[E]; };
template <> struct alignas(16) Vec<float, 4> { float v[4]; };
template <> struct alignas(8) Vec<float, 2> { float v[2]; };
template <> struct alignas(16) Vec<half_t, 8> { half_t v[8]; };
template <> struct alignas(8) Vec<half_t, 4> { half_t v[4]; };
template <> struct alignas(4) Vec<half_t, 2> { half_t v[2]; };

template <typename T> struct VecWidth { static constexpr int value = 16 / sizeof(T); };

// Widest access (16, 8 or 4 bytes, else one element) that divides a row of
// `row_elems` elements and every base address in `ptrs` (null entries are
// ignored): the vector width, in elements, a route can use for such rows.
template <typename T>
inline int widest_vector(int64_t row_elems, std::initializer_list<const void*> ptrs) {
    for (int bytes = 16; bytes > int(sizeof(T)); bytes /= 2) {
        bool ok = (row_elems * int64_t(sizeof(T))) % bytes == 0;
        for (const void* p : ptrs) ok = ok && (reinterpret_cast<uintptr_t>(p) % bytes == 0);
        if (ok) return bytes / int(sizeof(T));
    }
    return 1;
}

template <typename T, int E>
__device__ __forceinline__ Vec<T, E> load_vec(const T* __restrict__ p, int64_t i) {
    return reinterpret_cast<const Vec<T, E>*>(p)[i];
}
template <typename T, int E>
__device__ __forceinline__ void store_vec(T* __restrict__ p, int64_t i, const Vec<T, E>& v) {
    reinterpret_cast<Vec<T, E>*>(p)[i] = v;
}

// Streaming (nontemporal) accesses for data touched exactly once: the
// access carries the nontemporal hint, so the caches do not keep lines that
// will not be reused.  Values are moved as raw bits of the same size.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
template <int BYTES> struct RawBits;
template <> struct RawBits<16> { using type = u32x4; };
template <> struct RawBits<8> { using type = u32x2; };
template <> struct RawBits<4> { using type = uint32_t; };
template <> struct RawBits<2> { using type = uint16_t; };

template <typename T, int E>
__device__ __forceinline__ Vec<T, E> load_vec_stream(const T* __restrict__ p, int64_t i) {
    using R = typename RawBits<sizeof(Vec<T, E>)>::type;
    const R r = __builtin_nontemporal_load(reinterpret_cast<const R*>(p) + i);
    return __builtin_bit_cast(Vec<T, E>, r);
}
template <typename T, int E>
__device__ __forceinline__ void store_vec_stream(T* __restrict__ p, int64_t i, const Vec<T, E>& v) {
    using R = typename RawBits<sizeof(Vec<T, E>)>::type;
    __builtin_nontemporal_store(__builtin_bit_cast(R, v), reinterpret_cast<R*>(p) + i);
}

// A run of stores (a row, a tile) whose ends fall inside 128-byte lines
// shares those lines with the neighbouring runs, which other waves write.
// Nontemporal stores of such partial lines each go to memory on their own
// (measured: f16 rows of 2032 bytes 19 % slower than rows of 2048), so the
// vectors in the run's first and last partial line go through L2 with
// ordinary stores, where the two parts merge, and the rest stream.
// LineRun: the run's vectors [lo, hi), counted from its first, that lie in
// whole lines.
struct LineRun {
    int lo, hi;
};
template <typename T, int E>
__device__ __forceinline__ LineRun line_run(const T* run, int nvec) {
    constexpr int VB = E * int(sizeof(T));
    const int head = int(reinterpret_cast<uintptr_t>(run) & 127);  // bytes into its first line
    const int lo = head ? (128 - head) / VB : 0;
    const int hi = int(((int64_t(head) + int64_t(nvec) * VB) / 128 * 128 - head) / VB);
    return LineRun{lo, hi > lo ? hi : lo};
}
template <typename T, int E>
__device__ __forceinline__ void store_vec_run(T* __restrict__ run, int j, const Vec<T, E>& v,
                                              const LineRun& lr) {
    if (j >= lr.lo && j < lr.hi) store_vec_stream<T, E>(run, j, v);
    else store_vec<T, E>(run, j, v);
}

// Orders a wave's LDS writes before its later LDS reads from other lanes of
// the same wave: the LDS executes one wave's instructions in issue order, so
// only the compiler must be kept from moving accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Flat routes (GatedRMSNorm, SkipSimplifiedLayerNormalization): rows as one
// stream of aligned 16-byte vectors, per-column parameters from an LDS table
// of kFlatTable float32 slots with E of them ahead of column 0, so rows hold
// at most kFlatTable - E elements.
constexpr int kFlatTable = 1024;

// Elements k .. k + E - 1 of the 2E-element concatenation [lo, hi] of two
// 16-byte vectors (0 <= k < E): byte funnel shifts of their eight dwords.
// The dword offset is applied with value selects, not branches: an
// if / else-if chain on it, which the compiler could not prove uniform,
// was lowered into exec-masked blocks that left the last case's values
// unassigned (seen in the generated code and as wrong rows on the GPU).
template <typename T, int E>
__device__ __forceinline__ Vec<T, E> funnel16(const Vec<T, E>& lo, const Vec<T, E>& hi, int k) {
    static_assert(sizeof(Vec<T, E>) == 16, "16-byte vectors");
    const u32x4 a = __builtin_bit_cast(u32x4, lo), b = __builtin_bit_cast(u32x4, hi);
    const uint32_t c[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    const int byte = k * int(sizeof(T));
    const int q = byte >> 2;
    const uint32_t r = uint32_t(byte & 3);
    uint32_t w[5];  // dwords q .. q + 4 of [a, b]
#pragma unroll
    for (int j = 0; j < 5; ++j) {
        const uint32_t x01 = q == 0 ? c[j] : c[j + 1];
        const uint32_t x23 = q == 2 ? c[j + 2] : c[j + 3 < 8 ? j + 3 : 7];
        w[j] = q < 2 ? x01 : x23;
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __builtin_amdgcn_alignbyte(w[i + 1], w[i], r);
    return __builtin_bit_cast(Vec<T, E>, o);
}

// Wide-row kernels (one 1024-thread workgroup per row): sixteen-byte vectors
// per lane held in VGPRs and in LDS (9 x 16 KB of gfx950's 160 KB per
// workgroup), and the vectors per lane of each pipelined LDS chunk.
constexpr int kWideThreads = 1024;
constexpr int kWideRegs = 8;
constexpr int kWideLds = 9;
constexpr int kWideChunk = 2;

// Flat plan for rows of C <= kFlatTable - E elements: rt whole rows per wave
// such that the vectors they touch (at any offset from the grid) fit the
// wave's 64 * VPT vector slots, in the smaller tile (VPT = 2 for float16, 4
// for float32: 1024 element slots) unless `large` allows twice that and the
// smaller leaves over a quarter of its slots idle while the larger fills
// more; lpr = the largest power of two with lpr * rt <= 64 (1 beyond 64
// rows, which the lanes then take in turns).
struct FlatPlan {
    int vpt, rt, lpr_log;
    double fill;  // share of the tile's element slots that carry data
};

inline bool flat_plan(int64_t C, int vec_elems, bool large, FlatPlan* p) {
    if (C < 1 || C > kFlatTable - vec_elems) return false;
    const int small = 16 / vec_elems;
    p->fill = -1.0;
    for (int vpt : {small, 2 * small}) {
        if (vpt != small && !large) break;
        const int64_t te = int64_t(64) * vpt * vec_elems;
        const int64_t rt = (te - vec_elems + 1) / C;
        if (rt < 1) continue;
        const double fill = double(rt * C) / double(te);
        if (p->fill >= 0.75 || fill <= p->fill) continue;
        p->fill = fill;
        p->vpt = vpt;
        p->rt = int(rt);
    }
    if (p->fill < 0.0) return false;
    int lpr_log = 0;
    while ((int64_t(2) << lpr_log) * p->rt <= 64) ++lpr_log;
    p->lpr_log = lpr_log;
    return true;
}

// Host side: whether rows of row_bytes written at these bases (null ones
// skipped) do not all start on 128-byte lines.
inline int rows_off_lines(int64_t row_bytes, std::initializer_list<const void*> outs) {
    int off = row_bytes % 128 != 0;
    for (const void* p : outs) off |= p && reinterpret_cast<uintptr_t>(p) % 128 != 0;
    return off;
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(half_t x) { return static_cast<float>(x); }

// Round a float32 value to T (round to nearest even; v_cvt_f16_f32 keeps
// binary16 subnormals) -- the single narrowing step of every output.
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ half_t from_f32<half_t>(float x) { return static_cast<half_t>(x); }

// Residual sum of one element: float32 (x + skip), then + bias only when a
// bias exists (adding +0 would turn -0 into +0), then one rounding to T.
// Returns the T value widened back to float32, which is what the
// statistics and the normalization use.
template <typename T>
__device__ __forceinline__ float residual_sum(float x, float skip, bool has_bias, float bias, T& rounded) {
    float s = x + skip;
    if (has_bias) s = s + bias;
    rounded = from_f32<T>(s);
    return to_f32(rounded);
}

__device__ __forceinline__ float fmaf_(float a, float b, float c) { return __builtin_fmaf(a, b, c); }

// SiLU(v) = v / (1 + e^-v) in float32: v_exp_f32 on -v*log2(e) and
// v_rcp_f32 (about 1 ulp each).  For v << 0, e^-v overflows to +inf and the
// reciprocal gives 0, the correct limit.
__device__ __forceinline__ float silu_f32(float v) {
    const float e = __builtin_amdgcn_exp2f(-v * 1.4426950408889634f);
    return v * __builtin_amdgcn_rcpf(1.0f + e);
}

// 1 / sqrt(x) from a correctly rounded square root and an IEEE division:
// once per row or group, so exactness is preferred over speed.
__device__ __forceinline__ float inv_sqrt(float x) { return 1.0f / __builtin_sqrtf(x); }

// ---------------------------------------------------------------------------
// Cross-lane sums.  Every step adds a lane's value to its partner's; IEEE
// addition is commutative, so both partners hold bitwise the same sum and
// after the last step every lane of the segment holds the same total.

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}

// DPP controls (GFX9 encoding).
constexpr int kQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <-> 7-i within each 8
constexpr int kRowMirror = 0x140;      // lane i <-> 15-i within each 16

// Sum over aligned segments of L lanes (L a power of two, 1..64).
template <int L>
__device__ __forceinline__ float segment_sum(float v) {
    if constexpr (L >= 2) v = v + dpp_mov<kQuadXor1>(v);
    if constexpr (L >= 4) v = v + dpp_mov<kQuadXor2>(v);
    // After the quad steps each quad is uniform, so mirroring inside 8 lanes
    // pairs quad 0 with quad 1, and mirroring inside 16 pairs the halves.
    if constexpr (L >= 8) v = v + dpp_mov<kRowHalfMirror>(v);
    if constexpr (L >= 16) v = v + dpp_mov<kRowMirror>(v);
    if constexpr (L >= 32) v = v + __shfl_xor(v, 16, 64);
    if constexpr (L >= 64) v = v + __shfl_xor(v, 32, 64);
    return v;
}

// ---------------------------------------------------------------------------
// Moments (count, mean, M2 = sum of squared deviations) and their pairwise
// combination (Chan, Golub and LeVeque, "Updating formulae and a pairwise
// algorithm for computing sample variances", 1979).
struct Moments {
    float n, mean, m2;
};

__device__ __forceinline__ Moments merge(const Moments& a, const Moments& b) {
    if (b.n == 0.0f) return a;
    if (a.n == 0.0f) return b;
    const float n = a.n + b.n;
    const float d = b.mean - a.mean;
    const float wb = b.n / n;
    Moments r;
    r.n = n;
    r.mean = fmaf_(d, wb, a.mean);
    r.m2 = fmaf_(d * d, a.n * wb, a.m2 + b.m2);
    return r;
}

// The shift for sums about a row's first element: that element when it is
// finite, else 0.  With an infinite shift the shift element itself would add
// inf - inf = NaN, and the mean (shift + mean of the differences) would be
// NaN where the sum over the row is infinite.
__device__ __forceinline__ float row_shift(float s0) { return __builtin_isfinite(s0) ? s0 : 0.0f; }

// Per-thread accumulator with the shifted-data method: sums of (x - shift)
// and (x - shift)^2, shift = the first value seen, so a group whose values
// are all equal accumulates exact zeros.
struct ShiftedSums {
    float shift = 0.0f, s1 = 0.0f, s2 = 0.0f;
    __device__ __forceinline__ void add(float x, bool first) {
        if (first) shift = x;
        const float d = x - shift;
        s1 += d;
        s2 = fmaf_(d, d, s2);
    }
    __device__ __forceinline__ Moments moments(float n) const {
        Moments m;
        m.n = n;
        if (n == 0.0f) {
            m.mean = 0.0f;
            m.m2 = 0.0f;
            return m;
        }
        const float q = s1 / n;
        m.mean = shift + q;
        // Rounding can leave a tiny negative M2; clamp it, but keep NaN (an
        // infinite value gives inf - inf here), which fmaxf would turn into 0.
        const float m2 = fmaf_(-s1, q, s2);
        m.m2 = m2 < 0.0f ? 0.0f : m2;
        return m;
    }
};

// ---------------------------------------------------------------------------
// Unsigned division by a run-time invariant d >= 1 with one multiply-high
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994, unsigned case): exact for every 32-bit n.
struct FastDiv {
    uint32_t d, m, s1, s2;
};

__host__ __device__ inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;  // l = ceil(log2 d)
    FastDiv f;
    f.d = d;
    f.m = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
    f.s1 = l > 0 ? 1u : 0u;
    f.s2 = l > 0 ? l - 1 : 0u;
    return f;
}

__device__ __forceinline__ uint32_t fastdiv(uint32_t n, const FastDiv& f) {
    const uint32_t t = __umulhi(n, f.m);
    return (t + ((n - t) >> f.s1)) >> f.s2;
}

}  // namespace sn
