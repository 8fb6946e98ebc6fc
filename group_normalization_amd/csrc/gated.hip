// gated.hip -- GatedRMSNorm kernels for gfx950.
//
// Operator ("com.microsoft.GatedRMSNorm", Description): X is read as flat
// rows of C = numel(scale) contiguous elements; per row
// r = 1/sqrt(mean(X^2) + epsilon) and Y = X * r * scale * SiLU(gate), every
// intermediate in float32 and one narrowing store.
//
// Routes:
//   segment  L lanes per row (L = the row's vector count rounded up to a
//            power of two, at most 64), so 64/L rows share a wave and one
//            segmented butterfly (DPP quad/row-mirror steps, no LDS, no
//            barrier) reduces all of them at once.  A C = 128 float16 row is
//            16 lanes x one 16-byte vector: 4 rows per wave.  Rows wider
//            than 64 vectors use all 64 lanes with up to 16 vectors each.
//            Each thread loads RPT rows before computing, to keep enough
//            bytes in flight.  Element width: the widest of 16-, 8- and
//            4-byte vectors that divides the row and every base, else
//            scalars.
//   tile     float16 rows of 33 to 128 vectors of 8 or 4 bytes of which the
//            segment route would leave more than 40 % of the lanes idle (it
//            gives such a row 64 or 128 lane slots): each wave takes RT whole rows
//            packed back to back into its 64 * VPT vector slots
//            (RT = floor(64 * VPT / vectors per row)), so nearly every slot
//            carries data; per-vector sums of squares meet in LDS and each
//            row is summed by a power-of-two group of lanes, in order, then
//            by a butterfly over the group.  Elsewhere (and for float32) the
//            segment route measured as fast or faster: its idle lanes
//            re-read cached vectors, which costs issue slots but no HBM
//            traffic.
//   flat     rows of at most 1016 (float16) or 1020 (float32) elements read with
//            accesses narrower than
//            16 bytes (odd spans, narrow rows), where X, gate and Y share
//            their offset from the 16-byte grid and the tile is at least 3/4
//            full: the rows are read as one stream of aligned 16-byte
//            vectors, each wave taking whole rows packed back to back; the
//            squares meet in LDS, each row is summed by a power-of-two group
//            of lanes, and every element takes its row's r and its column's
//            scale from LDS (where exactly: flat_preferred below).
//   row      rows of 1025 to 4096 sixteen-byte vectors (8192 narrower
//            accesses): one 512- or 1024-thread workgroup per row holding
//            it in registers (at most four 16-byte vectors or eight
//            narrower accesses per thread); the waves' sums meet in LDS and
//            are added as a pairwise tree in wave order.
//   wide     rows of 16-byte vectors beyond the row route, up to 272 KB of X:
//            one 1024-thread workgroup per row holding X alone (8 vectors
//            per lane in VGPRs, up to 9 more in LDS); gate and scale are read
//            after the statistic (gated_wide_kernel).
//   phase    spans read element by element otherwise (odd spans, bases 2 or 6
//            bytes off the 16-byte grid) beyond the flat route, and longer
//            spans of 4- or 8-byte accesses, up to 4096 vectors: aligned
//            16-byte vectors across span boundaries, scale funnel-shifted
//            (gated_phase_kernel).
//   block    one 256-thread workgroup per row for wider rows; X is read
//            twice, four vectors per thread in flight per pass.
// scale is loaded once per thread and kept in registers as float32 (flat: an
// LDS table per workgroup).  X, gate and Y are touched once and move with
// nontemporal loads and stores, except that the flat route and the segment
// route's rows of more than 64 vectors write the vectors of 128-byte lines
// shared with another wave's rows through L2.
#include "device_common.h"
#include "skipnorm_internal.h"

namespace sn {
namespace {

// LINES: rows off the 128-byte grid; each wave's store of its 64 / L rows
// (one row, where LINES is used) writes the vectors in that run's first and
// last partial 128-byte line with ordinary stores (merged in L2) and streams
// the rest.
template <typename T, int E, int L, int VPL, int RPT, bool LINES>
__global__ void __launch_bounds__(256)
gated_segment_kernel(const T* __restrict__ X, const T* __restrict__ scale,
                     const T* __restrict__ gate, T* __restrict__ Y, int64_t rows,
                     int nvec, float span_f, float eps) {
    using V = Vec<T, E>;
    constexpr int SEGS = 256 / L;  // rows per block per step
    const int seg = threadIdx.x / L;
    const int l = threadIdx.x % L;
    const int64_t tile = int64_t(blockIdx.x) * SEGS * RPT;

    // No load sits behind a lane-dependent branch (the compiler would wait
    // for each in turn): padding lanes and rows past the end re-read the
    // last vector / row and discard the result.
    float sc[VPL][E];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const int idx = v * L + l;
        const V s = load_vec<T, E>(scale, idx < nvec ? idx : nvec - 1);
#pragma unroll
        for (int e = 0; e < E; ++e) sc[v][e] = to_f32(s.v[e]);
    }

    V xs[RPT][VPL], gs[RPT][VPL];
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        const int64_t row = tile + int64_t(k) * SEGS + seg;
        const int64_t rc = row < rows ? row : rows - 1;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            const int idx = v * L + l;
            const int ic = idx < nvec ? idx : nvec - 1;
            xs[k][v] = load_vec_stream<T, E>(X, rc * nvec + ic);
            gs[k][v] = load_vec_stream<T, E>(gate, rc * nvec + ic);
        }
    }

#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        const int64_t row = tile + int64_t(k) * SEGS + seg;
        float acc = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            const int idx = v * L + l;
            if (row < rows && idx < nvec) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float x = to_f32(xs[k][v].v[e]);
                    acc = fmaf_(x, x, acc);
                }
            }
        }
        // Every lane of the segment takes part, padding lanes with 0.
        const float total = segment_sum<L>(acc);
        const float r = inv_sqrt(total / span_f + eps);
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            const int idx = v * L + l;
            if (row < rows && idx < nvec) {
                V out;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float x = to_f32(xs[k][v].v[e]);
                    const float g = to_f32(gs[k][v].v[e]);
                    out.v[e] = from_f32<T>(x * r * sc[v][e] * silu_f32(g));
                }
                if constexpr (LINES) {
                    constexpr int RW = 64 / L;  // rows of one wave's store
                    const int64_t r0 = row - seg % RW;
                    const int64_t rn = rows - r0 < RW ? rows - r0 : RW;
                    T* run = Y + r0 * nvec * E;
                    store_vec_run<T, E>(run, (seg % RW) * nvec + idx, out,
                                        line_run<T, E>(run, int(rn * nvec)));
                } else {
                    store_vec_stream<T, E>(Y, row * nvec + idx, out);
                }
            }
        }
    }
}


// Tile route.  Wave w of the grid takes rows [w * rt, w * rt + rt) (fewer at
// the end), i.e. vectors [0, cnt) from the first of them; lane l holds the
// vectors l, l + 64, ... of that run.  A vector's row within the tile is
// j / nvec, taken as (j * magic) >> 32 with magic = floor(2^32 / nvec) + 1,
// exact because j < 64 * VPT <= 1024 and nvec <= 1024 (j * nvec < 2^32).
// Rows are summed by lpr = 2^lpr_log lanes each (rt * lpr <= 64).
template <typename T, int E, int VPT>
__global__ void __launch_bounds__(256)
gated_tile_kernel(const T* __restrict__ X, const T* __restrict__ scale,
                  const T* __restrict__ gate, T* __restrict__ Y, int64_t rows, int nvec,
                  int rt, int lpr_log, uint32_t magic, float span_f, float eps) {
    using V = Vec<T, E>;
    constexpr int SLOTS = 64 * VPT;
    __shared__ float part[4][SLOTS];
    __shared__ float row_r[4][64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r0 = (int64_t(blockIdx.x) * 4 + wave) * rt;
    const int64_t left = rows - r0;
    const int nr = left <= 0 ? 0 : (left < rt ? int(left) : rt);
    // Each wave works on its own LDS rows, so the waves of a block never wait
    // for one another; a wave past the last row has nothing to do.
    if (nr == 0) return;
    const int cnt = nr * nvec;
    const int64_t base = r0 * nvec;
    auto clamp = [&](int j) { return j < cnt ? j : cnt - 1; };
    auto row_of = [&](int j) { return int((uint64_t(uint32_t(j)) * magic) >> 32); };

    V xs[VPT], gs[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int jc = clamp(v * 64 + lane);
        xs[v] = load_vec_stream<T, E>(X, base + jc);
        gs[v] = load_vec_stream<T, E>(gate, base + jc);
    }
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int j = v * 64 + lane;
        float p = 0.0f;
        if (j < cnt) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float x = to_f32(xs[v].v[e]);
                p = fmaf_(x, x, p);
            }
        }
        part[wave][j] = p;
    }
    wave_lds_sync();
    // Row rr of the tile: lanes rr * lpr + k add its vectors k, k + lpr, ...
    // in order; then the lpr lanes meet in a butterfly (every lane of the
    // group ends with the same total).  A lane adds at most 2 * VPT + 1
    // vectors (lpr = 64 / rtp with rtp < 2 * rt and rt * nvec <= 64 * VPT),
    // read unconditionally from clamped slots so that the reads go out
    // together; the terms past the row add zero.
    const int lpr = 1 << lpr_log;
    const int rr = lane >> lpr_log, k = lane & (lpr - 1);
    const int row0 = (rr < nr ? rr : 0) * nvec;  // lanes past the last row read row 0
    float acc = 0.0f;
#pragma unroll
    for (int s = 0; s < 2 * VPT + 1; ++s) {
        const int i = k + s * lpr;
        const float pv = part[wave][row0 + (i < nvec ? i : nvec - 1)];
        acc += (i < nvec && rr < nr) ? pv : 0.0f;
    }
    for (int m = 1; m < lpr; m <<= 1) acc += __shfl_xor(acc, m, 64);
    if (rr < nr && k == 0) row_r[wave][rr] = inv_sqrt(acc / span_f + eps);
    wave_lds_sync();
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int j = v * 64 + lane;
        const int jc = clamp(j);
        const int row = row_of(jc);
        const V sv = load_vec<T, E>(scale, jc - row * nvec);
        const float r = row_r[wave][row];
        V out;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float x = to_f32(xs[v].v[e]);
            const float g = to_f32(gs[v].v[e]);
            out.v[e] = from_f32<T>(x * r * to_f32(sv.v[e]) * silu_f32(g));
        }
        if (j < cnt) store_vec_stream<T, E>(Y, base + j, out);
    }
}

// Flat route: the rows are one stream of elements.  Wave w takes the rt
// whole rows from r0 = w * rt on, elements [r0 * C, (r0 + rt) * C) (plus the
// offset `phase` of the data bases from the 16-byte grid, which X, gate and
// Y share), and reads the aligned 16-byte vectors that cover them; the first
// and last may hold a neighbouring wave's elements, which are read and left
// unused (never outside the 16-byte chunks that hold the tensors' own
// elements), and they are written element by element, the rest whole.  The
// squares go to LDS element by element; each row is summed by a power-of-two
// group of lanes (lane k of the group adds elements k, k + lpr, ... in
// order, then a butterfly over the group), and its r overwrites its first
// square.  Each element then takes r from its row and scale from an LDS
// table of C float32 values by its column.  NARROW (C < elements per
// vector): a vector spans several rows, so every element finds its own row;
// otherwise a vector spans at most two and the row changes once.  The scale
// table holds 1024 float32 slots, E of them ahead of column 0, so rows hold
// at most 1024 - E elements.

template <typename T, int VPT, bool NARROW>
__global__ void __launch_bounds__(256)
gated_flat_kernel(const T* __restrict__ X, const T* __restrict__ scale,
                  const T* __restrict__ gate, T* __restrict__ Y, int64_t rows, int C, int rt,
                  int lpr_log, int phase, FastDiv cdiv, float span_f, float eps) {
    constexpr int E = VecWidth<T>::value;
    constexpr int TE = 64 * VPT * E;  // element slots of a wave's tile
    using V = Vec<T, E>;
    __shared__ float sq[4][TE];
    // scale by column at sc[c]; E slots ahead of it keep the reads of
    // elements before a tile (columns down to 1 - E) inside the array.
    __shared__ float sc_tab[kFlatTable];
    float* sc = sc_tab + E;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r0 = (int64_t(blockIdx.x) * 4 + wave) * rt;
    const int64_t left = rows - r0;
    const int nr = left <= 0 ? 0 : (left < rt ? int(left) : rt);
    // A wave past the last row loads the last row (and discards it), so that
    // every wave reaches the barrier below with nothing out of bounds.
    const int64_t rl = nr > 0 ? r0 : rows - 1;
    const int span = (nr > 0 ? nr : 1) * C;
    const int64_t f0 = phase + rl * C;  // the tile's first element from the aligned base
    const int64_t v0 = f0 / E;
    const int off0 = int(f0 - v0 * E);
    const int nvt = (off0 + span + E - 1) / E;  // vectors the tile touches
    const T* xa = X - phase;
    const T* ga = gate - phase;
    T* ya = Y - phase;

    V xs[VPT], gs[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int i = v * 64 + lane;
        const int ic = i < nvt ? i : nvt - 1;
        xs[v] = load_vec_stream<T, E>(xa, v0 + ic);
        gs[v] = load_vec_stream<T, E>(ga, v0 + ic);
    }
    for (int c = threadIdx.x; c < C; c += 256) sc[c] = to_f32(scale[c]);
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int i = v * 64 + lane;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float x = to_f32(xs[v].v[e]);
            sq[wave][i * E + e] = x * x;
        }
    }
    __syncthreads();  // the scale table, and this wave's squares
    if (nr == 0) return;

    const int lpr = 1 << lpr_log;
    const int k = lane & (lpr - 1);
    for (int rb = 0; rb < nr; rb += 64 >> lpr_log) {
        const int rr = rb + (lane >> lpr_log);
        const bool has = rr < nr;
        const int first = off0 + (has ? rr : 0) * C;
        float acc = 0.0f;
        if (has)
            for (int c = k; c < C; c += lpr) acc += sq[wave][first + c];
        for (int m = 1; m < lpr; m <<= 1) acc += __shfl_xor(acc, m, 64);
        // The group's reads of this row are done (the butterfly used them).
        if (has && k == 0) sq[wave][first] = inv_sqrt(acc / span_f + eps);
    }
    wave_lds_sync();

    // The tile's ends fall inside 128-byte lines shared with the neighbouring
    // tiles: the vectors there are stored through L2.
    const LineRun run = line_run<T, E>(ya + v0 * E, nvt);
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int i = v * 64 + lane;
        const int t0 = i * E - off0;  // the vector's first element, from the tile's first
        float rv[E], sv[E];
        if constexpr (NARROW) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                int t = t0 + e;
                t = t < 0 ? 0 : (t < span ? t : span - 1);
                const int row = int(fastdiv(uint32_t(t), cdiv));
                rv[e] = sq[wave][off0 + row * C];
                sv[e] = sc[t - row * C];
            }
        } else {
            const int tc = t0 < 0 ? 0 : (t0 < span ? t0 : span - 1);
            const int row0 = int(fastdiv(uint32_t(tc), cdiv));
            const int row1 = row0 + 1 < nr ? row0 + 1 : row0;
            const float ra = sq[wave][off0 + row0 * C];
            const float rb = sq[wave][off0 + row1 * C];
            // Column of element 0: 1 - E to -1 for the vector that starts
            // before the tile, 0 to C - 1 for the others with elements in it
            // (clamped for the vectors past it, whose results are dropped).
            int c0 = t0 - row0 * C;
            c0 = c0 > C - 1 ? C - 1 : c0;
            const int b = C - c0;  // elements e >= b lie in the next row
            const float* sa = sc + c0;
            const float* sb = sc + (c0 - C);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const bool next = e >= b;
                rv[e] = next ? rb : ra;
                sv[e] = (next ? sb : sa)[e];
            }
        }
        V out;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float x = to_f32(xs[v].v[e]);
            const float g = to_f32(gs[v].v[e]);
            out.v[e] = from_f32<T>(x * rv[e] * sv[e] * silu_f32(g));
        }
        if (t0 >= 0 && t0 + E <= span) {
            store_vec_run<T, E>(ya + v0 * E, i, out, run);
        } else if (i < nvt) {
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (t0 + e >= 0 && t0 + e < span) ya[(v0 + i) * E + e] = out.v[e];
        }
    }
}

// Row route: a block of TPB threads (4, 8 or 16 waves) per row; thread t
// holds vectors t, t + TPB, ... (NV of them); lanes past the row re-read
// its last vector and discard it.  The wave sums are added as a pairwise
// tree in wave order.
template <typename T, int E, int NV, int TPB>
__global__ void __launch_bounds__(TPB)
gated_row_kernel(const T* __restrict__ X, const T* __restrict__ scale,
                 const T* __restrict__ gate, T* __restrict__ Y, int64_t rows, int nvec,
                 float span_f, float eps) {
    using V = Vec<T, E>;
    constexpr int W = TPB / 64;
    __shared__ float wave_part[W];
    const int t = threadIdx.x;
    auto clamp = [&](int j) { return j < nvec ? j : nvec - 1; };
    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const int64_t base = row * nvec;
        V xs[NV], gs[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int jc = clamp(v * TPB + t);
            xs[v] = load_vec_stream<T, E>(X, base + jc);
            gs[v] = load_vec_stream<T, E>(gate, base + jc);
        }
        float acc = 0.0f;
#pragma unroll
        for (int v = 0; v < NV; ++v)
            if (v * TPB + t < nvec) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float x = to_f32(xs[v].v[e]);
                    acc = fmaf_(x, x, acc);
                }
            }
        acc = segment_sum<64>(acc);
        if ((t & 63) == 0) wave_part[t >> 6] = acc;
        __syncthreads();
        float part[W];
#pragma unroll
        for (int w = 0; w < W; ++w) part[w] = wave_part[w];
#pragma unroll
        for (int s = 1; s < W; s *= 2)
#pragma unroll
            for (int w = 0; w + s < W; w += 2 * s) part[w] += part[w + s];
        const float total = part[0];
        __syncthreads();  // wave_part is rewritten for the next row
        const float r = inv_sqrt(total / span_f + eps);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int j = v * TPB + t;
            const V sv = load_vec<T, E>(scale, clamp(j));
            V out;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float x = to_f32(xs[v].v[e]);
                const float g = to_f32(gs[v].v[e]);
                out.v[e] = from_f32<T>(x * r * to_f32(sv.v[e]) * silu_f32(g));
            }
            if (j < nvec) store_vec_stream<T, E>(Y, base + j, out);
        }
    }
}

// Block route: two passes over X, four vectors per thread per step (the
// loads of a step go out together; lanes past the row re-read its last
// vector).  E == 1 is the scalar route.
// Spans read element by element otherwise (an odd span, or X, gate and Y
// sharing a base 2 or 6 bytes off a 16-byte boundary) and too long for the
// flat route: counted from the boundary at or below X's base, row r holds
// elements [a, a + C), a = r * C + phase; its lanes read the aligned
// 16-byte vectors of X and gate that cover them (the first and last may
// hold a neighbouring row's elements, read and left unused, never outside
// the 16-byte chunks that hold the tensors' own elements), write the
// interior vectors of Y whole and the two boundary vectors element by
// element.  scale is 16-byte aligned: a lane takes its elements' values
// from the two aligned vectors around them, funnel-shifted by the row's
// offset p = a mod E (uniform over the row).  WPR waves per row (1, 2 or 4
// in 256-thread blocks, or 8 and 16 in blocks of WPB = WPR waves), NV
// vectors per lane; the wave sums meet in LDS and are added in wave order.
template <typename T, int E, int NV, int WPR, int WPB>
__global__ void __launch_bounds__(64 * WPB)
gated_phase_kernel(const T* __restrict__ X, const T* __restrict__ scale,
                   const T* __restrict__ gate, T* __restrict__ Y, int64_t rows, int span, int phase,
                   int nvg, float span_f, float eps) {
    using V = Vec<T, E>;
    constexpr int LANES = 64 * WPR;
    static_assert(WPB % WPR == 0, "whole rows per block");
    __shared__ float wave_part[WPB];
    const int lane = threadIdx.x % LANES;
    const int64_t my_row = int64_t(blockIdx.x) * (WPB / WPR) + threadIdx.x / LANES;
    // With two rows per block the waves of a missing second row stay for the
    // barrier and store nothing.
    if (WPR != 2 && my_row >= rows) return;
    const bool live = my_row < rows;
    const int64_t row = live ? my_row : rows - 1;

    const int64_t a = row * span + phase;
    const int64_t v0 = a / E;                            // the row's first vector
    const int p = int(a - v0 * E);                       // its first element's place in it
    const int nvr = int((a + span + E - 1) / E - v0);    // vectors the row touches
    const T* x_a = X - phase;                            // 16-byte aligned bases
    const T* g_a = gate - phase;
    T* y_a = Y - phase;
    const int k_shift = (E - p) % E;
    const int pv = p > 0 ? 1 : 0;
    auto clamp = [&](int i) { return i < nvr ? i : nvr - 1; };
    V xs[NV], gs[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int i = clamp(v * LANES + lane);
        xs[v] = load_vec_stream<T, E>(x_a, v0 + i);
        gs[v] = load_vec_stream<T, E>(g_a, v0 + i);
    }
    // Element e of vector i lies in the row when lo_e <= e < hi_e.
    auto in_row = [&](int i, int e) { return i < nvr && e >= p - i * E && e < span + p - i * E; };
    auto whole = [&](int i) { return i < nvr && p - i * E <= 0 && span + p - i * E >= E; };
    float acc = 0.0f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int i = v * LANES + lane;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float x = to_f32(xs[v].v[e]);
            acc = in_row(i, e) ? fmaf_(x, x, acc) : acc;
        }
    }
    float total = segment_sum<64>(acc);
    if constexpr (WPR > 1) {
        if ((threadIdx.x & 63) == 0) wave_part[threadIdx.x >> 6] = total;
        __syncthreads();
        const int w0 = (threadIdx.x / LANES) * WPR;
        total = wave_part[w0];
#pragma unroll
        for (int w = 1; w < WPR; ++w) total += wave_part[w0 + w];
    }
    const float r = inv_sqrt(total / span_f + eps);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int i = v * LANES + lane;
        // scale of vector i's elements (row positions i*E - p + e).
        int lo = i - pv, hi = i - pv + 1;
        lo = lo < 0 ? 0 : (lo < nvg ? lo : nvg - 1);
        hi = hi < 0 ? 0 : (hi < nvg ? hi : nvg - 1);
        const V sv = funnel16<T, E>(load_vec<T, E>(scale, lo), load_vec<T, E>(scale, hi), k_shift);
        V out;
#pragma unroll
        for (int e = 0; e < E; ++e)
            out.v[e] = from_f32<T>(to_f32(xs[v].v[e]) * r * to_f32(sv.v[e]) * silu_f32(to_f32(gs[v].v[e])));
        if (live) {
            if (whole(i)) {
                store_vec_stream<T, E>(y_a, v0 + i, out);
            } else if (i < nvr) {
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (in_row(i, e)) y_a[(v0 + i) * E + e] = out.v[e];
            }
        }
    }
}

// Spans wider than the row route holds (4096 sixteen-byte vectors, 64 KB,
// with X and gate both in registers), up to kWideRegs + kWideLds vectors
// per lane (272 KB of X): one 1024-thread workgroup per span keeps X alone
// -- its first kWideRegs vectors per lane in VGPRs, the rest in LDS -- and
// reads gate and scale only to form the output, after the statistic, so
// every tensor is still read once.  Lane t holds vectors t + 1024 v; its
// LDS vectors t + 1024 (kWideRegs + j) sit at tail[1024 j + t].  Loads of
// the LDS part (and later of its gate and scale) stream through in chunks of
// kWideChunk vectors per lane, the next chunk's loads issued before the
// current one is used, every load unconditional with a clamped index.
template <typename T>
__global__ void __launch_bounds__(kWideThreads)
gated_wide_kernel(const T* __restrict__ X, const T* __restrict__ scale,
                  const T* __restrict__ gate, T* __restrict__ Y, int nvec, float span_f, float eps) {
    constexpr int E = VecWidth<T>::value;
    using V = Vec<T, E>;
    constexpr int L = kWideThreads, NV = kWideRegs, CH = kWideChunk;
    __shared__ V tail[kWideLds * L];
    __shared__ float wave_part[L / 64];
    const int t = threadIdx.x;
    const int64_t base = int64_t(blockIdx.x) * nvec;
    const int ntail = nvec > NV * L ? (nvec - NV * L + L - 1) / L : 0;  // uniform, <= kWideLds
    const int nch = (ntail + CH - 1) / CH;
    auto clamp = [&](int idx) { return idx < nvec ? idx : nvec - 1; };
    auto tail_idx = [&](int j) { return NV * L + j * L + t; };

    V xs[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) xs[v] = load_vec_stream<T, E>(X, base + clamp(v * L + t));
    V ax[CH], bx[CH];
    auto load_chunk = [&](int c, V(&x)[CH]) {
#pragma unroll
        for (int i = 0; i < CH; ++i) x[i] = load_vec_stream<T, E>(X, base + clamp(tail_idx(c * CH + i)));
    };
    if (nch > 0) load_chunk(0, ax);
    float acc = 0.0f;
#pragma unroll
    for (int v = 0; v < NV; ++v)
        if (v * L + t < nvec) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float x = to_f32(xs[v].v[e]);
                acc = fmaf_(x, x, acc);
            }
        }
    auto keep_chunk = [&](int c, const V(&x)[CH]) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int j = c * CH + i;
            if (tail_idx(j) < nvec) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float xv = to_f32(x[i].v[e]);
                    acc = fmaf_(xv, xv, acc);
                }
                tail[j * L + t] = x[i];
            }
        }
    };
    for (int c = 0; c < nch; c += 2) {
        load_chunk(c + 1 < nch ? c + 1 : nch - 1, bx);
        keep_chunk(c, ax);
        load_chunk(c + 2 < nch ? c + 2 : nch - 1, ax);
        if (c + 1 < nch) keep_chunk(c + 1, bx);
    }
    // Span total: butterfly in each wave, then the 16 wave sums in wave order
    // (each lane reads back only its own LDS vectors).
    float total = segment_sum<64>(acc);
    if ((t & 63) == 0) wave_part[t >> 6] = total;
    __syncthreads();
    total = wave_part[0];
#pragma unroll
    for (int w = 1; w < L / 64; ++w) total += wave_part[w];
    const float r = inv_sqrt(total / span_f + eps);

    auto form = [&](const V& xv, const V& gv, const V& sv) {
        V out;
#pragma unroll
        for (int e = 0; e < E; ++e)
            out.v[e] = from_f32<T>(to_f32(xv.v[e]) * r * to_f32(sv.v[e]) * silu_f32(to_f32(gv.v[e])));
        return out;
    };
    V ag[CH], as[CH], bg[CH], bs[CH];
    auto load_par = [&](int c, V(&g)[CH], V(&sc)[CH]) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int idx = clamp(tail_idx(c * CH + i));
            g[i] = load_vec_stream<T, E>(gate, base + idx);
            sc[i] = load_vec<T, E>(scale, idx);
        }
    };
    if (nch > 0) load_par(0, ag, as);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int idx = v * L + t;
        const V gv = load_vec_stream<T, E>(gate, base + clamp(idx));
        const V sv = load_vec<T, E>(scale, clamp(idx));
        const V out = form(xs[v], gv, sv);
        if (idx < nvec) store_vec_stream<T, E>(Y, base + idx, out);
    }
    auto out_chunk = [&](int c, const V(&g)[CH], const V(&sc)[CH]) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int j = c * CH + i;
            const int idx = tail_idx(j);
            if (idx < nvec) store_vec_stream<T, E>(Y, base + idx, form(tail[j * L + t], g[i], sc[i]));
        }
    };
    for (int c = 0; c < nch; c += 2) {
        load_par(c + 1 < nch ? c + 1 : nch - 1, bg, bs);
        out_chunk(c, ag, as);
        load_par(c + 2 < nch ? c + 2 : nch - 1, ag, as);
        if (c + 1 < nch) out_chunk(c + 1, bg, bs);
    }
}

template <typename T, int E>
__global__ void __launch_bounds__(256)
gated_block_kernel(const T* __restrict__ X, const T* __restrict__ scale,
                   const T* __restrict__ gate, T* __restrict__ Y, int64_t rows,
                   int64_t nvec, float span_f, float eps) {
    using V = Vec<T, E>;
    constexpr int U = 4;
    __shared__ float wave_part[4];
    const int t = threadIdx.x;
    auto clamp = [&](int64_t j) { return j < nvec ? j : nvec - 1; };
    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const int64_t base = row * nvec;
        float acc = 0.0f;
        for (int64_t j0 = t; j0 < nvec; j0 += 256 * U) {
            V xs[U];
#pragma unroll
            for (int u = 0; u < U; ++u) xs[u] = load_vec<T, E>(X, base + clamp(j0 + u * 256));
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (j0 + u * 256 < nvec) {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const float x = to_f32(xs[u].v[e]);
                        acc = fmaf_(x, x, acc);
                    }
                }
        }
        acc = segment_sum<64>(acc);
        if ((t & 63) == 0) wave_part[t >> 6] = acc;
        __syncthreads();
        const float total = (wave_part[0] + wave_part[1]) + (wave_part[2] + wave_part[3]);
        __syncthreads();  // wave_part is rewritten for the next row
        const float r = inv_sqrt(total / span_f + eps);
        for (int64_t j0 = t; j0 < nvec; j0 += 256 * U) {
            V xs[U], gs[U], ss[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t jc = clamp(j0 + u * 256);
                xs[u] = load_vec_stream<T, E>(X, base + jc);
                gs[u] = load_vec_stream<T, E>(gate, base + jc);
                ss[u] = load_vec<T, E>(scale, jc);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                V out;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float x = to_f32(xs[u].v[e]);
                    const float g = to_f32(gs[u].v[e]);
                    out.v[e] = from_f32<T>(x * r * to_f32(ss[u].v[e]) * silu_f32(g));
                }
                if (j0 + u * 256 < nvec) store_vec_stream<T, E>(Y, base + j0 + u * 256, out);
            }
        }
    }
}

template <typename T, int E, int L, int VPL>
hipError_t launch_segment(const GatedArgs& a, int nvec, hipStream_t stream) {
    // Vectors of X (and of gate) per thread in flight: 4 of 16 bytes; 16 of
    // 4 or 2 bytes (measured 1.1-1.6x faster than 4 where a row takes all
    // 64 lanes, the same elsewhere); 8 of 8 bytes where a row takes 64
    // lanes, else 4 (8 measured 2-3 % slower there).
    constexpr int VB = E * int(sizeof(T));
    constexpr int WANT = VB >= 16 ? 4 : VB == 8 ? (L == 64 ? 8 : 4) : 16;
    constexpr int RPT = VPL >= WANT ? 1 : WANT / VPL;
    constexpr int rows_per_block = (256 / L) * RPT;
    const int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(unsigned(blocks)), dim3(256), 0, stream,
                           static_cast<const T*>(a.X), static_cast<const T*>(a.scale),
                           static_cast<const T*>(a.gate), static_cast<T*>(a.Y), a.rows, nvec,
                           float(a.span), a.epsilon);
        return hipGetLastError();
    };
    // Rows of more than 64 vectors off the 128-byte grid store their shared
    // lines through L2 (f16 C = 1000 +4 %, f32 C = 264 / 280 +6 / +4 %);
    // shorter ones measured up to 13 % slower that way and keep streaming.
    if constexpr (VPL >= 2) {
        if (rows_off_lines(a.span * int64_t(sizeof(T)), {a.Y}))
            return go(gated_segment_kernel<T, E, L, VPL, RPT, true>);
    }
    return go(gated_segment_kernel<T, E, L, VPL, RPT, false>);
}

template <typename T, int E>
hipError_t launch_segment_for(const GatedArgs& a, int nvec, hipStream_t stream) {
    if (nvec <= 1) return launch_segment<T, E, 1, 1>(a, nvec, stream);
    if (nvec <= 2) return launch_segment<T, E, 2, 1>(a, nvec, stream);
    if (nvec <= 4) return launch_segment<T, E, 4, 1>(a, nvec, stream);
    if (nvec <= 8) return launch_segment<T, E, 8, 1>(a, nvec, stream);
    if (nvec <= 16) return launch_segment<T, E, 16, 1>(a, nvec, stream);
    if (nvec <= 32) return launch_segment<T, E, 32, 1>(a, nvec, stream);
    if (nvec <= 64) return launch_segment<T, E, 64, 1>(a, nvec, stream);
    if (nvec <= 128) return launch_segment<T, E, 64, 2>(a, nvec, stream);
    if (nvec <= 256) return launch_segment<T, E, 64, 4>(a, nvec, stream);
    if (nvec <= 512) return launch_segment<T, E, 64, 8>(a, nvec, stream);
    if (nvec <= 1024) return launch_segment<T, E, 64, 16>(a, nvec, stream);
    return hipErrorInvalidValue;  // callers check the width first
}

constexpr int64_t kMaxSegmentVectors = 1024;
// Widest rows of the row route: 16 waves of four 16-byte vectors per thread,
// or of eight narrower accesses (eight 16-byte ones would spill under the
// 1024-thread block's 128-VGPR limit).
constexpr int64_t kMaxRowVectors16 = 1024 * 4;
constexpr int64_t kMaxRowVectors = 1024 * 8;

template <typename T, int E, int NV, int TPB>
hipError_t launch_row(const GatedArgs& a, int nvec, hipStream_t stream) {
    const int64_t blocks = a.rows < (int64_t(1) << 20) ? a.rows : (int64_t(1) << 20);
    hipLaunchKernelGGL((gated_row_kernel<T, E, NV, TPB>), dim3(unsigned(blocks)), dim3(TPB), 0, stream,
                       static_cast<const T*>(a.X), static_cast<const T*>(a.scale),
                       static_cast<const T*>(a.gate), static_cast<T*>(a.Y), a.rows, nvec,
                       float(a.span), a.epsilon);
    return hipGetLastError();
}

template <typename T, int E, int TPB>
hipError_t launch_row_nv(const GatedArgs& a, int nvec, int nv, hipStream_t stream) {
    switch (nv) {
        case 2: return launch_row<T, E, 2, TPB>(a, nvec, stream);
        case 3: return launch_row<T, E, 3, TPB>(a, nvec, stream);
        case 4: return launch_row<T, E, 4, TPB>(a, nvec, stream);
        default: break;
    }
    if constexpr (E * sizeof(T) < 16) {
        switch (nv) {
            case 5: return launch_row<T, E, 5, TPB>(a, nvec, stream);
            case 6: return launch_row<T, E, 6, TPB>(a, nvec, stream);
            case 7: return launch_row<T, E, 7, TPB>(a, nvec, stream);
            case 8: return launch_row<T, E, 8, TPB>(a, nvec, stream);
            default: break;
        }
    }
    return hipErrorInvalidValue;  // callers check the width first
}

// Rows of more than 1024 vectors: 8 or 16 waves (512 or 1024 threads) of
// ceil(nvec / threads) vectors per thread, at most four 16-byte vectors or
// eight narrower accesses, whichever of the two leaves fewer lanes re-reading
// past the row's end; on a tie 512 threads, which hold more rows' bytes in
// flight per CU.  One 256-thread block of 8-16 vectors per thread ran
// float32 C = 16384 at 5.4 TB/s, 16 waves of four run it at 6.1; 3072
// vectors as 16 waves of four (a quarter of the loads discarded) ran at
// 5.0 TB/s against 5.4 on one 256-thread block of twelve.
template <typename T, int E>
hipError_t launch_row_for(const GatedArgs& a, int nvec, hipStream_t stream) {
    constexpr int kNvMax = E * sizeof(T) >= 16 ? 4 : 8;
    const int nv512 = (nvec + 511) / 512, nv1024 = (nvec + 1023) / 1024;
    if (nv512 <= kNvMax && 512 * nv512 <= 1024 * nv1024)
        return launch_row_nv<T, E, 512>(a, nvec, nv512, stream);
    return launch_row_nv<T, E, 1024>(a, nvec, nv1024, stream);
}

template <typename T, int NV, int WPR, int WPB>
hipError_t launch_phase_nv(const GatedArgs& a, int phase, int nvg, hipStream_t stream) {
    constexpr int E = VecWidth<T>::value;
    constexpr int rows_per_block = WPB / WPR;
    const int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL((gated_phase_kernel<T, E, NV, WPR, WPB>), dim3(unsigned(blocks)), dim3(64 * WPB), 0,
                       stream, static_cast<const T*>(a.X), static_cast<const T*>(a.scale),
                       static_cast<const T*>(a.gate), static_cast<T*>(a.Y), a.rows, int(a.span), phase, nvg,
                       float(a.span), a.epsilon);
    return hipGetLastError();
}

template <typename T, int WPR, int WPB = 4>
hipError_t launch_phase_w(const GatedArgs& a, int nmax, int phase, int nvg, hipStream_t stream) {
    const int need = (nmax + 64 * WPR - 1) / (64 * WPR);
    if (need <= 1) return launch_phase_nv<T, 1, WPR, WPB>(a, phase, nvg, stream);
    if (need <= 2) return launch_phase_nv<T, 2, WPR, WPB>(a, phase, nvg, stream);
    if (need <= 3) return launch_phase_nv<T, 3, WPR, WPB>(a, phase, nvg, stream);
    return launch_phase_nv<T, 4, WPR, WPB>(a, phase, nvg, stream);
}

// Vectors per lane of the phased route: four 16-byte vectors of X and of
// gate (deeper, the scale funnels would crowd the 1024-thread block's
// 128 VGPRs).
constexpr int kPhaseNv = 4;

// The phased route (see gated_phase_kernel) for spans that would be read
// element by element: taken when X, gate and Y share their offset from a
// 16-byte boundary, scale is 16-byte aligned, and a span touches more than
// 32 and at most 1024 * kPhaseNv vectors.  Returns false, having launched
// nothing, otherwise.
template <typename T>
bool launch_gated_phase(const GatedArgs& a, hipStream_t stream, const char** route, hipError_t* err) {
    constexpr int E = VecWidth<T>::value;
    const uintptr_t ph = reinterpret_cast<uintptr_t>(a.X) % 16;
    if (ph % sizeof(T) != 0 || reinterpret_cast<uintptr_t>(a.gate) % 16 != ph ||
        reinterpret_cast<uintptr_t>(a.Y) % 16 != ph || !aligned16(a.scale))
        return false;
    const int64_t nmax = a.span / E + 2;  // vectors a span can touch
    if (nmax <= 32 || nmax > 1024 * kPhaseNv) return false;
    const int phase = int(ph / sizeof(T));
    const int nvg = int((a.span + E - 1) / E);
    const int n = int(nmax);
    *route = "gated.phase.vec16";
    if (nmax <= 64 * kPhaseNv) *err = launch_phase_w<T, 1>(a, n, phase, nvg, stream);
    else if (nmax <= 128 * kPhaseNv) *err = launch_phase_w<T, 2>(a, n, phase, nvg, stream);
    else if (nmax <= 256 * kPhaseNv) *err = launch_phase_w<T, 4>(a, n, phase, nvg, stream);
    else if (nmax <= 512 * kPhaseNv) *err = launch_phase_w<T, 8, 8>(a, n, phase, nvg, stream);
    else *err = launch_phase_w<T, 16, 16>(a, n, phase, nvg, stream);
    return true;
}

// The wide route (see gated_wide_kernel): spans of 16-byte vectors beyond
// the row route, one 1024-thread workgroup per span.
constexpr int64_t kMaxWideVectors = int64_t(kWideThreads) * (kWideRegs + kWideLds);

template <typename T>
hipError_t launch_wide(const GatedArgs& a, int64_t nvec, hipStream_t stream) {
    hipLaunchKernelGGL(gated_wide_kernel<T>, dim3(unsigned(a.rows)), dim3(kWideThreads), 0, stream,
                       static_cast<const T*>(a.X), static_cast<const T*>(a.scale),
                       static_cast<const T*>(a.gate), static_cast<T*>(a.Y), int(nvec), float(a.span),
                       a.epsilon);
    return hipGetLastError();
}

template <typename T, int E>
hipError_t launch_block(const GatedArgs& a, int64_t nvec, hipStream_t stream) {
    const int64_t blocks = a.rows < (int64_t(1) << 20) ? a.rows : (int64_t(1) << 20);
    hipLaunchKernelGGL((gated_block_kernel<T, E>), dim3(unsigned(blocks)), dim3(256), 0, stream,
                       static_cast<const T*>(a.X), static_cast<const T*>(a.scale),
                       static_cast<const T*>(a.gate), static_cast<T*>(a.Y), a.rows, nvec,
                       float(a.span), a.epsilon);
    return hipGetLastError();
}

// Tile plan for rows of nvec vectors of vec_bytes each: taken for rows of
// 33 to 128 vectors of 8 or 4 bytes that fill less than 60 % of the segment
// route's lane slots (beyond that the segment route measured as fast), with
// the vectors per lane (4, 8 or 16, and no more than 64 bytes of each tensor
// per lane beyond 4 vectors, which keeps the held data at 32 VGPRs or less)
// that leave the fewest idle slots.
struct TilePlan {
    int vpt, rt, lpr_log;
    uint32_t magic;
};

bool gated_tile_plan(int64_t nvec, int vec_bytes, TilePlan* p) {
    if (vec_bytes != 8 && vec_bytes != 4) return false;
    if (nvec <= 32 || nvec > 128 || (nvec & (nvec - 1)) == 0) return false;
    int64_t lanes = 1;
    while (lanes < nvec && lanes < 64) lanes <<= 1;
    int64_t vpl = 1;
    while (lanes * vpl < nvec) vpl <<= 1;
    const double seg_eff = double(nvec) / double(lanes * vpl);
    if (seg_eff >= 0.6) return false;
    double best = 0.0;
    for (int vpt : {4, 8, 16}) {
        if (vpt > 4 && vpt * vec_bytes > 64) continue;
        const int64_t rt = 64 * vpt / nvec;
        if (rt < 1 || rt > 64) continue;
        const double eff = double(rt * nvec) / double(64 * vpt);
        if (eff > best + 1e-9) {
            best = eff;
            p->vpt = vpt;
            p->rt = int(rt);
        }
    }
    if (best <= seg_eff) return false;
    int rtp = 1;
    while (rtp < p->rt) rtp <<= 1;
    int lpr_log = 0;
    while ((1 << lpr_log) * rtp < 64) ++lpr_log;
    p->lpr_log = lpr_log;
    p->magic = uint32_t((uint64_t(1) << 32) / uint64_t(nvec) + 1);
    return true;
}

template <typename T, int E, int VPT>
hipError_t launch_tile(const GatedArgs& a, int nvec, const TilePlan& p, hipStream_t stream) {
    const int64_t tiles = (a.rows + p.rt - 1) / p.rt;
    const int64_t blocks = (tiles + 3) / 4;
    hipLaunchKernelGGL((gated_tile_kernel<T, E, VPT>), dim3(unsigned(blocks)), dim3(256), 0, stream,
                       static_cast<const T*>(a.X), static_cast<const T*>(a.scale),
                       static_cast<const T*>(a.gate), static_cast<T*>(a.Y), a.rows, nvec, p.rt,
                       p.lpr_log, p.magic, float(a.span), a.epsilon);
    return hipGetLastError();
}

template <typename T, int E>
hipError_t launch_tile_for(const GatedArgs& a, int nvec, const TilePlan& p, hipStream_t stream) {
    if (p.vpt == 4) return launch_tile<T, E, 4>(a, nvec, p, stream);
    if constexpr (E * sizeof(T) <= 8)
        if (p.vpt == 8) return launch_tile<T, E, 8>(a, nvec, p, stream);
    if constexpr (E * sizeof(T) <= 4)
        if (p.vpt == 16) return launch_tile<T, E, 16>(a, nvec, p, stream);
    return hipErrorInvalidValue;  // the plan only picks the widths above
}

// Where the automatic choice takes the flat route, for rows whose widest
// access (E elements of T) is narrower than 16 bytes, as measured on
// 2^27-element tensors against the segment and tile routes: tiles at least
// 3/4 full, and element-by-element rows of two elements or more (float32:
// from 8 elements on; the segment route's coalesced 4-byte loads win below),
// float16 pairs unless a row is one pair, and 8-byte rows whose segment lane
// group would be less than 3/4 full (float32: 0.6).  Float16 C = 3 to 301:
// 4.4-5.8 TB/s against 2.1-5.3 before; float32 C = 9 to 602: 5.3-5.6 against
// 4.3-5.2.
template <typename T>
bool flat_preferred(int64_t C, int E, const FlatPlan& p) {
    if (p.fill < 0.75) return false;
    const int64_t nvec = C / E;
    if (E == 1) return C >= (sizeof(T) == 2 ? 2 : 8);
    if (E * sizeof(T) == 4) return nvec >= 2;
    int64_t lanes = 1;
    while (lanes < nvec && lanes < 64) lanes <<= 1;
    int64_t vpl = 1;
    while (lanes * vpl < nvec) vpl <<= 1;
    return double(nvec) / double(lanes * vpl) < (sizeof(T) == 2 ? 0.75 : 0.6);
}

template <typename T, int VPT>
hipError_t launch_flat(const GatedArgs& a, const FlatPlan& p, int phase, hipStream_t stream) {
    const int C = int(a.span);
    const int64_t tiles = (a.rows + p.rt - 1) / p.rt;
    const int64_t blocks = (tiles + 3) / 4;
    const FastDiv cdiv = make_fastdiv(uint32_t(C));
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(unsigned(blocks)), dim3(256), 0, stream,
                           static_cast<const T*>(a.X), static_cast<const T*>(a.scale),
                           static_cast<const T*>(a.gate), static_cast<T*>(a.Y), a.rows, C, p.rt,
                           p.lpr_log, phase, cdiv, float(a.span), a.epsilon);
        return hipGetLastError();
    };
    if (C < VecWidth<T>::value) return go(gated_flat_kernel<T, VPT, true>);
    return go(gated_flat_kernel<T, VPT, false>);
}

template <typename T>
hipError_t launch_flat_for(const GatedArgs& a, const FlatPlan& p, int phase, hipStream_t stream) {
    constexpr int small = 16 / VecWidth<T>::value;
    if (p.vpt == small) return launch_flat<T, small>(a, p, phase, stream);
    return launch_flat<T, 2 * small>(a, p, phase, stream);
}

template <typename T>
hipError_t launch_gated_t(const GatedArgs& a, Route want, hipStream_t stream, const char** route) {
    // Widest access that divides the row and every tensor's base.
    int E = widest_vector<T>(a.span, {a.X, a.scale, a.gate, a.Y});
    if (want == Route::Scalar) E = 1;
    const int64_t nvec = a.span / E;
    // The flat route, forced or (rows read with accesses narrower than 16
    // bytes) where it measured faster, when X, gate and Y share their offset
    // from the 16-byte grid.
    if (want == Route::Flat || (want == Route::Auto && E * sizeof(T) < 16)) {
        const uintptr_t ph = reinterpret_cast<uintptr_t>(a.X) % 16;
        FlatPlan fp;
        if (ph % sizeof(T) == 0 && reinterpret_cast<uintptr_t>(a.gate) % 16 == ph &&
            reinterpret_cast<uintptr_t>(a.Y) % 16 == ph &&
            flat_plan(a.span, VecWidth<T>::value, want == Route::Flat || sizeof(T) == 4, &fp) &&
            (want == Route::Flat || flat_preferred<T>(a.span, E, fp))) {
            *route = "gated.flat.vec16";
            return launch_flat_for<T>(a, fp, int(ph / sizeof(T)), stream);
        }
    }
    // The phased route (aligned 16-byte vectors across span boundaries) for
    // spans read element by element beyond the flat route, and for spans of
    // more than 300 four-byte or 256 eight-byte vectors, where it measured
    // faster (f16 C = 766 / 1026 / 2050 / 8194 +17 / +14 / +40 / +26 %,
    // 1028 / 2052 / 4100 +20 / +21 / +15 %, f32 1026 / 2050 +22 / +6 %;
    // shorter ones keep the segment route: f16 C = 350 / 514 -5 / -4 %,
    // 380 / 1012 -10 / -3 %).
    const int vbytes = E * int(sizeof(T));
    const bool phase_pref = E == 1 || (vbytes == 4 && nvec > 300) || (vbytes == 8 && nvec > 256);
    if (want != Route::Scalar && want != Route::Block && phase_pref) {
        hipError_t err = hipSuccess;
        if (launch_gated_phase<T>(a, stream, route, &err)) return err;
    }
    if constexpr (sizeof(T) == 2) {
        TilePlan tp;
        if ((want == Route::Auto || want == Route::Flat) && E > 1 &&
            gated_tile_plan(nvec, int(E * sizeof(T)), &tp)) {
            if (E == 4) {
                *route = "gated.tile.vec8";
                return launch_tile_for<T, 4>(a, int(nvec), tp, stream);
            }
            *route = "gated.tile.vec4";
            return launch_tile_for<T, 2>(a, int(nvec), tp, stream);
        }
    }
    if (want != Route::Block && nvec <= kMaxSegmentVectors) {
        if (E * sizeof(T) == 16) {
            *route = "gated.segment.vec16";
            return launch_segment_for<T, VecWidth<T>::value>(a, int(nvec), stream);
        }
        if (E * sizeof(T) == 8) {
            *route = "gated.segment.vec8";
            return launch_segment_for<T, 8 / sizeof(T)>(a, int(nvec), stream);
        }
        if constexpr (sizeof(T) == 2) {
            if (E == 2) {
                *route = "gated.segment.vec4";
                return launch_segment_for<T, 2>(a, int(nvec), stream);
            }
        }
        *route = "gated.segment.scalar";
        return launch_segment_for<T, 1>(a, int(nvec), stream);
    }
    if (want != Route::Block && nvec <= (E * sizeof(T) == 16 ? kMaxRowVectors16 : kMaxRowVectors)) {
        if (E * sizeof(T) == 16) {
            *route = "gated.row.vec16";
            return launch_row_for<T, VecWidth<T>::value>(a, int(nvec), stream);
        }
        if (E * sizeof(T) == 8) {
            *route = "gated.row.vec8";
            return launch_row_for<T, 8 / sizeof(T)>(a, int(nvec), stream);
        }
        if constexpr (sizeof(T) == 2) {
            if (E == 2) {
                *route = "gated.row.vec4";
                return launch_row_for<T, 2>(a, int(nvec), stream);
            }
        }
        *route = "gated.row.scalar";
        return launch_row_for<T, 1>(a, int(nvec), stream);
    }
    // Wider spans of 16-byte vectors: the wide route while a span fits one
    // workgroup's registers and LDS (one workgroup per span keeps the grid
    // below 2^32 work-items).
    if (want != Route::Block && E == VecWidth<T>::value && nvec <= kMaxWideVectors &&
        a.rows < (int64_t(1) << 22)) {
        *route = "gated.wide.vec16";
        return launch_wide<T>(a, nvec, stream);
    }
    // The block route: wider rows, or forced (then with scalar accesses).
    if (want == Route::Block) E = 1;
    const int64_t bvec = a.span / E;
    if (E * sizeof(T) == 16) {
        *route = "gated.block.vec16";
        return launch_block<T, VecWidth<T>::value>(a, bvec, stream);
    }
    if (E * sizeof(T) == 8) {
        *route = "gated.block.vec8";
        return launch_block<T, 8 / sizeof(T)>(a, bvec, stream);
    }
    if constexpr (sizeof(T) == 2) {
        if (E == 2) {
            *route = "gated.block.vec4";
            return launch_block<T, 2>(a, bvec, stream);
        }
    }
    *route = "gated.block";
    return launch_block<T, 1>(a, bvec, stream);
}

}  // namespace

hipError_t launch_gated(const GatedArgs& a, Route want, hipStream_t stream, const char** route) {
    if (a.rows == 0) {
        *route = "gated.empty";
        return hipSuccess;
    }
    if (a.dtype == 0) return launch_gated_t<float>(a, want, stream, route);
    return launch_gated_t<half_t>(a, want, stream, route);
}

}  // namespace sn
