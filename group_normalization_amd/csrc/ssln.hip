// ssln.hip -- SkipSimplifiedLayerNormalization kernels for gfx950.
//
// Operator ("com.microsoft.SkipSimplifiedLayerNormalization", Description,
// Inputs, Outputs): per row, S = input + skip (+ bias) rounded to T,
// r = 1/sqrt(mean(S^2) + epsilon), output = S * r * gamma; optional outputs
// S, mean (zero for the simplified form) and inv_std_var (r).
//
// The same kernels with the mean removed (CENTER) give the non-simplified
// skip layer normalization: mean = mean(S), r = 1/sqrt(mean((S - mean)^2) +
// epsilon), output = (S - mean) * r * gamma (+ beta).
//
// Routes:
//   segment  rows of at most 48 accesses: a power-of-two group of lanes per
//          row, several rows per wave and per thread (ssln_segment_kernel).
//   wave   one wave64 per row (wave2: two; rows of up to 4 sixteen-byte,
//          8 eight-byte or 16 narrower accesses per lane); lane l holds the
//          row's vectors l, l+64, ...
//          in VGPRs as T (the rounded S is exactly representable in T), so
//          the row is read once and written once, with nontemporal loads
//          and stores (gamma and bias, shared by every row, stay cached).
//          E elements per access: the widest of 16-, 8- and 4-byte vectors
//          that divides the row and every base address, else scalars.
//   rowblock, row8, row16  the same with 4, 8 or 16 waves (a 256-, 512-
//          or 1024-thread workgroup) per row for wider rows, at the same
//          accesses per lane, and 16 waves of up to 8 sixteen-byte vectors
//          per lane for the widest (128 KB rows: 65536 float16 / 32768
//          float32 elements): the wave sums meet in LDS and are added in
//          wave order.
//   phase  rows that would otherwise be read element by element (an odd
//          row length, or data tensors sharing a base 2 or 6 bytes off a
//          16-byte boundary), and rows of 4- or 8-byte accesses where it
//          measured faster (phase_preferred): aligned 16-byte vectors read
//          across row boundaries, boundary elements masked
//          (ssln_phase_kernel).
//   wide   rows of 16-byte vectors beyond the register routes, up to 272 KB:
//          one 1024-thread workgroup per row, S held in VGPRs (8 vectors
//          per lane) and LDS (up to 9 more), so still one read and one write
//          (ssln_wide_kernel).
//   block  one 256-thread workgroup per row for any wider row: S is formed
//          twice (once for the statistic, once for the output; three times
//          with the mean removed), reading the inputs again each time.
// Statistic: each lane accumulates its own squares in float32 (FMA), then a
// fixed butterfly sums the 64 lanes (DPP inside 16-lane rows, then two
// cross-row exchanges), so every lane holds the same total and the result
// does not depend on which optional outputs were requested.
#include <type_traits>

#include "device_common.h"
#include "skipnorm_internal.h"

namespace sn {
namespace {

constexpr int kWavesPerBlock = 4;

// v with its raw bits ANDed with m (all ones keeps v, zero makes every
// element +0).
template <typename T, int E>
__device__ __forceinline__ Vec<T, E> mask_bits(const Vec<T, E>& v, uint32_t m) {
    using R = typename RawBits<sizeof(Vec<T, E>)>::type;
    return __builtin_bit_cast(Vec<T, E>, R(__builtin_bit_cast(R, v) & R(m)));
}

// WPR waves per row: 1, 2 or 4 (four, two or one rows per 256-thread
// block), or 8 and 16 (one row per block of WPB = WPR waves).  Lane l of the
// row's 64*WPR lanes holds vectors l, l + 64*WPR, ...
// CENTER: remove the row mean (skip layer normalization) instead of the
// simplified root-mean-square form.
template <typename T, int E, int NV, bool FULL, int WPR, bool CENTER, int WPB>
__global__ void __launch_bounds__(64 * WPB)
ssln_wave_kernel(const T* __restrict__ input, const T* __restrict__ skip,
                 const T* __restrict__ gamma, const T* __restrict__ beta,
                 const T* __restrict__ bias, T* __restrict__ output, float* __restrict__ mean,
                 float* __restrict__ inv_std_var, T* __restrict__ sum,
                 int64_t rows, int nvec, float hidden_f, float eps, uint32_t beta_mask,
                 int lines) {
    using V = Vec<T, E>;
    constexpr int LANES = 64 * WPR;
    static_assert(WPB % WPR == 0, "whole rows per block");
    __shared__ float wave_part[WPB];
    const int lane = threadIdx.x % LANES;
    const int64_t my_row = int64_t(blockIdx.x) * (WPB / WPR) + threadIdx.x / LANES;
    // A whole wave (WPR = 1) or block (WPR = 4) leaves; with two rows per
    // block the waves of a missing second row stay for the barrier and
    // store nothing.
    if (WPR != 2 && my_row >= rows) return;
    const bool live = my_row < rows;
    const int64_t row = live ? my_row : rows - 1;
    const int64_t base = row * nvec;
    const bool has_bias = bias != nullptr;
    // lines: rows that do not all start on 128-byte lines (a uniform
    // argument): the vectors in lines shared with the neighbouring rows are
    // stored through L2.  Rows that fill the lanes exactly (FULL) keep plain
    // streaming stores: their widths are whole lines, and the check alone
    // cost 2-4 % there.
    const bool use_lines = !FULL && lines;
    const LineRun out_run = line_run<T, E>(output + base * E, nvec);
    const LineRun sum_run = line_run<T, E>(sum ? sum + base * E : output, nvec);

    // Issue every load of the row before any arithmetic.  No load sits behind
    // a lane-dependent branch (that makes the compiler wait for each one in
    // turn): lanes past the row's end re-read its last vector and discard it.
    auto clamp = [&](int idx) { return FULL || idx < nvec ? idx : nvec - 1; };
    V xs[NV], ks[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int idx = clamp(v * LANES + lane);
        xs[v] = load_vec_stream<T, E>(input, base + idx);
        ks[v] = load_vec_stream<T, E>(skip, base + idx);
    }
    // With the mean removed, everything is taken about the row's first
    // element S[0] (every lane forms it from the same inputs, bit for bit,
    // after the row's loads are out): S - S[0] is exact for nearby values
    // and the mean of the differences is small, so rows far from zero keep
    // their accuracy in float32.
    // With accesses of 4 bytes or less, bias loads go out with the data,
    // unconditionally (gamma's address in place of an absent bias, its
    // values unused): a load whose use sits behind a branch, even a uniform
    // one, is moved into it and waited for there, one round trip per vector
    // (skip layer norm f16 rows of 186: 6.9 % faster).  Wider accesses keep
    // each vector's bias load beside its use: there the preload measured
    // within +-2 % (the 16 x 2048 x 4096 float16 workload 2.3 % slower), and
    // 1024-thread workgroups would spill.
    constexpr bool kBiasAhead = E * sizeof(T) <= 4 && (64 * WPB < 1024 || 3 * NV * int(E * sizeof(T) / 4) <= 64);
    const T* bias_src = has_bias ? bias : gamma;  // gamma holds a row's vectors
    V bvs[kBiasAhead ? NV : 1];
    if constexpr (kBiasAhead) {
#pragma unroll
        for (int v = 0; v < NV; ++v) bvs[v] = load_vec<T, E>(bias_src, clamp(v * LANES + lane));
    }
    float shift = 0.0f;
    if constexpr (CENTER) {
        T rounded;
        if constexpr (kBiasAhead) {
            const float b0 = to_f32(bias_src[0]);
            shift = residual_sum<T>(to_f32(input[row * nvec * E]), to_f32(skip[row * nvec * E]), has_bias,
                                    has_bias ? b0 : 0.0f, rounded);
        } else {
            shift = residual_sum<T>(to_f32(input[row * nvec * E]), to_f32(skip[row * nvec * E]), has_bias,
                                    has_bias ? to_f32(bias[0]) : 0.0f, rounded);
        }
        shift = row_shift(shift);
    }

    // S for every lane (lanes past the row's end form their re-read vector
    // and add nothing to the sums), so that no use of a load is behind a
    // lane branch.
    V ss[NV];
    float acc = 0.0f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int idx = v * LANES + lane;
        const bool valid = FULL || idx < nvec;
        if constexpr (kBiasAhead) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float s = residual_sum<T>(to_f32(xs[v].v[e]), to_f32(ks[v].v[e]), has_bias,
                                                to_f32(bvs[v].v[e]), ss[v].v[e]);
                if constexpr (CENTER) {
                    acc += valid ? s - shift : 0.0f;
                } else {
                    const float q = valid ? s : 0.0f;
                    acc = fmaf_(q, q, acc);
                }
            }
            if (valid && sum && live) {
                if (use_lines) store_vec_run<T, E>(sum + base * E, idx, ss[v], sum_run);
                else store_vec_stream<T, E>(sum, base + idx, ss[v]);
            }
        } else {
            V bv = {};
            if (has_bias) bv = load_vec<T, E>(bias, clamp(idx));  // cached; outside the lane branch
            if (valid) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float s = residual_sum<T>(to_f32(xs[v].v[e]), to_f32(ks[v].v[e]), has_bias,
                                                    to_f32(bv.v[e]), ss[v].v[e]);
                    if constexpr (CENTER) acc += s - shift;
                    else acc = fmaf_(s, s, acc);
                }
                if (sum && live) {
                    if (use_lines) store_vec_run<T, E>(sum + base * E, idx, ss[v], sum_run);
                    else store_vec_stream<T, E>(sum, base + idx, ss[v]);
                }
            }
        }
    }

    // Row total of the lanes' partial sums: butterfly inside the wave, then
    // the row's waves in order through LDS.
    auto row_total = [&](float part) {
        float total = segment_sum<64>(part);
        if constexpr (WPR > 1) {
            __syncthreads();  // earlier readers of wave_part are done
            if ((threadIdx.x & 63) == 0) wave_part[threadIdx.x >> 6] = total;
            __syncthreads();
            const int w0 = (threadIdx.x / LANES) * WPR;  // the row's first wave
            total = wave_part[w0];
#pragma unroll
            for (int w = 1; w < WPR; ++w) total += wave_part[w0 + w];
        }
        return total;
    };
    // Simplified: r = 1/sqrt(mean(S^2) + eps), no centre.  With the mean
    // removed: md = mean(S - S[0]) (the mean is S[0] + md), then the squared
    // deviations from the S held in registers (a second pass over registers,
    // not memory).
    float md = 0.0f, r;
    if constexpr (!CENTER) {
        r = inv_sqrt(row_total(acc) / hidden_f + eps);
    } else {
        md = row_total(acc) / hidden_f;
        float dev = 0.0f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int idx = v * LANES + lane;
            if (FULL || idx < nvec) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float d = (to_f32(ss[v].v[e]) - shift) - md;
                    dev = fmaf_(d, d, dev);
                }
            }
        }
        r = inv_sqrt(row_total(dev) / hidden_f + eps);
    }
    if (live && lane == 0) {
        if (inv_std_var) inv_std_var[row] = r;
        if (mean) mean[row] = shift + md;
    }

#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int idx = v * LANES + lane;
        const V gv = load_vec<T, E>(gamma, clamp(idx));
        // beta's load and add are unconditional: without a beta the host
        // passes gamma's address and a zero mask, so the added value is +0.
        // (A load whose use sits behind a branch, even a uniform one, is
        // moved into it and waited for on the spot.)
        V bt = {};
        if constexpr (CENTER) bt = mask_bits(load_vec<T, E>(beta, clamp(idx)), beta_mask);
        V out;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if constexpr (CENTER) {
                float y = ((to_f32(ss[v].v[e]) - shift) - md) * r * to_f32(gv.v[e]);
                y = y + to_f32(bt.v[e]);
                out.v[e] = from_f32<T>(y);
            } else {
                out.v[e] = from_f32<T>(to_f32(ss[v].v[e]) * r * to_f32(gv.v[e]));
            }
        }
        if ((FULL || idx < nvec) && live) {
            if (use_lines) store_vec_run<T, E>(output + base * E, idx, out, out_run);
            else store_vec_stream<T, E>(output, base + idx, out);
        }
    }
}

// Rows wider than one workgroup's registers hold (more than 1024 lanes x
// kWideRegs sixteen-byte vectors: 128 KB, 65536 float16 / 32768 float32
// elements), up to kWideRegs + kWideLds vectors per lane (272 KB): one
// 1024-thread workgroup per row keeps the row's first kWideRegs vectors per
// lane in VGPRs, as the widest wave route does, and S of the rest in LDS
// (gfx950 gives a workgroup up to 160 KB), so the row is still read once and
// written once.  Lane t holds vectors t + 1024 v; its LDS vectors are
// t + 1024 (kWideRegs + j), stored at tail[1024 j + t] (consecutive lanes,
// consecutive 16-byte slots).  The LDS part streams through in chunks of
// kWideChunk vectors per lane, the next chunk's loads issued before the
// current one is formed (ping-pong buffers, every load unconditional with
// its index clamped, so none waits behind a branch); bias (or gamma's
// address in its place) is fetched with the chunk.  Output and the
// parameters of the LDS part follow the same pattern.
template <typename T, bool CENTER>
__global__ void __launch_bounds__(kWideThreads)
ssln_wide_kernel(const T* __restrict__ input, const T* __restrict__ skip,
                 const T* __restrict__ gamma, const T* __restrict__ beta,
                 const T* __restrict__ biasp, bool has_bias, T* __restrict__ output,
                 float* __restrict__ mean, float* __restrict__ inv_std_var, T* __restrict__ sum,
                 int nvec, float hidden_f, float eps, uint32_t beta_mask) {
    constexpr int E = VecWidth<T>::value;
    using V = Vec<T, E>;
    constexpr int L = kWideThreads, NV = kWideRegs, CH = kWideChunk;
    __shared__ V tail[kWideLds * L];
    __shared__ float wave_part[L / 64];
    const int t = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int64_t base = row * nvec;
    // LDS vectors per lane (at most kWideLds: the host checks the width) and
    // chunks of them; both uniform.
    const int ntail = nvec > NV * L ? (nvec - NV * L + L - 1) / L : 0;
    const int nch = (ntail + CH - 1) / CH;
    auto clamp = [&](int idx) { return idx < nvec ? idx : nvec - 1; };
    auto tail_idx = [&](int j) { return NV * L + j * L + t; };

    V xs[NV], ks[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int idx = clamp(v * L + t);
        xs[v] = load_vec_stream<T, E>(input, base + idx);
        ks[v] = load_vec_stream<T, E>(skip, base + idx);
    }
    V ax[CH], ak[CH], ab[CH], bx[CH], bk[CH], bb[CH];
    auto load_chunk = [&](int c, V(&x)[CH], V(&k)[CH], V(&b)[CH]) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int idx = clamp(tail_idx(c * CH + i));
            x[i] = load_vec_stream<T, E>(input, base + idx);
            k[i] = load_vec_stream<T, E>(skip, base + idx);
            b[i] = load_vec<T, E>(biasp, idx);
        }
    };
    if (nch > 0) load_chunk(0, ax, ak, ab);

    float shift = 0.0f;  // as in ssln_wave_kernel: statistics about S[0]
    if constexpr (CENTER) {
        T rounded;
        shift = row_shift(residual_sum<T>(to_f32(input[base * E]), to_f32(skip[base * E]), has_bias,
                                          to_f32(biasp[0]), rounded));
    }

    V ss[NV];
    float acc = 0.0f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int idx = v * L + t;
        const V bv = load_vec<T, E>(biasp, clamp(idx));
        if (idx < nvec) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float s = residual_sum<T>(to_f32(xs[v].v[e]), to_f32(ks[v].v[e]), has_bias,
                                                to_f32(bv.v[e]), ss[v].v[e]);
                if constexpr (CENTER) acc += s - shift;
                else acc = fmaf_(s, s, acc);
            }
            if (sum) store_vec_stream<T, E>(sum, base + idx, ss[v]);
        }
    }
    auto form_chunk = [&](int c, const V(&x)[CH], const V(&k)[CH], const V(&b)[CH]) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int j = c * CH + i;
            const int idx = tail_idx(j);
            if (idx < nvec) {
                V sv;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float s = residual_sum<T>(to_f32(x[i].v[e]), to_f32(k[i].v[e]), has_bias,
                                                    to_f32(b[i].v[e]), sv.v[e]);
                    if constexpr (CENTER) acc += s - shift;
                    else acc = fmaf_(s, s, acc);
                }
                tail[j * L + t] = sv;
                if (sum) store_vec_stream<T, E>(sum, base + idx, sv);
            }
        }
    };
    for (int c = 0; c < nch; c += 2) {
        load_chunk(c + 1 < nch ? c + 1 : nch - 1, bx, bk, bb);
        form_chunk(c, ax, ak, ab);
        load_chunk(c + 2 < nch ? c + 2 : nch - 1, ax, ak, ab);
        if (c + 1 < nch) form_chunk(c + 1, bx, bk, bb);
    }

    // Row total: butterfly in each wave, then the 16 wave sums in wave order.
    auto row_total = [&](float part) {
        float total = segment_sum<64>(part);
        __syncthreads();  // earlier readers of wave_part are done; tail is complete
        if ((t & 63) == 0) wave_part[t >> 6] = total;
        __syncthreads();
        total = wave_part[0];
#pragma unroll
        for (int w = 1; w < L / 64; ++w) total += wave_part[w];
        return total;
    };
    // Each lane reads back only its own LDS vectors, so the barriers in
    // row_total are for wave_part alone.
    float md = 0.0f, r;
    if constexpr (!CENTER) {
        r = inv_sqrt(row_total(acc) / hidden_f + eps);
    } else {
        md = row_total(acc) / hidden_f;
        float dev = 0.0f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            if (v * L + t < nvec) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float d = (to_f32(ss[v].v[e]) - shift) - md;
                    dev = fmaf_(d, d, dev);
                }
            }
        }
        for (int j = 0; j < ntail; ++j) {
            if (tail_idx(j) < nvec) {
                const V sv = tail[j * L + t];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float d = (to_f32(sv.v[e]) - shift) - md;
                    dev = fmaf_(d, d, dev);
                }
            }
        }
        r = inv_sqrt(row_total(dev) / hidden_f + eps);
    }
    if (t == 0) {
        if (inv_std_var) inv_std_var[row] = r;
        if (mean) mean[row] = shift + md;
    }

    auto normalize = [&](const V& sv, const V& gv, const V& bt) {
        V out;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if constexpr (CENTER) {
                float y = ((to_f32(sv.v[e]) - shift) - md) * r * to_f32(gv.v[e]);
                y = y + to_f32(bt.v[e]);
                out.v[e] = from_f32<T>(y);
            } else {
                out.v[e] = from_f32<T>(to_f32(sv.v[e]) * r * to_f32(gv.v[e]));
            }
        }
        return out;
    };
    // Parameters of the LDS part: gamma (and beta, masked to +0 without one).
    V ag[CH], at[CH], bg[CH], bt2[CH];
    auto load_par = [&](int c, V(&g)[CH], V(&bt)[CH]) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int idx = clamp(tail_idx(c * CH + i));
            g[i] = load_vec<T, E>(gamma, idx);
            if constexpr (CENTER) bt[i] = mask_bits(load_vec<T, E>(beta, idx), beta_mask);
            else bt[i] = V{};
        }
    };
    if (nch > 0) load_par(0, ag, at);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int idx = v * L + t;
        const V gv = load_vec<T, E>(gamma, clamp(idx));
        V bt = {};
        if constexpr (CENTER) bt = mask_bits(load_vec<T, E>(beta, clamp(idx)), beta_mask);
        const V out = normalize(ss[v], gv, bt);
        if (idx < nvec) store_vec_stream<T, E>(output, base + idx, out);
    }
    auto out_chunk = [&](int c, const V(&g)[CH], const V(&bt)[CH]) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int j = c * CH + i;
            const int idx = tail_idx(j);
            if (idx < nvec) store_vec_stream<T, E>(output, base + idx, normalize(tail[j * L + t], g[i], bt[i]));
        }
    };
    for (int c = 0; c < nch; c += 2) {
        load_par(c + 1 < nch ? c + 1 : nch - 1, bg, bt2);
        out_chunk(c, ag, at);
        load_par(c + 2 < nch ? c + 2 : nch - 1, ag, at);
        if (c + 1 < nch) out_chunk(c + 1, bg, bt2);
    }
}

// Rows off the 16-byte grid: a row length that is not a whole number of
// 16-byte vectors, or data tensors (input, skip, output, S) whose common
// base address sits off a 16-byte boundary.  Counted from the boundary at
// or below that base, row r holds elements [a, a + hidden), a = r * hidden +
// phase; its lanes read the aligned 16-byte vectors that cover them (the
// first and last may hold a neighbouring row's elements, read and left
// unused, never outside the 16-byte chunks that hold the tensors' own
// elements), write the interior vectors whole and the two boundary vectors
// element by element.  gamma, beta and bias are 16-byte aligned: a lane
// takes its elements' values from the two aligned vectors around them,
// funnel-shifted by the row's offset p = a mod E (uniform over the row).
// Without a bias or beta the host passes gamma's address and a zero mask
// (the loads stay unconditional).  Otherwise the arithmetic, its order and
// the row reduction are those of ssln_wave_kernel.
template <typename T, int E, int NV, int WPR, bool CENTER, int WPB>
__global__ void __launch_bounds__(64 * WPB)
ssln_phase_kernel(const T* __restrict__ input, const T* __restrict__ skip,
                  const T* __restrict__ gamma, const T* __restrict__ beta,
                  const T* __restrict__ bias, T* __restrict__ output, float* __restrict__ mean,
                  float* __restrict__ inv_std_var, T* __restrict__ sum,
                  int64_t rows, int hidden, int phase, int nvg, float hidden_f, float eps,
                  uint32_t beta_mask, uint32_t bias_mask) {
    using V = Vec<T, E>;
    constexpr int LANES = 64 * WPR;
    static_assert(WPB % WPR == 0, "whole rows per block");
    __shared__ float wave_part[WPB];
    const int lane = threadIdx.x % LANES;
    const int64_t my_row = int64_t(blockIdx.x) * (WPB / WPR) + threadIdx.x / LANES;
    if (WPR != 2 && my_row >= rows) return;
    const bool live = my_row < rows;
    const int64_t row = live ? my_row : rows - 1;
    const bool has_bias = bias_mask != 0;

    const int64_t a = row * hidden + phase;
    const int64_t v0 = a / E;                              // the row's first vector
    const int p = int(a - v0 * E);                         // its first element's place in it
    const int nvr = int((a + hidden + E - 1) / E - v0);    // vectors the row touches
    const T* in_a = input - phase;                         // 16-byte aligned bases
    const T* sk_a = skip - phase;
    T* out_a = output - phase;
    T* sum_a = sum ? sum - phase : nullptr;
    const int k_shift = (E - p) % E;
    const int pv = p > 0 ? 1 : 0;
    // The parameter values of vector i's elements (row positions i*E - p + e).
    auto param = [&](const T* base, int i) {
        int lo = i - pv, hi = i - pv + 1;
        lo = lo < 0 ? 0 : (lo < nvg ? lo : nvg - 1);
        hi = hi < 0 ? 0 : (hi < nvg ? hi : nvg - 1);
        return funnel16<T, E>(load_vec<T, E>(base, lo), load_vec<T, E>(base, hi), k_shift);
    };

    auto clamp = [&](int i) { return i < nvr ? i : nvr - 1; };
    V xs[NV], ks[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int i = clamp(v * LANES + lane);
        xs[v] = load_vec_stream<T, E>(in_a, v0 + i);
        ks[v] = load_vec_stream<T, E>(sk_a, v0 + i);
    }
    float shift = 0.0f;
    if constexpr (CENTER) {
        T rounded;
        shift = row_shift(residual_sum<T>(to_f32(input[row * hidden]), to_f32(skip[row * hidden]), has_bias,
                                          has_bias ? to_f32(bias[0]) : 0.0f, rounded));
    }
    // Element e of vector i lies in the row when lo_e <= e < hi_e.
    auto in_row = [&](int i, int e) { return i < nvr && e >= p - i * E && e < hidden + p - i * E; };
    auto whole = [&](int i) { return i < nvr && p - i * E <= 0 && hidden + p - i * E >= E; };

    V ss[NV];
    float acc = 0.0f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int i = v * LANES + lane;
        const V bv = mask_bits(param(bias, i), bias_mask);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float s = residual_sum<T>(to_f32(xs[v].v[e]), to_f32(ks[v].v[e]), has_bias,
                                            to_f32(bv.v[e]), ss[v].v[e]);
            const bool ok = in_row(i, e);
            if constexpr (CENTER) acc += ok ? s - shift : 0.0f;
            else acc = ok ? fmaf_(s, s, acc) : acc;
        }
        if (sum_a && live) {
            if (whole(i)) {
                store_vec_stream<T, E>(sum_a, v0 + i, ss[v]);
            } else if (i < nvr) {
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (in_row(i, e)) sum_a[(v0 + i) * E + e] = ss[v].v[e];
            }
        }
    }

    auto row_total = [&](float part) {
        float total = segment_sum<64>(part);
        if constexpr (WPR > 1) {
            __syncthreads();
            if ((threadIdx.x & 63) == 0) wave_part[threadIdx.x >> 6] = total;
            __syncthreads();
            const int w0 = (threadIdx.x / LANES) * WPR;
            total = wave_part[w0];
#pragma unroll
            for (int w = 1; w < WPR; ++w) total += wave_part[w0 + w];
        }
        return total;
    };
    float md = 0.0f, r;
    if constexpr (!CENTER) {
        r = inv_sqrt(row_total(acc) / hidden_f + eps);
    } else {
        md = row_total(acc) / hidden_f;
        float dev = 0.0f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int i = v * LANES + lane;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float d = (to_f32(ss[v].v[e]) - shift) - md;
                dev = in_row(i, e) ? fmaf_(d, d, dev) : dev;
            }
        }
        r = inv_sqrt(row_total(dev) / hidden_f + eps);
    }
    if (live && lane == 0) {
        if (inv_std_var) inv_std_var[row] = r;
        if (mean) mean[row] = shift + md;
    }

#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int i = v * LANES + lane;
        const V gv = param(gamma, i);
        V bt = {};
        if constexpr (CENTER) bt = mask_bits(param(beta, i), beta_mask);
        V out;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if constexpr (CENTER) {
                float y = ((to_f32(ss[v].v[e]) - shift) - md) * r * to_f32(gv.v[e]);
                y = y + to_f32(bt.v[e]);
                out.v[e] = from_f32<T>(y);
            } else {
                out.v[e] = from_f32<T>(to_f32(ss[v].v[e]) * r * to_f32(gv.v[e]));
            }
        }
        if (live) {
            if (whole(i)) {
                store_vec_stream<T, E>(out_a, v0 + i, out);
            } else if (i < nvr) {
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (in_row(i, e)) out_a[(v0 + i) * E + e] = out.v[e];
            }
        }
    }
}

// Rows too wide for the register-resident routes: one workgroup per row,
// S formed again in every pass (two passes; three with the mean removed),
// four accesses per thread per step whose loads go out together (lanes past
// the row re-read its last access).  E == 1 is the scalar route.  bias and
// beta are read unconditionally: the host passes gamma's address for an
// absent one and the flags say whether to use the value.
template <typename T, int E, bool CENTER>
__global__ void __launch_bounds__(256)
ssln_block_kernel(const T* __restrict__ input, const T* __restrict__ skip,
                  const T* __restrict__ gamma, const T* __restrict__ beta,
                  const T* __restrict__ bias, T* __restrict__ output, float* __restrict__ mean,
                  float* __restrict__ inv_std_var, T* __restrict__ sum,
                  int64_t rows, int64_t nvec, float hidden_f, float eps, bool has_bias,
                  bool has_beta) {
    using V = Vec<T, E>;
    constexpr int U = 4;
    __shared__ float wave_part[kWavesPerBlock];
    const int t = threadIdx.x;
    auto clamp = [&](int64_t j) { return j < nvec ? j : nvec - 1; };
    auto block_total = [&](float acc) {
        acc = segment_sum<64>(acc);
        if ((t & 63) == 0) wave_part[t >> 6] = acc;
        __syncthreads();
        const float total = (wave_part[0] + wave_part[1]) + (wave_part[2] + wave_part[3]);
        __syncthreads();  // wave_part is rewritten next
        return total;
    };
    // S (rounded to T) of the U accesses j0, j0 + 256, ... of the row.
    auto form = [&](int64_t base, int64_t j0, V (&ss)[U]) {
        V xs[U], ks[U], bs[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t jc = clamp(j0 + u * 256);
            xs[u] = load_vec_stream<T, E>(input, base + jc);
            ks[u] = load_vec_stream<T, E>(skip, base + jc);
            bs[u] = load_vec<T, E>(bias, jc);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e)
                residual_sum<T>(to_f32(xs[u].v[e]), to_f32(ks[u].v[e]), has_bias, to_f32(bs[u].v[e]),
                                ss[u].v[e]);
    };
    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const int64_t base = row * nvec;
        float shift = 0.0f;  // sums about S[0], as in the register routes
        if constexpr (CENTER) {
            T r0;
            shift = row_shift(residual_sum<T>(to_f32(input[base * E]), to_f32(skip[base * E]), has_bias,
                                              to_f32(bias[0]), r0));
        }
        float acc = 0.0f;
        for (int64_t j0 = t; j0 < nvec; j0 += 256 * U) {
            V ss[U];
            form(base, j0, ss);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (j0 + u * 256 >= nvec) continue;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float sv = to_f32(ss[u].v[e]);
                    if constexpr (CENTER) acc += sv - shift;
                    else acc = fmaf_(sv, sv, acc);
                }
                if (sum) store_vec_stream<T, E>(sum, base + j0 + u * 256, ss[u]);
            }
        }
        float md = 0.0f, r;
        if constexpr (!CENTER) {
            r = inv_sqrt(block_total(acc) / hidden_f + eps);
        } else {
            md = block_total(acc) / hidden_f;
            float dev = 0.0f;
            for (int64_t j0 = t; j0 < nvec; j0 += 256 * U) {
                V ss[U];
                form(base, j0, ss);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (j0 + u * 256 >= nvec) continue;
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const float d = (to_f32(ss[u].v[e]) - shift) - md;
                        dev = fmaf_(d, d, dev);
                    }
                }
            }
            r = inv_sqrt(block_total(dev) / hidden_f + eps);
        }
        if (t == 0) {
            if (inv_std_var) inv_std_var[row] = r;
            if (mean) mean[row] = shift + md;
        }
        for (int64_t j0 = t; j0 < nvec; j0 += 256 * U) {
            V ss[U], gs[U], bt[U];
            form(base, j0, ss);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t jc = clamp(j0 + u * 256);
                gs[u] = load_vec<T, E>(gamma, jc);
                bt[u] = load_vec<T, E>(beta, jc);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                V out;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float sv = to_f32(ss[u].v[e]);
                    if constexpr (CENTER) {
                        float y = ((sv - shift) - md) * r * to_f32(gs[u].v[e]);
                        if (has_beta) y = y + to_f32(bt[u].v[e]);
                        out.v[e] = from_f32<T>(y);
                    } else {
                        out.v[e] = from_f32<T>(sv * r * to_f32(gs[u].v[e]));
                    }
                }
                if (j0 + u * 256 < nvec) store_vec_stream<T, E>(output, base + j0 + u * 256, out);
            }
        }
    }
}

// Rows of at most 48 accesses: L lanes per row (the row's access count
// rounded up to a power of two), 64 / L rows per wave and RPT rows per
// thread in flight; each lane holds one access of each of its rows, and a
// row's sums are a butterfly inside its L-lane segment (no LDS, no
// barrier).  Lanes past the row's end re-read its last access and discard
// it; rows past the last re-read the last row and store nothing.
template <typename T, int E, int L, int RPT, bool CENTER>
__global__ void __launch_bounds__(256)
ssln_segment_kernel(const T* __restrict__ input, const T* __restrict__ skip,
                    const T* __restrict__ gamma, const T* __restrict__ beta,
                    const T* __restrict__ bias, T* __restrict__ output, float* __restrict__ mean,
                    float* __restrict__ inv_std_var, T* __restrict__ sum,
                    int64_t rows, int nvec, float hidden_f, float eps, uint32_t beta_mask) {
    using V = Vec<T, E>;
    constexpr int SEGS = 256 / L;  // rows per block per step
    const int seg = threadIdx.x / L, l = threadIdx.x % L;
    const int first_lane = (threadIdx.x & 63) & ~(L - 1);  // the segment's lane 0 in the wave
    const int64_t tile = int64_t(blockIdx.x) * SEGS * RPT;
    const int ic = l < nvec ? l : nvec - 1;
    const bool has_bias = bias != nullptr;

    V xs[RPT], ks[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        const int64_t row = tile + int64_t(k) * SEGS + seg;
        const int64_t rc = row < rows ? row : rows - 1;
        xs[k] = load_vec_stream<T, E>(input, rc * nvec + ic);
        ks[k] = load_vec_stream<T, E>(skip, rc * nvec + ic);
    }
    const V gv = load_vec<T, E>(gamma, ic);
    V bt = {};
    if constexpr (CENTER) bt = mask_bits(load_vec<T, E>(beta, ic), beta_mask);
    V bv = {};
    if (has_bias) bv = load_vec<T, E>(bias, ic);

#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        const int64_t row = tile + int64_t(k) * SEGS + seg;
        const bool store = row < rows && l < nvec;
        V ss;
#pragma unroll
        for (int e = 0; e < E; ++e)
            residual_sum<T>(to_f32(xs[k].v[e]), to_f32(ks[k].v[e]), has_bias, to_f32(bv.v[e]), ss.v[e]);
        // With the mean removed, sums are taken about the row's first element
        // S[0], which the segment's lane 0 holds.
        float shift = 0.0f, md = 0.0f, r;
        if constexpr (CENTER) shift = row_shift(__shfl(to_f32(ss.v[0]), first_lane, 64));
        float part = 0.0f;
        if (l < nvec) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float sv = to_f32(ss.v[e]);
                if constexpr (CENTER) part += sv - shift;
                else part = fmaf_(sv, sv, part);
            }
        }
        if constexpr (!CENTER) {
            r = inv_sqrt(segment_sum<L>(part) / hidden_f + eps);
        } else {
            md = segment_sum<L>(part) / hidden_f;
            float dev = 0.0f;
            if (l < nvec) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float d = (to_f32(ss.v[e]) - shift) - md;
                    dev = fmaf_(d, d, dev);
                }
            }
            r = inv_sqrt(segment_sum<L>(dev) / hidden_f + eps);
        }
        V out;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if constexpr (CENTER)
                out.v[e] = from_f32<T>(((to_f32(ss.v[e]) - shift) - md) * r * to_f32(gv.v[e]) +
                                       to_f32(bt.v[e]));
            else
                out.v[e] = from_f32<T>(to_f32(ss.v[e]) * r * to_f32(gv.v[e]));
        }
        if (store) {
            store_vec_stream<T, E>(output, row * nvec + l, out);
            if (sum) store_vec_stream<T, E>(sum, row * nvec + l, ss);
        }
        if (row < rows && l == 0) {
            if (inv_std_var) inv_std_var[row] = r;
            if (mean) mean[row] = shift + md;
        }
    }
}

// ------------------------------------------------------------------ flat route
// Rows that would otherwise be read with accesses narrower than 16 bytes
// (odd widths, bases off the 4-byte grid) and hold at most kFlatTable - E
// elements: the rows as one stream of elements, as in the GatedRMSNorm flat
// route.  Wave w takes the rt whole rows from r0 = w * rt on, elements
// [r0 * C, (r0 + rt) * C) (plus the offset `phase` of the data bases from
// the 16-byte grid, which input, skip, output and S share), and reads the
// aligned 16-byte vectors that cover them; the first and last may hold a
// neighbouring wave's elements, which are read and left unused (never
// outside the 16-byte chunks that hold the tensors' own elements), and they
// are written element by element, the rest whole (vectors in 128-byte
// lines shared with the neighbouring tiles through L2).  S is formed per
// element with its column's bias from a per-workgroup LDS table of (gamma,
// bias) by column (E slots ahead of column 0 keep the reads of elements
// before a tile inside it), its square -- with the mean removed, S itself
// -- goes to the wave's LDS, and each row is summed there by a power-of-two
// group of lanes (lane k adds elements k, k + lpr, ... into four partial
// sums, then a butterfly over the group).  The group's first lane writes the row's
// statistics and leaves them in place of the row's first LDS entries (r;
// with the mean removed s0, d, r, rows of at least 3 elements), which the
// elements then read by row.  NARROW (C < elements per vector): a vector
// spans several rows, so every element finds its own row; otherwise a
// vector spans at most two and the row changes once.  With the mean
// removed, the statistics are taken about the row's first element s0 as in
// the other routes: d = mean(S - s0), then the squares of (S - s0) - d.
template <typename T, int VPT, bool NARROW, bool CENTER>
__global__ void __launch_bounds__(256)
ssln_flat_kernel(const T* __restrict__ input, const T* __restrict__ skip,
                 const T* __restrict__ gamma, const T* __restrict__ beta,
                 const T* __restrict__ bias, T* __restrict__ output, float* __restrict__ mean,
                 float* __restrict__ inv_std_var, T* __restrict__ sum, int64_t rows, int C, int rt,
                 int lpr_log, int phase, FastDiv cdiv, float hidden_f, float eps) {
    constexpr int E = VecWidth<T>::value;
    constexpr int TE = 64 * VPT * E;  // element slots of a wave's tile
    using V = Vec<T, E>;
    __shared__ float sq[4][TE];
    __shared__ float2 gb_tab[kFlatTable];                // (gamma, bias) by column
    __shared__ float beta_tab[CENTER ? kFlatTable : 1];  // beta by column
    float2* gb = gb_tab + E;
    float* bt = beta_tab + (CENTER ? E : 0);
    const bool has_bias = bias != nullptr;
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
    const T* ia = input - phase;
    const T* ka = skip - phase;
    T* oa = output - phase;
    T* sa = sum ? sum - phase : nullptr;

    V xs[VPT], ss[VPT];  // input; skip, then S
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int i = v * 64 + lane;
        const int ic = i < nvt ? i : nvt - 1;
        xs[v] = load_vec_stream<T, E>(ia, v0 + ic);
        ss[v] = load_vec_stream<T, E>(ka, v0 + ic);
    }
    // The tables: each thread's (at most kFlatTable / 256) columns are loaded
    // at once (indices clamped, no load behind a branch), then stored.
    // Every table load is unconditional (gamma's address in place of an
    // absent bias or beta, its values unused) and every value is converted
    // outside the lane branch that guards the LDS store: a load whose use
    // sits behind a branch is waited for there, one round trip each.
    constexpr int kFill = kFlatTable / 256;
    const T* bias_src = has_bias ? bias : gamma;
    const T* beta_src = beta ? beta : gamma;
    T gv[kFill], bv[kFill], tv[kFill];
#pragma unroll
    for (int j = 0; j < kFill; ++j) {
        const int c = threadIdx.x + j * 256;
        const int cc = c < C ? c : C - 1;
        gv[j] = gamma[cc];
        bv[j] = bias_src[cc];
        if constexpr (CENTER) tv[j] = beta_src[cc];
    }
#pragma unroll
    for (int j = 0; j < kFill; ++j) {
        const int c = threadIdx.x + j * 256;
        const float2 g_b = make_float2(to_f32(gv[j]), has_bias ? to_f32(bv[j]) : 0.0f);
        const float t_v = CENTER && beta ? to_f32(tv[j]) : 0.0f;
        if (c < C) {
            gb[c] = g_b;
            if constexpr (CENTER) bt[c] = t_v;
        }
    }
    __syncthreads();  // the tables
    if (nr == 0) return;

    // Where vector v's elements fall: row of element 0 (relative to the
    // tile) and the column of element 0 (1 - E to -1 for the vector that
    // starts before the tile; clamped for those past it, whose results are
    // dropped); elements e >= C - column lie in the next row.  Each element
    // reads its column's parameters at an immediate offset from one of two
    // table bases (this row's, the next row's).
    int row_a[VPT], col_a[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int t0 = (v * 64 + lane) * E - off0;
        const int tc = t0 < 0 ? 0 : (t0 < span ? t0 : span - 1);
        row_a[v] = int(fastdiv(uint32_t(tc), cdiv));
        const int c0 = t0 - row_a[v] * C;
        col_a[v] = c0 > C - 1 ? C - 1 : c0;
    }
    // NARROW: element e's row and column from its own position.
    auto narrow_rc = [&](int v, int e, int& row, int& col) {
        int t = (v * 64 + lane) * E - off0 + e;
        t = t < 0 ? 0 : (t < span ? t : span - 1);
        row = int(fastdiv(uint32_t(t), cdiv));
        col = t - row * C;
    };

#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int i = v * 64 + lane;
        const float2* pa = gb + col_a[v];
        const float2* pb = gb + (col_a[v] - C);
        const int b = C - col_a[v];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float bv;
            if constexpr (NARROW) {
                int row, col;
                narrow_rc(v, e, row, col);
                bv = gb[col].y;
            } else {
                bv = (e >= b ? pb : pa)[e].y;
            }
            const float sv = residual_sum<T>(to_f32(xs[v].v[e]), to_f32(ss[v].v[e]), has_bias, bv,
                                             ss[v].v[e]);
            sq[wave][i * E + e] = CENTER ? sv : sv * sv;
        }
    }
    wave_lds_sync();

    const int lpr = 1 << lpr_log;
    const int k = lane & (lpr - 1);
    // Lane k of a row's group adds f(element) over k, k + lpr, ... into four
    // partial sums (elements k + 4j lpr, k + (4j + 1) lpr, ...: four LDS reads
    // in flight), added as ((p0 + p1) + (p2 + p3)); then a butterfly over
    // the group (every lane ends with the same total).
    auto row_sum = [&](int first, bool has, auto f) {
        float p0 = 0.0f, p1 = 0.0f, p2 = 0.0f, p3 = 0.0f;
        if (has) {
            int c = k;
            for (; c + 3 * lpr < C; c += 4 * lpr) {
                const float a0 = sq[wave][first + c], a1 = sq[wave][first + c + lpr];
                const float a2 = sq[wave][first + c + 2 * lpr], a3 = sq[wave][first + c + 3 * lpr];
                p0 = f(p0, a0);
                p1 = f(p1, a1);
                p2 = f(p2, a2);
                p3 = f(p3, a3);
            }
            if (c < C) p0 = f(p0, sq[wave][first + c]);
            if (c + lpr < C) p1 = f(p1, sq[wave][first + c + lpr]);
            if (c + 2 * lpr < C) p2 = f(p2, sq[wave][first + c + 2 * lpr]);
        }
        float acc = (p0 + p1) + (p2 + p3);
        for (int m = 1; m < lpr; m <<= 1) acc += __shfl_xor(acc, m, 64);
        return acc;
    };
    for (int rb = 0; rb < nr; rb += 64 >> lpr_log) {
        const int rr = rb + (lane >> lpr_log);
        const bool has = rr < nr;
        const int first = off0 + (has ? rr : 0) * C;
        float r, s0 = 0.0f, md = 0.0f;
        if constexpr (!CENTER) {
            const float acc = row_sum(first, has, [](float p, float x) { return p + x; });
            r = inv_sqrt(acc / hidden_f + eps);
            // The group's reads of this row are done (the butterfly used them).
            if (has && k == 0) sq[wave][first] = r;
        } else {
            s0 = row_shift(sq[wave][first]);
            md = row_sum(first, has, [&](float p, float x) { return p + (x - s0); }) / hidden_f;
            const float dev = row_sum(first, has, [&](float p, float x) {
                const float d = (x - s0) - md;
                return fmaf_(d, d, p);
            });
            r = inv_sqrt(dev / hidden_f + eps);
            if (has && k == 0) {
                sq[wave][first + 1] = md;
                sq[wave][first + 2] = r;
            }
        }
        if (has && k == 0) {
            if (inv_std_var) inv_std_var[r0 + rr] = r;
            if (mean) mean[r0 + rr] = CENTER ? s0 + md : 0.0f;
        }
    }
    wave_lds_sync();

    const LineRun orun = line_run<T, E>(oa + v0 * E, nvt);
    const LineRun srun = line_run<T, E>(sa ? sa + v0 * E : oa + v0 * E, nvt);
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int i = v * 64 + lane;
        const int t0 = i * E - off0;  // the vector's first element, from the tile's first
        V out;
        if constexpr (NARROW) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                int row, c;
                narrow_rc(v, e, row, c);
                const int at = off0 + row * C;  // the row's first LDS entry
                const float sv = to_f32(ss[v].v[e]);
                if constexpr (CENTER)
                    out.v[e] = from_f32<T>(((sv - sq[wave][at]) - sq[wave][at + 1]) * sq[wave][at + 2] *
                                           gb[c].x + bt[c]);
                else
                    out.v[e] = from_f32<T>(sv * sq[wave][at] * gb[c].x);
            }
        } else {
            // The statistics of this vector's (at most) two rows, once.
            const int ra = off0 + row_a[v] * C;
            const int rb = off0 + (row_a[v] + 1 < nr ? row_a[v] + 1 : row_a[v]) * C;
            const float r_a = sq[wave][CENTER ? ra + 2 : ra], r_b = sq[wave][CENTER ? rb + 2 : rb];
            float s0_a = 0.0f, s0_b = 0.0f, md_a = 0.0f, md_b = 0.0f;
            if constexpr (CENTER) {
                s0_a = sq[wave][ra];
                s0_b = sq[wave][rb];
                md_a = sq[wave][ra + 1];
                md_b = sq[wave][rb + 1];
            }
            const float2* pa = gb + col_a[v];
            const float2* pb = gb + (col_a[v] - C);
            const float* qa = bt + col_a[v];
            const float* qb = bt + (col_a[v] - C);
            const int b = C - col_a[v];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const bool next = e >= b;
                const float sv = to_f32(ss[v].v[e]);
                const float g = (next ? pb : pa)[e].x;
                if constexpr (CENTER)
                    out.v[e] = from_f32<T>(((sv - (next ? s0_b : s0_a)) - (next ? md_b : md_a)) *
                                           (next ? r_b : r_a) * g + (next ? qb : qa)[e]);
                else
                    out.v[e] = from_f32<T>(sv * (next ? r_b : r_a) * g);
            }
        }
        if (t0 >= 0 && t0 + E <= span) {
            store_vec_run<T, E>(oa + v0 * E, i, out, orun);
            if (sa) store_vec_run<T, E>(sa + v0 * E, i, ss[v], srun);
        } else if (i < nvt) {
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (t0 + e >= 0 && t0 + e < span) {
                    oa[(v0 + i) * E + e] = out.v[e];
                    if (sa) sa[(v0 + i) * E + e] = ss[v].v[e];
                }
        }
    }
}

template <typename T, int E, int L>
hipError_t launch_segment(const SslnArgs& a, int nvec, hipStream_t stream) {
    // About 64 bytes of each input per thread in flight, at most 16 rows.
    constexpr int VB = E * int(sizeof(T));
    constexpr int RPT = 64 / VB < 16 ? 64 / VB : 16;
    constexpr int rows_per_block = (256 / L) * RPT;
    const int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
    auto args = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(256), 0, stream,
                           static_cast<const T*>(a.input), static_cast<const T*>(a.skip),
                           static_cast<const T*>(a.gamma),
                           static_cast<const T*>(a.beta ? a.beta : a.gamma),
                           static_cast<const T*>(a.bias), static_cast<T*>(a.output), a.mean,
                           a.inv_std_var, static_cast<T*>(a.sum), a.rows, nvec, float(a.hidden),
                           a.epsilon, a.beta ? ~0u : 0u);
    };
    if (a.center) args(ssln_segment_kernel<T, E, L, RPT, true>);
    else args(ssln_segment_kernel<T, E, L, RPT, false>);
    return hipGetLastError();
}

template <typename T, int E>
hipError_t launch_segment_for(const SslnArgs& a, int nvec, hipStream_t stream) {
    if (nvec <= 1) return launch_segment<T, E, 1>(a, nvec, stream);
    if (nvec <= 2) return launch_segment<T, E, 2>(a, nvec, stream);
    if (nvec <= 4) return launch_segment<T, E, 4>(a, nvec, stream);
    if (nvec <= 8) return launch_segment<T, E, 8>(a, nvec, stream);
    if (nvec <= 16) return launch_segment<T, E, 16>(a, nvec, stream);
    if (nvec <= 32) return launch_segment<T, E, 32>(a, nvec, stream);
    return launch_segment<T, E, 64>(a, nvec, stream);
}

template <typename T, int E, int NV, int WPR, int WPB>
hipError_t launch_wave_nv(const SslnArgs& a, int nvec, hipStream_t stream) {
    constexpr int rows_per_block = WPB / WPR;
    const int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
    const float hidden_f = float(a.hidden);
    const int lines = rows_off_lines(a.hidden * int64_t(sizeof(T)), {a.output, a.sum});
    auto args = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(64 * WPB), 0, stream,
                           static_cast<const T*>(a.input), static_cast<const T*>(a.skip),
                           static_cast<const T*>(a.gamma),
                           static_cast<const T*>(a.beta ? a.beta : a.gamma),
                           static_cast<const T*>(a.bias), static_cast<T*>(a.output), a.mean,
                           a.inv_std_var, static_cast<T*>(a.sum), a.rows, nvec, hidden_f, a.epsilon,
                           a.beta ? ~0u : 0u, lines);
    };
    const bool full = nvec == 64 * WPR * NV;
    if (a.center) {
        if (full) args(ssln_wave_kernel<T, E, NV, true, WPR, true, WPB>);
        else args(ssln_wave_kernel<T, E, NV, false, WPR, true, WPB>);
    } else {
        if (full) args(ssln_wave_kernel<T, E, NV, true, WPR, false, WPB>);
        else args(ssln_wave_kernel<T, E, NV, false, WPR, false, WPB>);
    }
    return hipGetLastError();
}

template <typename T, int E, int MAXNV, int WPR, int WPB = kWavesPerBlock>
hipError_t launch_wave(const SslnArgs& a, int nvec, hipStream_t stream) {
    const int need = (nvec + 64 * WPR - 1) / (64 * WPR);
    if (need <= 1) return launch_wave_nv<T, E, 1, WPR, WPB>(a, nvec, stream);
    if (need <= 2) return launch_wave_nv<T, E, 2, WPR, WPB>(a, nvec, stream);
    if (need <= 3) return launch_wave_nv<T, E, 3, WPR, WPB>(a, nvec, stream);
    if (need <= 4) return launch_wave_nv<T, E, 4, WPR, WPB>(a, nvec, stream);
    if constexpr (MAXNV >= 8) {
        if (need <= 6) return launch_wave_nv<T, E, 6, WPR, WPB>(a, nvec, stream);
        if (need <= 8) return launch_wave_nv<T, E, 8, WPR, WPB>(a, nvec, stream);
    }
    if constexpr (MAXNV >= 16) {
        if (need <= 12) return launch_wave_nv<T, E, 12, WPR, WPB>(a, nvec, stream);
        if (need <= 16) return launch_wave_nv<T, E, 16, WPR, WPB>(a, nvec, stream);
    }
    if constexpr (MAXNV >= 32) {
        if (need <= 24) return launch_wave_nv<T, E, 24, WPR, WPB>(a, nvec, stream);
        if (need <= 32) return launch_wave_nv<T, E, 32, WPR, WPB>(a, nvec, stream);
    }
    return hipErrorInvalidValue;  // callers check the width first
}

// Accesses per lane: a row goes to the fewest waves (1, 2, 4, 8 or 16) that
// keep it within kNvLane<T, E> accesses per lane -- about 64 VGPRs of row
// data, which leaves room for 8 waves per SIMD (measured on 4096-wide
// float16 rows: two waves of 4 vectors per lane 6.1 TB/s, one wave of 8
// vectors 5.7 TB/s; float32 rows of 8192: eight waves of 4 vectors 5.9 TB/s,
// four waves of 8 vectors 5.4 TB/s).
template <typename T, int E> constexpr int kNvLane = E * sizeof(T) >= 16 ? 4 : E * sizeof(T) == 8 ? 8 : 16;
// Accesses per lane of the widest register rows (sixteen waves): twice
// kNvLane for 16-byte vectors (8, about 100 VGPRs: 128 KB rows), kNvLane for
// narrower accesses (deeper ones spill under the 1024-thread block's
// 128-VGPR limit).
template <typename T, int E> constexpr int kNvWidest = E * sizeof(T) >= 16 ? 2 * kNvLane<T, E> : kNvLane<T, E>;
template <typename T, int E> constexpr int64_t kMaxRegisterRow = int64_t(1024) * kNvWidest<T, E> * E;

template <typename T, int E>
hipError_t launch_ssln_width(const SslnArgs& a, hipStream_t stream, const char** route) {
    static const char* const kNames[6][4] = {
        {"ssln.wave.scalar", "ssln.wave.vec4", "ssln.wave.vec8", "ssln.wave.vec16"},
        {"ssln.wave2.scalar", "ssln.wave2.vec4", "ssln.wave2.vec8", "ssln.wave2.vec16"},
        {"ssln.rowblock.scalar", "ssln.rowblock.vec4", "ssln.rowblock.vec8", "ssln.rowblock.vec16"},
        {"ssln.segment.scalar", "ssln.segment.vec4", "ssln.segment.vec8", "ssln.segment.vec16"},
        {"ssln.row8.scalar", "ssln.row8.vec4", "ssln.row8.vec8", "ssln.row8.vec16"},
        {"ssln.row16.scalar", "ssln.row16.vec4", "ssln.row16.vec8", "ssln.row16.vec16"}};
    constexpr int kName = E == 1 ? 0 : E * sizeof(T) == 16 ? 3 : E * sizeof(T) == 8 ? 2 : 1;
    constexpr int NVL = kNvLane<T, E>;
    const int64_t nvec = a.hidden / E;
    // Lane groups for rows of up to 48 accesses (64 lanes for 33-48: 1.01-1.11x
    // the one-wave route on float16 rows of 264-384; from 49 sixteen-byte
    // accesses on the one-wave route measured faster, 1.09-1.16x on float16
    // rows of 392-512), and for
    // rows of up to 64 accesses narrower than 16 bytes, where the one-wave
    // route holds one small access per lane (49-63 accesses: f16 elements
    // 2.0-2.1x, f16 pairs 1.7-2.0x, f32 elements 1.3-1.6x, 8-byte accesses
    // 0.96-1.28x).
    if (nvec <= (E * int(sizeof(T)) < 16 ? 64 : 48)) {
        *route = kNames[3][kName];
        return launch_segment_for<T, E>(a, int(nvec), stream);
    }
    if (nvec <= 64 * NVL) {
        *route = kNames[0][kName];
        return launch_wave<T, E, NVL, 1>(a, int(nvec), stream);
    }
    if (nvec <= 128 * NVL) {
        *route = kNames[1][kName];
        return launch_wave<T, E, NVL, 2>(a, int(nvec), stream);
    }
    if (nvec <= 256 * NVL) {
        *route = kNames[2][kName];
        return launch_wave<T, E, NVL, 4>(a, int(nvec), stream);
    }
    if (nvec <= 512 * NVL) {
        *route = kNames[4][kName];
        return launch_wave<T, E, NVL, 8, 8>(a, int(nvec), stream);
    }
    *route = kNames[5][kName];
    if (nvec <= 1024 * NVL) return launch_wave<T, E, NVL, 16, 16>(a, int(nvec), stream);
    return launch_wave<T, E, kNvWidest<T, E>, 16, 16>(a, int(nvec), stream);  // up to kMaxRegisterRow
}

template <typename T, int NV, int WPR, int WPB>
hipError_t launch_phase_nv(const SslnArgs& a, int phase, int nvg, hipStream_t stream) {
    constexpr int E = VecWidth<T>::value;
    constexpr int rows_per_block = WPB / WPR;
    const int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
    const T* g = static_cast<const T*>(a.gamma);
    auto args = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(64 * WPB), 0, stream,
                           static_cast<const T*>(a.input), static_cast<const T*>(a.skip), g,
                           a.beta ? static_cast<const T*>(a.beta) : g,
                           a.bias ? static_cast<const T*>(a.bias) : g, static_cast<T*>(a.output), a.mean,
                           a.inv_std_var, static_cast<T*>(a.sum), a.rows, int(a.hidden), phase, nvg,
                           float(a.hidden), a.epsilon, a.beta ? ~0u : 0u, a.bias ? ~0u : 0u);
    };
    if (a.center) args(ssln_phase_kernel<T, E, NV, WPR, true, WPB>);
    else args(ssln_phase_kernel<T, E, NV, WPR, false, WPB>);
    return hipGetLastError();
}

template <typename T, int MAXNV, int WPR, int WPB = kWavesPerBlock>
hipError_t launch_phase(const SslnArgs& a, int nmax, int phase, int nvg, hipStream_t stream) {
    const int need = (nmax + 64 * WPR - 1) / (64 * WPR);
    if (need <= 1) return launch_phase_nv<T, 1, WPR, WPB>(a, phase, nvg, stream);
    if (need <= 2) return launch_phase_nv<T, 2, WPR, WPB>(a, phase, nvg, stream);
    if (need <= 3) return launch_phase_nv<T, 3, WPR, WPB>(a, phase, nvg, stream);
    if (need <= 4) return launch_phase_nv<T, 4, WPR, WPB>(a, phase, nvg, stream);
    if constexpr (MAXNV >= 8) {
        if (need <= 6) return launch_phase_nv<T, 6, WPR, WPB>(a, phase, nvg, stream);
        if (need <= 8) return launch_phase_nv<T, 8, WPR, WPB>(a, phase, nvg, stream);
    }
    return hipErrorInvalidValue;  // the caller checks the width first
}

// The phased route for rows off the 16-byte grid (see ssln_phase_kernel):
// taken when the data tensors share their offset from a 16-byte boundary,
// gamma, beta and bias are 16-byte aligned, and the row needs more than
// lane groups' 48 vectors and at most sixteen waves of four.  Returns
// false, having launched nothing, otherwise.
template <typename T>
bool launch_ssln_phase(const SslnArgs& a, hipStream_t stream, const char** route, hipError_t* err) {
    constexpr int E = VecWidth<T>::value;
    constexpr int NVL = kNvLane<T, E>;
    const uintptr_t ph = reinterpret_cast<uintptr_t>(a.input) % 16;
    auto same = [&](const void* q) { return !q || reinterpret_cast<uintptr_t>(q) % 16 == ph; };
    if (ph % sizeof(T) != 0 || !same(a.skip) || !same(a.output) || !same(a.sum)) return false;
    if (!aligned16(a.gamma) || (a.beta && !aligned16(a.beta)) || (a.bias && !aligned16(a.bias)))
        return false;
    const int64_t nmax = a.hidden / E + 2;  // vectors a row can touch
    // From 33 vectors on (f16 rows of 248 elements, f32 of 124) a wave of
    // 16-byte vectors beats the one-wave-per-row element route (f16 hidden
    // 255 / 301 / 375 +14 / +30 / +37 %, f32 187 +13 %); below that it leaves
    // too many lanes idle (f16 57-127: 17-44 % slower).  Deeper than four
    // vectors per lane its parameter funnels spill under the 1024-thread
    // block's 128-VGPR limit.
    if (nmax <= 32 || nmax > 1024 * NVL) return false;
    const int phase = int(ph / sizeof(T));
    const int nvg = int((a.hidden + E - 1) / E);
    const int n = int(nmax);
    *route = "ssln.phase.vec16";
    if (nmax <= 64 * NVL) *err = launch_phase<T, NVL, 1>(a, n, phase, nvg, stream);
    else if (nmax <= 128 * NVL) *err = launch_phase<T, NVL, 2>(a, n, phase, nvg, stream);
    else if (nmax <= 256 * NVL) *err = launch_phase<T, NVL, 4>(a, n, phase, nvg, stream);
    else if (nmax <= 512 * NVL) *err = launch_phase<T, NVL, 8, 8>(a, n, phase, nvg, stream);
    else *err = launch_phase<T, NVL, 16, 16>(a, n, phase, nvg, stream);
    return true;
}

// The flat route (see ssln_flat_kernel): rows of at most kFlatTable - E
// elements whose data tensors (input, skip, output, S) share their offset
// from a 16-byte boundary; with the mean removed, rows of at least three
// elements.  Returns false, having launched nothing, when it does not apply.
template <typename T>
bool launch_ssln_flat(const SslnArgs& a, bool forced, hipStream_t stream, const char** route,
                      hipError_t* err) {
    constexpr int EV = VecWidth<T>::value;
    const uintptr_t ph = reinterpret_cast<uintptr_t>(a.input) % 16;
    auto same = [&](const void* q) { return !q || reinterpret_cast<uintptr_t>(q) % 16 == ph; };
    if (ph % sizeof(T) != 0 || !same(a.skip) || !same(a.output) || !same(a.sum)) return false;
    if (a.center && a.hidden < 3) return false;
    FlatPlan fp;
    if (!flat_plan(a.hidden, EV, forced || sizeof(T) == 4, &fp)) return false;
    const int C = int(a.hidden);
    const int phase = int(ph / sizeof(T));
    const int64_t tiles = (a.rows + fp.rt - 1) / fp.rt;
    const int64_t blocks = (tiles + 3) / 4;
    const FastDiv cdiv = make_fastdiv(uint32_t(C));
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(unsigned(blocks)), dim3(256), 0, stream,
                           static_cast<const T*>(a.input), static_cast<const T*>(a.skip),
                           static_cast<const T*>(a.gamma), static_cast<const T*>(a.beta),
                           static_cast<const T*>(a.bias), static_cast<T*>(a.output), a.mean,
                           a.inv_std_var, static_cast<T*>(a.sum), a.rows, C, fp.rt, fp.lpr_log,
                           phase, cdiv, float(a.hidden), a.epsilon);
        return hipGetLastError();
    };
    auto by_vpt = [&](auto vpt, auto center) {
        constexpr int VPT = decltype(vpt)::value;
        constexpr bool CTR = decltype(center)::value;
        if (C < EV) return go(ssln_flat_kernel<T, VPT, true, CTR>);
        return go(ssln_flat_kernel<T, VPT, false, CTR>);
    };
    auto by_center = [&](auto vpt) {
        if (a.center) return by_vpt(vpt, std::true_type{});
        return by_vpt(vpt, std::false_type{});
    };
    constexpr int small = 16 / EV;
    *route = "ssln.flat.vec16";
    *err = fp.vpt == small ? by_center(std::integral_constant<int, small>{})
                           : by_center(std::integral_constant<int, 2 * small>{});
    return true;
}

// Where the automatic choice takes the flat route, by the access width E the
// other routes would use, as measured on 2^27-element tensors (outputs Y and
// S) against them:
//   element rows: float16 up to 247 elements (the phased route beyond:
//     f16 255-1015 3.6-3.8 against 3.8-5.3 TB/s), 191 with the mean
//     removed; float32 up to 255, 1020 with the mean removed.  f16 C = 9 /
//     33 / 99 / 127 / 247 at 5.7 / 5.5 / 5.5 / 5.8 / 4.0 TB/s against 2.7
//     / 2.6 / 2.0 / 2.6 / 3.2 (lane groups or one wave of scalars).
//   float16 pairs (4-byte accesses): rows of 10 to 300 elements (+2 to
//     +110 %, f16 70 / 130 at 5.7 / 5.1 against 3.7 / 2.4 TB/s); with the
//     mean removed (two passes over LDS) only where the pairs fill less than
//     70 % of their lane group's or wave's slots.
//   float32 pairs (8-byte accesses): rows of 42 elements or more (+3 to +32
//     %; shorter rows fill their lane groups well and lost up to 17 %).
//   16-byte rows and float16 8-byte rows keep their routes (mixed, -37 to
//   +8 %).
template <typename T>
bool flat_preferred(const SslnArgs& a, int E) {
    const int64_t h = a.hidden;
    const int bytes = E * int(sizeof(T));
    if (E == 1) {
        if (sizeof(T) == 2) return h <= (a.center ? 191 : 247);
        return h <= (a.center ? 1020 : 255);
    }
    if (bytes == 4 && sizeof(T) == 2) {
        if (h < 10 || h > 300) return false;
        if (!a.center) return true;
        const int64_t nvec = h / E;
        int64_t slots = 64 * ((nvec + 63) / 64);  // one wave of up to 64 lanes per pass
        if (nvec <= 64) {
            slots = 1;
            while (slots < nvec) slots <<= 1;  // a power-of-two lane group
        }
        return double(nvec) / double(slots) < 0.7;
    }
    if (bytes == 8 && sizeof(T) == 4) return h >= 42;
    return false;
}

// The wide route (see ssln_wide_kernel): rows of 16-byte vectors beyond
// the register routes, one 1024-thread workgroup per row.
template <typename T>
constexpr int64_t kMaxWideRow = int64_t(kWideThreads) * (kWideRegs + kWideLds) * VecWidth<T>::value;

template <typename T>
hipError_t launch_ssln_wide(const SslnArgs& a, hipStream_t stream) {
    constexpr int EV = VecWidth<T>::value;
    const T* g = static_cast<const T*>(a.gamma);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(unsigned(a.rows)), dim3(kWideThreads), 0, stream,
                           static_cast<const T*>(a.input), static_cast<const T*>(a.skip), g,
                           a.beta ? static_cast<const T*>(a.beta) : g,
                           a.bias ? static_cast<const T*>(a.bias) : g, a.bias != nullptr,
                           static_cast<T*>(a.output), a.mean, a.inv_std_var, static_cast<T*>(a.sum),
                           int(a.hidden / EV), float(a.hidden), a.epsilon, a.beta ? ~0u : 0u);
        return hipGetLastError();
    };
    if (a.center) return go(ssln_wide_kernel<T, true>);
    return go(ssln_wide_kernel<T, false>);
}

// Where the automatic choice takes the phased route (rows that touch 33 to
// 4096 aligned vectors and that the flat route does not take), by the access
// width E the other routes would use, as measured on 2^27-element tensors
// (outputs Y and S) against them:
//   element rows: always (1.2-2.3x).
//   float16 pairs (4-byte accesses): always (hidden 302-16382 +7 to +37 %;
//     with the mean removed +0 to +14 %).
//   float32 pairs (8-byte accesses): always (1022-8190 +1 to +16 %).
//   float16 quads (8-byte accesses), the mean not removed: rows of more than
//     256 of them, or whose lane group or wave leaves more than a fifth of
//     its slots idle (260 / 380 / 2044 / 4092 / 4100 +9 to +16 %; rows that
//     fill their slots lose: 252 / 508 / 764 -33 / -11 / -4 %); with the
//     mean removed, never (2044 +4 %, 4100 -6 %).
template <typename T>
bool phase_preferred(const SslnArgs& a, int E) {
    const int bytes = E * int(sizeof(T));
    if (E == 1 || bytes == 4 || (bytes == 8 && sizeof(T) == 4)) return true;
    if (bytes != 8 || a.center) return false;
    const int64_t nvec = a.hidden / E;
    if (nvec > 256) return true;
    int64_t slots = 1;
    if (nvec <= 64) {
        while (slots < nvec) slots <<= 1;  // the lane group
    } else {
        const int64_t need = (nvec + 63) / 64;  // one wave, as launch_wave picks its depth
        slots = 64 * (need <= 4 ? need : need <= 6 ? 6 : 8);
    }
    return double(nvec) / double(slots) < 0.8;
}

template <typename T>
hipError_t launch_ssln_t(const SslnArgs& a, Route want, hipStream_t stream, const char** route) {
    // Widest access that divides the row and every tensor's base.
    int E = widest_vector<T>(a.hidden, {a.input, a.skip, a.gamma, a.beta, a.bias, a.output, a.sum});
    if (want == Route::Scalar) E = 1;
    hipError_t err = hipSuccess;
    if (want == Route::Flat) {  // forced where it applies, else automatic
        if (launch_ssln_flat<T>(a, true, stream, route, &err)) return err;
        want = Route::Auto;
    }
    // The flat route where it measured faster (flat_preferred), then the
    // phased route where it did (phase_preferred).
    if (want == Route::Auto || want == Route::Vector) {
        if (flat_preferred<T>(a, E) && launch_ssln_flat<T>(a, false, stream, route, &err)) return err;
        if (phase_preferred<T>(a, E) && launch_ssln_phase<T>(a, stream, route, &err)) return err;
    }
    int64_t max_regs = kMaxRegisterRow<T, 1>;
    if constexpr (sizeof(T) == 2) {
        if (E == 8) max_regs = kMaxRegisterRow<T, 8>;
        if (E == 4) max_regs = kMaxRegisterRow<T, 4>;
        if (E == 2) max_regs = kMaxRegisterRow<T, 2>;
    } else {
        if (E == 4) max_regs = kMaxRegisterRow<T, 4>;
        if (E == 2) max_regs = kMaxRegisterRow<T, 2>;
    }
    if (want != Route::Block && a.hidden <= max_regs) {
        if constexpr (sizeof(T) == 2) {
            if (E == 8) return launch_ssln_width<T, 8>(a, stream, route);
            if (E == 4) return launch_ssln_width<T, 4>(a, stream, route);
            if (E == 2) return launch_ssln_width<T, 2>(a, stream, route);
        } else {
            if (E == 4) return launch_ssln_width<T, 4>(a, stream, route);
            if (E == 2) return launch_ssln_width<T, 2>(a, stream, route);
        }
        return launch_ssln_width<T, 1>(a, stream, route);
    }
    // Wider rows of 16-byte vectors: the wide route while a row fits one
    // workgroup's registers and LDS (a grid of one workgroup per row stays
    // below 2^32 work-items).
    if (want != Route::Block && E == VecWidth<T>::value && a.hidden <= kMaxWideRow<T> &&
        a.rows < (int64_t(1) << 22)) {
        *route = "ssln.wide.vec16";
        return launch_ssln_wide<T>(a, stream);
    }
    // Wider rows (or forced, then with scalar accesses): the block route.
    if (want == Route::Block) E = 1;
    static const char* const kBlockNames[4] = {"ssln.block", "ssln.block.vec4", "ssln.block.vec8",
                                               "ssln.block.vec16"};
    *route = kBlockNames[E == 1 ? 0 : E * sizeof(T) == 16 ? 3 : E * sizeof(T) == 8 ? 2 : 1];
    const int64_t blocks = a.rows < 65536 * 16 ? a.rows : 65536 * 16;
    auto block = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(256), 0, stream,
                           static_cast<const T*>(a.input), static_cast<const T*>(a.skip),
                           static_cast<const T*>(a.gamma),
                           static_cast<const T*>(a.beta ? a.beta : a.gamma),
                           static_cast<const T*>(a.bias ? a.bias : a.gamma), static_cast<T*>(a.output),
                           a.mean, a.inv_std_var, static_cast<T*>(a.sum), a.rows, a.hidden / E,
                           float(a.hidden), a.epsilon, a.bias != nullptr, a.beta != nullptr);
        return hipGetLastError();
    };
    auto by_width = [&](auto center) {
        constexpr bool C = decltype(center)::value;
        if constexpr (sizeof(T) == 2) {
            if (E == 8) return block(ssln_block_kernel<T, 8, C>);
            if (E == 4) return block(ssln_block_kernel<T, 4, C>);
            if (E == 2) return block(ssln_block_kernel<T, 2, C>);
        } else {
            if (E == 4) return block(ssln_block_kernel<T, 4, C>);
            if (E == 2) return block(ssln_block_kernel<T, 2, C>);
        }
        return block(ssln_block_kernel<T, 1, C>);
    };
    if (a.center) return by_width(std::true_type{});
    return by_width(std::false_type{});
}

}  // namespace

hipError_t launch_ssln(const SslnArgs& a, Route want, hipStream_t stream, const char** route) {
    if (a.rows == 0) {
        *route = "ssln.empty";
        return hipSuccess;
    }
    if (a.dtype == 0) return launch_ssln_t<float>(a, want, stream, route);
    return launch_ssln_t<half_t>(a, want, stream, route);
}

}  // namespace sn
