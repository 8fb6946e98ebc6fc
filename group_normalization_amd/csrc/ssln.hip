// ssln.hip -- SkipSimplifiedLayerNormalization kernels for gfx950.
//
// Operator ("com.microsoft.SkipSimplifiedLayerNormalization", Description,
// Inputs, Outputs): per row, S = input + skip (+ bias) rounded to T,
// r = 1/sqrt(mean(S^2) + epsilon), output = S * r * gamma; optional outputs
// S, mean (zero for the simplified form) and inv_std_var (r).
//
// Routes:
//   wave   one wave64 per row (rows up to 8192 elements); lane l holds the
//          row's vectors l, l+64, ...
//          in VGPRs as T (the rounded S is exactly representable in T), so
//          the row is read once and written once, with nontemporal loads
//          and stores (gamma and bias, shared by every row, stay cached).
//          E elements per access: 16-byte vectors (4 x f32 / 8 x f16) or
//          scalars.
//   rowblock  the same with four waves (one 256-thread workgroup) per row
//          for wider rows (up to 32768 float16 / 16384 float32 elements): the
//          wave sums meet in LDS and are added in wave order.
//   block  one 256-thread workgroup per row for any other row (scalar
//          accesses, wider rows): S is formed twice (once for the statistic,
//          once for the output), reading the inputs twice.
// Statistic: each lane accumulates its own squares in float32 (FMA), then a
// fixed butterfly sums the 64 lanes (DPP inside 16-lane rows, then two
// cross-row exchanges), so every lane holds the same total and the result
// does not depend on which optional outputs were requested.
#include "device_common.h"
#include "skipnorm_internal.h"

namespace sn {
namespace {

constexpr int kWavesPerBlock = 4;

// WPR waves per row: 1 (four rows per 256-thread block) or 4 (one row per
// block, for rows wider than one wave's registers).  Lane l of the row's
// 64*WPR lanes holds vectors l, l + 64*WPR, ...
template <typename T, int E, int NV, bool FULL, int WPR>
__global__ void __launch_bounds__(256)
ssln_wave_kernel(const T* __restrict__ input, const T* __restrict__ skip,
                 const T* __restrict__ gamma, const T* __restrict__ bias,
                 T* __restrict__ output, float* __restrict__ mean,
                 float* __restrict__ inv_std_var, T* __restrict__ sum,
                 int64_t rows, int nvec, float hidden_f, float eps) {
    using V = Vec<T, E>;
    constexpr int LANES = 64 * WPR;
    __shared__ float wave_part[WPR > 1 ? WPR : 1];
    const int lane = threadIdx.x % LANES;
    const int64_t row = int64_t(blockIdx.x) * (kWavesPerBlock / WPR) + threadIdx.x / LANES;
    if (row >= rows) return;  // whole wave (WPR = 1) or whole block (WPR = 4)
    const int64_t base = row * nvec;
    const bool has_bias = bias != nullptr;

    // Issue every load of the row before any arithmetic.
    V xs[NV], ks[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int idx = v * LANES + lane;
        if (FULL || idx < nvec) {
            xs[v] = load_vec_stream<T, E>(input, base + idx);
            ks[v] = load_vec_stream<T, E>(skip, base + idx);
        }
    }

    V ss[NV];
    float acc = 0.0f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int idx = v * LANES + lane;
        if (FULL || idx < nvec) {
            V bv = {};
            if (has_bias) bv = load_vec<T, E>(bias, idx);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float s = residual_sum<T>(to_f32(xs[v].v[e]), to_f32(ks[v].v[e]), has_bias,
                                                to_f32(bv.v[e]), ss[v].v[e]);
                acc = fmaf_(s, s, acc);
            }
            if (sum) store_vec_stream<T, E>(sum, base + idx, ss[v]);
        }
    }

    float total = segment_sum<64>(acc);
    if constexpr (WPR > 1) {
        if ((threadIdx.x & 63) == 0) wave_part[threadIdx.x >> 6] = total;
        __syncthreads();
        total = wave_part[0];
#pragma unroll
        for (int w = 1; w < WPR; ++w) total += wave_part[w];
    }
    const float r = inv_sqrt(total / hidden_f + eps);
    if (lane == 0) {
        if (inv_std_var) inv_std_var[row] = r;
        if (mean) mean[row] = 0.0f;
    }

#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int idx = v * LANES + lane;
        if (FULL || idx < nvec) {
            const V gv = load_vec<T, E>(gamma, idx);
            V out;
#pragma unroll
            for (int e = 0; e < E; ++e)
                out.v[e] = from_f32<T>(to_f32(ss[v].v[e]) * r * to_f32(gv.v[e]));
            store_vec_stream<T, E>(output, base + idx, out);
        }
    }
}

template <typename T>
__global__ void __launch_bounds__(256)
ssln_block_kernel(const T* __restrict__ input, const T* __restrict__ skip,
                  const T* __restrict__ gamma, const T* __restrict__ bias,
                  T* __restrict__ output, float* __restrict__ mean,
                  float* __restrict__ inv_std_var, T* __restrict__ sum,
                  int64_t rows, int64_t hidden, float hidden_f, float eps) {
    __shared__ float wave_part[kWavesPerBlock];
    const bool has_bias = bias != nullptr;
    const int t = threadIdx.x;
    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const int64_t base = row * hidden;
        float acc = 0.0f;
        for (int64_t j = t; j < hidden; j += 256) {
            T rounded;
            const float s = residual_sum<T>(to_f32(input[base + j]), to_f32(skip[base + j]), has_bias,
                                            has_bias ? to_f32(bias[j]) : 0.0f, rounded);
            if (sum) sum[base + j] = rounded;
            acc = fmaf_(s, s, acc);
        }
        acc = segment_sum<64>(acc);
        if ((t & 63) == 0) wave_part[t >> 6] = acc;
        __syncthreads();
        const float total = (wave_part[0] + wave_part[1]) + (wave_part[2] + wave_part[3]);
        __syncthreads();  // wave_part is rewritten by the next row
        const float r = inv_sqrt(total / hidden_f + eps);
        if (t == 0) {
            if (inv_std_var) inv_std_var[row] = r;
            if (mean) mean[row] = 0.0f;
        }
        for (int64_t j = t; j < hidden; j += 256) {
            T rounded;
            const float s = residual_sum<T>(to_f32(input[base + j]), to_f32(skip[base + j]), has_bias,
                                            has_bias ? to_f32(bias[j]) : 0.0f, rounded);
            output[base + j] = from_f32<T>(s * r * to_f32(gamma[j]));
        }
    }
}

template <typename T, int E, int NV, int WPR>
hipError_t launch_wave_nv(const SslnArgs& a, int nvec, hipStream_t stream) {
    constexpr int rows_per_block = kWavesPerBlock / WPR;
    const int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
    const float hidden_f = float(a.hidden);
    auto args = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(256), 0, stream,
                           static_cast<const T*>(a.input), static_cast<const T*>(a.skip),
                           static_cast<const T*>(a.gamma), static_cast<const T*>(a.bias),
                           static_cast<T*>(a.output), a.mean, a.inv_std_var,
                           static_cast<T*>(a.sum), a.rows, nvec, hidden_f, a.epsilon);
    };
    if (nvec == 64 * WPR * NV) args(ssln_wave_kernel<T, E, NV, true, WPR>);
    else args(ssln_wave_kernel<T, E, NV, false, WPR>);
    return hipGetLastError();
}

template <typename T, int E, int MAXNV, int WPR>
hipError_t launch_wave(const SslnArgs& a, int nvec, hipStream_t stream) {
    const int need = (nvec + 64 * WPR - 1) / (64 * WPR);
    if (need <= 1) return launch_wave_nv<T, E, 1, WPR>(a, nvec, stream);
    if (need <= 2) return launch_wave_nv<T, E, 2, WPR>(a, nvec, stream);
    if (need <= 3) return launch_wave_nv<T, E, 3, WPR>(a, nvec, stream);
    if (need <= 4) return launch_wave_nv<T, E, 4, WPR>(a, nvec, stream);
    if (need <= 6) return launch_wave_nv<T, E, 6, WPR>(a, nvec, stream);
    if (need <= 8) return launch_wave_nv<T, E, 8, WPR>(a, nvec, stream);
    if constexpr (MAXNV >= 16) {
        if (need <= 12) return launch_wave_nv<T, E, 12, WPR>(a, nvec, stream);
        if (need <= 16) return launch_wave_nv<T, E, 16, WPR>(a, nvec, stream);
    }
    if constexpr (MAXNV >= 32) {
        if (need <= 24) return launch_wave_nv<T, E, 24, WPR>(a, nvec, stream);
        if (need <= 32) return launch_wave_nv<T, E, 32, WPR>(a, nvec, stream);
    }
    return hipErrorInvalidValue;  // callers check the width first
}

// Widest row (in vectors per lane) each instantiation keeps in registers:
// one wave per row up to 8192 elements; four waves per row up to 16 vectors
// per lane (32768 float16 or 16384 float32 elements).
template <typename T> constexpr int kMaxNvVector = sizeof(T) == 2 ? 16 : 32;
constexpr int kMaxNvRowBlock = 16;
constexpr int kMaxNvScalar = 32;                                           // 2048 elements

template <typename T>
hipError_t launch_ssln_t(const SslnArgs& a, Route want, hipStream_t stream, const char** route) {
    constexpr int EV = VecWidth<T>::value;
    const int64_t nvec = a.hidden / EV;
    const bool vec_ok = a.hidden % EV == 0 && nvec <= 256 * kMaxNvRowBlock &&
                        aligned16(a.input) && aligned16(a.skip) && aligned16(a.gamma) &&
                        (!a.bias || aligned16(a.bias)) && aligned16(a.output) &&
                        (!a.sum || aligned16(a.sum));
    Route r = want;
    if (r == Route::Auto || r == Route::Vector || r == Route::Split) r = vec_ok ? Route::Vector : Route::Scalar;
    if (r == Route::Scalar && a.hidden > 64 * kMaxNvScalar) r = Route::Block;

    if (r == Route::Vector) {
        if (nvec <= 64 * kMaxNvVector<T>) {
            *route = "ssln.wave.vec16";
            return launch_wave<T, EV, kMaxNvVector<T>, 1>(a, int(nvec), stream);
        }
        *route = "ssln.rowblock.vec16";
        return launch_wave<T, EV, kMaxNvRowBlock, 4>(a, int(nvec), stream);
    }
    if (r == Route::Scalar) {
        *route = "ssln.wave.scalar";
        return launch_wave<T, 1, kMaxNvScalar, 1>(a, int(a.hidden), stream);
    }
    *route = "ssln.block";
    const int64_t blocks = a.rows < 65536 * 16 ? a.rows : 65536 * 16;
    hipLaunchKernelGGL(ssln_block_kernel<T>, dim3(unsigned(blocks)), dim3(256), 0, stream,
                       static_cast<const T*>(a.input), static_cast<const T*>(a.skip),
                       static_cast<const T*>(a.gamma), static_cast<const T*>(a.bias),
                       static_cast<T*>(a.output), a.mean, a.inv_std_var, static_cast<T*>(a.sum),
                       a.rows, a.hidden, float(a.hidden), a.epsilon);
    return hipGetLastError();
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
