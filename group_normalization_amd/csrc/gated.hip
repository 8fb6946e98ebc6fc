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
//   block    one 256-thread workgroup per row for wider rows; X is read twice.
// scale is loaded once per thread and kept in registers as float32.  X, gate
// and Y are touched once and move with nontemporal loads and stores.
#include "device_common.h"
#include "skipnorm_internal.h"

namespace sn {
namespace {

template <typename T, int E, int L, int VPL, int RPT>
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
                store_vec_stream<T, E>(Y, row * nvec + idx, out);
            }
        }
    }
}

template <typename T>
__global__ void __launch_bounds__(256)
gated_block_kernel(const T* __restrict__ X, const T* __restrict__ scale,
                   const T* __restrict__ gate, T* __restrict__ Y, int64_t rows,
                   int64_t span, float span_f, float eps) {
    __shared__ float wave_part[4];
    const int t = threadIdx.x;
    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const int64_t base = row * span;
        float acc = 0.0f;
        for (int64_t j = t; j < span; j += 256) {
            const float x = to_f32(X[base + j]);
            acc = fmaf_(x, x, acc);
        }
        acc = segment_sum<64>(acc);
        if ((t & 63) == 0) wave_part[t >> 6] = acc;
        __syncthreads();
        const float total = (wave_part[0] + wave_part[1]) + (wave_part[2] + wave_part[3]);
        __syncthreads();
        const float r = inv_sqrt(total / span_f + eps);
        for (int64_t j = t; j < span; j += 256) {
            const float x = to_f32(X[base + j]);
            const float g = to_f32(gate[base + j]);
            Y[base + j] = from_f32<T>(x * r * to_f32(scale[j]) * silu_f32(g));
        }
    }
}

template <typename T, int E, int L, int VPL>
hipError_t launch_segment(const GatedArgs& a, int nvec, hipStream_t stream) {
    constexpr int RPT = VPL >= 4 ? 1 : 4 / VPL;
    constexpr int rows_per_block = (256 / L) * RPT;
    const int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL((gated_segment_kernel<T, E, L, VPL, RPT>), dim3(unsigned(blocks)), dim3(256),
                       0, stream, static_cast<const T*>(a.X), static_cast<const T*>(a.scale),
                       static_cast<const T*>(a.gate), static_cast<T*>(a.Y), a.rows, nvec,
                       float(a.span), a.epsilon);
    return hipGetLastError();
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

template <typename T>
hipError_t launch_gated_t(const GatedArgs& a, Route want, hipStream_t stream, const char** route) {
    // Widest access that divides the row and every tensor's base.
    int E = widest_vector<T>(a.span, {a.X, a.scale, a.gate, a.Y});
    if (want == Route::Scalar) E = 1;
    const int64_t nvec = a.span / E;
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
    *route = "gated.block";
    const int64_t blocks = a.rows < 65536 * 16 ? a.rows : 65536 * 16;
    hipLaunchKernelGGL(gated_block_kernel<T>, dim3(unsigned(blocks)), dim3(256), 0, stream,
                       static_cast<const T*>(a.X), static_cast<const T*>(a.scale),
                       static_cast<const T*>(a.gate), static_cast<T*>(a.Y), a.rows, a.span,
                       float(a.span), a.epsilon);
    return hipGetLastError();
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
