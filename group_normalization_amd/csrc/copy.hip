// copy.hip -- 16-byte vector copy kernel: the copy-bandwidth reference and
// the calibration kernel of known traffic for hardware byte counters.
// Nontemporal loads and stores, one pass (no grid-stride loop) for sizes up
// to 2^31 blocks of 4 KiB.
#include "device_common.h"
#include "skipnorm_internal.h"

namespace sn {
namespace {

constexpr int kCopyUnroll = 4;

__global__ void __launch_bounds__(256)
copy16_kernel(const Vec<float, 4>* __restrict__ src, Vec<float, 4>* __restrict__ dst, int64_t n) {
    const int64_t stride = int64_t(gridDim.x) * 256 * kCopyUnroll;
    for (int64_t i = int64_t(blockIdx.x) * 256 * kCopyUnroll + threadIdx.x; i < n; i += stride) {
        Vec<float, 4> v[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u)
            if (i + u * 256 < n) v[u] = load_vec_stream<float, 4>(reinterpret_cast<const float*>(src), i + u * 256);
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u)
            if (i + u * 256 < n) store_vec_stream<float, 4>(reinterpret_cast<float*>(dst), i + u * 256, v[u]);
    }
}

}  // namespace

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
    const int64_t n = int64_t(bytes / 16);
    if (n == 0) return hipSuccess;
    int64_t blocks = (n + 256 * kCopyUnroll - 1) / (256 * kCopyUnroll);
    hipLaunchKernelGGL(copy16_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream,
                       static_cast<const Vec<float, 4>*>(src), static_cast<Vec<float, 4>*>(dst), n);
    return hipGetLastError();
}

}  // namespace sn
