// skipnorm_internal.h -- argument blocks and kernel launchers shared between
// the C-ABI front end (skipnorm_api.cpp) and the kernel sources.  Internal.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace sn {

enum class Route { Auto = 0, Scalar = 1, Vector = 2, Block = 3, Split = 4, Flat = 5 };

// ---------------------------------------------------------------- SSLN
// Also the non-simplified form (center = true: the row mean is removed and
// beta, if given, added).
struct SslnArgs {
    int dtype;  // 0 = float32, 1 = float16
    int64_t rows, hidden;
    const void *input, *skip, *gamma, *beta, *bias;
    float epsilon;
    void* output;
    float *mean, *inv_std_var;
    void* sum;
    bool center;
};
// Enqueues the op; *route receives the name of the kernel family used.
hipError_t launch_ssln(const SslnArgs& a, Route want, hipStream_t stream, const char** route);

// ---------------------------------------------------------------- Gated
struct GatedArgs {
    int dtype;
    int64_t rows, span;
    const void *X, *scale, *gate;
    float epsilon;
    void* Y;
};
hipError_t launch_gated(const GatedArgs& a, Route want, hipStream_t stream, const char** route);

// ---------------------------------------------------------------- SGN
struct SgnArgs {
    int dtype, param_dtype;
    int64_t N, C, H, W, groups;
    bool channels_last;
    int activation;
    const void *X, *gamma, *beta, *skip, *bias;
    bool skip_broadcast;
    float epsilon;
    void *Y, *S;
    void* workspace;
    uint64_t tag;                     // unique per call (publication tags)
    long long exchange_timeout_ticks; // bounded wait of the cluster route
    // Clear the publication slots before a cluster launch (the call is being
    // captured into a graph, whose replays repeat `tag`).
    bool clear_tags;
    // Phase timestamps of the single-launch routes (measurement builds with
    // SN_PHASE_TRACE only; nullptr otherwise).
    unsigned long long* trace = nullptr;
};
// Measurement builds (SN_PHASE_TRACE): the workspace grows by
// kTraceBytes, where the leader of each of the first kTraceBlocks
// workgroups of a single-launch SkipGroupNorm route records the 100 MHz
// wall clock at kTraceStamps phase boundaries.
constexpr int kTraceStamps = 8;
constexpr unsigned kTraceBlocks = 65536;
constexpr size_t kTraceBytes = size_t(kTraceBlocks) * kTraceStamps * 8;
// Blocks of the statistics pass per (n, group) partial-sum row; a function
// of the shapes and T only, so that the workspace size does not depend on
// the route taken.
int64_t sgn_partials_per_group(int dtype, int64_t N, int64_t C, int64_t H, int64_t W,
                               int64_t groups, bool channels_last);
size_t sgn_workspace_bytes(int dtype, int64_t N, int64_t C, int64_t H, int64_t W,
                           int64_t groups, bool channels_last);
hipError_t launch_sgn(const SgnArgs& a, Route want, hipStream_t stream, const char** route);

// The device address of the library's static SkipGroupNorm scratch on the
// current device (kStaticScratchBytes, 256-byte aligned), looked up on the
// first call on each device.  Allocates nothing.
constexpr size_t kStaticScratchBytes = size_t(8) << 20;
hipError_t static_scratch(void** ptr);

// ---------------------------------------------------------------- copy
hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace sn
