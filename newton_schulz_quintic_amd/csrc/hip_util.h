// HIP helpers shared by the library's kernels and entry points.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "internal.h"

namespace nsq {

#define NSQ_HIP(call)                                                                    \
    do {                                                                                 \
        hipError_t e_ = (call);                                                          \
        if (e_ != hipSuccess)                                                            \
            return ::nsq::fail(NS_ERR_HIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
    } while (0)

// Kernel timing (see ns_timing_enable). A timed launch goes out through
// hipExtLaunchKernelGGL with a start and a stop event that the dispatch itself
// records, so a pair spans the kernel's execution only (the figure rocprofv3
// reports), not the launch's dispatch. kTimeProduct covers the B X product
// kernel (all but the final step); kTimeSyrkX / kTimeSyrkA the two symmetric
// products; kTimeFinal the last B X; kTimeSmall the small-class kernel (every
// step of every small matrix in one launch).
enum TimingKind {
    kTimeProduct = 0,
    kTimeRoute = 1,
    kTimeNorm = 2,
    kTimeFinal = 3,
    kTimeSyrkX = 4,
    kTimeSyrkA = 5,
    kTimeSmall = 6,
    kTimeKinds = 7
};

// Whether launches of `kind` are timed now.
bool timing_on(int kind);
// An event pair for one launch of `kind` performing `work` (flops or bytes);
// returns an opaque slot, or -1 when timing is off or no event is free.
int timing_pair(int kind, double work, hipEvent_t *start, hipEvent_t *stop);
// The launch that was given the pair of `slot` went out (`ok`) or failed.
void timing_close(int slot, bool ok);

// Pinned host staging buffers for the per-call tables (staging.hip). Acquire
// a buffer of at least `bytes` (host pointer and the device's pointer to the
// same memory), fill it, enqueue the kernel that reads it, then release it
// with that stream so it is reused only after the kernel ends.
// Without may_grow the call uses only slots already large enough (see
// staging_reserve) and allocates nothing.
ns_status staging_acquire(size_t bytes, int *slot, void **ptr, void **dev_ptr, bool may_grow = true);
ns_status staging_reserve(size_t bytes);
// Calls under stream capture: slots of `bytes` reserved up front, each taken
// for good by one captured call (its graph's replays read it).
ns_status staging_reserve_capture(size_t bytes);
ns_status staging_acquire_capture(size_t bytes, void **ptr, void **dev_ptr);
ns_status staging_release(int slot, hipStream_t stream, bool used);

// The launches of one timed step of a call: `work` is what they perform
// together, counted with the first of them.
struct TimedScope {
    int kind;
    double work;
    bool on;
    TimedScope(int k, double w) : kind(k), work(w), on(timing_on(k)) {}
    template <typename F, typename... Args>
    void launch(F kernel, dim3 grid, dim3 block, hipStream_t st, Args... args) {
        hipEvent_t a = nullptr, b = nullptr;
        const int slot = on ? timing_pair(kind, work, &a, &b) : -1;
        work = 0.0;
        if (slot < 0) {
            hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
            return;
        }
        hipExtLaunchKernelGGL(kernel, grid, block, 0, st, a, b, 0, args...);
        timing_close(slot, hipPeekAtLastError() == hipSuccess);
    }
};

}  // namespace nsq
