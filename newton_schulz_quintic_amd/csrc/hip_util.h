// HIP helpers shared by the library's kernels and entry points.
#pragma once

#include <hip/hip_runtime.h>

#include "internal.h"

namespace nsq {

#define NSQ_HIP(call)                                                                    \
    do {                                                                                 \
        hipError_t e_ = (call);                                                          \
        if (e_ != hipSuccess)                                                            \
            return ::nsq::fail(NS_ERR_HIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
    } while (0)

// Kernel timing (see ns_timing_enable): a scope that records a HIP event pair
// around the launches made while it is alive, when timing is enabled.
// kTimeProduct covers the B X product kernel (all but the final step);
// kTimeSyrkX / kTimeSyrkA the two symmetric products; kTimeFinal the last B X.
enum TimingKind {
    kTimeProduct = 0,
    kTimeRoute = 1,
    kTimeNorm = 2,
    kTimeFinal = 3,
    kTimeSyrkX = 4,
    kTimeSyrkA = 5,
    kTimeKinds = 6
};

bool timing_enabled();
// Returns an opaque slot (or -1 when timing is off). `work` is the algorithmic
// work the bracketed launches perform (flops or bytes).
int timing_start(int kind, hipStream_t stream, double work);
void timing_stop(int slot, hipStream_t stream);

// Pinned host staging buffers for the per-call tables (staging.hip). Acquire
// a buffer of at least `bytes` (host pointer and the device's pointer to the
// same memory), fill it, enqueue the kernel that reads it, then release it
// with that stream so it is reused only after the kernel ends.
ns_status staging_acquire(size_t bytes, int *slot, void **ptr, void **dev_ptr);
ns_status staging_release(int slot, hipStream_t stream, bool used);

struct TimedScope {
    int slot;
    hipStream_t stream;
    TimedScope(int kind, hipStream_t s, double work) : slot(timing_start(kind, s, work)), stream(s) {}
    ~TimedScope() { timing_stop(slot, stream); }
};

}  // namespace nsq
