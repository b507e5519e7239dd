// Kernel timing hooks (ns_timing_enable / ns_timing_read): HIP event pairs
// recorded by the library's own kernel dispatches (hipExtLaunchKernelGGL), one
// pair per timed launch.

#include <mutex>
#include <vector>

#include "hip_util.h"

namespace nsq {

namespace {
struct Rec {
    hipEvent_t start, stop;
    int kind;
    double work;
    bool closed;
};
std::mutex g_mu;
uint32_t g_mask = 0;   // bit k: record launches of kind k
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}
}  // namespace

bool timing_on(int kind) {
    std::lock_guard<std::mutex> lk(g_mu);
    return kind >= 0 && kind < kTimeKinds && (g_mask & (1u << kind));
}

int timing_pair(int kind, double work, hipEvent_t *start, hipEvent_t *stop) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (kind < 0 || kind >= kTimeKinds || !(g_mask & (1u << kind))) return -1;
    Rec r{take_event(), take_event(), kind, work, false};
    if (!r.start || !r.stop) {
        if (r.start) g_pool.push_back(r.start);
        if (r.stop) g_pool.push_back(r.stop);
        return -1;
    }
    g_recs.push_back(r);
    *start = r.start;
    *stop = r.stop;
    return (int)g_recs.size() - 1;
}

void timing_close(int slot, bool ok) {
    if (slot < 0) return;
    std::lock_guard<std::mutex> lk(g_mu);
    if (slot < (int)g_recs.size()) g_recs[slot].closed = ok;
}

}  // namespace nsq

using namespace nsq;

// Events are made ahead, when timing is switched on: creating them on demand
// inside a measured loop costs host time that the loop would then report.
constexpr size_t kPoolEvents = 4096;

extern "C" ns_status ns_timing_enable(int32_t kinds) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_mask = kinds == -1 ? (1u << kTimeKinds) - 1 : (uint32_t)kinds & ((1u << kTimeKinds) - 1);
    while (g_mask && g_pool.size() + 2 * g_recs.size() < kPoolEvents) {
        hipEvent_t e = nullptr;
        NSQ_HIP(hipEventCreate(&e));
        g_pool.push_back(e);
    }
    return NS_OK;
}

extern "C" ns_status ns_timing_read(int32_t kind, double *total_ms, int64_t *launches,
                                    double *work) {
    if (kind < 0 || kind >= kTimeKinds) return fail(NS_ERR_INVALID_ARG, "timing kind %d", kind);
    std::lock_guard<std::mutex> lk(g_mu);
    double ms_sum = 0.0, work_sum = 0.0;
    int64_t count = 0;
    std::vector<Rec> keep;
    for (Rec &r : g_recs) {
        if (r.kind != kind) {
            keep.push_back(r);
            continue;
        }
        if (r.closed) {
            hipError_t e = hipEventSynchronize(r.stop);
            float ms = 0.f;
            if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
            if (e != hipSuccess) return fail(NS_ERR_HIP, "timing event: %s", hipGetErrorString(e));
            ms_sum += ms;
            work_sum += r.work;
            ++count;
        }
        g_pool.push_back(r.start);
        g_pool.push_back(r.stop);
    }
    g_recs.swap(keep);
    if (total_ms) *total_ms = ms_sum;
    if (launches) *launches = count;
    if (work) *work = work_sum;
    return NS_OK;
}
