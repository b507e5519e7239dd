// Pinned host staging for the per-call device tables of the batched
// Newton-Schulz entry point. The first kernel of a call reads the tables
// straight from this buffer (it is mapped into the device's address space) and
// copies them into the workspace for the later kernels. A buffer is reused only
// after the event recorded behind that kernel has completed, so the host never
// overwrites data a pending kernel still reads. All kMaxSlots buffers are made
// on the first call: a host that runs calls ahead of the GPU then never pays
// for pinned allocation (several ms each) in its steady state.

#include <mutex>
#include <vector>

#include "hip_util.h"

namespace nsq {

namespace {
struct Slot {
    void *ptr = nullptr;
    void *dev = nullptr;   // the same memory as the device addresses it
    size_t cap = 0;
    hipEvent_t done = nullptr;
    bool in_use = false;     // handed out and not yet released
    bool pending = false;    // a kernel may still be reading it
};
std::mutex g_mu;
std::vector<Slot> g_slots;
constexpr size_t kMaxSlots = 8;

bool idle(Slot &s) {
    if (s.in_use) return false;
    if (s.pending && hipEventQuery(s.done) == hipSuccess) s.pending = false;
    return !s.pending;
}
}  // namespace

// Makes every slot hold at least `bytes` (allocating pinned memory now), so
// that later calls whose tables fit never allocate.
ns_status staging_reserve(size_t bytes) {
    std::lock_guard<std::mutex> lk(g_mu);
    while (g_slots.size() < kMaxSlots) {
        g_slots.emplace_back();
        NSQ_HIP(hipEventCreateWithFlags(&g_slots.back().done, hipEventDisableTiming));
    }
    for (Slot &s : g_slots) {
        if (s.cap >= bytes) continue;
        if (s.in_use) return fail(NS_ERR_INVALID_ARG, "table staging is in use by another thread's call");
        if (s.pending) {
            NSQ_HIP(hipEventSynchronize(s.done));
            s.pending = false;
        }
        if (s.ptr) NSQ_HIP(hipHostFree(s.ptr));
        s.ptr = s.dev = nullptr;
        s.cap = 0;
        NSQ_HIP(hipHostMalloc(&s.ptr, bytes, hipHostMallocDefault));
        NSQ_HIP(hipHostGetDevicePointer(&s.dev, s.ptr, 0));
        s.cap = bytes;
    }
    return NS_OK;
}

// Without may_grow, only slots that already hold `bytes` are used (waiting for
// one to become free if need be) and nothing is allocated.
ns_status staging_acquire(size_t bytes, int *slot, void **ptr, void **dev_ptr, bool may_grow) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!may_grow) {
        int pick = -1;
        for (size_t i = 0; i < g_slots.size() && pick < 0; ++i)
            if (g_slots[i].cap >= bytes && idle(g_slots[i])) pick = (int)i;
        for (size_t i = 0; i < g_slots.size() && pick < 0; ++i)
            if (g_slots[i].cap >= bytes && !g_slots[i].in_use) {
                NSQ_HIP(hipEventSynchronize(g_slots[i].done));
                g_slots[i].pending = false;
                pick = (int)i;
            }
        if (pick < 0)
            return fail(NS_ERR_WORKSPACE, "the call's tables take %zu bytes, more than the table staging reserved "
                        "without allocating (ns_noalloc_init)", bytes);
        g_slots[pick].in_use = true;
        *slot = pick;
        *ptr = g_slots[pick].ptr;
        *dev_ptr = g_slots[pick].dev;
        return NS_OK;
    }
    while (g_slots.size() < kMaxSlots) {
        g_slots.emplace_back();
        Slot &s = g_slots.back();
        NSQ_HIP(hipEventCreateWithFlags(&s.done, hipEventDisableTiming));
        const size_t cap = std::max<size_t>(bytes, 1 << 20);
        NSQ_HIP(hipHostMalloc(&s.ptr, cap, hipHostMallocDefault));
        NSQ_HIP(hipHostGetDevicePointer(&s.dev, s.ptr, 0));
        s.cap = cap;
    }
    int pick = -1;
    for (size_t i = 0; i < g_slots.size(); ++i)
        if (idle(g_slots[i]) && (pick < 0 || g_slots[i].cap >= bytes)) {
            pick = (int)i;
            if (g_slots[i].cap >= bytes) break;
        }
    if (pick < 0 && g_slots.size() < kMaxSlots) {
        g_slots.emplace_back();
        pick = (int)g_slots.size() - 1;
        NSQ_HIP(hipEventCreateWithFlags(&g_slots[pick].done, hipEventDisableTiming));
    }
    if (pick < 0) {
        // every slot is busy: wait for the oldest free-able one
        for (size_t i = 0; i < g_slots.size() && pick < 0; ++i)
            if (!g_slots[i].in_use) {
                NSQ_HIP(hipEventSynchronize(g_slots[i].done));
                g_slots[i].pending = false;
                pick = (int)i;
            }
        if (pick < 0) return fail(NS_ERR_HIP, "no free table staging buffer (too many concurrent calls)");
    }
    Slot &s = g_slots[pick];
    if (s.cap < bytes) {
        if (s.ptr) NSQ_HIP(hipHostFree(s.ptr));
        s.ptr = s.dev = nullptr;
        s.cap = 0;
        const size_t cap = std::max<size_t>(bytes, 1 << 20);
        NSQ_HIP(hipHostMalloc(&s.ptr, cap, hipHostMallocDefault));
        NSQ_HIP(hipHostGetDevicePointer(&s.dev, s.ptr, 0));
        s.cap = cap;
    }
    s.in_use = true;
    *slot = pick;
    *ptr = s.ptr;
    *dev_ptr = s.dev;
    return NS_OK;
}

// Calls made while their stream is being captured into a graph: the graph's
// replays read the tables from the staging long after the call returns, so
// such a call takes a slot of its own for the life of the process.
namespace {
std::vector<Slot> g_capture;
size_t g_capture_taken = 0;
constexpr size_t kCaptureSlots = 8;
}  // namespace

ns_status staging_reserve_capture(size_t bytes) {
    std::lock_guard<std::mutex> lk(g_mu);
    while (g_capture.size() < kCaptureSlots) {
        Slot s;
        NSQ_HIP(hipHostMalloc(&s.ptr, bytes, hipHostMallocDefault));
        NSQ_HIP(hipHostGetDevicePointer(&s.dev, s.ptr, 0));
        s.cap = bytes;
        g_capture.push_back(s);
    }
    return NS_OK;
}

ns_status staging_acquire_capture(size_t bytes, void **ptr, void **dev_ptr) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_capture.empty())
        return fail(NS_ERR_INVALID_ARG, "a call under stream capture needs the staging that ns_noalloc_init reserves");
    if (g_capture_taken >= g_capture.size())
        return fail(NS_ERR_WORKSPACE, "all %zu table staging slots for calls under stream capture are taken",
                    g_capture.size());
    Slot &s = g_capture[g_capture_taken];
    if (s.cap < bytes)
        return fail(NS_ERR_WORKSPACE, "the call's tables take %zu bytes, more than a capture slot's %zu", bytes, s.cap);
    ++g_capture_taken;
    *ptr = s.ptr;
    *dev_ptr = s.dev;
    return NS_OK;
}

ns_status staging_release(int slot, hipStream_t stream, bool used) {
    std::lock_guard<std::mutex> lk(g_mu);
    Slot &s = g_slots[slot];
    s.in_use = false;
    if (used) {
        NSQ_HIP(hipEventRecord(s.done, stream));
        s.pending = true;
    }
    return NS_OK;
}

}  // namespace nsq
