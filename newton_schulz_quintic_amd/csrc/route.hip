// Pack / unpack: move the row pieces of every tensor between the S shard
// buffers and the S home buffers of one GPU, as laid out by the route plan.
//
// "core.optimizer.layer_sharded_a2a": route_to_ns_home gathers each param's
// row shards into the complete matrix at its home, route_from_ns_home scatters
// the results back. "...owner_planning": OwnerGatherPlan.reconstruct_full
// concatenates per-rank shards in buffer order; OwnerScatterPlan.unpack
// extracts each rank's flat result shard.
//
// One launch moves every piece. The pieces are cut into chunks (16 KiB)
// numbered globally; each workgroup takes one chunk (a contiguous range of
// them only past 2^23 chunks, 128 GiB), so the workgroups in flight together
// touch neighbouring chunks: four chunks per workgroup measured 10 % slower on
// a 13 GiB plan and 16 % slower on one of 12 000 small pieces. A chunk moves
// with 16-byte loads and stores when both ends are 16-byte aligned
// (narrower accesses otherwise); a full aligned chunk has all of each thread's
// loads in flight before its stores. A piece cut along a dimension other than
// the first (the TP stage's partition_dim in route_to_ns_home) is contiguous
// in its shard buffer and a run of equal strided blocks in the home buffer;
// its chunks map each 16-, 4- or 2-byte unit to its run. HBM-bound: every byte
// is read once and written once. Plans that move more than the 256 MB last-level cache (MALL)
// load and store with non-temporal hints; smaller ones keep their output
// cache-resident for the kernel that reads it next.

#include <cstdlib>
#include <type_traits>

#include "hip_util.h"

namespace nsq {
namespace {

constexpr int kRouteThreads = 256;
#ifndef NSQ_ROUTE_GRID
#define NSQ_ROUTE_GRID 8388608   // 2^23 workgroups x 256 threads stays below 2^32 work-items
#endif
constexpr int kRouteMaxGrid = NSQ_ROUTE_GRID;

struct PtrSet {
    char *p[NS_MAX_SHARDS];
};

// A 16-byte load, with the non-temporal hint on large plans (their data is
// not read again; 2 % faster on a 13 GiB plan).
template <bool NT, typename V>
__device__ inline V load16(const V *p) {
    if constexpr (NT) {
        V v;
        v.x = __builtin_nontemporal_load(&p->x);
        v.y = __builtin_nontemporal_load(&p->y);
        v.z = __builtin_nontemporal_load(&p->z);
        v.w = __builtin_nontemporal_load(&p->w);
        return v;
    } else {
        return *p;
    }
}

// UA: the misaligned branch moves 16 bytes per access (plans with a piece or
// a buffer off 16-byte alignment); otherwise it moves 2 bytes per access, which
// keeps the aligned kernel's register budget (64, eight waves per SIMD).
template <bool NT, bool UA>
__device__ inline void copy_chunk(const char *__restrict__ src, char *__restrict__ dst, int64_t len) {
    const int t = threadIdx.x;
    const uintptr_t mis = reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst);
    if ((mis & 15) == 0) {
        const uint4 *s4 = reinterpret_cast<const uint4 *>(src);
        uint4 *d4 = reinterpret_cast<uint4 *>(dst);
        const int64_t n16 = len >> 4;
        constexpr int kPer = (int)(kRouteChunkBytes / 16 / kRouteThreads);   // 16-byte units per thread
        static_assert(kRouteChunkBytes % (16 * kRouteThreads) == 0, "whole units per thread");
        if (n16 == kRouteChunkBytes / 16) {
            // full chunk: all of this thread's loads in flight before the stores
            uint4 v[kPer];
#pragma unroll
            for (int k = 0; k < kPer; ++k) v[k] = load16<NT>(s4 + t + kRouteThreads * k);
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
                if constexpr (NT) {
                    __builtin_nontemporal_store(v[k].x, &d4[t + kRouteThreads * k].x);
                    __builtin_nontemporal_store(v[k].y, &d4[t + kRouteThreads * k].y);
                    __builtin_nontemporal_store(v[k].z, &d4[t + kRouteThreads * k].z);
                    __builtin_nontemporal_store(v[k].w, &d4[t + kRouteThreads * k].w);
                } else {
                    d4[t + kRouteThreads * k] = v[k];
                }
            }
        } else {
            for (int64_t i = t; i < n16; i += kRouteThreads) d4[i] = s4[i];
        }
        for (int64_t i = (n16 << 4) + 2 * t; i < len; i += 2 * kRouteThreads)
            *reinterpret_cast<uint16_t *>(dst + i) = *reinterpret_cast<const uint16_t *>(src + i);
    } else if constexpr (!UA) {
        for (int64_t i = 2 * t; i < len; i += 2 * kRouteThreads)
            *reinterpret_cast<uint16_t *>(dst + i) = *reinterpret_cast<const uint16_t *>(src + i);
    } else {
        // Ends 2-byte aligned (elements are 2 or 4 bytes): a 2-byte head up to
        // the first 16-byte boundary of dst, then 16-byte stores fed by
        // 16-byte loads at src's own alignment (the GPU's unaligned access
        // mode serves them as one load; four per thread in flight), then a
        // 2-byte tail. Every access stays inside [src, src + len).
        const int n = (int)len;   // a chunk: at most kRouteChunkBytes
        const int head = min(n, (int)((16 - (reinterpret_cast<uintptr_t>(dst) & 15)) & 15));
        if (2 * t < head)
            *reinterpret_cast<uint16_t *>(dst + 2 * t) = *reinterpret_cast<const uint16_t *>(src + 2 * t);
        const char *s = src + head;
        char *d = dst + head;
        const int n16 = (n - head) >> 4;
        typedef int v4i __attribute__((ext_vector_type(4)));
        typedef v4i __attribute__((aligned(2))) v4i_u;   // 16 bytes at 2-byte alignment
        for (int i0 = t; i0 < n16; i0 += 4 * kRouteThreads) {
            v4i v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = i0 + k * kRouteThreads;
                // no non-temporal hint: neighbouring lanes' loads share cache lines
                if (i < n16) v[k] = *reinterpret_cast<const v4i_u *>(s + 16 * i);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = i0 + k * kRouteThreads;
                if (i < n16) {
                    if constexpr (NT) __builtin_nontemporal_store(v[k], reinterpret_cast<v4i *>(d + 16 * i));
                    else *reinterpret_cast<v4i *>(d + 16 * i) = v[k];
                }
            }
        }
        for (int i = head + (n16 << 4) + 2 * t; i < n; i += 2 * kRouteThreads)
            *reinterpret_cast<uint16_t *>(dst + i) = *reinterpret_cast<const uint16_t *>(src + i);
    }
}

// One chunk of a strided piece: shard bytes [off, off + len) of the piece
// (contiguous at sp), whose byte p sits in the home at
// hp + (p / run) * stride + p % run. Units of W bytes never straddle a run:
// W divides run, stride, off and both bases. IDX is the integer type of byte
// offsets inside the piece (32-bit when the piece is under 4 GiB: its
// division is several times cheaper). 16-byte units keep each thread's four
// loads in flight before the stores; narrower ones (pieces at odd offsets)
// copy unit by unit, so the kernel's register budget stays that of the
// contiguous path.
template <int W, bool NT, typename IDX>
__device__ inline void copy_chunk_strided(char *__restrict__ sp, char *__restrict__ hp, int64_t off, int64_t len,
                                          int64_t run, int64_t stride, bool to_home) {
    typedef typename std::conditional<W == 16, uint4, typename std::conditional<W == 4, uint32_t, uint16_t>::type>::type U;
    const int64_t nu = len / W;
    const IDX run_i = (IDX)run;
    auto home_off = [&](int64_t p) -> int64_t {
        const IDX r = (IDX)p / run_i;
        return (int64_t)r * stride + (int64_t)((IDX)p - r * run_i);
    };
    static_assert(kRouteChunkBytes == 4 * 16 * kRouteThreads, "four 16-byte units per thread in a full chunk");
    if (W == 16 && nu == 4 * kRouteThreads) {   // full chunk: the four loads in flight before the stores
        const int64_t p0 = off + (int64_t)threadIdx.x * 16, step = 16 * kRouteThreads;
        const int64_t h0 = home_off(p0), h1 = home_off(p0 + step), h2 = home_off(p0 + 2 * step),
                      h3 = home_off(p0 + 3 * step);
        const char *src = to_home ? sp : hp;
        char *dst = to_home ? hp : sp;
        const int64_t s0 = to_home ? p0 : h0, s1 = to_home ? p0 + step : h1, s2 = to_home ? p0 + 2 * step : h2,
                      s3 = to_home ? p0 + 3 * step : h3;
        const int64_t d0 = to_home ? h0 : p0, d1 = to_home ? h1 : p0 + step, d2 = to_home ? h2 : p0 + 2 * step,
                      d3 = to_home ? h3 : p0 + 3 * step;
        const uint4 v0 = load16<NT>(reinterpret_cast<const uint4 *>(src + s0));
        const uint4 v1 = load16<NT>(reinterpret_cast<const uint4 *>(src + s1));
        const uint4 v2 = load16<NT>(reinterpret_cast<const uint4 *>(src + s2));
        const uint4 v3 = load16<NT>(reinterpret_cast<const uint4 *>(src + s3));
        auto put = [&](int64_t d, const uint4 &v) {
            uint4 *q = reinterpret_cast<uint4 *>(dst + d);
            if constexpr (NT) {
                __builtin_nontemporal_store(v.x, &q->x);
                __builtin_nontemporal_store(v.y, &q->y);
                __builtin_nontemporal_store(v.z, &q->z);
                __builtin_nontemporal_store(v.w, &q->w);
            } else {
                *q = v;
            }
        };
        put(d0, v0);
        put(d1, v1);
        put(d2, v2);
        put(d3, v3);
    } else {
        for (int64_t u = threadIdx.x; u < nu; u += kRouteThreads) {
            const int64_t p = off + u * W;
            U *h = reinterpret_cast<U *>(hp + home_off(p));
            U *sh = reinterpret_cast<U *>(sp + p);
            if (to_home)
                *h = *sh;
            else
                *sh = *h;
        }
    }
}

// to_home = 1: shard -> home (pack); 0: home -> shard (unpack).
// Workgroup b copies the contiguous chunk range [b per, (b + 1) per): it finds
// the piece holding its first chunk by binary search over the pieces' first
// chunk numbers, then walks forward through the pieces.
constexpr int64_t kMallBytes = 256ll << 20;

// Workgroups per launch. NS_ROUTE_MAX_GRID lowers the cap, so that small
// plans give each workgroup several chunks (tests; the bits are the same).
int64_t route_max_grid() {
    if (const char *env = getenv("NS_ROUTE_MAX_GRID")) {
        const long long v = atoll(env);
        if (v >= 1 && v < kRouteMaxGrid) return v;
    }
    return kRouteMaxGrid;
}
template <bool NT, bool UA>
__global__ __launch_bounds__(kRouteThreads) void route_copy_kernel(const RouteSeg *__restrict__ segs,
                                                                   int32_t nseg, int64_t total_chunks,
                                                                   int64_t per, PtrSet shard, PtrSet home,
                                                                   int32_t to_home) {
    const int64_t c0 = (int64_t)blockIdx.x * per;
    const int64_t c1 = c0 + per < total_chunks ? c0 + per : total_chunks;
    if (c0 >= c1) return;
    int32_t lo = 0, hi = nseg - 1;
    while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (segs[mid].chunk_begin <= c0)
            lo = mid;
        else
            hi = mid - 1;
    }
    RouteSeg g = segs[lo];
    for (int64_t c = c0; c < c1; ++c) {
        while (lo + 1 < nseg && segs[lo + 1].chunk_begin <= c) g = segs[++lo];
        const int64_t off = (c - g.chunk_begin) * kRouteChunkBytes;
        const int64_t rem = g.len - off;
        const int64_t len = rem < kRouteChunkBytes ? rem : kRouteChunkBytes;
        if (g.run_len == g.len) {   // one run: contiguous on both sides
            char *sp = shard.p[g.shard] + g.shard_off + off;
            char *hp = home.p[g.home] + g.home_off + off;
            if (to_home)
                copy_chunk<NT, UA>(sp, hp, len);
            else
                copy_chunk<NT, UA>(hp, sp, len);
        } else {
            char *sp = shard.p[g.shard] + g.shard_off;
            char *hp = home.p[g.home] + g.home_off;
            const uintptr_t mis = reinterpret_cast<uintptr_t>(sp) | reinterpret_cast<uintptr_t>(hp) |
                                  (uintptr_t)g.run_len | (uintptr_t)g.home_stride;
            if (g.len <= (int64_t)UINT32_MAX) {
                if ((mis & 15) == 0)
                    copy_chunk_strided<16, NT, uint32_t>(sp, hp, off, len, g.run_len, g.home_stride, to_home);
                else if ((mis & 3) == 0)
                    copy_chunk_strided<4, NT, uint32_t>(sp, hp, off, len, g.run_len, g.home_stride, to_home);
                else
                    copy_chunk_strided<2, NT, uint32_t>(sp, hp, off, len, g.run_len, g.home_stride, to_home);
            } else {
                if ((mis & 15) == 0)
                    copy_chunk_strided<16, NT, int64_t>(sp, hp, off, len, g.run_len, g.home_stride, to_home);
                else if ((mis & 3) == 0)
                    copy_chunk_strided<4, NT, int64_t>(sp, hp, off, len, g.run_len, g.home_stride, to_home);
                else
                    copy_chunk_strided<2, NT, int64_t>(sp, hp, off, len, g.run_len, g.home_stride, to_home);
            }
        }
    }
}

ns_status route_launch(const ns_route_plan *plan, const void *const *shard_bufs,
                       const void *const *home_bufs, int32_t to_home, void *stream) {
    if (!plan) return fail(NS_ERR_INVALID_ARG, "plan is NULL");
    if (!plan->device_table && !plan->segs.empty())
        return fail(NS_ERR_PLAN_MISMATCH, "route plan not uploaded (call ns_route_plan_upload)");
    const int32_t S = plan->num_shards;
    if (S > 0 && (!shard_bufs || !home_bufs))
        return fail(NS_ERR_INVALID_ARG, "buffer pointer arrays are required");
    PtrSet sh{}, ho{};
    bool aligned = plan->aligned16;
    for (int32_t s = 0; s < S; ++s) {
        if (!shard_bufs[s] && plan->shard_elems[s] > 0)
            return fail(NS_ERR_INVALID_ARG, "shard buffer %d is NULL but holds %lld elements", s,
                        (long long)plan->shard_elems[s]);
        if (!home_bufs[s] && plan->home_elems[s] > 0)
            return fail(NS_ERR_INVALID_ARG, "home buffer %d is NULL but holds %lld elements", s,
                        (long long)plan->home_elems[s]);
        const uintptr_t align = (uintptr_t)shard_bufs[s] | (uintptr_t)home_bufs[s];
        if (align % plan->elem_bytes)
            return fail(NS_ERR_INVALID_ARG, "buffers of shard/home %d not %d-byte aligned", s,
                        plan->elem_bytes);
        sh.p[s] = (char *)shard_bufs[s];
        ho.p[s] = (char *)home_bufs[s];
        aligned = aligned && align % 16 == 0;
    }
    if (plan->segs.empty()) return NS_OK;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int64_t max_grid = route_max_grid();
    const int64_t per = (plan->total_chunks + max_grid - 1) / max_grid;   // chunks per workgroup
    const int64_t grid = (plan->total_chunks + per - 1) / per;
    {
        TimedScope ts(kTimeRoute, 2.0 * (double)plan->total_bytes);
        const RouteSeg *table = reinterpret_cast<const RouteSeg *>(plan->device_table);
        const bool nt = plan->total_bytes > kMallBytes;
        auto go = [&](auto kernel) {
            ts.launch(kernel, dim3((unsigned)grid), dim3(kRouteThreads), st, table, (int32_t)plan->segs.size(),
                      plan->total_chunks, per, sh, ho, to_home);
        };
        if (aligned) nt ? go(route_copy_kernel<true, false>) : go(route_copy_kernel<false, false>);
        else nt ? go(route_copy_kernel<true, true>) : go(route_copy_kernel<false, true>);
    }
    NSQ_HIP(hipGetLastError());
    return NS_OK;
}

}  // namespace
}  // namespace nsq

using namespace nsq;

extern "C" ns_status ns_route_plan_upload(ns_route_plan *plan, void *device_table, void *stream) {
    if (!plan) return fail(NS_ERR_INVALID_ARG, "plan is NULL");
    if (!device_table) return fail(NS_ERR_INVALID_ARG, "device_table is NULL");
    if (reinterpret_cast<uintptr_t>(device_table) % 16)
        return fail(NS_ERR_INVALID_ARG, "device_table must be 16-byte aligned");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (!plan->segs.empty()) {
        NSQ_HIP(hipMemcpyAsync(device_table, plan->segs.data(), plan->segs.size() * sizeof(RouteSeg),
                               hipMemcpyHostToDevice, st));
        NSQ_HIP(hipStreamSynchronize(st));
    }
    plan->device_table = device_table;
    return NS_OK;
}

extern "C" ns_status ns_pack_shards(const ns_route_plan *plan, const void *const *shard_bufs,
                                    void *const *home_bufs, void *stream) {
    return route_launch(plan, shard_bufs, const_cast<const void *const *>(home_bufs), 1, stream);
}

extern "C" ns_status ns_unpack_shards(const ns_route_plan *plan, const void *const *home_bufs,
                                      void *const *shard_bufs, void *stream) {
    return route_launch(plan, const_cast<const void *const *>(shard_bufs), home_bufs, 0, stream);
}
