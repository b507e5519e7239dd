// Host planner: tensor view, Newton-Schulz cost, LPT home assignment and the
// route plan (offsets of every row piece in the shard and home buffers).
//
// Pages: "core.distributed.fsdp.src.megatron_fsdp.experimental.owner_planning"
// (select_ge_2d_params, ns_cost_fn, _OwnerWork, assign_owner_work,
// OwnerGatherPlan) and "core.optimizer.layer_sharded_a2a" (params_by_home,
// route_to_ns_home and its cached `plan` of index groupings and offsets).
// Pure host code: no GPU is touched here.

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <numeric>

#include "internal.h"

#ifndef NSQ_ROUTE_BAND
#define NSQ_ROUTE_BAND 262144
#endif

namespace {
// The pieces segs[first..] of one tensor, each `runs` strided runs (a slice
// along a dimension after the first), cut into bands of B runs (B home rows
// of about NSQ_ROUTE_BAND bytes) and ordered band by band: every shard's piece
// of a band of home rows, then the next band. Chunks are numbered in segment
// order, so the workgroups in flight together fill whole home rows instead of
// one shard's column block of many rows: column shards of the dense-transformer
// set measured 5.3 -> 5.6 TB/s. Row shards are one run each and stay whole.
void band_pieces(std::vector<nsq::RouteSeg> &segs, size_t first, int64_t runs) {
    if (NSQ_ROUTE_BAND <= 0 || first == segs.size() || runs <= 1) return;
    if (segs[first].run_len == segs[first].len) return;   // single runs: contiguous pieces
    const int64_t B = std::max<int64_t>(1, (int64_t)NSQ_ROUTE_BAND / segs[first].home_stride);
    if (B >= runs) return;
    std::vector<nsq::RouteSeg> mine(segs.begin() + (std::ptrdiff_t)first, segs.end());
    segs.resize(first);
    for (int64_t r0 = 0; r0 < runs; r0 += B)
        for (nsq::RouteSeg g : mine) {
            g.shard_off += r0 * g.run_len;
            g.home_off += r0 * g.home_stride;
            g.len = std::min(B, runs - r0) * g.run_len;
            segs.push_back(g);
        }
}
}  // namespace

namespace nsq {

static thread_local std::string g_last_error;

ns_status fail(ns_status code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

void clear_error() { g_last_error.clear(); }

ns_status matrix_view(const ns_shape &s, int64_t idx, int64_t *rows, int64_t *cols) {
    if (s.ndim < 0 || s.ndim > NS_MAX_DIMS)
        return fail(NS_ERR_INVALID_ARG, "tensor %lld: ndim %d outside [0, %d]", (long long)idx,
                    s.ndim, NS_MAX_DIMS);
    for (int d = 0; d < s.ndim; ++d)
        if (s.dims[d] < 0)
            return fail(NS_ERR_INVALID_ARG, "tensor %lld: negative dim %d", (long long)idx, d);
    if (s.ndim < 2) {
        *rows = *cols = -1;
        return NS_OK;
    }
    int64_t c = 1;
    for (int d = 1; d < s.ndim; ++d)
        if (__builtin_mul_overflow(c, s.dims[d], &c))
            return fail(NS_ERR_OVERFLOW, "tensor %lld: element count overflows", (long long)idx);
    int64_t numel;
    if (__builtin_mul_overflow(c, s.dims[0], &numel))
        return fail(NS_ERR_OVERFLOW, "tensor %lld: element count overflows", (long long)idx);
    *rows = s.dims[0];
    *cols = c;
    return NS_OK;
}

static uint64_t fnv1a(uint64_t h, const void *data, size_t len) {
    const unsigned char *p = static_cast<const unsigned char *>(data);
    for (size_t i = 0; i < len; ++i) {
        h ^= p[i];
        h *= 1099511628211ull;
    }
    return h;
}

}  // namespace nsq

using namespace nsq;

extern "C" const char *ns_last_error(void) { return g_last_error.c_str(); }

extern "C" const char *ns_version(void) { return "ns-mi355x 0.1 (gfx950)"; }

// ns_cost_fn: numel * (min(rows, cols) * steps + 1), exact in uint64.
static ns_status cost_of(int64_t rows, int64_t cols, int32_t steps, int64_t idx, uint64_t *out) {
    uint64_t numel, t, cost;
    uint64_t m = (uint64_t)std::min(rows, cols);
    if (__builtin_mul_overflow((uint64_t)rows, (uint64_t)cols, &numel) ||
        __builtin_mul_overflow(m, (uint64_t)steps, &t) || __builtin_add_overflow(t, 1ull, &t) ||
        __builtin_mul_overflow(numel, t, &cost))
        return fail(NS_ERR_OVERFLOW, "tensor %lld: cost overflows uint64", (long long)idx);
    *out = cost;
    return NS_OK;
}

extern "C" ns_status ns_plan(int32_t n, const ns_shape *shapes, int32_t steps, int32_t num_homes,
                             const int64_t *split_rows, uint64_t *cost_out, int32_t *home_out,
                             uint64_t *load_out, int32_t *order_out) {
    if (n < 0) return fail(NS_ERR_INVALID_ARG, "n = %d < 0", n);
    if (n > 0 && (!shapes || !home_out))
        return fail(NS_ERR_INVALID_ARG, "shapes and home_out are required");
    if (steps < 0) return fail(NS_ERR_INVALID_ARG, "steps = %d < 0", steps);
    if (num_homes < 1 || num_homes > NS_MAX_SHARDS)
        return fail(NS_ERR_INVALID_ARG, "num_homes = %d outside [1, %d]", num_homes, NS_MAX_SHARDS);

    std::vector<uint64_t> cost(n, 0);
    std::vector<char> part(n, 0);
    std::vector<std::vector<int32_t>> cand(n);
    for (int32_t i = 0; i < n; ++i) {
        int64_t rows, cols;
        ns_status st = matrix_view(shapes[i], i, &rows, &cols);
        if (st) return st;
        if (rows < 0) continue;  // select_ge_2d_params: fewer than 2 dims
        part[i] = 1;
        if ((st = cost_of(rows, cols, steps, i, &cost[i]))) return st;
        if (split_rows) {
            int64_t sum = 0;
            for (int32_t s = 0; s < num_homes; ++s) {
                int64_t r = split_rows[(int64_t)i * num_homes + s];
                if (r < 0) return fail(NS_ERR_INVALID_ARG, "tensor %d: negative split rows", i);
                if (__builtin_add_overflow(sum, r, &sum))
                    return fail(NS_ERR_OVERFLOW, "tensor %d: split rows overflow", i);
                if (r > 0) cand[i].push_back(s);  // a holder of part of the tensor
            }
            if (sum != rows)
                return fail(NS_ERR_SPLIT_SUM, "tensor %d: split rows sum to %lld, not %lld", i,
                            (long long)sum, (long long)rows);
            if (cand[i].empty())
                return fail(NS_ERR_NO_CANDIDATE, "tensor %d: no shard holds any of its rows", i);
        } else {
            cand[i].resize(num_homes);
            std::iota(cand[i].begin(), cand[i].end(), 0);
        }
    }

    // assign_owner_work: single-candidate tensors first (index order), then the
    // rest by descending cost (ties by index); least-loaded holder, ties to
    // the first holder in buffer order.
    std::vector<int32_t> order;
    order.reserve(n);
    for (int32_t i = 0; i < n; ++i)
        if (part[i] && cand[i].size() == 1) order.push_back(i);
    size_t n_single = order.size();
    for (int32_t i = 0; i < n; ++i)
        if (part[i] && cand[i].size() > 1) order.push_back(i);
    std::stable_sort(order.begin() + n_single, order.end(),
                     [&](int32_t x, int32_t y) { return cost[x] > cost[y]; });

    std::vector<uint64_t> load(num_homes, 0);
    std::vector<int32_t> home(n, -1);
    for (int32_t i : order) {
        int32_t best = -1;
        for (int32_t s : cand[i])
            if (best < 0 || load[s] < load[best]) best = s;
        home[i] = best;
        if (__builtin_add_overflow(load[best], cost[i], &load[best]))
            return fail(NS_ERR_OVERFLOW, "home %d: load overflows uint64", best);
    }

    std::copy(home.begin(), home.end(), home_out);
    if (cost_out) std::copy(cost.begin(), cost.end(), cost_out);
    if (load_out) std::copy(load.begin(), load.end(), load_out);
    if (order_out) {
        std::copy(order.begin(), order.end(), order_out);
        std::fill(order_out + order.size(), order_out + n, -1);
    }
    return NS_OK;
}

// Route plan for shards cut along a per-tensor dimension (0 = rows). Shard s
// holds, for every tensor in index order, its slice of width split[i][s] along
// shard_dim[i], flattened row-major; homes hold complete tensors in index order.
static ns_status route_plan_build(int32_t n, const ns_shape *shapes, int32_t num_shards,
                                  const int64_t *split, const int32_t *shard_dim, const int32_t *home,
                                  int32_t elem_bytes, ns_route_plan **out) {
    if (!out) return fail(NS_ERR_INVALID_ARG, "out is NULL");
    if (n < 0) return fail(NS_ERR_INVALID_ARG, "n = %d < 0", n);
    if (num_shards < 1 || num_shards > NS_MAX_SHARDS)
        return fail(NS_ERR_INVALID_ARG, "num_shards = %d outside [1, %d]", num_shards,
                    NS_MAX_SHARDS);
    if (elem_bytes != 2 && elem_bytes != 4)
        return fail(NS_ERR_DTYPE, "elem_bytes = %d (must be 2 or 4)", elem_bytes);
    if (n > 0 && (!shapes || !split || !home))
        return fail(NS_ERR_INVALID_ARG, "shapes, split sizes and home are required");

    const int32_t S = num_shards;
    auto plan = new ns_route_plan();
    plan->n = n;
    plan->num_shards = S;
    plan->elem_bytes = elem_bytes;
    if (n > 0) {
        plan->shapes.assign(shapes, shapes + n);
        plan->split_rows.assign(split, split + (size_t)n * S);
    }
    plan->shard_dim.assign(n, 0);
    plan->shard_elems.assign(S, 0);
    plan->home_elems.assign(S, 0);
    plan->home_offset.assign(n, 0);
    plan->shard_offset.assign((size_t)n * S, 0);
    // per tensor: runs (product of the dims before shard_dim), extent of
    // shard_dim, inner (product of the dims after it)
    std::vector<int64_t> outer(n), extent(n), inner(n);

    auto bad = [&](ns_status st) {
        delete plan;
        return st;
    };
    for (int32_t i = 0; i < n; ++i) {
        int64_t rows, cols;
        ns_status st = matrix_view(shapes[i], i, &rows, &cols);
        if (st) return bad(st);
        if (rows < 0)
            return bad(fail(NS_ERR_INVALID_ARG, "tensor %d: routed tensors need ndim >= 2", i));
        if (home[i] < 0 || home[i] >= S)
            return bad(fail(NS_ERR_HOME_RANGE, "tensor %d: home %d outside [0, %d)", i, home[i], S));
        const int32_t d = shard_dim ? shard_dim[i] : 0;
        if (d < 0 || d >= shapes[i].ndim)
            return bad(fail(NS_ERR_INVALID_ARG, "tensor %d: shard_dim %d outside [0, %d)", i, d, shapes[i].ndim));
        plan->shard_dim[i] = d;
        int64_t o = 1, in = 1;   // no overflow: their product with the extent is the element count
        for (int32_t k = 0; k < d; ++k) o *= shapes[i].dims[k];
        for (int32_t k = d + 1; k < shapes[i].ndim; ++k) in *= shapes[i].dims[k];
        outer[i] = o;
        extent[i] = shapes[i].dims[d];
        inner[i] = in;
        int64_t sum = 0;
        for (int32_t s = 0; s < S; ++s) {
            int64_t r = split[(int64_t)i * S + s];
            if (r < 0) return bad(fail(NS_ERR_INVALID_ARG, "tensor %d: negative split size", i));
            if (__builtin_add_overflow(sum, r, &sum))
                return bad(fail(NS_ERR_OVERFLOW, "tensor %d: split sizes overflow", i));
        }
        if (sum != extent[i])
            return bad(fail(NS_ERR_SPLIT_SUM, "tensor %d: split sizes sum to %lld, not %lld (dim %d)", i,
                            (long long)sum, (long long)extent[i], d));
    }
    // Offsets: shard buffers hold the tensors' slices in index order; home
    // buffers hold the complete tensors homed there in index order.
    for (int32_t i = 0; i < n; ++i) {
        const int64_t numel = outer[i] * extent[i] * inner[i];
        int64_t &ho = plan->home_elems[home[i]];
        plan->home_offset[i] = ho;
        if (__builtin_add_overflow(ho, numel, &ho))
            return bad(fail(NS_ERR_OVERFLOW, "home buffer size overflows"));
        int64_t start = 0;
        const size_t first_seg = plan->segs.size();
        for (int32_t s = 0; s < S; ++s) {
            const int64_t w = split[(int64_t)i * S + s];
            int64_t &so = plan->shard_elems[s];
            plan->shard_offset[(size_t)i * S + s] = so;
            const int64_t piece = outer[i] * w * inner[i];   // <= numel, no overflow
            if (__builtin_add_overflow(so, piece, &so))
                return bad(fail(NS_ERR_OVERFLOW, "shard buffer size overflows"));
            if (piece > 0) {
                RouteSeg g{};
                g.shard = s;
                g.home = home[i];
                g.shard_off = plan->shard_offset[(size_t)i * S + s] * elem_bytes;
                g.home_off = (plan->home_offset[i] + start * inner[i]) * elem_bytes;
                g.len = piece * elem_bytes;
                g.run_len = w * inner[i] * elem_bytes;
                g.home_stride = extent[i] * inner[i] * elem_bytes;
                plan->segs.push_back(g);
            }
            start += w;
        }
        band_pieces(plan->segs, first_seg, outer[i]);
    }
    for (int32_t s = 0; s < S; ++s) {
        int64_t b;
        if (__builtin_mul_overflow(plan->shard_elems[s], (int64_t)elem_bytes, &b) ||
            __builtin_mul_overflow(plan->home_elems[s], (int64_t)elem_bytes, &b))
            return bad(fail(NS_ERR_OVERFLOW, "buffer byte size overflows"));
    }
    int64_t chunks = 0, bytes = 0;
    bool aligned = true;
    for (RouteSeg &g : plan->segs) {
        g.chunk_begin = chunks;
        chunks += (g.len + kRouteChunkBytes - 1) / kRouteChunkBytes;
        bytes += g.len;
        aligned = aligned && (g.shard_off | g.home_off) % 16 == 0 &&
                  (g.run_len == g.len || (g.run_len | g.home_stride) % 16 == 0);
    }
    plan->aligned16 = aligned;
    plan->total_chunks = chunks;
    plan->total_bytes = bytes;

    uint64_t h = 1469598103934665603ull;
    h = fnv1a(h, &n, sizeof n);
    h = fnv1a(h, &S, sizeof S);
    h = fnv1a(h, &elem_bytes, sizeof elem_bytes);
    for (int32_t i = 0; i < n; ++i) {
        h = fnv1a(h, &shapes[i].ndim, sizeof(int32_t));
        h = fnv1a(h, shapes[i].dims, sizeof(int64_t) * shapes[i].ndim);
        h = fnv1a(h, &home[i], sizeof(int32_t));
        h = fnv1a(h, &plan->shard_dim[i], sizeof(int32_t));
    }
    if (n > 0) h = fnv1a(h, split, sizeof(int64_t) * (size_t)n * S);
    plan->fingerprint = h;
    *out = plan;
    return NS_OK;
}

extern "C" ns_status ns_route_plan_create(int32_t n, const ns_shape *shapes, int32_t num_shards,
                                          const int64_t *split_rows, const int32_t *home,
                                          int32_t elem_bytes, ns_route_plan **out) {
    return route_plan_build(n, shapes, num_shards, split_rows, nullptr, home, elem_bytes, out);
}

extern "C" ns_status ns_route_plan_create_axis(int32_t n, const ns_shape *shapes, int32_t num_shards,
                                               const int64_t *split_sizes, const int32_t *shard_dim,
                                               const int32_t *home, int32_t elem_bytes, ns_route_plan **out) {
    return route_plan_build(n, shapes, num_shards, split_sizes, shard_dim, home, elem_bytes, out);
}

extern "C" ns_status ns_route_plan_query(const ns_route_plan *plan, int64_t *shard_elems,
                                         int64_t *home_elems, int64_t *home_offset,
                                         int64_t *shard_offset, size_t *device_table_bytes,
                                         uint64_t *fingerprint) {
    if (!plan) return fail(NS_ERR_INVALID_ARG, "plan is NULL");
    if (shard_elems) std::copy(plan->shard_elems.begin(), plan->shard_elems.end(), shard_elems);
    if (home_elems) std::copy(plan->home_elems.begin(), plan->home_elems.end(), home_elems);
    if (home_offset) std::copy(plan->home_offset.begin(), plan->home_offset.end(), home_offset);
    if (shard_offset)
        std::copy(plan->shard_offset.begin(), plan->shard_offset.end(), shard_offset);
    if (device_table_bytes)
        *device_table_bytes = std::max<size_t>(16, plan->segs.size() * sizeof(RouteSeg));
    if (fingerprint) *fingerprint = plan->fingerprint;
    return NS_OK;
}

extern "C" void ns_route_plan_destroy(ns_route_plan *plan) { delete plan; }

extern "C" ns_status ns_wave_plan(int32_t n, const ns_shape *shapes, const int32_t *ready_order,
                                  int32_t slots, int32_t *wave_of, int32_t *num_waves) {
    if (n < 0) return fail(NS_ERR_INVALID_ARG, "n = %d < 0", n);
    if (slots < 1) return fail(NS_ERR_INVALID_ARG, "slots = %d < 1", slots);
    if (!num_waves || (n > 0 && (!shapes || !wave_of)))
        return fail(NS_ERR_INVALID_ARG, "shapes, wave_of and num_waves are required");
    std::vector<char> eligible(n, 0), seen(n, 0);
    for (int32_t i = 0; i < n; ++i) {
        int64_t rows, cols;
        ns_status st = matrix_view(shapes[i], i, &rows, &cols);
        if (st) return st;
        eligible[i] = rows >= 0;
    }
    std::vector<int32_t> order(n);
    for (int32_t k = 0; k < n; ++k) {
        const int32_t i = ready_order ? ready_order[k] : n - 1 - k;
        if (i < 0 || i >= n || seen[i])
            return fail(NS_ERR_INVALID_ARG, "ready_order is not a permutation of 0..%d", n - 1);
        seen[i] = 1;
        order[k] = i;
    }
    int64_t k = 0;
    std::vector<int32_t> w(n, -1);
    for (int32_t i : order)
        if (eligible[i]) w[i] = (int32_t)(k++ / slots);
    std::copy(w.begin(), w.end(), wave_of);
    *num_waves = (int32_t)((k + slots - 1) / slots);
    return NS_OK;
}
