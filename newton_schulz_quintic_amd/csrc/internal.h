// Internal declarations shared by the library's translation units.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "ns.h"

namespace nsq {

// Records a message for ns_last_error() and returns `code`.
ns_status fail(ns_status code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// (rows, cols) view of a shape, with overflow and sign checks.
// Returns NS_OK, NS_ERR_INVALID_ARG or NS_ERR_OVERFLOW (message set).
ns_status matrix_view(const ns_shape &s, int64_t idx, int64_t *rows, int64_t *cols);

// One piece moved by pack/unpack: `len` bytes, contiguous in shard buffer
// `shard` from byte `shard_off`; in home buffer `home` they are runs of
// `run_len` bytes, run k at byte home_off + k * home_stride (a row shard is a
// single run; a slice along another dimension is one run per index of the
// dimensions before it). Chunks of kRouteChunkBytes (counted on the shard side)
// are numbered globally; this piece owns chunks
// [chunk_begin, chunk_begin + ceil(len / kRouteChunkBytes)).
struct RouteSeg {
    int64_t shard_off;
    int64_t home_off;
    int64_t len;
    int64_t chunk_begin;
    int64_t run_len;
    int64_t home_stride;
    int32_t shard;
    int32_t home;
    int64_t pad;
};
static_assert(sizeof(RouteSeg) == 64, "RouteSeg layout");

#ifndef NSQ_ROUTE_CHUNK
#define NSQ_ROUTE_CHUNK 16384
#endif
constexpr int64_t kRouteChunkBytes = NSQ_ROUTE_CHUNK;

}  // namespace nsq

struct ns_route_plan {
    int32_t n = 0;
    int32_t num_shards = 0;
    int32_t elem_bytes = 0;
    std::vector<ns_shape> shapes;      // [n] as given
    std::vector<int64_t> split_rows;   // [n * num_shards] as given (sizes along shard_dim)
    std::vector<int32_t> shard_dim;    // [n]
    std::vector<int64_t> shard_elems, home_elems, home_offset, shard_offset;
    std::vector<nsq::RouteSeg> segs;
    int64_t total_chunks = 0;
    int64_t total_bytes = 0;
    bool aligned16 = false;   // every piece starts (and every run and stride is) a multiple of 16 bytes
    uint64_t fingerprint = 0;
    void *device_table = nullptr;
};
