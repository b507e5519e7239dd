/* A plain C99 caller of the library's host-only entry points, built against
 * include/ns.h with no C++ and no HIP headers. Expected values are worked by
 * hand from the contracts in ns.h (the cost formula of [owner_planning]
 * ns_cost_fn, the LPT rule of assign_owner_work, the shard offsets of
 * [layer_sharded] route_to_ns_home). Prints "ok" and exits 0 when all hold. */
#include <stdio.h>
#include <string.h>

#include "ns.h"

static int failures = 0;
#define CHECK(cond)                                                        \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "%s:%d: %s failed\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                    \
        }                                                                  \
    } while (0)

static ns_shape shape2(int64_t r, int64_t c) {
    ns_shape s;
    memset(&s, 0, sizeof s);
    s.ndim = 2;
    s.dims[0] = r;
    s.dims[1] = c;
    return s;
}

int main(void) {
    const char *v = ns_version();
    CHECK(v != NULL && v[0] != '\0');

    /* planning: (4, 5), (6, 7) and a 1-D (3,) over 2 homes, 5 steps.
     * cost = rows cols (min(rows, cols) 5 + 1): 20 * 21 = 420, 42 * 31 = 1302;
     * LPT: tensor 1 to home 0 (tie on empty homes: first), tensor 0 to home 1. */
    {
        ns_shape sh[3];
        uint64_t cost[3], load[2];
        int32_t home[3], order[3];
        sh[0] = shape2(4, 5);
        sh[1] = shape2(6, 7);
        memset(&sh[2], 0, sizeof sh[2]);
        sh[2].ndim = 1;
        sh[2].dims[0] = 3;
        CHECK(ns_plan(3, sh, 5, 2, NULL, cost, home, load, order) == NS_OK);
        CHECK(cost[0] == 420 && cost[1] == 1302 && cost[2] == 0);
        CHECK(home[0] == 1 && home[1] == 0 && home[2] == -1);
        CHECK(load[0] == 1302 && load[1] == 420);
        CHECK(order[0] == 1 && order[1] == 0 && order[2] == -1);
    }

    /* route plan: tensor 0 (4 x 5) split 1 + 3 rows, tensor 1 (6 x 7) all in
     * shard 0; homes 1 and 0. Shard 0 holds 1*5 + 6*7 = 47 elements, shard 1
     * 3*5 = 15; tensor 1 follows tensor 0's pieces: offsets 5 and 15. */
    {
        ns_shape sh[2];
        const int64_t split[4] = {1, 3, 6, 0};
        const int32_t home[2] = {1, 0};
        int64_t shard_elems[2], home_elems[2], home_off[2], shard_off[4];
        size_t table_bytes = 0;
        ns_route_plan *plan = NULL;
        sh[0] = shape2(4, 5);
        sh[1] = shape2(6, 7);
        CHECK(ns_route_plan_create(2, sh, 2, split, home, 2, &plan) == NS_OK && plan != NULL);
        if (plan) {
            CHECK(ns_route_plan_query(plan, shard_elems, home_elems, home_off, shard_off, &table_bytes, NULL) ==
                  NS_OK);
            CHECK(shard_elems[0] == 47 && shard_elems[1] == 15);
            CHECK(home_elems[0] == 42 && home_elems[1] == 20);
            CHECK(home_off[0] == 0 && home_off[1] == 0);
            CHECK(shard_off[0] == 0 && shard_off[1] == 0 && shard_off[2] == 5 && shard_off[3] == 15);
            CHECK(table_bytes > 0);
            ns_route_plan_destroy(plan);
        }
    }

    /* waves: five eligible tensors, reverse index order, 2 slots -> 3 waves */
    {
        ns_shape sh[5];
        int32_t wave[5], nw = 0, i;
        for (i = 0; i < 5; ++i) sh[i] = shape2(8, 8);
        CHECK(ns_wave_plan(5, sh, NULL, 2, wave, &nw) == NS_OK);
        CHECK(nw == 3 && wave[4] == 0 && wave[3] == 0 && wave[2] == 1 && wave[1] == 1 && wave[0] == 2);
    }

    /* workspace size of one 1024^2 bf16 matrix: positive, minimum <= full */
    {
        ns_shape sh = shape2(1024, 1024);
        size_t bytes = 0, min_bytes = 0;
        CHECK(ns_workspace_bytes(1, &sh, NS_BF16, &bytes, &min_bytes) == NS_OK);
        CHECK(bytes > 0 && min_bytes > 0 && min_bytes <= bytes);
    }

    /* errors: a shape with more than NS_MAX_DIMS dimensions, a SPLIT_SUM */
    {
        ns_shape sh = shape2(4, 5);
        int32_t home[1];
        const int64_t split[2] = {1, 2};
        sh.ndim = NS_MAX_DIMS + 1;
        CHECK(ns_plan(1, &sh, 5, 1, NULL, NULL, home, NULL, NULL) == NS_ERR_INVALID_ARG);
        CHECK(ns_last_error()[0] != '\0');
        sh.ndim = 2;
        CHECK(ns_plan(1, &sh, 5, 2, split, NULL, home, NULL, NULL) == NS_ERR_SPLIT_SUM);
    }

    if (failures) return 1;
    printf("ok\n");
    return 0;
}
