/* A plain C99 caller of the GPU entry points through ns.h and HIP's C runtime
 * API, no C++ and no torch. Two checks:
 *  - ns_orthogonalize_batched on a 64 x 256 bf16 matrix whose rows are
 *    orthogonal with equal norms (a Sylvester-Hadamard block tiled along the
 *    columns, times per-column signs): every singular value of X0 is 1/sqrt(m),
 *    so the result is kappa * G with kappa = p^5(1/sqrt(m)) / sqrt(n),
 *    p(s) = a s + b s^3 + c s^5 (closed form, evaluated here in double); every
 *    element, times sqrt(n), must be within 2e-2 of kappa sqrt(n) G.
 *  - pack then unpack through a route plan (uneven row splits, a home with
 *    nothing) returns the shard buffers bit for bit.
 * Prints "ok" and exits 0 when both hold. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ns.h"

#define HIPCHECK(x)                                                                   \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
            return 2;                                                                 \
        }                                                                             \
    } while (0)
#define NSCHECK(x)                                                                      \
    do {                                                                                \
        ns_status s_ = (x);                                                             \
        if (s_ != NS_OK) {                                                              \
            fprintf(stderr, "%s:%d: %s: %d %s\n", __FILE__, __LINE__, #x, s_, ns_last_error()); \
            return 3;                                                                   \
        }                                                                               \
    } while (0)

static float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

int main(void) {
    enum { M = 64, N = 256 };
    const double a = 3.4445, b = -4.7750, c = 2.0315;
    static uint16_t g[M * N], y[M * N];
    int h[M][M];
    int i, j, k, r;
    HIPCHECK(hipSetDevice(0));

    /* Sylvester-Hadamard M x M, tiled N / M times, column j times sign(j) */
    h[0][0] = 1;
    for (k = 1; k < M; k *= 2)
        for (i = 0; i < k; ++i)
            for (j = 0; j < k; ++j) {
                h[i][j + k] = h[i][j];
                h[i + k][j] = h[i][j];
                h[i + k][j + k] = -h[i][j];
            }
    for (i = 0; i < M; ++i)
        for (j = 0; j < N; ++j) {
            const int sign = ((j * 2654435761u) >> 7) & 1 ? -1 : 1;
            g[i * N + j] = h[i][j % M] * sign > 0 ? 0x3F80 : 0xBF80; /* +1 / -1 in bf16 */
        }

    {
        ns_shape sh;
        void *din = NULL, *dout = NULL, *ws = NULL;
        size_t bytes = 0, min_bytes = 0;
        const void *ins[1];
        void *outs[1];
        double s = 1.0 / sqrt((double)M), worst = 0.0;
        memset(&sh, 0, sizeof sh);
        sh.ndim = 2;
        sh.dims[0] = M;
        sh.dims[1] = N;
        HIPCHECK(hipMalloc(&din, sizeof g));
        HIPCHECK(hipMalloc(&dout, sizeof g));
        HIPCHECK(hipMemcpy(din, g, sizeof g, hipMemcpyHostToDevice));
        NSCHECK(ns_workspace_bytes(1, &sh, NS_BF16, &bytes, &min_bytes));
        HIPCHECK(hipMalloc(&ws, bytes));
        ins[0] = din;
        outs[0] = dout;
        NSCHECK(ns_orthogonalize_batched(1, &sh, ins, outs, NS_BF16, 5, (float)a, (float)b, (float)c, 1e-7f, NULL,
                                         ws, bytes, NULL));
        HIPCHECK(hipDeviceSynchronize());
        HIPCHECK(hipMemcpy(y, dout, sizeof y, hipMemcpyDeviceToHost));
        for (k = 0; k < 5; ++k) s = a * s + b * s * s * s + c * s * s * s * s * s;
        for (i = 0; i < M * N; ++i) {
            const double want = s * (double)bf16_to_f32(g[i]);
            const double err = fabs((double)bf16_to_f32(y[i]) * sqrt((double)N) - want);
            if (err > worst) worst = err;
        }
        if (!(worst <= 2e-2)) {
            fprintf(stderr, "NS: max abs err %g (sqrt(n) scale)\n", worst);
            return 1;
        }
        HIPCHECK(hipFree(ws));
        HIPCHECK(hipFree(dout));
        HIPCHECK(hipFree(din));
    }

    {   /* route round trip: tensors (5 x 3) and (4 x 2) over 3 shards, homes 2 and 0 */
        ns_shape sh[2];
        const int64_t split[6] = {2, 3, 0, 0, 4, 0};
        const int32_t home[2] = {2, 0};
        int64_t shard_elems[3], home_elems[3];
        size_t table_bytes = 0;
        ns_route_plan *plan = NULL;
        void *table = NULL, *sb[3], *hb[3], *back[3];
        uint16_t host[64], got[64];
        for (r = 0; r < 64; ++r) host[r] = (uint16_t)(0x1000 + 37 * r);
        memset(sh, 0, sizeof sh);
        sh[0].ndim = 2; sh[0].dims[0] = 5; sh[0].dims[1] = 3;
        sh[1].ndim = 2; sh[1].dims[0] = 4; sh[1].dims[1] = 2;
        NSCHECK(ns_route_plan_create(2, sh, 3, split, home, 2, &plan));
        NSCHECK(ns_route_plan_query(plan, shard_elems, home_elems, NULL, NULL, &table_bytes, NULL));
        HIPCHECK(hipMalloc(&table, table_bytes));
        NSCHECK(ns_route_plan_upload(plan, table, NULL));
        for (k = 0; k < 3; ++k) {
            sb[k] = hb[k] = back[k] = NULL;
            if (shard_elems[k]) {
                HIPCHECK(hipMalloc(&sb[k], (size_t)shard_elems[k] * 2));
                HIPCHECK(hipMalloc(&back[k], (size_t)shard_elems[k] * 2));
                HIPCHECK(hipMemcpy(sb[k], host, (size_t)shard_elems[k] * 2, hipMemcpyHostToDevice));
            }
            if (home_elems[k]) HIPCHECK(hipMalloc(&hb[k], (size_t)home_elems[k] * 2));
        }
        NSCHECK(ns_pack_shards(plan, (const void *const *)sb, hb, NULL));
        NSCHECK(ns_unpack_shards(plan, (const void *const *)hb, back, NULL));
        HIPCHECK(hipDeviceSynchronize());
        for (k = 0; k < 3; ++k)
            if (shard_elems[k]) {
                HIPCHECK(hipMemcpy(got, back[k], (size_t)shard_elems[k] * 2, hipMemcpyDeviceToHost));
                if (memcmp(got, host, (size_t)shard_elems[k] * 2) != 0) {
                    fprintf(stderr, "route round trip differs in shard %d\n", k);
                    return 1;
                }
                HIPCHECK(hipFree(sb[k]));
                HIPCHECK(hipFree(back[k]));
            }
        for (k = 0; k < 3; ++k)
            if (hb[k]) HIPCHECK(hipFree(hb[k]));
        HIPCHECK(hipFree(table));
        ns_route_plan_destroy(plan);
    }
    printf("ok\n");
    return 0;
}
