/*
 * ns.h -- C ABI of the MI355X (gfx950) Newton-Schulz library.
 *
 * One GPU. Plain pointers and sizes; no C++ or torch types. Every call returns
 * an ns_status (0 = NS_OK, negative = error). Every argument is checked, and
 * every group and wave of a call is planned, before anything is enqueued: on
 * any error other than NS_ERR_HIP nothing has been enqueued on the stream and
 * no output has been written. NS_ERR_HIP reports a failing HIP runtime call;
 * work enqueued before it (earlier launches of the same call) may still run.
 * ns_last_error() returns a message for the calling thread's last failure.
 *
 * Memory: the library never allocates device memory. Every device buffer (shard
 * buffers, home buffers, the route plan's device table, the Newton-Schulz
 * workspace, inputs and outputs) belongs to the caller. Device pointers must
 * stay valid until the work enqueued on the stream has finished.
 *
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the null stream).
 * Work is enqueued asynchronously in stream order; calls do not synchronise
 * the host unless stated.
 *
 * Environment (tuning and tests; read at each call; results are the same bits
 * whichever is set):
 *   NS_TILE=128|256      product tile edge for bf16 groups (default: 256 when
 *                        the group has enough 256-tiles to fill the GPU)
 *   NS_KMAJOR_MAX=K      largest padded m for which B.X reads X in place
 *                        (default 1024; larger m keep a transposed copy)
 *   NS_SMALL_MAX=M       largest m of the small size class (default 128, at
 *                        most 128; 0 sends every matrix down the tiled path)
 *   NS_ROUTE_MAX_GRID=W  cap on pack/unpack workgroups (default 2^23, one
 *                        16 KiB chunk each; a lower cap gives each several)
 *   NS_STAGE_RUN=R       input-staging tiles per workgroup, 1..16 (default:
 *                        1, or 4 for calls with 32768 staging tiles and more)
 *
 * Pages cited (by title, then section):
 *   [owner_planning] "core.distributed.fsdp.src.megatron_fsdp.experimental.
 *                     owner_planning" (Megatron-FSDP API docs)
 *   [layer_sharded]  "core.optimizer.layer_sharded_a2a" (Megatron Core API docs)
 *   [issue]          "[GTP][Muon] Optimize Muon step performance" (GitHub issue)
 */
#ifndef NS_MI355X_NS_H
#define NS_MI355X_NS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t ns_status;

#define NS_OK                 0
#define NS_ERR_INVALID_ARG   -1  /* null pointer, negative size, bad shape, bad order, ...   */
#define NS_ERR_NO_CANDIDATE  -2  /* a participating tensor has no rows in any shard          */
#define NS_ERR_HOME_RANGE    -3  /* a home index outside [0, num_shards)                     */
#define NS_ERR_SPLIT_SUM     -4  /* a tensor's split rows do not sum to its first dimension  */
#define NS_ERR_OVERFLOW      -5  /* a size, offset or cost does not fit in 63 / 64 bits      */
#define NS_ERR_PLAN_MISMATCH -6  /* a route plan used with buffers it was not built for      */
#define NS_ERR_WORKSPACE     -7  /* workspace too small (or its table not uploaded)          */
#define NS_ERR_DTYPE         -8  /* unsupported dtype or element size                        */
#define NS_ERR_HIP           -9  /* a HIP runtime call failed (message names it)             */

#define NS_MAX_DIMS   8
#define NS_MAX_SHARDS 64

/* Thread-local message describing the calling thread's last failed call.
 * Never NULL; empty if no call on this thread has failed. */
const char *ns_last_error(void);

/* A tensor's full shape. It is viewed as a matrix (rows, cols) =
 * (dims[0], dims[1] * ... * dims[ndim-1]), row-major and contiguous
 * [owner_planning, ns_cost_fn]. Tensors with ndim < 2 do not take part
 * [owner_planning, select_ge_2d_params]. */
typedef struct ns_shape {
    int32_t ndim;                 /* 0 .. NS_MAX_DIMS */
    int64_t dims[NS_MAX_DIMS];    /* dims[d] >= 0 for d < ndim; the rest ignored */
} ns_shape;

typedef enum ns_dtype { NS_BF16 = 0, NS_F32 = 1 } ns_dtype;

/* ------------------------------------------------------------------------ *
 * Planning (host only; no GPU needed)
 * ------------------------------------------------------------------------ */

/* Cost estimate and owner ("home") assignment for n tensors over num_homes
 * homes [owner_planning, ns_cost_fn and assign_owner_work].
 *
 * cost[i]  = rows * cols * (min(rows, cols) * steps + 1), exact in uint64
 *            (NS_ERR_OVERFLOW if it does not fit).
 * Candidates of tensor i: the homes s with split_rows[i*num_homes + s] > 0, in
 * ascending s (buffer order); every home if split_rows is NULL.
 * Assignment (LPT): tensors with a single candidate first, in index order; then
 * the others by descending cost (ties: ascending index); each goes to its
 * least-loaded candidate, ties to the first candidate in buffer order.
 *
 * n            number of tensors (>= 0); shapes: [n] (may be NULL iff n == 0).
 * steps        Newton-Schulz steps in the cost (>= 0).
 * num_homes    1 .. NS_MAX_SHARDS.
 * split_rows   [n * num_homes] rows of tensor i held by shard s, each row of the
 *              table summing to dims[0]; or NULL.
 * cost_out     [n] or NULL: cost per tensor (0 for tensors with ndim < 2).
 * home_out     [n] (required): home per tensor, -1 for tensors with ndim < 2.
 * load_out     [num_homes] or NULL: summed cost per home.
 * order_out    [n] or NULL: participating tensors in assignment order, then -1
 *              for the entries left over.
 * Errors: INVALID_ARG, SPLIT_SUM, NO_CANDIDATE, OVERFLOW. Outputs untouched on error. */
ns_status ns_plan(int32_t n, const ns_shape *shapes, int32_t steps, int32_t num_homes,
                  const int64_t *split_rows, uint64_t *cost_out, int32_t *home_out,
                  uint64_t *load_out, int32_t *order_out);

/* ------------------------------------------------------------------------ *
 * Routing: S simulated row-shard buffers <-> S home buffers on one GPU
 * [layer_sharded, route_to_ns_home / route_from_ns_home / params_by_home;
 *  owner_planning, OwnerGatherPlan / OwnerScatterPlan]
 * ------------------------------------------------------------------------ */

/* Immutable, host-side description of one routing: the offsets of every piece
 * in the shard and home buffers. It is a pure function of (shapes, split_rows,
 * home, num_shards, elem_bytes), built once and reused while those are unchanged
 * [layer_sharded, route_to_ns_home `plan` argument]. The caller owns it.
 *
 * Layouts (flat, row-major, contiguous, in elements):
 *  - shard buffer s: for every tensor i in increasing index order, the
 *    split_rows[i][s] rows of tensor i that shard s holds, end to end. Shard s
 *    holds the rows starting at sum_{s' < s} split_rows[i][s'] (shards split a
 *    tensor in buffer order).
 *  - home buffer h: the complete tensors i with home[i] == h, in increasing
 *    index order [layer_sharded, params_by_home]; empty homes hold nothing.
 * Tensors must have ndim >= 2 (view (rows, cols) as above); zero-size tensors
 * and zero-row splits are allowed. */
typedef struct ns_route_plan ns_route_plan;

/* n >= 0 tensors; num_shards 1 .. NS_MAX_SHARDS; split_rows [n * num_shards]
 * (each row sums to dims[0]); home [n] in [0, num_shards); elem_bytes 2 or 4.
 * *out receives a new plan (release with ns_route_plan_destroy).
 * Errors: INVALID_ARG, SPLIT_SUM, HOME_RANGE, OVERFLOW, DTYPE. */
ns_status ns_route_plan_create(int32_t n, const ns_shape *shapes, int32_t num_shards,
                               const int64_t *split_rows, const int32_t *home,
                               int32_t elem_bytes, ns_route_plan **out);

/* Route plan for shards cut along any dimension [layer_sharded,
 * route_to_ns_home / route_from_ns_home: `shard_dim`, 0 for the GTP_remat
 * stage, the param's partition_dim for the TP stage]. Tensor i is split along
 * shard_dim[i] (0 <= shard_dim[i] < ndim; NULL = all 0, which is
 * ns_route_plan_create) into split_sizes[i * num_shards + s] slices, summing
 * to dims[shard_dim[i]]. Shard buffer s holds, for every tensor in increasing
 * index order, its slice along that dimension (the slices follow each other
 * in buffer order), flattened row-major; home buffers are as above. Pack and
 * unpack move a slice along dimension d > 0 as strided runs in the home
 * buffer. The two-stage exchange (rows within the GTP_remat group, then
 * partition_dim within the TP group) is two plans applied in turn.
 * ns_orthogonalize_routed accepts only plans whose tensors are split along
 * dimension 0 or held by a single shard. Errors as ns_route_plan_create, plus
 * INVALID_ARG for a shard_dim out of range. */
ns_status ns_route_plan_create_axis(int32_t n, const ns_shape *shapes, int32_t num_shards,
                                    const int64_t *split_sizes, const int32_t *shard_dim,
                                    const int32_t *home, int32_t elem_bytes, ns_route_plan **out);

/* Any output pointer may be NULL.
 * shard_elems [S], home_elems [S]: buffer sizes in elements.
 * home_offset [n]: element offset of tensor i in its home buffer.
 * shard_offset [n * S]: element offset of tensor i's piece in shard buffer s.
 * device_table_bytes: size of the device table ns_route_plan_upload writes.
 * fingerprint: 64-bit hash of everything the plan was built from. */
ns_status ns_route_plan_query(const ns_route_plan *plan, int64_t *shard_elems,
                              int64_t *home_elems, int64_t *home_offset,
                              int64_t *shard_offset, size_t *device_table_bytes,
                              uint64_t *fingerprint);

/* Copy the plan's segment table to caller-owned device memory of at least
 * device_table_bytes (16-byte aligned), on `stream`, and wait for the copy.
 * Must be called once before pack/unpack; the plan remembers the address. */
ns_status ns_route_plan_upload(ns_route_plan *plan, void *device_table, void *stream);

/* Release a plan (NULL is a no-op). Work already enqueued keeps running. */
void ns_route_plan_destroy(ns_route_plan *plan);

/* Forward routing (gather): for every tensor i, concatenate its row pieces from
 * shard buffers 0..S-1 (buffer order) into its slot in home buffer home[i]
 * [owner_planning, OwnerGatherPlan.reconstruct_full; layer_sharded,
 * route_to_ns_home]. Bit copy. shard_bufs [S] and home_bufs [S] are arrays of
 * device pointers of num_shards entries; an entry may be NULL only if that
 * buffer has zero elements. Buffers must not overlap. One kernel launch.
 * Errors: INVALID_ARG, PLAN_MISMATCH (plan not uploaded), HIP. */
ns_status ns_pack_shards(const ns_route_plan *plan, const void *const *shard_bufs,
                         void *const *home_bufs, void *stream);

/* Backward routing (scatter): the inverse of ns_pack_shards on the same plan;
 * every shard buffer receives its rows of every tensor back from the home
 * buffers [owner_planning, OwnerScatterPlan.unpack; layer_sharded,
 * route_from_ns_home]. Same conventions as ns_pack_shards. */
ns_status ns_unpack_shards(const ns_route_plan *plan, const void *const *home_bufs,
                           void *const *shard_bufs, void *stream);

/* ------------------------------------------------------------------------ *
 * Newton-Schulz orthogonalisation [owner_planning, ns_cost_fn;
 * issue, "Current Progress": shape-batched NS, SYRK symmetric kernels]
 * ------------------------------------------------------------------------ */

/* Device workspace (bytes) that lets ns_orthogonalize_batched run all n
 * tensors at once. A smaller workspace is accepted down to the amount needed
 * for the largest single tensor; tensors are then processed in consecutive
 * groups that fit (results are identical). *min_bytes (may be NULL) receives
 * that minimum. Errors: INVALID_ARG, DTYPE, OVERFLOW. */
ns_status ns_workspace_bytes(int32_t n, const ns_shape *shapes, ns_dtype dtype,
                             size_t *bytes, size_t *min_bytes);

/* For every tensor i with ndim >= 2 and numel > 0: view it as (rows, cols);
 * if rows > cols work on its transpose so that m = min <= n = max; normalise
 * X0 = G / (||G||_F + eps); run `steps` steps of
 *     A = X X^T,  B = b A + c A A,  X = a X + B X
 * and write X (transposed back if it was transposed) to out[i] in the input's
 * shape and dtype [owner_planning, ns_cost_fn].
 *
 * Precision: bf16 tensors keep X, A and B' in bf16 between products; every
 * product runs on bf16 MFMA with fp32 accumulation, and the norm and the
 * epilogues are computed in fp32 and rounded once (round to nearest even).
 * The step is evaluated as X' = B' X with B' = a I + B, an exact rewrite of
 * a X + B X: B' = c ((b / c) A + A A) + a I (b A + a I when c == 0) is summed
 * in fp32 from the old A tile onward and rounded once, so a + B_ii cancels
 * before rounding. The normalisation X0 = G / (||G||_F + eps) is applied in
 * fp32 inside the first step's products (A0 = s^2 G G^T, B0' stored scaled
 * by s), so X0 itself is never rounded. f32 tensors keep everything in fp32
 * (f32 MFMA).
 *
 * Input range: ||G||_F^2, and the entries of G G^T, must be within fp32 range
 * (||G||_F below about 1.8e19; gradients and momenta are far below it). A
 * tensor past it, or one holding inf or NaN, comes out as all NaN (never as
 * silent zeros).
 *
 * Size classes: tensors with m <= 128 are padded to 128 and run every step in
 * one workgroup per tensor; the others are padded to 256 and tiled across the
 * GPU. Both give the same bits.
 *
 * in[i], out[i]   device pointers, contiguous row-major, 2-byte (bf16) or
 *                 4-byte (f32) aligned; out[i] may equal in[i]; distinct outputs
 *                 must not overlap. Entries of tensors with numel == 0 or
 *                 ndim < 2 are ignored (and may be NULL).
 * steps >= 0; a, b, c: coefficients (quintic 3.4445, -4.7750, 2.0315); eps >= 0.
 * order   [n] permutation of 0..n-1 giving the dispatch order (e.g. ns_plan's
 *         order), or NULL for descending cost. Results do not depend on it.
 * workspace/workspace_bytes  device memory, 256-byte aligned, at least the
 *         minimum from ns_workspace_bytes. The call uses it as scratch until its
 *         work on `stream` has finished; two calls in flight at once (e.g. on
 *         different streams) must not share a workspace. The per-call device
 *         tables are written to pinned host staging owned by the library; the
 *         call's first kernel reads them from there and copies them into the
 *         workspace.
 * Errors: INVALID_ARG, DTYPE, WORKSPACE, OVERFLOW, HIP. */
ns_status ns_orthogonalize_batched(int32_t n, const ns_shape *shapes,
                                   const void *const *in, void *const *out, ns_dtype dtype,
                                   int32_t steps, float a, float b, float c, float eps,
                                   const int32_t *order, void *workspace,
                                   size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * ns_orthogonalize_batched with no workspace argument. Its scratch is a
 * 64 MiB array in device memory that the library defines and that every GPU
 * it runs on holds for the life of the process (one array per GPU, shared by
 * every call on that GPU).
 *
 * ns_noalloc_init: call once per device, with that device current, before
 * the first ns_orthogonalize_batched_noalloc on it and outside any region
 * that may not allocate: it looks up the array's device address and reserves
 * the pinned host staging the calls' tables go through (8 slots of 1 MiB
 * for calls in stream order, 8 more for calls under stream capture). Calling
 * it again is harmless. Errors: HIP, INVALID_ARG (device index >= 64, or the
 * staging busy in another thread's call).
 *
 * Stream capture: a call made while its stream is being captured into a HIP
 * graph (this entry point or any other NS entry point) copies its tables
 * into one of the 8 capture slots and keeps that slot for the life of the
 * process, since every replay of the graph reads them. A ninth captured call
 * fails with NS_ERR_WORKSPACE, and a captured call before any ns_noalloc_init
 * with NS_ERR_INVALID_ARG, before anything is captured. Replays run like the
 * call itself: on the scratch array (or the workspace given), in the order
 * of the stream they are launched on.
 *
 * ns_orthogonalize_batched_noalloc: arguments, results and errors as for
 * ns_orthogonalize_batched (same bits), on the current device's array; it
 * calls no allocating routine. NS_ERR_WORKSPACE if the largest tensor alone
 * needs more than 64 MiB of scratch (ns_workspace_bytes' minimum), or if the
 * call's tables exceed 1 MiB; NS_ERR_INVALID_ARG if ns_noalloc_init was not
 * called on the device. Larger sets run in groups that fit, with the same
 * bits. Nothing in the array needs clearing between calls: every byte a call
 * reads, it writes first. Calls that overlap on one GPU (e.g. on two streams)
 * share the array and race; keep them in one stream order. */
ns_status ns_noalloc_init(void);
ns_status ns_orthogonalize_batched_noalloc(int32_t n, const ns_shape *shapes, const void *const *in,
                                           void *const *out, ns_dtype dtype, int32_t steps, float a, float b,
                                           float c, float eps, const int32_t *order, void *stream);

/* ns_orthogonalize_batched on strided views: tensor i's input row r starts
 * at in[i] + r * in_ld[i] elements and its output row at out[i] + r *
 * out_ld[i] (rows as given, i.e. dims[0]; a row holds dims[1] * ... *
 * dims[ndim-1] contiguous elements). Row strides must be >= that row length;
 * in_ld / out_ld may be NULL for contiguous rows. For NS on sub-blocks of a
 * larger matrix in place, e.g. the Q, K and V blocks of a fused weight split
 * by rows or by columns ([issue], "Current Progress": split-QKV support).
 * Views may share memory only as in == out with equal strides (in place);
 * distinct outputs must not overlap. Results are bit-identical to
 * ns_orthogonalize_batched on contiguous copies. Other arguments and errors
 * as for ns_orthogonalize_batched (workspace from ns_workspace_bytes). */
ns_status ns_orthogonalize_strided(int32_t n, const ns_shape *shapes, const void *const *in,
                                   const int64_t *in_ld, void *const *out, const int64_t *out_ld,
                                   ns_dtype dtype, int32_t steps, float a, float b, float c, float eps,
                                   const int32_t *order, void *workspace, size_t workspace_bytes,
                                   void *stream);

/* ------------------------------------------------------------------------ *
 * Gram-space Newton-Schulz [issue, "Secondary (parked)": gram_once, the exact
 * Gram-space reformulation hardened with an fp32 Gram and a trace ridge]
 * ------------------------------------------------------------------------ */

/* Workspace for ns_orthogonalize_gram (fp32 X0 and nine m x m arrays
 * per tensor), as for ns_workspace_bytes. Errors: INVALID_ARG, DTYPE, OVERFLOW. */
ns_status ns_gram_workspace_bytes(int32_t n, const ns_shape *shapes, ns_dtype dtype, size_t *bytes,
                                  size_t *min_bytes);

/* The same iteration as ns_orthogonalize_batched, evaluated in the m x m Gram
 * space, all in fp32 (f32 MFMA; bf16 inputs are widened exactly): with X0 the
 * normalised, wide-oriented input, G = X0 X0^T + ridge (tr(G) / m) I is formed
 * once; then Q_0 = I and, per step, A = Q G Q^T, Q = a Q + (b A + c A A) Q,
 * evaluated as Q' = (a I + b A + c A A) Q; the output is Q_k X0 in the input's
 * shape and dtype. ridge = 0 is exactly the NS iteration (in exact
 * arithmetic); ridge > 0 regularises a near-singular Gram and changes the
 * result. Every Q_k is a polynomial in G, so in exact arithmetic the m x m
 * products are symmetric; in fp32 they are not, and are computed as full
 * products (forcing symmetry loses about a decimal digit on ill-conditioned
 * inputs); only G is formed as an upper-tile product. The products are
 * 4 (2 m^3) per step instead of about 4 m^2 n: cheaper when n >> m, but in
 * fp32 (157 TFLOP/s dense on MI355X, against 2.5 PFLOP/s bf16).
 * ridge: finite, >= 0. Other arguments and errors as for
 * ns_orthogonalize_batched (workspace from ns_gram_workspace_bytes). */
ns_status ns_orthogonalize_gram(int32_t n, const ns_shape *shapes, const void *const *in, void *const *out,
                                ns_dtype dtype, int32_t steps, float a, float b, float c, float eps,
                                float ridge, const int32_t *order, void *workspace, size_t workspace_bytes,
                                void *stream);

/* ------------------------------------------------------------------------ *
 * Fused routing: Newton-Schulz straight from and back to the shard buffers
 * [layer_sharded, route_to_ns_home / route_from_ns_home around the
 *  orthogonalisation; owner_planning, OwnerGatherPlan.reconstruct_full and
 *  OwnerScatterPlan.unpack]
 * ------------------------------------------------------------------------ */

/* Workspace (bytes) for ns_orthogonalize_routed on `plan`, and the minimum
 * (*min_bytes, may be NULL), as for ns_workspace_bytes. dtype must have the
 * plan's elem_bytes. Errors: INVALID_ARG, DTYPE, PLAN_MISMATCH, OVERFLOW. */
ns_status ns_routed_workspace_bytes(const ns_route_plan *plan, ns_dtype dtype, size_t *bytes,
                                    size_t *min_bytes);

/* The result of ns_pack_shards, then ns_orthogonalize_batched on all of the
 * plan's tensors (in the home buffers), then ns_unpack_shards into shard_out,
 * without home buffers: the first kernel reads each tensor's rows from its
 * pieces in the shard buffers and the last one writes the result rows to the
 * same offsets of the output shard buffers. Bit-identical to that sequence
 * (same kernels, same arithmetic). The homes play no part: on one GPU every
 * tensor of the plan is orthogonalised by the one call.
 *
 * plan        from ns_route_plan_create (no upload needed); its elem_bytes
 *             must match dtype.
 * shard_in    [num_shards] device pointers, layouts as in the route plan; an
 *             entry may be NULL only if that shard has zero elements.
 * shard_out   [num_shards] likewise; shard_out[s] may equal shard_in[s]
 *             (in place); otherwise buffers must not overlap.
 * steps, a, b, c, eps, order, workspace, workspace_bytes, stream: as for
 *             ns_orthogonalize_batched (order indexes the plan's tensors;
 *             the workspace minimum comes from ns_routed_workspace_bytes).
 * Errors: INVALID_ARG, DTYPE, PLAN_MISMATCH, WORKSPACE, OVERFLOW, HIP. */
ns_status ns_orthogonalize_routed(const ns_route_plan *plan, const void *const *shard_in,
                                  void *const *shard_out, ns_dtype dtype, int32_t steps, float a,
                                  float b, float c, float eps, const int32_t *order,
                                  void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------ *
 * Wave dispatch: Newton-Schulz started wave by wave as gradients become ready
 * [issue, "Current Progress": backward/forward overlap with dynamic wave
 *  dispatch]
 * ------------------------------------------------------------------------ */

/* Static wave partition (host only). Eligible tensors (ndim >= 2) are taken in
 * the order their gradients become ready -- ready_order [n], a permutation, or
 * NULL for reverse index order (the order a backward pass produces them) --
 * and each run of `slots` consecutive ones forms a wave (e.g. 3000 tensors on
 * 1000 slots: 3 waves). wave_of [n] receives each tensor's wave (-1 for
 * tensors with ndim < 2); *num_waves the number of waves.
 * Errors: INVALID_ARG (slots < 1, bad order, NULL outputs), OVERFLOW. */
ns_status ns_wave_plan(int32_t n, const ns_shape *shapes, const int32_t *ready_order, int32_t slots,
                       int32_t *wave_of, int32_t *num_waves);

/* ns_orthogonalize_batched run wave by wave on `stream`: for w = 0 ..
 * num_waves-1 the stream first waits for ready_events[w] (a hipEvent_t passed
 * as void*, recorded on any stream when wave w's inputs are complete; the
 * array or an entry may be NULL for no wait), then orthogonalises the tensors
 * with wave_of[i] == w. Tensors with wave_of[i] < 0 are left alone. Results
 * are bit-identical to ns_orthogonalize_batched on the same tensors (no
 * result depends on which tensors share a call). The workspace minimum is that
 * of ns_workspace_bytes on all n shapes; the waves reuse it in stream order.
 * Every wave is planned before the first event wait is enqueued, so an
 * argument error enqueues nothing; an invalid event handle fails in
 * hipStreamWaitEvent (NS_ERR_HIP) after the earlier waves were enqueued.
 * Other arguments and errors as for ns_orthogonalize_batched. */
ns_status ns_orthogonalize_waves(int32_t n, const ns_shape *shapes, const void *const *in,
                                 void *const *out, ns_dtype dtype, int32_t steps, float a, float b,
                                 float c, float eps, const int32_t *wave_of, int32_t num_waves,
                                 void *const *ready_events, void *workspace, size_t workspace_bytes,
                                 void *stream);

/* ------------------------------------------------------------------------ *
 * Measurement support
 * ------------------------------------------------------------------------ */

/* Kernel timing: for the kinds enabled (bit k of `kinds` enables kind k;
 * -1 enables all, 0 disables), every launch of that kind goes out through
 * hipExtLaunchKernelGGL with a HIP event pair that its dispatch records, so a
 * pair spans that kernel's execution only (what rocprofv3's kernel trace
 * reports), not its dispatch. Enable only the kinds being measured. Enabling
 * creates a pool of 4096 events up front (so no measured loop pays for event
 * creation); it needs the GPU and returns NS_ERR_HIP if event creation fails.
 * ns_timing_read waits for the events of one kind, returns their sums and
 * clears them. Not thread-safe against concurrent batched calls.
 * kind: 0 = the B X product kernel (every step but the last),
 *       1 = pack/unpack kernel, 2 = input staging (with steps = 0, also the
 *       scaling kernel after it),
 *       3 = the final B X launch of each call (it writes the caller's output),
 *       4 = the A = X X^T product kernel, 5 = the B = b A + c A A product kernel,
 *       6 = the small-class kernel (every step of the matrices with m <= 128).
 * total_ms: summed durations; launches: number of launches; work: summed
 * algorithmic work of those launches (flops for kinds 0, 3, 4, 5, 6; bytes
 * moved for kind 1; bytes read + written for kind 2). */
ns_status ns_timing_enable(int32_t kinds);
ns_status ns_timing_read(int32_t kind, double *total_ms, int64_t *launches, double *work);

/* Library version string. */
const char *ns_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NS_MI355X_NS_H */
