// Batched Newton-Schulz orthogonalisation on gfx950.
//
// "core.distributed.fsdp.src.megatron_fsdp.experimental.owner_planning",
// ns_cost_fn: view each tensor as (rows, cols) = (shape[0], prod shape[1:]),
// normalise, work on the transpose when rows > cols, then per step
//     A = X X^T,   X = a X + (b A + c A A) X.
// "[GTP][Muon] Optimize Muon step performance", Current Progress: shape-batched
// NS and SYRK (symmetric) kernels.
//
// Design (one GPU, every matrix of a group in flight at once):
//  * Workspace per matrix, padded to multiples of 128 in both dims and kept
//    zero in the padding: X and X^T (two copies each, ping-pong), A and B.
//    Padding removes every bounds check from the product main loop; zero
//    padding stays zero through every step (products with zero rows/cols).
//  * All three products have the form C = P Q^T with P and Q row-major and
//    contiguous along the contraction (K) axis:
//        A   = X X^T  : P = Q = X
//        A A          : P = Q = A          (A is symmetric, so A A = A A^T)
//        B X          : P = B, Q = X^T     (X^T kept as its own array)
//    so one MFMA main loop serves all of them: 128x128 output tiles, 4 waves of
//    64x64, K panels of 128 bytes staged through double-buffered, padded LDS.
//  * The symmetric products compute only tiles on or above the diagonal and
//    store each off-diagonal tile twice (itself and its mirror), so A and B are
//    exactly symmetric.
//  * Epilogues in fp32, rounded once: A; B = b A + c (A A); X' = a X + B X
//    (written as X' and X'^T, or on the last step straight to the output in the
//    input's orientation, shape and dtype).
//  * Norm: per-chunk fp32 sums of squares in a fixed order (no atomics), then a
//    tile pass that reduces the partials, scales, and writes X0 and X0^T
//    (transposing tall inputs through LDS).
//  * Workgroup ids are remapped so consecutive tiles land on the same XCD (the
//    hardware hands workgroups to the 8 XCDs round-robin), sharing its L2.

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "hip_util.h"

namespace nsq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 128;          // product output tile (rows and cols); padding unit
constexpr int kThreads = 256;       // 4 waves
constexpr int kPanelBytes = 128;    // K bytes per LDS row per stage
constexpr int kLdsStride = 144;     // padded LDS row stride in bytes (conflict-free fragment reads)
constexpr int kOperandLds = kTile * kLdsStride;
constexpr int kStageLds = 2 * kOperandLds;
constexpr int kLdsBytes = 2 * kStageLds;  // double-buffered P and Q panels: 73728 B
constexpr int kNormChunk = 16384;   // elements per norm partial
constexpr int kNormTile = 64;       // norm apply tile edge
constexpr int kNumXcd = 8;

// Per-matrix descriptor in device memory.
struct NsProb {
    char *x[2];        // X ping/pong: mp x np (ld np)
    char *xt[2];       // X^T ping/pong: np x mp (ld mp)
    char *a;           // mp x mp
    char *b;           // mp x mp
    const char *in;    // input, rows x cols
    char *out;         // output, rows x cols
    float *partials;   // nparts fp32 partial sums of squares
    int32_t m, n;      // oriented sizes (m <= n)
    int32_t mp, np;    // padded to kTile
    int32_t tall;      // input had rows > cols
    int32_t nparts;
};

struct TileRef {
    int32_t prob;
    uint16_t ti, tj;
};
static_assert(sizeof(TileRef) == 8, "TileRef layout");

template <typename T> struct Mfma;

template <> struct Mfma<__bf16> {
    typedef bf16x8 frag;  // 8 consecutive k per lane
    static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mfma<float> {
    typedef f32x4 frag;   // 4 consecutive k per lane, one 32x32x2 MFMA per element
    static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0], b[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[1], b[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[2], b[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[3], b[3], c, 0, 0, 0);
        return c;
    }
};

template <typename T> __device__ __forceinline__ float to_f32(T v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v) { return (T)v; }

// Bijection from hardware workgroup id to logical tile id such that the
// workgroups of one XCD (hardware ids congruent mod 8) get a contiguous range.
__device__ __forceinline__ int xcd_remap(int b, int g) {
    const int xcd = b % kNumXcd, local = b / kNumXcd;
    const int per = g / kNumXcd, rem = g % kNumXcd;
    return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

enum Mode { kSyrkX = 0, kSyrkA = 1, kGemmBX = 2 };

// C = P Q^T over K (elements) for one 128x128 tile; P rows [row0, row0+128),
// Q rows [col0, col0+128). ld in bytes. Every access is in bounds by padding.
template <typename T>
__device__ __forceinline__ void tile_product(const char *__restrict__ P, const char *__restrict__ Q,
                                             int64_t ldp, int64_t ldq, int K, char *lds,
                                             f32x16 (&acc)[2][2]) {
    typedef typename Mfma<T>::frag frag;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lrow = t >> 3, lc16 = (t & 7) * 16;
    const int nk = (int)((int64_t)K * sizeof(T) / kPanelBytes);

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    uint4 pr[4], qr[4];
    auto gload = [&](int kb) {
        const int64_t kbyte = (int64_t)kb * kPanelBytes + lc16;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int row = it * 32 + lrow;
            pr[it] = *reinterpret_cast<const uint4 *>(P + row * ldp + kbyte);
            qr[it] = *reinterpret_cast<const uint4 *>(Q + row * ldq + kbyte);
        }
    };
    auto lstore = [&](int buf) {
        char *base = lds + buf * kStageLds;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int row = it * 32 + lrow;
            *reinterpret_cast<uint4 *>(base + row * kLdsStride + lc16) = pr[it];
            *reinterpret_cast<uint4 *>(base + kOperandLds + row * kLdsStride + lc16) = qr[it];
        }
    };

    gload(0);
    lstore(0);
    __syncthreads();
    const int frow_a = (wm * 64 + (lane & 31)) * kLdsStride + (lane >> 5) * 16;
    const int frow_b = (wn * 64 + (lane & 31)) * kLdsStride + (lane >> 5) * 16;
    for (int kb = 0; kb < nk; ++kb) {
        const bool more = kb + 1 < nk;
        if (more) gload(kb + 1);
        const char *sp = lds + (kb & 1) * kStageLds;
        const char *sq = sp + kOperandLds;
#pragma unroll
        for (int kg = 0; kg < kPanelBytes / 32; ++kg) {
            frag fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                fa[i] = *reinterpret_cast<const frag *>(sp + frow_a + i * 32 * kLdsStride + kg * 32);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                fb[j] = *reinterpret_cast<const frag *>(sq + frow_b + j * 32 * kLdsStride + kg * 32);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = Mfma<T>::mma(fa[i], fb[j], acc[i][j]);
        }
        if (more) lstore((kb + 1) & 1);
        __syncthreads();
    }
}

// Store 4 consecutive-row values of one column into a row-major array at
// [col][row..row+3] (the mirror / transposed copy), as one vector store.
template <typename T>
__device__ __forceinline__ void store4(char *base, int64_t ld_elems, int col, int row, const T v[4]) {
    T *p = reinterpret_cast<T *>(base) + (int64_t)col * ld_elems + row;
    if constexpr (sizeof(T) == 2) {
        typedef __bf16 b4 __attribute__((ext_vector_type(4)));
        b4 w = {v[0], v[1], v[2], v[3]};
        *reinterpret_cast<b4 *>(p) = w;
    } else {
        *reinterpret_cast<f32x4 *>(p) = f32x4{v[0], v[1], v[2], v[3]};
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads, 2) void ns_product_kernel(const NsProb *__restrict__ probs,
                                                                 const TileRef *__restrict__ tiles,
                                                                 int32_t ntiles, int32_t mode,
                                                                 int32_t cur, int32_t last, float ca,
                                                                 float cb, float cc) {
    __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
    const int tile_id = xcd_remap(blockIdx.x, gridDim.x);
    if (tile_id >= ntiles) return;
    const TileRef tr = tiles[tile_id];
    const NsProb pr = probs[tr.prob];
    const int64_t es = sizeof(T);
    const int row0 = tr.ti * kTile, col0 = tr.tj * kTile;

    const char *P, *Q;
    int64_t ldp, ldq;
    int K;
    if (mode == kSyrkX) {
        P = pr.x[cur] + row0 * (int64_t)pr.np * es;
        Q = pr.x[cur] + col0 * (int64_t)pr.np * es;
        ldp = ldq = pr.np * es;
        K = pr.np;
    } else if (mode == kSyrkA) {
        P = pr.a + row0 * (int64_t)pr.mp * es;
        Q = pr.a + col0 * (int64_t)pr.mp * es;
        ldp = ldq = pr.mp * es;
        K = pr.mp;
    } else {
        P = pr.b + row0 * (int64_t)pr.mp * es;
        Q = pr.xt[cur] + col0 * (int64_t)pr.mp * es;
        ldp = ldq = pr.mp * es;
        K = pr.mp;
    }

    f32x16 acc[2][2];
    if (mode == kSyrkA && cc == 0.f) {
        // c == 0: B = b A; the A A product is not needed.
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    } else {
        tile_product<T>(P, Q, ldp, ldq, K, lds, acc);
    }

    // Epilogue. Accumulator element (i, j, v) of this lane sits at tile row
    // wm*64 + i*32 + 8*(v/4) + 4*(lane/32) + v%4 and tile column
    // wn*64 + j*32 + lane%32.
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const bool mirror = tr.ti != tr.tj;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int gc = col0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int gr = row0 + wm * 64 + i * 32 + 8 * q + 4 * (lane >> 5);
                T val[4];
                if (mode == kSyrkX) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) val[e] = from_f32<T>(acc[i][j][4 * q + e]);
                    T *A = reinterpret_cast<T *>(pr.a);
#pragma unroll
                    for (int e = 0; e < 4; ++e) A[(int64_t)(gr + e) * pr.mp + gc] = val[e];
                    if (mirror) store4<T>(pr.a, pr.mp, gc, gr, val);
                } else if (mode == kSyrkA) {
                    const T *A = reinterpret_cast<const T *>(pr.a);
                    T *B = reinterpret_cast<T *>(pr.b);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float old = to_f32<T>(A[(int64_t)(gr + e) * pr.mp + gc]);
                        val[e] = from_f32<T>(cb * old + cc * acc[i][j][4 * q + e]);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) B[(int64_t)(gr + e) * pr.mp + gc] = val[e];
                    if (mirror) store4<T>(pr.b, pr.mp, gc, gr, val);
                } else {
                    const T *X = reinterpret_cast<const T *>(pr.x[cur]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float old = to_f32<T>(X[(int64_t)(gr + e) * pr.np + gc]);
                        val[e] = from_f32<T>(ca * old + acc[i][j][4 * q + e]);
                    }
                    if (!last) {
                        T *Xn = reinterpret_cast<T *>(pr.x[cur ^ 1]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) Xn[(int64_t)(gr + e) * pr.np + gc] = val[e];
                        store4<T>(pr.xt[cur ^ 1], pr.mp, gc, gr, val);
                    } else {
                        T *O = reinterpret_cast<T *>(pr.out);
                        if (gc < pr.n) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const int r = gr + e;
                                if (r < pr.m) {
                                    if (pr.tall)
                                        O[(int64_t)gc * pr.m + r] = val[e];   // out is n x m
                                    else
                                        O[(int64_t)r * pr.n + gc] = val[e];   // out is m x n
                                }
                            }
                        }
                    }
                }
            }
        }
    }
}

// Fixed-order fp32 sum over a workgroup (every thread gets the total).
__device__ __forceinline__ float block_sum(float v, float *red) {
    red[threadIdx.x] = v;
    __syncthreads();
#pragma unroll
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
        __syncthreads();
    }
    const float total = red[0];
    __syncthreads();
    return total;
}

struct NormPart {
    int32_t prob;
    int32_t part;
};

// Sum of squares of one kNormChunk-element chunk of one input, in fp32.
template <typename T>
__global__ __launch_bounds__(kThreads) void ns_norm_partial_kernel(const NsProb *__restrict__ probs,
                                                                   const NormPart *__restrict__ list,
                                                                   int32_t count) {
    __shared__ float red[kThreads];
    const int bid = blockIdx.x;
    if (bid >= count) return;
    const NormPart np_ = list[bid];
    const NsProb pr = probs[np_.prob];
    const int64_t numel = (int64_t)pr.m * pr.n;
    const int64_t start = (int64_t)np_.part * kNormChunk;
    const int64_t end = min(numel, start + (int64_t)kNormChunk);
    const T *in = reinterpret_cast<const T *>(pr.in);
    float s = 0.f;
    constexpr int kVec = 16 / sizeof(T);
    if ((reinterpret_cast<uintptr_t>(in) & 15) == 0 && end - start == kNormChunk) {
        const uint4 *v4 = reinterpret_cast<const uint4 *>(in + start);
        for (int k = threadIdx.x; k < kNormChunk / kVec; k += kThreads) {
            uint4 raw = v4[k];
            const T *e = reinterpret_cast<const T *>(&raw);
#pragma unroll
            for (int u = 0; u < kVec; ++u) {
                const float f = to_f32<T>(e[u]);
                s += f * f;
            }
        }
    } else {
        for (int64_t k = start + threadIdx.x; k < end; k += kThreads) {
            const float f = to_f32<T>(in[k]);
            s += f * f;
        }
    }
    const float total = block_sum(s, red);
    if (threadIdx.x == 0) pr.partials[np_.part] = total;
}

// One workgroup per matrix: reduce its partial sums in a fixed order and store
// the scale 1 / (||G||_F + eps) after the partials.
__global__ __launch_bounds__(kThreads) void ns_norm_finish_kernel(const NsProb *__restrict__ probs,
                                                                  int32_t count, float eps) {
    __shared__ float red[kThreads];
    const int bid = blockIdx.x;
    if (bid >= count) return;
    const NsProb pr = probs[bid];
    float s = 0.f;
    for (int p = threadIdx.x; p < pr.nparts; p += kThreads) s += pr.partials[p];
    const float nrm = sqrtf(block_sum(s, red));
    if (threadIdx.x == 0) pr.partials[pr.nparts] = 1.0f / (nrm + eps);
}

// Scale and write one 64x64 tile of X0 (mp x np) and
// X0^T, zero in the padding. With write_out (steps == 0) the scaled input goes
// straight to the output instead.
template <typename T>
__global__ __launch_bounds__(kThreads) void ns_norm_apply_kernel(const NsProb *__restrict__ probs,
                                                                 const TileRef *__restrict__ tiles,
                                                                 int32_t count, int32_t write_out) {
    __shared__ float tile[kNormTile][kNormTile + 1];
    const int bid = blockIdx.x;
    if (bid >= count) return;
    const TileRef tr = tiles[bid];
    const NsProb pr = probs[tr.prob];
    const float scale = pr.partials[pr.nparts];

    const T *in = reinterpret_cast<const T *>(pr.in);
    const int i0 = tr.ti * kNormTile, j0 = tr.tj * kNormTile;  // X rows / cols
    // tile[r][c] = X0[i0 + r][j0 + c]
    for (int e = threadIdx.x; e < kNormTile * kNormTile; e += kThreads) {
        const int a = e / kNormTile, b = e % kNormTile;  // b runs fastest: coalesced input reads
        float v = 0.f;
        if (!pr.tall) {
            const int i = i0 + a, j = j0 + b;
            if (i < pr.m && j < pr.n) v = to_f32<T>(in[(int64_t)i * pr.n + j]);
            tile[a][b] = to_f32<T>(from_f32<T>(v * scale));
        } else {
            const int j = j0 + a, i = i0 + b;  // input is n x m: row j, col i
            if (i < pr.m && j < pr.n) v = to_f32<T>(in[(int64_t)j * pr.m + i]);
            tile[b][a] = to_f32<T>(from_f32<T>(v * scale));
        }
    }
    __syncthreads();
    if (write_out) {
        T *O = reinterpret_cast<T *>(pr.out);
        for (int e = threadIdx.x; e < kNormTile * kNormTile; e += kThreads) {
            const int a = e / kNormTile, b = e % kNormTile;
            if (!pr.tall) {
                const int i = i0 + a, j = j0 + b;
                if (i < pr.m && j < pr.n) O[(int64_t)i * pr.n + j] = from_f32<T>(tile[a][b]);
            } else {
                const int j = j0 + a, i = i0 + b;
                if (i < pr.m && j < pr.n) O[(int64_t)j * pr.m + i] = from_f32<T>(tile[b][a]);
            }
        }
        return;
    }
    T *X = reinterpret_cast<T *>(pr.x[0]);
    T *XT = reinterpret_cast<T *>(pr.xt[0]);
    for (int e = threadIdx.x; e < kNormTile * kNormTile; e += kThreads) {
        const int a = e / kNormTile, b = e % kNormTile;
        X[(int64_t)(i0 + a) * pr.np + (j0 + b)] = from_f32<T>(tile[a][b]);
        XT[(int64_t)(j0 + a) * pr.mp + (i0 + b)] = from_f32<T>(tile[b][a]);
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

struct MatInfo {
    int64_t rows, cols, m, n, mp, np;
    bool tall, active;
    int64_t nparts, syrk_tiles, gemm_tiles, norm_tiles;
    size_t buf_bytes;
};

ns_status describe(int32_t n, const ns_shape *shapes, ns_dtype dtype, std::vector<MatInfo> &info) {
    if (n < 0) return fail(NS_ERR_INVALID_ARG, "n = %d < 0", n);
    if (n > 0 && !shapes) return fail(NS_ERR_INVALID_ARG, "shapes is NULL");
    if (dtype != NS_BF16 && dtype != NS_F32) return fail(NS_ERR_DTYPE, "dtype %d", (int)dtype);
    const int64_t es = dtype == NS_BF16 ? 2 : 4;
    info.resize(n);
    for (int32_t i = 0; i < n; ++i) {
        MatInfo &mi = info[i];
        ns_status st = matrix_view(shapes[i], i, &mi.rows, &mi.cols);
        if (st) return st;
        mi.active = mi.rows > 0 && mi.cols > 0;
        if (!mi.active) {
            mi = MatInfo{mi.rows, mi.cols, 0, 0, 0, 0, false, false, 0, 0, 0, 0, 0};
            continue;
        }
        mi.tall = mi.rows > mi.cols;
        mi.m = std::min(mi.rows, mi.cols);
        mi.n = std::max(mi.rows, mi.cols);
        if (mi.n > (int64_t)65535 * kNormTile || mi.m * mi.n > ((int64_t)1 << 40))
            return fail(NS_ERR_OVERFLOW, "tensor %d: %lld x %lld is too large", i,
                        (long long)mi.rows, (long long)mi.cols);
        mi.mp = round_up(mi.m, kTile);
        mi.np = round_up(mi.n, kTile);
        const int64_t tm = mi.mp / kTile, tn = mi.np / kTile;
        mi.syrk_tiles = tm * (tm + 1) / 2;
        mi.gemm_tiles = tm * tn;
        mi.norm_tiles = (mi.mp / kNormTile) * (mi.np / kNormTile);
        mi.nparts = (mi.m * mi.n + kNormChunk - 1) / kNormChunk;
        const size_t xb = align256((size_t)(mi.mp * mi.np * es));
        const size_t ab = align256((size_t)(mi.mp * mi.mp * es));
        mi.buf_bytes = 4 * xb + 2 * ab;
    }
    return NS_OK;
}

struct TableSizes {
    size_t probs, syrk, gemm, parts, ntiles, partials, total;
};

TableSizes table_sizes(const std::vector<MatInfo> &info) {
    int64_t np = 0, sy = 0, ge = 0, pa = 0, nt = 0, ps = 0;
    for (const MatInfo &mi : info) {
        if (!mi.active) continue;
        ++np;
        sy += mi.syrk_tiles;
        ge += mi.gemm_tiles;
        pa += mi.nparts;
        nt += mi.norm_tiles;
        ++ps;
    }
    TableSizes t;
    t.probs = align256(np * sizeof(NsProb));
    t.syrk = align256(sy * sizeof(TileRef));
    t.gemm = align256(ge * sizeof(TileRef));
    t.parts = align256(pa * sizeof(NormPart));
    t.ntiles = align256(nt * sizeof(TileRef));
    t.partials = align256((pa + ps) * sizeof(float));  // partials + one scale per matrix
    t.total = t.probs + t.syrk + t.gemm + t.parts + t.ntiles + t.partials;
    return t;
}

template <typename T>
ns_status run_group(const std::vector<int32_t> &group, const std::vector<MatInfo> &info,
                    const void *const *in, void *const *out, int32_t steps, float a, float b,
                    float c, float eps, char *ws, const TableSizes &tsz, hipStream_t st) {
    // Host tables for this group.
    std::vector<NsProb> probs;
    std::vector<TileRef> syrk, gemm, ntiles;
    std::vector<NormPart> parts;
    char *base = ws + tsz.total;
    float *partials = reinterpret_cast<float *>(ws + tsz.total - tsz.partials);
    int64_t part_off = 0;
    double f_syrk_x = 0, f_syrk_a = 0, f_gemm = 0, norm_bytes = 0;
    const int64_t es = sizeof(T);
    for (int32_t idx : group) {
        const MatInfo &mi = info[idx];
        NsProb p{};
        const size_t xb = align256((size_t)(mi.mp * mi.np * es));
        const size_t ab = align256((size_t)(mi.mp * mi.mp * es));
        p.x[0] = base;
        p.x[1] = base + xb;
        p.xt[0] = base + 2 * xb;
        p.xt[1] = base + 3 * xb;
        p.a = base + 4 * xb;
        p.b = base + 4 * xb + ab;
        base += mi.buf_bytes;
        p.in = static_cast<const char *>(in[idx]);
        p.out = static_cast<char *>(out[idx]);
        p.partials = partials + part_off;
        part_off += mi.nparts + 1;
        p.m = (int32_t)mi.m;
        p.n = (int32_t)mi.n;
        p.mp = (int32_t)mi.mp;
        p.np = (int32_t)mi.np;
        p.tall = mi.tall;
        p.nparts = (int32_t)mi.nparts;
        const int32_t pid = (int32_t)probs.size();
        probs.push_back(p);
        const int tm = (int)(mi.mp / kTile), tn = (int)(mi.np / kTile);
        for (int ti = 0; ti < tm; ++ti)
            for (int tj = ti; tj < tm; ++tj) syrk.push_back(TileRef{pid, (uint16_t)ti, (uint16_t)tj});
        for (int ti = 0; ti < tm; ++ti)
            for (int tj = 0; tj < tn; ++tj) gemm.push_back(TileRef{pid, (uint16_t)ti, (uint16_t)tj});
        for (int64_t k = 0; k < mi.nparts; ++k) parts.push_back(NormPart{pid, (int32_t)k});
        const int nm = (int)(mi.mp / kNormTile), nn = (int)(mi.np / kNormTile);
        for (int ti = 0; ti < nm; ++ti)
            for (int tj = 0; tj < nn; ++tj) ntiles.push_back(TileRef{pid, (uint16_t)ti, (uint16_t)tj});
        const double m = (double)mi.m, n = (double)mi.n;
        f_syrk_x += m * (m + 1) * n;
        f_syrk_a += c != 0.f ? m * m * (m + 1) : 0.0;
        f_gemm += 2 * m * m * n;
        norm_bytes += 2.0 * m * n * es + 2.0 * (double)mi.mp * (double)mi.np * es;
    }
    if (probs.empty()) return NS_OK;

    // One upload of every table (stream-ordered after earlier groups' kernels).
    std::vector<char> host(tsz.total - tsz.partials, 0);
    auto put = [&](size_t off, const void *src, size_t bytes) {
        if (bytes) std::memcpy(host.data() + off, src, bytes);
    };
    const size_t o_syrk = tsz.probs, o_gemm = o_syrk + tsz.syrk, o_parts = o_gemm + tsz.gemm,
                 o_ntiles = o_parts + tsz.parts;
    put(0, probs.data(), probs.size() * sizeof(NsProb));
    put(o_syrk, syrk.data(), syrk.size() * sizeof(TileRef));
    put(o_gemm, gemm.data(), gemm.size() * sizeof(TileRef));
    put(o_parts, parts.data(), parts.size() * sizeof(NormPart));
    put(o_ntiles, ntiles.data(), ntiles.size() * sizeof(TileRef));
    NSQ_HIP(hipMemcpyAsync(ws, host.data(), host.size(), hipMemcpyHostToDevice, st));

    const NsProb *d_probs = reinterpret_cast<const NsProb *>(ws);
    const TileRef *d_syrk = reinterpret_cast<const TileRef *>(ws + o_syrk);
    const TileRef *d_gemm = reinterpret_cast<const TileRef *>(ws + o_gemm);
    const NormPart *d_parts = reinterpret_cast<const NormPart *>(ws + o_parts);
    const TileRef *d_ntiles = reinterpret_cast<const TileRef *>(ws + o_ntiles);

    {
        TimedScope ts(kTimeNorm, st, norm_bytes);
        hipLaunchKernelGGL(ns_norm_partial_kernel<T>, dim3((unsigned)parts.size()), dim3(kThreads), 0,
                           st, d_probs, d_parts, (int32_t)parts.size());
        hipLaunchKernelGGL(ns_norm_finish_kernel, dim3((unsigned)probs.size()), dim3(kThreads), 0, st,
                           d_probs, (int32_t)probs.size(), eps);
        hipLaunchKernelGGL(ns_norm_apply_kernel<T>, dim3((unsigned)ntiles.size()), dim3(kThreads), 0,
                           st, d_probs, d_ntiles, (int32_t)ntiles.size(), steps == 0 ? 1 : 0);
    }
    NSQ_HIP(hipGetLastError());
    int cur = 0;
    for (int32_t s = 0; s < steps; ++s) {
        const int last = s == steps - 1;
        {
            TimedScope ts(kTimeProduct, st, f_syrk_x);
            hipLaunchKernelGGL(ns_product_kernel<T>, dim3((unsigned)syrk.size()), dim3(kThreads), 0,
                               st, d_probs, d_syrk, (int32_t)syrk.size(), (int32_t)kSyrkX, cur, last,
                               a, b, c);
        }
        {
            TimedScope ts(kTimeProduct, st, f_syrk_a);
            hipLaunchKernelGGL(ns_product_kernel<T>, dim3((unsigned)syrk.size()), dim3(kThreads), 0,
                               st, d_probs, d_syrk, (int32_t)syrk.size(), (int32_t)kSyrkA, cur, last,
                               a, b, c);
        }
        {
            TimedScope ts(kTimeProduct, st, f_gemm);
            hipLaunchKernelGGL(ns_product_kernel<T>, dim3((unsigned)gemm.size()), dim3(kThreads), 0,
                               st, d_probs, d_gemm, (int32_t)gemm.size(), (int32_t)kGemmBX, cur, last,
                               a, b, c);
        }
        NSQ_HIP(hipGetLastError());
        cur ^= 1;
    }
    return NS_OK;
}

}  // namespace
}  // namespace nsq

using namespace nsq;

extern "C" ns_status ns_workspace_bytes(int32_t n, const ns_shape *shapes, ns_dtype dtype,
                                        size_t *bytes, size_t *min_bytes) {
    if (!bytes) return fail(NS_ERR_INVALID_ARG, "bytes is NULL");
    std::vector<MatInfo> info;
    ns_status st = describe(n, shapes, dtype, info);
    if (st) return st;
    const TableSizes t = table_sizes(info);
    size_t all = t.total, biggest = 0;
    for (const MatInfo &mi : info) {
        all += mi.buf_bytes;
        biggest = std::max(biggest, mi.buf_bytes);
    }
    *bytes = all;
    if (min_bytes) *min_bytes = t.total + biggest;
    return NS_OK;
}

extern "C" ns_status ns_orthogonalize_batched(int32_t n, const ns_shape *shapes,
                                              const void *const *in, void *const *out,
                                              ns_dtype dtype, int32_t steps, float a, float b,
                                              float c, float eps, const int32_t *order,
                                              void *workspace, size_t workspace_bytes,
                                              void *stream) {
    std::vector<MatInfo> info;
    ns_status st = describe(n, shapes, dtype, info);
    if (st) return st;
    if (steps < 0) return fail(NS_ERR_INVALID_ARG, "steps = %d < 0", steps);
    if (!(eps >= 0.f) || !std::isfinite(a) || !std::isfinite(b) || !std::isfinite(c))
        return fail(NS_ERR_INVALID_ARG, "coefficients must be finite and eps >= 0");
    if (n == 0) return NS_OK;
    if (!in || !out) return fail(NS_ERR_INVALID_ARG, "in and out are required");
    const size_t es = dtype == NS_BF16 ? 2 : 4;
    for (int32_t i = 0; i < n; ++i) {
        if (!info[i].active) continue;
        if (!in[i] || !out[i]) return fail(NS_ERR_INVALID_ARG, "tensor %d: NULL in/out", i);
        if ((reinterpret_cast<uintptr_t>(in[i]) | reinterpret_cast<uintptr_t>(out[i])) % es)
            return fail(NS_ERR_INVALID_ARG, "tensor %d: in/out not %zu-byte aligned", i, es);
    }
    // Dispatch order: caller's permutation, else descending cost (ties by index).
    std::vector<int32_t> ord(n);
    if (order) {
        std::vector<char> seen(n, 0);
        for (int32_t k = 0; k < n; ++k) {
            const int32_t i = order[k];
            if (i < 0 || i >= n || seen[i])
                return fail(NS_ERR_INVALID_ARG, "order is not a permutation of 0..%d", n - 1);
            seen[i] = 1;
            ord[k] = i;
        }
    } else {
        for (int32_t k = 0; k < n; ++k) ord[k] = k;
        auto cost = [&](int32_t i) {
            const MatInfo &mi = info[i];
            return (double)mi.m * (double)mi.n * ((double)mi.m * steps + 1);
        };
        std::stable_sort(ord.begin(), ord.end(), [&](int32_t x, int32_t y) { return cost(x) > cost(y); });
    }
    const TableSizes tsz = table_sizes(info);
    size_t biggest = 0;
    for (const MatInfo &mi : info) biggest = std::max(biggest, mi.buf_bytes);
    if (!workspace) return fail(NS_ERR_WORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
        return fail(NS_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < tsz.total + biggest)
        return fail(NS_ERR_WORKSPACE, "workspace of %zu bytes < minimum %zu", workspace_bytes,
                    tsz.total + biggest);
    // Groups of consecutive matrices (in dispatch order) whose buffers fit.
    const size_t room = workspace_bytes - tsz.total;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    std::vector<int32_t> group;
    size_t used = 0;
    auto flush = [&]() -> ns_status {
        if (group.empty()) return NS_OK;
        ns_status r = dtype == NS_BF16
                          ? run_group<__bf16>(group, info, in, out, steps, a, b, c, eps,
                                              static_cast<char *>(workspace), tsz, hs)
                          : run_group<float>(group, info, in, out, steps, a, b, c, eps,
                                             static_cast<char *>(workspace), tsz, hs);
        group.clear();
        used = 0;
        return r;
    };
    for (int32_t i : ord) {
        if (!info[i].active) continue;
        if (used + info[i].buf_bytes > room && (st = flush())) return st;
        group.push_back(i);
        used += info[i].buf_bytes;
    }
    return flush();
}
