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
//  * Workspace per matrix, oriented so m <= n, padded to multiples of 256 in
//    both dims and kept zero in the padding: X (two copies, ping-pong), A and
//    B, and X^T (two copies) where B X reads it (below). Padding removes every
//    bounds check from the product main loop; zero padding stays zero through
//    every step (products with zero rows/cols).
//  * All three products run one MFMA main loop over K panels:
//        A   = X X^T  : P = Q = X        (C = P Q^T, both read along rows)
//        A A          : P = Q = A        (A A = A A^T, A symmetric)
//        B X          : P = B, Q = X     (C = P Q, Q read K-major: stage kb
//                                         holds 64 rows of X and the MFMA
//                                         fragments come from LDS transpose
//                                         reads; f32 and 128-tile calls past
//                                         K = 1024: C = P Q^T with Q = X^T, a
//                                         copy each step writes)
//    Panels of 128 bytes of K per row go global -> LDS with buffer_load ... lds
//    into two stage buffers; every wave loads a slice of both panels.
//    bf16 256 x 256 tiles run on 4 waves of 128 x 128 whose accumulators stay
//    in fixed AGPRs under a hand-written stage schedule (ns_pinned_kernel);
//    128 x 128 tiles (small groups, f32) on 4 waves of 64 x 64
//    (ns_product_kernel). bf16 runs v_mfma_f32_16x16x32_bf16, f32
//    v_mfma_f32_32x32x2f32.
//  * The symmetric products compute only tiles on or above the diagonal and
//    store each off-diagonal tile twice (itself and its mirror), so A and B are
//    exactly symmetric.
//  * Epilogues in fp32, rounded once: A; B = b A + c (A A); X' = a X + B X.
//    The rounded tile is staged in LDS column-major; the tile is then written
//    row-major through LDS transpose reads and, for the symmetric products'
//    mirror (and X'^T where it is kept), column-major from plain LDS rows,
//    both as 16-byte stores. The last step's epilogue writes straight to the
//    caller's output in the input's orientation, shape and dtype.
//  * Input staging: the input goes unscaled into X0 (tall inputs transposed
//    through LDS; X0^T too where it is kept) with per-tile fp32 sums of
//    squares, each workgroup taking a run of 128 x 128 tiles along one band of
//    input rows; the products reduce those sums in a fixed order (no atomics)
//    and fold the scale into the first step's epilogues.
//  * Workgroup ids are remapped so consecutive tiles land on the same XCD (the
//    hardware hands workgroups to the 8 XCDs round-robin), sharing its L2, and
//    tiles are taken in groups of 4 x 8 so a run of tiles reuses operand panels.

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <type_traits>
#include <vector>

#include "hip_util.h"

namespace nsq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kPad = 256;           // tiled matrices are padded to a multiple of this (zero padding)
constexpr int kSmallPad = 128;      // ... matrices of the small size class to a multiple of this
constexpr int kSmallM = 128;        // largest m of the small size class
constexpr int kPrepTile = 128;      // tile edge of the input-staging pass
constexpr int kPrepThreads = 512;   // its threads (8 waves, 4 input loads each)
constexpr int kScaleSlots = 256;    // width of the fixed-order reduction of the norm partials
constexpr int kNumXcd = 8;
// Every workspace row is padded by this many bytes past its padded width, so
// the row stride is an odd multiple of 256 bytes: a K panel (the same bytes of
// 256 consecutive rows) then spreads over the L2 channels instead of landing
// on a few of them, as a power-of-two stride makes it do.
constexpr int kRowPadBytes = 256;
// The no-allocation entry point: its scratch array (one per GPU) and the most
// table bytes a call may stage (the pinned staging that ns_noalloc_init makes).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
constexpr size_t kNoAllocTableBytes = size_t(1) << 20;
// Tables up to this size are read by the staging workgroups straight from the
// pinned host staging; larger ones are copied to the workspace first.
constexpr size_t kTablesFromHostMax = size_t(256) << 10;

// Per-matrix descriptor in device memory.
struct NsProb {
    char *x0, *x1;     // X ping/pong: mp x np (row stride ldx)
    char *xt0, *xt1;   // X^T ping/pong: np x mp (row stride ldxt); null when kmajor
    char *a;           // A: mp x mp (row stride ldt)
    char *b;           // B: mp x mp (row stride ldt)
    char *g, *q0, *q1, *t;   // Gram-space only: G, Q ping/pong, Q G; mp x mp fp32 (row stride ldt)
    char *qt0, *qt1, *at;    // Gram-space only: Q^T ping/pong, A^T
    float *partials;   // nparts fp32 sums of squares, one per staging tile
    int32_t m, n;      // oriented sizes (m <= n)
    int32_t mp, np;    // padded to kPad (kSmallPad for the small size class)
    int32_t ldx;       // row stride of X (elements, > np)
    int32_t ldxt;      // row stride of X^T (elements, > mp)
    int32_t ldt;       // row stride of A and B (elements, > mp)
    int32_t kmajor;    // B X reads X K-major (as stored); X^T is not kept
    int32_t tall;      // input had rows > cols
    int32_t nparts;    // (mp / kPrepTile) * (np / kPrepTile)
    int32_t vec_in;    // every input piece allows 16-byte accesses (aligned base, row bytes % 16 == 0)
    int32_t vec_out;   // ... every output piece
};

// Rows [row0, next piece's row0) of a tensor as stored (rows x cols,
// row-major with row strides ld_in / ld_out elements): element (r, c) of the
// input is at in + ((r - row0) ld_in + c) es, of the output at
// out + ((r - row0) ld_out + c) es. An unrouted tensor is one piece (strided
// for a sub-block of a larger matrix, e.g. one of Q, K, V in a fused weight);
// a routed one has a piece per shard buffer that holds some of its rows
// (route_to_ns_home / route_from_ns_home of "core.optimizer.layer_sharded_a2a"
// move exactly these pieces). Pieces of a tensor are sorted by row0, the first
// has row0 = 0 and none is empty.
struct RowPiece {
    int64_t row0;
    const char *in;
    char *out;
    int64_t ld_in, ld_out;
};
static_assert(sizeof(RowPiece) == 40, "RowPiece layout");

// A tile of one tensor: (ti, tj) in the tile grid of the launch that uses it.
// pieces[piece .. piece + npiece) are the pieces holding the tensor rows (as
// stored) that the tile reads or writes; npiece >= 1.
struct TileRef {
    int32_t prob;
    uint16_t ti, tj;
    int32_t piece, npiece;
};
static_assert(sizeof(TileRef) == 16, "TileRef layout");

// A run of input-staging tiles of one tensor: `count` consecutive
// kPrepTile x kPrepTile tiles q0 .. q0 + count - 1 of input row band `band`
// (input rows band * kPrepTile onwards, as stored; a row band of a tall G is a
// column band of X). pieces[piece .. piece + npiece) hold the band's rows.
struct StageRun {
    int32_t prob;
    uint16_t band, q0;
    int32_t piece;
    uint16_t npiece, count;
};
static_assert(sizeof(StageRun) == 16, "StageRun layout");

// The piece among band[0 .. n) (sorted by row0, band[0].row0 <= row) holding
// row `row`.
__device__ __forceinline__ const RowPiece &find_piece(const RowPiece *band, int n, int64_t row) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (band[mid].row0 <= row) lo = mid;
        else hi = mid - 1;
    }
    return band[lo];
}

template <typename T> struct Mfma;

// The MFMA of each element type and its lane layouts. A K step is KB bytes of
// k; operand lane l holds row l % BLK of the block and the 16-byte chunk
// (KB / 16) kg + l / BLK of K step kg; output lane l holds column l % BLK of
// the BLK x BLK block and, for q < NQ, rows out_row(l, q) .. + 4.
template <> struct Mfma<__bf16> {
    // v_mfma_f32_16x16x32_bf16: 32 k per step, 8 consecutive k per lane
    typedef bf16x8 frag;
    typedef f32x4 acc;
    static constexpr int BLK = 16, KB = 64, NQ = 1;
    static __device__ __forceinline__ int out_row(int lane, int) { return 4 * (lane >> 4); }
    static __device__ __forceinline__ acc mma(frag a, frag b, acc c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mfma<float> {
    // v_mfma_f32_32x32x2f32: 8 k per step, 4 consecutive k per lane, one MFMA per element
    typedef f32x4 frag;
    typedef f32x16 acc;
    static constexpr int BLK = 32, KB = 32, NQ = 4;
    static __device__ __forceinline__ int out_row(int lane, int q) { return 8 * q + 4 * (lane >> 5); }
    static __device__ __forceinline__ acc mma(frag a, frag b, acc c) {
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0], b[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[1], b[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[2], b[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[3], b[3], c, 0, 0, 0);
        return c;
    }
};

template <typename T> __device__ __forceinline__ float to_f32(T v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v) { return (T)v; }

#define NSQ_GLOBAL __attribute__((address_space(1)))
#define NSQ_LDS __attribute__((address_space(3)))
template <typename T> __device__ __forceinline__ NSQ_GLOBAL T *gp(const char *p) {
    return (NSQ_GLOBAL T *)(p);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Bijection from hardware workgroup id to logical tile id such that the
// workgroups of one XCD (hardware ids congruent mod 8) get a contiguous range.
__device__ __forceinline__ int xcd_remap(int b, int g) {
    const int xcd = b % kNumXcd, local = b / kNumXcd;
    const int per = g / kNumXcd, rem = g % kNumXcd;
    return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// Product launches. NS: kSyrkX, kSyrkA, kGemmBX. Gram-space NS ("[GTP][Muon]
// Optimize Muon step performance", "Secondary (parked)", gram_once): the
// iterate is X_k = Q_k X0 with the m x m Gram G = X0 X0^T computed once, so a
// step is A = Q G Q^T, Q' = (a I + b A + c A A) Q on m x m matrices, and the
// result is Q_k X0. In exact arithmetic Q_k is a polynomial in G, so all of
// these are symmetric; in fp32 they are not, and forcing them symmetric
// (copying one triangle over the other, or averaging) multiplies the error on
// ill-conditioned inputs about tenfold. So only G (exactly symmetric: its
// (i, j) and (j, i) sum the same products) is an upper-tile product; the
// others are full products, and each matrix that is later a right operand
// is also written transposed, so those products read K-major rows (the last
// one, Q X0, reads X0 as stored, like B' X).
enum Mode {
    kSyrkX = 0,    // A = s_final X X^T                             upper tiles
    kSyrkA = 1,    // B' = s_final (s_init A + A A) + s_diag I      upper tiles
    kGemmBX = 2,   // X' = B' X
    kGramG = 3,    // G = s^2 X0 X0^T + ridge (tr G / m) I          upper tiles
    kGramB0 = 4,   // Q1 = s_final (s_init G + G G) + s_diag I, also Q1^T   (step 0: Q0 = I)
    kGramQG = 5,   // T = Q G
    kGramTQ = 6,   // A = T Q, also A^T
    kGramAA = 7,   // B' = s_final (s_init A + A A) + s_diag I
    kGramBQ = 8,   // Q' = B' Q, also Q'^T
    kGramOut = 9,  // out = s Q X0 (last launch, the caller's output)
};
constexpr bool symmetric_mode(int mode) { return mode == kSyrkX || mode == kSyrkA || mode == kGramG; }
// Modes that always write their result transposed (the next products' K-major
// operand); B X also writes X'^T unless the next B X reads X' K-major.
constexpr bool writes_transpose(int mode) {
    return mode == kGramB0 || mode == kGramTQ || mode == kGramBQ;
}

// Output tile of BM x BM computed by WM x WN waves; each wave owns a
// (BM/WM) x (BM/WN) sub-tile made of the element type's MFMA output blocks
// (Geo<T>: rows wm BM/WM .., column blocks col_blk(wn, 0 ..)). K is staged in
// panels of ROWB bytes per row, in a ring of NBUF stage buffers.
template <int BM_, int WM_, int WN_, int ROWB_, int NBUF_> struct TileCfg {
    static constexpr int BM = BM_, WM = WM_, WN = WN_, ROWB = ROWB_, NBUF = NBUF_;
    static constexpr int WAVES = WM * WN;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int PANEL = BM * ROWB;
    static constexpr int STAGE = 2 * PANEL;     // P panel then Q panel
    static constexpr int RING = NBUF * STAGE;
    static constexpr int RPW = BM / WAVES;      // panel rows each wave loads
    static constexpr int RPI = 1024 / ROWB;     // panel rows per 1 KiB wave load
    static constexpr int LOADS = RPW / RPI;     // loads per wave per panel
    static_assert(ROWB == 64 || ROWB == 128, "panel row size");
    // The wave's MFMA blocks for element type T: NBM x NBN blocks of BLK x BLK,
    // KG K steps (k-groups) per stage. col_blk(wn, j) is the first tile column
    // of the wave's column block j: the blocks of a wave are WN apart.
    template <typename T> struct Geo {
        static constexpr int BLK = Mfma<T>::BLK;
        static constexpr int NBM = BM / WM / BLK, NBN = BM / WN / BLK;
        static constexpr int KG = ROWB / Mfma<T>::KB;
        static_assert(NBM * BLK * WM == BM && NBN * BLK * WN == BM && KG >= 1, "whole blocks");
        static __device__ __forceinline__ int col_blk(int wn, int j) { return (j * WN + wn) * BLK; }
    };
    static_assert(RPW % RPI == 0, "each wave loads whole row groups");
    static_assert(NBUF >= 2 && NBUF <= 5, "ring depth");
};
// The accumulators of one wave.
template <typename T, class C>
using AccTile = typename Mfma<T>::acc[C::template Geo<T>::NBM][C::template Geo<T>::NBN];

// Build-time alternatives of the 256-tile configuration, kept for measuring
// (64-byte panel rows in up to 5 ring buffers, or 4 waves across; all
// measured slower than these defaults).
#ifndef NSQ_BIG_ROWB
#define NSQ_BIG_ROWB 128
#endif
#ifndef NSQ_BIG_NBUF
#define NSQ_BIG_NBUF 2
#endif
#ifndef NSQ_BIG_WN
#define NSQ_BIG_WN 4
#endif
typedef TileCfg<256, 2, NSQ_BIG_WN, NSQ_BIG_ROWB, NSQ_BIG_NBUF> Big;   // 8 waves, 2 per SIMD, 128 x 64 per wave
typedef TileCfg<128, 2, 2, 128, 2> Small;                     // 4 waves, 64 x 64 per wave (two per CU)

// Operand staging. Each stage holds, per operand, ROWB bytes of K for each of
// the tile's BM rows. Panel row r sits at r * ROWB bytes; its 16-byte chunk c
// (8 bf16 / 4 f32 consecutive k) sits in slot c ^ swz(r), which makes the
// fragment reads (16 or 32 consecutive rows, one chunk each) hit distinct
// banks in every 16 lanes:
//   ROWB = 128: swz(r) = (r >> 1) & 7
//   ROWB = 64:  swz(r) = ((r >> 1) & 3) ^ ((r >> 3) & 1)
// Global -> LDS uses buffer_load ... lds: lane l's 16 bytes land at M0 + 16 l,
// so each lane fetches whatever global chunk belongs at its LDS slot; one wave
// instruction moves 1 KiB (1024 / ROWB rows).
template <int ROWB> __device__ __forceinline__ int swz(int r) {
    if constexpr (ROWB == 128) return (r >> 1) & 7;
    else return ((r >> 1) & 3) ^ ((r >> 3) & 1);
}

// s_waitcnt vmcnt(N), the other counters left alone (gfx9 encoding).
template <int N> __device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier that waits for this wave's LDS operations but not for its
// global loads (the ring keeps later stages in flight across it).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// MFMA operand fragment for the block starting at panel row `blk`, k-group
// kg of the stage: lane l gets row blk + l % BLK, chunk (KB / 16) kg + l / BLK.
template <typename T, int ROWB>
__device__ __forceinline__ typename Mfma<T>::frag operand_frag(const char *region, int lane, int blk, int kg) {
    typedef typename Mfma<T>::frag frag;
    const int row = blk + lane % Mfma<T>::BLK;
    const int c = (Mfma<T>::KB / 16) * kg + lane / Mfma<T>::BLK;
    return *reinterpret_cast<const frag *>(region + row * ROWB + ((c ^ swz<ROWB>(row)) << 4));
}

// K-major Q panels (the Q operand read from a row-major matrix whose rows run
// along K, e.g. X for X' = B' X): a stage holds KW = ROWB / es rows of K, each
// the BM tile columns (BM es bytes). The 16-byte unit u of panel row k sits at
// unit position u ^ swq(k), which puts the rows read together on distinct
// banks: bf16 fragments come from LDS transpose reads, each 16 lanes reading
// four consecutive rows and 32 lanes rows k0 .. k0 + 3 and k0 + 8 .. k0 + 11
// of the same 32 bytes (XOR 4 (k % 4) moves the four rows' pieces to four bank
// groups, XOR 2 ((k / 8) % 2) the second four rows to the other half of each),
// f32 fragments from 4-byte reads of rows k and k + 4 (XOR 8 ((k / 4) % 2)).
template <int ES> __device__ __forceinline__ int swq(int k) {
    if constexpr (ES == 2) return (4 * (k & 3)) ^ (2 * ((k >> 3) & 1));
    else return 8 * ((k >> 2) & 1);
}

// MFMA operand fragment of tile columns blk .. blk + BLK, k-group kg, from a
// K-major panel (RB bytes per row): lane l gets column blk + l % BLK and the
// fragment's consecutive k. bf16: each 16-lane group g takes columns
// blk .. blk + 16, k from 32 kg + 8 g, four per transpose read (lane t
// addresses row k0 + t / 4, columns blk + 4 (t % 4) .. + 4, and receives
// column blk + t of rows k0 .. k0 + 3). f32: k = 8 kg + 4 (l / 32) + e.
template <typename T, int RB>
__device__ __forceinline__ typename Mfma<T>::frag kmajor_frag(const char *region, int lane, int blk, int kg) {
    constexpr int ES = sizeof(T);
    auto at = [&](int k, int c) -> const char * {
        const int byte = c * ES;
        return region + k * RB + ((((byte >> 4) ^ swq<ES>(k))) << 4) + (byte & 15);
    };
    if constexpr (ES == 2) {
        static_assert(Mfma<T>::BLK == 16 && Mfma<T>::KB == 64, "bf16 fragment layout");
        const int t = lane & 15, g = lane >> 4;
        const int c0 = blk, k0 = 32 * kg + 8 * g;
        s16x4 v[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
            v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (NSQ_LDS s16x4 *)at(k0 + 4 * h + (t >> 2), c0 + 4 * (t & 3)));
        typedef short s16x8 __attribute__((ext_vector_type(8)));
        const s16x8 w = {v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]};
        return __builtin_bit_cast(typename Mfma<T>::frag, w);
    } else {
        const int c = blk + (lane & 31), k0 = 8 * kg + 4 * (lane >> 5);
        typename Mfma<T>::frag f;
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = *reinterpret_cast<const float *>(at(k0 + e, c));
        return f;
    }
}

// Rounding is spelled out wherever a product meets a sum (an explicit
// multiply before the accumulation, separate rounded multiply and add in the
// epilogue), so that no tile configuration's instruction choice can change a
// result bit.
//
// acc += P Q^T over nk stages for one BM x BM tile. P, Q point at the tile's
// first operand row; ldp, ldq are row strides in bytes; `extent_*` is the byte
// size the buffer resources may address from P and Q. QK: Q is K-major
// instead, a row-major matrix with K along its rows (C = P Q): Q points at its
// row 0, tile column 0, and stage kb reads its rows kb KW .. kb KW + KW.
template <typename T, class C, bool QK = false>
__device__ __forceinline__ void tile_product(const char *P, const char *Q, int ldp, int ldq, int extent_p,
                                             int extent_q, int nk, char *lds, AccTile<T, C> &acc) {
    typedef typename Mfma<T>::frag frag;
    typedef typename C::template Geo<T> G;
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int wm = wave / C::WN, wn = wave % C::WN;

    const __amdgpu_buffer_rsrc_t rp =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(P), (short)0, extent_p, 0x00020000);
    const __amdgpu_buffer_rsrc_t rq =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(Q), (short)0, extent_q, 0x00020000);
    constexpr int ROWB = C::ROWB, CPR = ROWB / 16;   // 16-byte chunks per panel row
    int voff_p[C::LOADS], voff_q[C::LOADS];
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
        const int row = wave * C::RPW + i * C::RPI + lane / CPR;
        const int chunk = ((lane % CPR) ^ swz<ROWB>(row)) << 4;
        voff_p[i] = row * ldp + chunk;
        voff_q[i] = row * ldq + chunk;
    }
    // K-major Q: a 1 KiB wave load covers RPQ panel rows of UPR units; each
    // wave loads KW / WAVES consecutive rows (the same LDS bytes as a P slice)
    constexpr int ES = sizeof(T), KW = ROWB / ES, RB = C::BM * ES, UPR = RB / 16, RPQ = 64 / UPR;
    static_assert(!QK || (KW % C::WAVES == 0 && (KW / C::WAVES) == C::LOADS * RPQ), "K-major Q slices");
    if constexpr (QK) {
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i) {
            const int k = wave * (KW / C::WAVES) + i * RPQ + lane / UPR;
            voff_q[i] = k * ldq + (((lane % UPR) ^ swq<ES>(k)) << 4);
        }
    }
    const int q_stage = QK ? KW * ldq : ROWB;   // byte step of Q per stage
    const int a_blk = wm * (C::BM / C::WM);
    // This wave's loads of stage kb: rows [wave RPW, (wave + 1) RPW) of both
    // panels into ring buffer kb % NBUF, 1 KiB per instruction.
    auto issue = [&](int kb) {
        char *sp = lds + (kb % C::NBUF) * C::STAGE + wave * C::RPW * ROWB;
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rp, (NSQ_LDS void *)(sp + i * C::RPI * ROWB), 16,
                                                     (int)voff_p[i], kb * ROWB, 0, 0);
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (NSQ_LDS void *)(sp + C::PANEL + i * C::RPI * ROWB), 16,
                                                     (int)voff_q[i], kb * q_stage, 0, 0);
    };
    // Wait until this wave's loads of the current stage have landed, leaving
    // the n stages issued after it in flight.
    constexpr int L = 2 * C::LOADS;
    auto wait_stage = [&](int n) {
        if constexpr (C::NBUF >= 5) {
            if (n >= 3) { wait_vmcnt<3 * L>(); return; }
        }
        if constexpr (C::NBUF >= 4) {
            if (n >= 2) { wait_vmcnt<2 * L>(); return; }
        }
        if constexpr (C::NBUF >= 3) {
            if (n >= 1) { wait_vmcnt<L>(); return; }
        }
        wait_vmcnt<0>();
    };

#pragma unroll
    for (int s = 0; s < C::NBUF - 1; ++s)
        if (s < nk) issue(s);
    for (int kb = 0; kb < nk; ++kb) {
        // Every wave's loads of stage kb have landed and every wave is done
        // with stage kb - 1, whose buffer the next loads overwrite.
        wait_stage(min(C::NBUF - 2, nk - 1 - kb));
        lds_barrier();
        if (kb + C::NBUF - 1 < nk) issue(kb + C::NBUF - 1);
        const char *sp = lds + (kb % C::NBUF) * C::STAGE, *sq = sp + C::PANEL;
        // fragments for k-group kg + 1 are read while the MFMAs of kg run
        frag fa[2][G::NBM], fb[2][G::NBN];
#pragma unroll
        for (int i = 0; i < G::NBM; ++i) fa[0][i] = operand_frag<T, ROWB>(sp, lane, a_blk + G::BLK * i, 0);
#pragma unroll
        for (int j = 0; j < G::NBN; ++j)
            fb[0][j] = QK ? kmajor_frag<T, RB>(sq, lane, G::col_blk(wn, j), 0)
                          : operand_frag<T, ROWB>(sq, lane, G::col_blk(wn, j), 0);
#pragma unroll
        for (int kg = 0; kg < G::KG; ++kg) {
            const int cb = kg & 1, nb = cb ^ 1;
            if (kg + 1 < G::KG) {
#pragma unroll
                for (int i = 0; i < G::NBM; ++i)
                    fa[nb][i] = operand_frag<T, ROWB>(sp, lane, a_blk + G::BLK * i, kg + 1);
#pragma unroll
                for (int j = 0; j < G::NBN; ++j)
                    fb[nb][j] = QK ? kmajor_frag<T, RB>(sq, lane, G::col_blk(wn, j), kg + 1)
                                   : operand_frag<T, ROWB>(sq, lane, G::col_blk(wn, j), kg + 1);
            }
            __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of this k-group's MFMAs
#pragma unroll
            for (int i = 0; i < G::NBM; ++i)
#pragma unroll
                for (int j = 0; j < G::NBN; ++j) acc[i][j] = Mfma<T>::mma(fa[cb][i], fb[cb][j], acc[i][j]);
        }
    }
}

// --- epilogue staging ------------------------------------------------------
// The rounded tile D (BM x BM, D[r][c]) is staged column-major: LDS row c holds
// D[0..BM)[c] (BM * es bytes), its 16-byte unit u at unit position
// u ^ swt(c). swt maps 16 consecutive columns to 16 distinct positions, so the
// staging writes (16 consecutive columns of bf16, 8 bytes each, or 32 of f32,
// 16 bytes each) spread over the banks, and it maps 4 consecutive columns to
// positions that differ in bits 1-2, so a transpose read (4 columns x 32
// bytes) touches 8 distinct positions.
__device__ __forceinline__ int swt(int c) { return ((c & 3) << 1) | (((c >> 2) & 1) << 3) | ((c >> 3) & 1); }

template <typename T, int BM>
__device__ __forceinline__ int stage_off(int c, int r) {   // byte offset of D[r][c]
    const int byte = r * (int)sizeof(T);
    return c * (BM * (int)sizeof(T)) + ((((byte >> 4) ^ swt(c)) << 4) | (byte & 15));
}

// D[r..r+3][c] = v into the staging area.
template <typename T, int BM>
__device__ __forceinline__ void stage4(char *lds, int r, int c, const float v[4]) {
    char *p = lds + stage_off<T, BM>(c, r);
    if constexpr (sizeof(T) == 2) {
        typedef __bf16 b4 __attribute__((ext_vector_type(4)));
        *reinterpret_cast<b4 *>(p) = b4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    } else {
        *reinterpret_cast<f32x4 *>(p) = f32x4{v[0], v[1], v[2], v[3]};
    }
}

// Row-major chunks of D: 16 bytes of row r starting at column c.
//   bf16: blocks of 16 rows x 32 columns; lane (t = l % 16, g = l / 16) takes
//         row r0 + t, columns c0 + 8 g .. + 8, from two LDS transpose reads:
//         lane t addresses column c + t / 4, rows r0 + 4 (t % 4) .. + 4 of the
//         staging, and receives rows r0 + t of columns c .. c + 3.
//   f32:  blocks of 16 rows x 16 columns; lane (t, g) takes row r0 + t,
//         columns c0 + 4 g .. + 4, from four 4-byte reads.
template <typename T, int BM> struct RowChunks {
    static constexpr int BCOLS = sizeof(T) == 2 ? 32 : 16;
    static constexpr int BLOCKS = (BM / 16) * (BM / BCOLS);
};

template <typename T, int BM>
__device__ __forceinline__ i32x4 row_chunk(const char *lds, int blk, int lane, int &r, int &c) {
    constexpr int BC = RowChunks<T, BM>::BCOLS;
    const int t = lane & 15, g = lane >> 4;
    const int r0 = (blk % (BM / 16)) * 16, c0 = (blk / (BM / 16)) * BC;
    r = r0 + t;
    if constexpr (sizeof(T) == 2) {
        c = c0 + 8 * g;
        s16x4 v[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const char *a = lds + stage_off<T, BM>(c + 4 * h + (t >> 2), r0 + 4 * (t & 3));
            v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((NSQ_LDS s16x4 *)a);
        }
        const s16x4 lo = v[0], hi = v[1];
        i32x4 w;
        w[0] = (int)(uint16_t)lo[0] | ((int)(uint16_t)lo[1] << 16);
        w[1] = (int)(uint16_t)lo[2] | ((int)(uint16_t)lo[3] << 16);
        w[2] = (int)(uint16_t)hi[0] | ((int)(uint16_t)hi[1] << 16);
        w[3] = (int)(uint16_t)hi[2] | ((int)(uint16_t)hi[3] << 16);
        return w;
    } else {
        c = c0 + 4 * g;
        i32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = *reinterpret_cast<const int *>(lds + stage_off<T, BM>(c + e, r));
        return w;
    }
}

// Column-major chunks of D (rows of the staging): 16 bytes of column c
// starting at row r = 16 u / es.
template <typename T, int BM>
__device__ __forceinline__ i32x4 col_chunk(const char *lds, int idx, int &c, int &r) {
    constexpr int NU = BM * (int)sizeof(T) / 16;
    c = idx / NU;
    const int u = idx % NU;
    r = u * (16 / (int)sizeof(T));
    return *reinterpret_cast<const i32x4 *>(lds + c * (BM * (int)sizeof(T)) + ((u ^ swt(c)) << 4));
}

template <typename T>
__device__ __forceinline__ void store16(char *base, int64_t elem, i32x4 w) {
    *(NSQ_GLOBAL i32x4 *)(base + elem * (int64_t)sizeof(T)) = w;
}

// 16 bytes at an address aligned only to the element size: one access in the
// GPU's unaligned access mode (caller tensors at arbitrary element offsets).
typedef i32x4 __attribute__((aligned(2))) i32x4_a2;   // 16 bytes, 2-byte alignment
template <typename T>
__device__ __forceinline__ i32x4 load16_unaligned(const char *p) {
    return *(const NSQ_GLOBAL i32x4_a2 *)p;
}
template <typename T>
__device__ __forceinline__ void store16_unaligned(char *p, i32x4 w) {
    *(NSQ_GLOBAL i32x4_a2 *)p = w;
}

// Bounds-checked store of the 16 / es elements of chunk w at [row][col] of the
// caller's output (rows x cols as stored), row in piece pc.
template <typename T>
__device__ __forceinline__ void store_chunk_in_piece(const NsProb &pr, const RowPiece &pc, int64_t rows,
                                                     int64_t cols, int64_t row, int64_t col, i32x4 w) {
    constexpr int E = 16 / (int)sizeof(T);
    if (row >= rows || col >= cols) return;
    char *dst = pc.out + (row - pc.row0) * pc.ld_out * (int64_t)sizeof(T);
    if (col + E <= cols) {
        if (pr.vec_out) store16<T>(dst, col, w);
        else store16_unaligned<T>(dst + col * (int64_t)sizeof(T), w);
        return;
    }
    T vals[E];
    __builtin_memcpy(vals, &w, 16);
    NSQ_GLOBAL T *p = gp<T>(dst);
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (col + e < cols) p[col + e] = vals[e];
}

// The same with the row spread over band[0 .. nband) (rows sorted by row0).
template <typename T>
__device__ __forceinline__ void store_chunk_checked(const NsProb &pr, const RowPiece *band, int nband,
                                                    int64_t rows, int64_t cols, int64_t row, int64_t col, i32x4 w) {
    if (row >= rows || col >= cols) return;
    store_chunk_in_piece<T>(pr, find_piece(band, nband, row), rows, cols, row, col, w);
}

template <typename T, class C>
__device__ __forceinline__ void zero_acc(AccTile<T, C> &acc) {
    typedef typename C::template Geo<T> G;
#pragma unroll
    for (int i = 0; i < G::NBM; ++i)
#pragma unroll
        for (int j = 0; j < G::NBN; ++j)
#pragma unroll
            for (int v = 0; v < 4 * Mfma<T>::NQ; ++v) acc[i][j][v] = 0.f;
}

// acc = s * M[row0 + r][col0 + c] for this wave's accumulator elements, M
// row-major with row stride ld bytes. The BM x BM tile of M goes global -> LDS
// first (load_init_tile: coalesced, rows of BM * es bytes, the 16-byte unit u
// of row r at unit position u ^ 2 (r % 4)); each lane then picks its
// accumulator layout (four consecutive rows of one column) out of it
// (init_quad): for bf16 with LDS transpose reads (in each 16-lane group lane t
// addresses row r0 + t / 4, columns c0 + 4 (t % 4) .. + 4, and receives rows
// r0 .. r0 + 3 of column c0 + t), for f32 with four 4-byte reads. Ends with a
// barrier: the LDS is free again.
template <typename T, class C>
__device__ __forceinline__ void load_init_tile(const char *M, int ld, int row0, int col0, char *lds) {
    constexpr int ES = sizeof(T), RB = C::BM * ES, RPI = 1024 / RB, NI = C::BM / RPI / C::WAVES;
    static_assert(C::BM % (RPI * C::WAVES) == 0, "whole 1 KiB loads per wave");
    const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
    const char *base = M + (int64_t)row0 * ld + (int64_t)col0 * ES;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0, C::BM * ld, 0x00020000);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int blk = wave * NI + i;                        // 1 KiB block of the staged tile
        const int row = blk * RPI + (lane * 16) / RB;
        const int pos = ((lane * 16) % RB) >> 4;              // unit position in the LDS row
        const int voff = row * ld + ((pos ^ (2 * (row & 3))) << 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (NSQ_LDS void *)(lds + blk * 1024), 16, voff, 0, 0, 0);
    }
    __syncthreads();   // waits for this wave's loads, then for every wave's
}

// s * the staged tile's rows rb .. rb + 3 of this lane's column: cb + lane %
// BLK (bf16: cb + 16 ((lane / 16) % (BLK / 16)) + lane % 16).
template <typename T, int BM, int BLK>
__device__ __forceinline__ void init_quad(const char *lds, int lane, int rb, int cb, float s, float out[4]) {
    constexpr int ES = sizeof(T), RB = BM * ES;
    auto at = [&](int r, int c) -> const char * {
        const int byte = c * ES;
        return lds + r * RB + ((((byte >> 4) ^ (2 * (r & 3)))) << 4) + (byte & 15);
    };
    float old[4];
    if constexpr (ES == 2) {
        const int t = lane & 15, c0 = cb + 16 * ((lane >> 4) & (BLK / 16 - 1));
        const s16x4 w = __builtin_amdgcn_ds_read_tr16_b64_v4i16((NSQ_LDS s16x4 *)at(rb + (t >> 2), c0 + 4 * (t & 3)));
#pragma unroll
        for (int e = 0; e < 4; ++e) old[e] = __builtin_bit_cast(float, (uint32_t)(uint16_t)w[e] << 16);   // bf16 -> fp32
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) old[e] = *reinterpret_cast<const float *>(at(rb + e, cb + lane % BLK));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = s * old[e];
}

template <typename T, class C>
__device__ __forceinline__ void init_acc(const char *M, int ld, int row0, int col0, float s, char *lds,
                                         AccTile<T, C> &acc) {
    typedef typename C::template Geo<T> G;
    const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
    const int wm = wave / C::WN, wn = wave % C::WN;
    load_init_tile<T, C>(M, ld, row0, col0, lds);
#pragma unroll
    for (int i = 0; i < G::NBM; ++i)
#pragma unroll
        for (int j = 0; j < G::NBN; ++j)
#pragma unroll
            for (int q = 0; q < Mfma<T>::NQ; ++q) {
                float v[4];
                init_quad<T, C::BM, G::BLK>(lds, lane, wm * (C::BM / C::WM) + i * G::BLK + Mfma<T>::out_row(lane, q),
                                            G::col_blk(wn, j), s, v);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] = v[e];
            }
    __syncthreads();   // every wave is done with the staged tile
}

// Accumulator values -> the values stored (before rounding to the stored
// type): times s_final (B X: as they are), plus s_diag on the matrix diagonal
// (rows < m) for the modes that add one. Element e sits at tile row r + e,
// tile column c of a tile whose first row is row0; diag_tile: ti == tj.
template <int MODE>
__device__ __forceinline__ void finish4(float v[4], float s_final, float s_diag, bool diag_tile, int r, int c,
                                        int row0, int m) {
    constexpr bool kDiag = MODE == kSyrkA || MODE == kGramB0 || MODE == kGramG || MODE == kGramAA;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (MODE != kGemmBX) v[e] = __fmul_rn(s_final, v[e]);
        if constexpr (kDiag)
            if (diag_tile && r + e == c && row0 + r + e < m) v[e] = __fadd_rn(v[e], s_diag);
    }
}

// The normalisation scale 1 / (||G||_F + eps) of one matrix from its partial
// sums of squares, reduced in a fixed order: partial k goes to slot
// k % kScaleSlots (summed in increasing k), then the slots are summed as a
// binary tree. Independent of the workgroup size (>= kScaleSlots threads), so
// every kernel that needs it gets the same bits. `red` is kScaleSlots floats of
// LDS; ends with a barrier.
__device__ __forceinline__ float norm_scale(const float *partials, int nparts, float eps, float *red,
                                            float *total_out = nullptr) {
    const int t = threadIdx.x;
    if (t < kScaleSlots) {
        float v = 0.f;
        for (int k = t; k < nparts; k += kScaleSlots) v += partials[k];
        red[t] = v;
    }
    __syncthreads();
#pragma unroll
    for (int w = kScaleSlots / 2; w > 0; w >>= 1) {
        if (t < w) red[t] += red[t + w];
        __syncthreads();
    }
    const float total = red[0];
    __syncthreads();
    if (total_out) *total_out = total;
    // A sum of squares past fp32 range (||G||_F above about 1.8e19), or an
    // input holding inf or NaN, gives a NaN scale: every output element is then
    // NaN, rather than the zeros a zero scale would give.
    if (!(total <= 3.402823466e38f)) return __builtin_nanf("");
    return 1.0f / (sqrtf(total) + eps);
}

// The first step's products fold the normalisation s = 1 / (||G||_F + eps)
// into their scales (X0 in the workspace holds G unscaled): A0 = s^2 G G^T,
// B0' scaled by s, and in the Gram space G = s^2 X0 X0^T (ridge times
// tr(G) / m on the diagonal) and out = s Q X0. `lds` holds kScaleSlots floats
// of scratch; ends with a barrier.
template <int MODE>
__device__ __forceinline__ void fold_norm(const NsProb &pr, float eps, char *lds, float &s_final, float &s_diag) {
    float total;
    const float sc = norm_scale(pr.partials, pr.nparts, eps, reinterpret_cast<float *>(lds), &total);
    if constexpr (MODE == kSyrkX) s_final = sc * sc;
    else if constexpr (MODE == kSyrkA) {
        s_final *= sc;
        s_diag *= sc;
    } else if constexpr (MODE == kGramG) {
        s_final = sc * sc;
        s_diag *= sc * sc * total / (float)pr.m;   // ridge * tr(G) / m, tr(G) = s^2 ||input||^2
    } else if constexpr (MODE == kGramOut) {
        s_final = sc;
    }
}

// One product launch: MODE picks the operands and epilogue.
//   kSyrkX : A = X X^T                          P = X, Q = X     upper tiles, mirrored
//   kSyrkA : B' = s_final (s_init A + A A^T) + s_diag I
//                                               P = A, Q = A     upper tiles, mirrored
//   kGemmBX: X' = B' X                          P = B', Q = X read K-major
// The step X' = a X + B X with B = b A + c A A is computed as X' = B' X with
// B' = a I + B: the a X term becomes a on B's diagonal (added in fp32 before
// B' is rounded), so the B X product needs no old tile. The A A product's
// accumulators start at s_init times the old A tile: with (s_init, s_final) =
// (b / c, c), B = b A + c A A up to fp32 rounding; when c == 0 (or b / c is
// not finite, where c A A is below fp32 resolution of b A) the host passes
// (b, 1) and do_product = 0, so B = b A. s_diag = a, added for rows < m only.
// FIRST (the first step): X0 in the workspace holds the input G unscaled, and
// the normalisation X0 = s G, s = 1 / (||G||_F + eps), is folded in here:
// A0 = s^2 (G G^T), and B0' is stored scaled by s, so X1 = (s B0') G.
// LAST (kGemmBX only): the final step writes B' X straight to the caller's
// output in the input's orientation instead of into the workspace.
// LDS bytes of one product tile: the operand ring, or the staged output tile.
template <typename T, class C> constexpr int tile_lds_bytes() {
    return C::RING > C::BM * C::BM * (int)sizeof(T) ? C::RING : C::BM * C::BM * (int)sizeof(T);
}

// Epilogue, part 2, of one BM x BM tile: writes the tile staged in `lds` (in
// the type it is stored in: the workspace type, or the output's for the last
// launch) to its destinations. Every wave of the workgroup calls it after the
// staging barrier.
template <typename T, class C, int MODE, bool LAST, typename TO>
__device__ __forceinline__ void write_staged(const NsProb &pr, const TileRef tr, int32_t cur,
                                             const RowPiece *__restrict__ pieces, const char *lds) {
    typedef typename std::conditional<LAST, TO, T>::type TS;
    constexpr int BM = C::BM, ES = sizeof(T), SES = sizeof(TS);
    const int row0 = tr.ti * BM, col0 = tr.tj * BM;
    const int ldx = pr.ldx, ldxt = pr.ldxt, ldt = pr.ldt;
    char *xn = cur ? pr.x0 : pr.x1;
    char *xtn = cur ? pr.xt0 : pr.xt1;
    char *qn = cur ? pr.q0 : pr.q1;
    char *A = pr.a, *B = pr.b;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // A diagonal tile of the A A product writes its lower half from its upper
    // half, so the stored B' is symmetric bit for bit whatever order the
    // matrix cores sum in (elements (i, j) and (j, i) start from the same
    // s_init A value and add the same products, in the same k order). Row r's
    // elements left of the diagonal are staged column r's, which the row
    // stores below pick up with one extra 16-byte read per chunk.
    const bool mirror_lower = MODE == kSyrkA && tr.ti == tr.tj;

    // Epilogue, part 2: write the staged tile.
    constexpr int NU = BM * SES / 16;                // 16-byte units per staged column
    constexpr int COL_CHUNKS = BM * NU;
    if constexpr (!LAST) {
        // row-major: the tile itself, at (row0, col0)
        char *D = MODE == kSyrkX ? A : MODE == kSyrkA ? B : MODE == kGemmBX ? xn : MODE == kGramG ? pr.g
                : MODE == kGramQG ? pr.t : MODE == kGramTQ ? A : MODE == kGramAA ? B : qn;   // B0, BQ: next Q
        const int ldd = MODE == kGemmBX ? ldx : ldt;
        // Fixed trip counts, unrolled by 4: the LDS reads of four iterations
        // go out before their stores instead of one read-wait-store at a time.
        static_assert(RowChunks<T, BM>::BLOCKS % C::WAVES == 0, "whole row blocks per wave");
#pragma unroll 4
        for (int it = 0; it < RowChunks<T, BM>::BLOCKS / C::WAVES; ++it) {
            const int blk = wave + it * C::WAVES;
            int r, c;
            i32x4 w = row_chunk<T, BM>(lds, blk, lane, r, c);
            if (mirror_lower && c < r) {   // elements c .. c + 16/es - 1 of row r; those left of r mirrored
                constexpr int E = 16 / ES;
                const i32x4 lo = *reinterpret_cast<const i32x4 *>(lds + r * (BM * ES) + (((c * ES >> 4) ^ swt(r)) << 4));
                T up[E], dn[E];
                __builtin_memcpy(up, &w, 16);
                __builtin_memcpy(dn, &lo, 16);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (c + e < r) up[e] = dn[e];
                __builtin_memcpy(&w, up, 16);
            }
            store16<T>(D, (int64_t)(row0 + r) * ldd + col0 + c, w);
        }
        // column-major: the mirror tile at (col0, row0), or the transpose
        if (writes_transpose(MODE) || (MODE == kGemmBX && !pr.kmajor) || (symmetric_mode(MODE) && tr.ti != tr.tj)) {
            char *qtn = cur ? pr.qt0 : pr.qt1;
            char *E = MODE == kGemmBX ? xtn : MODE == kGramTQ ? pr.at : MODE == kGramB0 || MODE == kGramBQ ? qtn : D;
            const int lde = MODE == kGemmBX ? ldxt : ldt;
            static_assert(COL_CHUNKS % C::THREADS == 0, "whole column chunks per thread");
#pragma unroll 4
            for (int it = 0; it < COL_CHUNKS / C::THREADS; ++it) {
                const int idx = threadIdx.x + it * C::THREADS;
                int c, r;
                const i32x4 w = col_chunk<T, BM>(lds, idx, c, r);
                store16<T>(E, (int64_t)(col0 + c) * lde + row0 + r, w);
            }
        }
    } else {
        const int m = pr.m, n = pr.n;
        const RowPiece *band = pieces + tr.piece;
        static_assert(RowChunks<TS, BM>::BLOCKS % C::WAVES == 0 && COL_CHUNKS % C::THREADS == 0,
                      "whole chunks per wave and thread");
        // A tile whose output rows lie in one piece (the usual case) reads
        // that piece once: a descriptor load inside the loop would make each
        // chunk wait for it, and with it for every store issued before
        // (the same counter tracks both).
        const bool one = tr.npiece == 1;
        const RowPiece pc0 = band[0];
        auto put = [&](int64_t rows, int64_t cols, int64_t row, int64_t col, i32x4 w) {
            if (one) store_chunk_in_piece<TS>(pr, pc0, rows, cols, row, col, w);
            else store_chunk_checked<TS>(pr, band, tr.npiece, rows, cols, row, col, w);
        };
        if (!pr.tall) {   // out is m x n: row-major chunks
#pragma unroll 4
            for (int it = 0; it < RowChunks<TS, BM>::BLOCKS / C::WAVES; ++it) {
                const int blk = wave + it * C::WAVES;
                int r, c;
                const i32x4 w = row_chunk<TS, BM>(lds, blk, lane, r, c);
                put(m, n, row0 + r, col0 + c, w);
            }
        } else {          // out is n x m: column-major chunks
#pragma unroll 4
            for (int it = 0; it < COL_CHUNKS / C::THREADS; ++it) {
                const int idx = threadIdx.x + it * C::THREADS;
                int c, r;
                const i32x4 w = col_chunk<TS, BM>(lds, idx, c, r);
                put(n, m, col0 + c, row0 + r, w);
            }
        }
    }
}

// One BM x BM tile `tr` of matrix `pr` for the product MODE (see Mode). The
// caller's workgroup runs it whole; `lds` is tile_lds_bytes() of LDS, free on
// entry and free again on return.
template <typename T, class C, int MODE, bool LAST, typename TO = T>
__device__ __forceinline__ void run_tile(const NsProb &pr, const TileRef tr, int32_t cur, float s_init,
                                         float s_final, float s_diag, int32_t do_product, int32_t first,
                                         float eps, const RowPiece *__restrict__ pieces, char *lds) {
    static_assert(!LAST || MODE == kGemmBX || MODE == kGramOut, "only B X or the Gram-space output writes out");
    static_assert(MODE != kGramOut || LAST, "the Gram-space output launch is a last launch");
    constexpr int BM = C::BM, ES = sizeof(T);
    const int mp = pr.mp, np = pr.np;
    const int row0 = tr.ti * BM, col0 = tr.tj * BM;
    const int ldx = pr.ldx, ldxt = pr.ldxt, ldt = pr.ldt;
    char *xc = cur ? pr.x1 : pr.x0;
    char *xtc = cur ? pr.xt1 : pr.xt0;
    char *qc = cur ? pr.q1 : pr.q0;
    char *A = pr.a, *B = pr.b;
    if (first) fold_norm<MODE>(pr, eps, lds, s_final, s_diag);

    // K stages of the NS products: the K extent (n for X X^T, m for A A and
    // B' X) rounded up to a whole stage; the zero padding past it adds nothing.
    // The Gram-space products run over the padded extents.
    constexpr int KW = C::ROWB / ES;
    constexpr bool kTrim = MODE == kSyrkX || MODE == kSyrkA || MODE == kGemmBX;
    const int nk_n = kTrim ? (pr.n + KW - 1) / KW : np / KW;
    const int nk_m = kTrim ? (pr.m + KW - 1) / KW : mp / KW;
    typedef typename C::template Geo<T> G;
    AccTile<T, C> acc;
    if constexpr (MODE == kSyrkX || MODE == kGramG) {
        zero_acc<T, C>(acc);
        const int ld = ldx * ES;
        tile_product<T, C>(xc + (int64_t)row0 * ld, xc + (int64_t)col0 * ld, ld, ld, BM * ld, BM * ld,
                           nk_n, lds, acc);
    } else if constexpr (MODE == kSyrkA || MODE == kGramB0 || MODE == kGramAA) {
        // S S with S symmetric (A, G): the Q operand is S's rows; the general
        // A A of the Gram space reads A^T's rows instead
        const int ld = ldt * ES;
        char *S = MODE == kSyrkA ? A : MODE == kGramB0 ? pr.g : A;
        char *SQ = MODE == kGramAA ? pr.at : S;
        // the accumulators start at s_init times the old tile S[row0.., col0..]
        init_acc<T, C>(S, ld, row0, col0, s_init, lds, acc);
        if (do_product)
            tile_product<T, C>(S + (int64_t)row0 * ld, SQ + (int64_t)col0 * ld, ld, ld, BM * ld, BM * ld, nk_m,
                               lds, acc);
    } else if constexpr (MODE == kGemmBX || MODE == kGramOut) {
        // B' X, or Q X0 in the Gram space: X read K-major, as stored, or (B' X
        // with a long K) the rows of the stored X^T
        zero_acc<T, C>(acc);
        char *P = MODE == kGemmBX ? B : qc;
        const int ldp = ldt * ES;
        if (MODE == kGramOut || pr.kmajor) {
            char *X = MODE == kGemmBX ? xc : pr.x0;
            const int ldq = ldx * ES;
            tile_product<T, C, true>(P + (int64_t)row0 * ldp, X + (int64_t)col0 * ES, ldp, ldq, BM * ldp,
                                            mp * ldq - col0 * ES, nk_m, lds, acc);
        } else {
            const int ldq = ldxt * ES;
            tile_product<T, C>(P + (int64_t)row0 * ldp, xtc + (int64_t)col0 * ldq, ldp, ldq, BM * ldp, BM * ldq,
                               nk_m, lds, acc);
        }
    } else {   // the other Gram-space products, all with K = mp
        char *qtc = cur ? pr.qt1 : pr.qt0;
        char *P = MODE == kGramQG ? qc : MODE == kGramTQ ? pr.t : MODE == kGramBQ ? B : qc;
        char *Q = MODE == kGramQG ? pr.g : qtc;   // G symmetric; else the transposes kept for this
        const int ldp = ldt * ES, ldq = ldt * ES;
        zero_acc<T, C>(acc);
        tile_product<T, C>(P + (int64_t)row0 * ldp, Q + (int64_t)col0 * ldq, ldp, ldq, BM * ldp, BM * ldq,
                           nk_m, lds, acc);
    }

    // Epilogue, part 1: scaling, rounding, staging. Accumulator element
    // (i, j, 4 q + e) of this lane sits at tile row wm*BM/WM + BLK i +
    // out_row(lane, q) + e and tile column col_blk(wn, j) + lane % BLK. The
    // tile is staged in the type it is stored in: the workspace type, or the
    // output's.
    typedef typename std::conditional<LAST, TO, T>::type TS;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    __syncthreads();   // every wave is done reading operand panels
#pragma unroll
    for (int i = 0; i < G::NBM; ++i) {
#pragma unroll
        for (int j = 0; j < G::NBN; ++j) {
            const int c = G::col_blk(wn, j) + lane % G::BLK;
#pragma unroll
            for (int q = 0; q < Mfma<T>::NQ; ++q) {
                const int r = wm * (BM / C::WM) + i * G::BLK + Mfma<T>::out_row(lane, q);
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
                finish4<MODE>(v, s_final, s_diag, tr.ti == tr.tj, r, c, row0, pr.m);
                stage4<TS, BM>(lds, r, c, v);
            }
        }
    }
    __syncthreads();
    write_staged<T, C, MODE, LAST, TO>(pr, tr, cur, pieces, lds);
}

// One product launch: every tile of `tiles` (hardware workgroup ids remapped
// so each XCD takes a contiguous range of the list).
template <typename T, class C, int MODE, bool LAST, typename TO = T>
__global__ __launch_bounds__(C::THREADS, C::BM == 256 ? 1 : 2) void ns_product_kernel(
    const NsProb *__restrict__ probs, const TileRef *__restrict__ tiles, int32_t ntiles, int32_t cur,
    float s_init, float s_final, float s_diag, int32_t do_product, int32_t first, float eps,
    const RowPiece *__restrict__ pieces) {
    __shared__ __attribute__((aligned(1024))) char lds[tile_lds_bytes<T, C>()];
    const int tile_id = xcd_remap(blockIdx.x, gridDim.x);
    if (tile_id >= ntiles) return;
    const TileRef tr = tiles[tile_id];
    run_tile<T, C, MODE, LAST, TO>(probs[tr.prob], tr, cur, s_init, s_final, s_diag, do_product, first, eps,
                                   pieces, lds);
}


// --- bf16 256-tiles on four waves, accumulators in fixed registers -----------
// The bf16 256 x 256 tiles of X X^T, A A and B' X run here by default: four
// waves of 128 x 128 (one per SIMD), the same two stage buffers filled by
// direct-to-LDS loads as the 8-wave kernel, and each wave's 8 x 8 blocks of
// 16 x 16 accumulators held in the AGPRs a0..a255 for the whole tile: every
// MFMA names its block's registers (acc_pinned.h), because the register
// allocator, left to itself, moves a tile this size between registers inside
// the K loop. One K stage is an unrolled schedule (pinned_stage.inc): k-group
// 0's MFMAs in pairs with k-group 1's fragment reads between them, then
// k-group 1's pairs with, after the first pair, the wait for the next stage
// and the barrier, and then the loads two stages ahead and the next stage's
// first fragment reads. Same MFMA, same k order and the same epilogue
// arithmetic as the 8-wave kernel, so the two give the same bits.
#include "acc_pinned.h"

typedef TileCfg<256, 2, 2, 128, 2> Quad;   // 4 waves, 128 x 128 per wave, two 64 KiB stages

// Pinned accumulators += P Q^T over nk >= 1 stages of the 256 tile; operands
// and QK as in tile_product. Wave (wm, wn) = (wave / 2, wave % 2) owns tile
// rows wm 128 .. + 128 and columns wn 128 .. + 128; its block q = 8 i + j
// covers rows wm 128 + 16 i .., columns wn 128 + 16 j ... Load n < 8 of a
// stage brings rows wave 64 + 8 n .. + 8 of the P panel, load 8 + n the same
// rows of the Q panel (K-major Q: its k-rows wave 16 + 2 n, + 1, the same LDS
// bytes).
template <bool QK>
__device__ __forceinline__ void pinned_product(const char *P, const char *Q, int ldp, int ldq, int extent_p,
                                               int extent_q, int nk, char *lds) {
    typedef Quad C;
    constexpr int ROWB = C::ROWB, PANEL = C::PANEL, STAGE = C::STAGE;
    constexpr int KW = ROWB / 2, RB = C::BM * 2;   // K-major: KW k-rows of RB bytes per stage
    static_assert(C::WAVES == 4 && C::LOADS == 8 && C::RPI == 8, "load layout");
    const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const __amdgpu_buffer_rsrc_t rp =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(P), (short)0, extent_p, 0x00020000);
    const __amdgpu_buffer_rsrc_t rq =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(Q), (short)0, extent_q, 0x00020000);
    int voff_p[8], voff_q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = wave * 64 + 8 * i + (lane >> 3);
        const int chunk = ((lane & 7) ^ swz<ROWB>(row)) << 4;
        voff_p[i] = row * ldp + chunk;
        if constexpr (QK) {
            const int k = wave * 16 + 2 * i + (lane >> 5);
            voff_q[i] = k * ldq + (((lane & 31) ^ swq<2>(k)) << 4);
        } else {
            voff_q[i] = row * ldq + chunk;
        }
    }
    const int q_stage = QK ? KW * ldq : ROWB;   // byte step of Q per stage
    auto ld = [&](int n, int kb, int buf) {
        char *dst = lds + buf * STAGE + (n < 8 ? 0 : PANEL) + (wave * 64 + 8 * (n & 7)) * ROWB;
        if (n < 8)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rp, (NSQ_LDS void *)dst, 16, voff_p[n & 7], kb * ROWB, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (NSQ_LDS void *)dst, 16, voff_q[n & 7], kb * q_stage, 0, 0);
    };
    // fragment x < 8: P block x (rows wm 128 + 16 x ..); x >= 8: Q block x - 8
    const int fsw = swz<ROWB>(lane & 15);
    const int a_off = (wm * 128 + (lane & 15)) * ROWB, b_off = PANEL + (wn * 128 + (lane & 15)) * ROWB;
    bf16x8 F[2][16];
    auto rf = [&](int slot, int buf, int kg, int x) {
        const char *sb = lds + buf * STAGE;
        if (QK && x >= 8) {
            F[slot][x] = kmajor_frag<__bf16, RB>(sb + PANEL, lane, wn * 128 + 16 * (x - 8), kg);
        } else {
            const int c = ((4 * kg + (lane >> 4)) ^ fsw) << 4;
            F[slot][x] = *reinterpret_cast<const bf16x8 *>(
                sb + (x < 8 ? a_off + 16 * x * ROWB : b_off + 16 * (x - 8) * ROWB) + c);
        }
    };
    // stage 0 landed in buffer 0, stage 1 on its way to buffer 1, stage 0's
    // first fragments read
#pragma unroll
    for (int n = 0; n < 16; ++n) ld(n, 0, 0);
    wait_vmcnt<0>();
    lds_barrier();
    if (nk > 1) {
#pragma unroll
        for (int n = 0; n < 16; ++n) ld(n, 1, 1);
    }
#pragma unroll
    for (int n = 0; n < 16; ++n) rf(0, 0, 0, n < 8 ? 8 + n : n - 8);
    // Stage kb in buffer PAR = kb % 2. W: a stage kb + 1 exists (wait for it,
    // barrier, read its first fragments); L: a stage kb + 2 exists (load it
    // into buffer PAR once every wave is past the barrier).
    auto stage = [&](auto par, auto w, auto l, int kb) {
        constexpr int PAR = decltype(par)::value;
        constexpr bool W = decltype(w)::value, L = decltype(l)::value;
#include "pinned_stage.inc"
    };
    typedef std::integral_constant<int, 0> B0;
    typedef std::integral_constant<int, 1> B1;
    typedef std::true_type Y;
    typedef std::false_type N;
    int kb = 0;
    for (; kb + 3 < nk; kb += 2) {
        stage(B0{}, Y{}, Y{}, kb);
        stage(B1{}, Y{}, Y{}, kb + 1);
    }
    if (nk - kb == 3) {
        stage(B0{}, Y{}, Y{}, kb);
        stage(B1{}, Y{}, N{}, kb + 1);
        stage(B0{}, N{}, N{}, kb + 2);
    } else if (nk - kb == 2) {
        stage(B0{}, Y{}, N{}, kb);
        stage(B1{}, N{}, N{}, kb + 1);
    } else {
        stage(B0{}, N{}, N{}, kb);
    }
    pinned::drain();
}

// Pinned accumulators = s * M[row0 + r][col0 + c] (the 256 tile of M, row
// stride ld bytes), through LDS as in init_acc; ends with a barrier.
__device__ __forceinline__ void pinned_init(const char *M, int ld, int row0, int col0, float s, char *lds) {
    const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    load_init_tile<__bf16, Quad>(M, ld, row0, col0, lds);
    pinned::init_each_block([&](auto qc) -> f32x4 {
        constexpr int q = decltype(qc)::value;
        float v[4];
        init_quad<__bf16, 256, 16>(lds, lane, wm * 128 + 16 * (q >> 3) + 4 * (lane >> 4), wn * 128 + 16 * (q & 7), s,
                                   v);
        return f32x4{v[0], v[1], v[2], v[3]};
    });
    __syncthreads();
}

// One 256 x 256 tile for MODE in {kSyrkX, kSyrkA, kGemmBX} on four waves:
// operands, scales and results as run_tile's. The descriptor comes in as a
// __restrict__ pointer that every mode reads: inlining then tags each other
// memory access of the tile, the LDS transpose reads included, as not
// aliasing it, and with such a tag the compiler does not make an LDS read
// wait for the direct-to-LDS loads in flight (untagged, a transpose read
// would wait for the next stage's loads; the schedule's own waits order the
// stages).
template <int MODE, bool LAST>
__device__ __forceinline__ void pinned_tile(const NsProb *__restrict__ prp, const TileRef tr, int32_t cur,
                                            float s_init, float s_final, float s_diag, int32_t do_product,
                                            int32_t first, float eps, const RowPiece *__restrict__ pieces,
                                            char *lds) {
    static_assert(MODE == kSyrkX || MODE == kSyrkA || MODE == kGemmBX, "NS products only");
    static_assert(!LAST || MODE == kGemmBX, "only B X writes out");
    typedef __bf16 T;
    const NsProb &pr = *prp;
    constexpr int BM = Quad::BM, ES = 2, KW = Quad::ROWB / ES;
    const int row0 = tr.ti * BM, col0 = tr.tj * BM;
    char *xc = cur ? pr.x1 : pr.x0;
    char *xtc = cur ? pr.xt1 : pr.xt0;
    if (first) fold_norm<MODE>(pr, eps, lds, s_final, s_diag);
    const int nk_n = (pr.n + KW - 1) / KW, nk_m = (pr.m + KW - 1) / KW;
    if constexpr (MODE == kSyrkX) {
        const int ld = pr.ldx * ES;
        pinned::zero();
        pinned_product<false>(xc + (int64_t)row0 * ld, xc + (int64_t)col0 * ld, ld, ld, BM * ld, BM * ld, nk_n, lds);
    } else if constexpr (MODE == kSyrkA) {
        const int ld = pr.ldt * ES;
        pinned_init(pr.a, ld, row0, col0, s_init, lds);
        if (do_product)
            pinned_product<false>(pr.a + (int64_t)row0 * ld, pr.a + (int64_t)col0 * ld, ld, ld, BM * ld, BM * ld,
                                  nk_m, lds);
    } else {
        const int ldp = pr.ldt * ES;
        pinned::zero();
        if (pr.kmajor) {
            const int ldq = pr.ldx * ES;
            pinned_product<true>(pr.b + (int64_t)row0 * ldp, xc + (int64_t)col0 * ES, ldp, ldq, BM * ldp,
                                 pr.mp * ldq - col0 * ES, nk_m, lds);
        } else {
            const int ldq = pr.ldxt * ES;
            pinned_product<false>(pr.b + (int64_t)row0 * ldp, xtc + (int64_t)col0 * ldq, ldp, ldq, BM * ldp,
                                  BM * ldq, nk_m, lds);
        }
    }
    // Epilogue, part 1: block q = 8 i + j's element e of this lane sits at tile
    // row wm 128 + 16 i + 4 (lane / 16) + e, column wn 128 + 16 j + lane % 16.
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    __syncthreads();   // every wave is done reading operand panels
    pinned::each_block([&](auto qc, f32x4 a) {
        constexpr int q = decltype(qc)::value;
        const int r = wm * 128 + 16 * (q >> 3) + 4 * (lane >> 4), c = wn * 128 + 16 * (q & 7) + (lane & 15);
        float v[4] = {a[0], a[1], a[2], a[3]};
        finish4<MODE>(v, s_final, s_diag, tr.ti == tr.tj, r, c, row0, pr.m);
        stage4<T, BM>(lds, r, c, v);
    });
    __syncthreads();
    write_staged<T, Quad, MODE, LAST, T>(pr, tr, cur, pieces, lds);
}

template <int MODE, bool LAST>
__global__ __launch_bounds__(Quad::THREADS, 1) void ns_pinned_kernel(
    const NsProb *__restrict__ probs, const TileRef *__restrict__ tiles, int32_t ntiles, int32_t cur,
    float s_init, float s_final, float s_diag, int32_t do_product, int32_t first, float eps,
    const RowPiece *__restrict__ pieces) {
    __shared__ __attribute__((aligned(1024))) char lds[tile_lds_bytes<__bf16, Quad>()];
    const int tile_id = xcd_remap(blockIdx.x, gridDim.x);
    if (tile_id >= ntiles) return;
    const TileRef tr = tiles[tile_id];
    pinned_tile<MODE, LAST>(probs + tr.prob, tr, cur, s_init, s_final, s_diag, do_product, first, eps, pieces, lds);
}

// Ends a phase of the small-matrix kernel: every thread's global stores of
// this phase are complete (release at workgroup scope), the workgroup meets,
// and its later loads see them (acquire at workgroup scope). Only this
// workgroup reads what it wrote, and it runs on one CU, so workgroup scope is
// enough; agent scope would write back and invalidate the XCD's whole L2 at
// every phase.
// The explicit vmcnt(0) makes every store of this thread complete at the L2
// before the barrier, whatever path the next phase's direct-to-LDS loads take.
__device__ __forceinline__ void phase_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    wait_vmcnt<0>();
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// The small size class ("[GTP][Muon] Optimize Muon step performance", Current
// Progress: shape-batched NS over many small tensors): one workgroup runs
// every step of one matrix with m <= kSmallM (padded to 128 x np), phase after
// phase: the X X^T tile, the A A tile, then the np / 128 tiles of B' X
// (bx_tiles[mats[i].piece ..] with their output pieces), each phase finished
// by the whole workgroup before the next starts. The tiles are the product
// kernel's 128-tiles, so the bits equal the tiled path's.
template <typename T>
__global__ __launch_bounds__(Small::THREADS, 2) void ns_small_kernel(
    const NsProb *__restrict__ probs, const TileRef *__restrict__ mats, const TileRef *__restrict__ bx_tiles,
    int32_t steps, float sa_init, float sa_final, float s_diag, int32_t sa_product, float eps,
    const RowPiece *__restrict__ pieces) {
    __shared__ __attribute__((aligned(1024))) char lds[tile_lds_bytes<T, Small>()];
    const TileRef m = mats[blockIdx.x];
    const NsProb &pr = probs[m.prob];
    const TileRef diag{m.prob, 0, 0, 0, 1};
    int32_t cur = 0;
    for (int32_t s = 0; s < steps; ++s) {
        const int32_t first = s == 0;
        run_tile<T, Small, kSyrkX, false>(pr, diag, cur, 1.f, 1.f, 0.f, 1, first, eps, pieces, lds);
        phase_fence();
        run_tile<T, Small, kSyrkA, false>(pr, diag, cur, sa_init, sa_final, s_diag, sa_product, first, eps, pieces,
                                          lds);
        phase_fence();
        for (int32_t k = 0; k < m.npiece; ++k) {
            const TileRef tr = bx_tiles[m.piece + k];
            if (k > 0) __syncthreads();   // the previous tile's epilogue is done with the LDS
            if (s + 1 < steps)
                run_tile<T, Small, kGemmBX, false>(pr, tr, cur, 1.f, 1.f, 0.f, 1, first, eps, pieces, lds);
            else
                run_tile<T, Small, kGemmBX, true>(pr, tr, cur, 1.f, 1.f, 0.f, 1, first, eps, pieces, lds);
        }
        phase_fence();
        cur ^= 1;
    }
}

// Input staging, one kPrepTile x kPrepTile tile of X (m x n, oriented) per
// workgroup: the input G goes unscaled into X0, and into X0^T unless the
// matrix is kmajor (zero in the padding), and the tile's fp32 sum of squares
// goes to partials[ti * (np / kPrepTile) + tj], summed in a fixed order. The
// tile is read as stored (rows of G; for a tall G those are columns of X),
// copied straight to the matching array (X0, or X0^T for a tall G) with
// 16-byte stores, and staged in LDS (rows of kPrepTile * es bytes, the 16-byte
// unit u of row r at unit position u ^ 2 (r % 4)) when the other array is
// kept; that array's rows come out of LDS with transpose reads (bf16) or
// 4-byte reads (f32).
//
// This is the first kernel of a call: its descriptor and tile list are read
// from the pinned host staging buffer, and the workgroups also copy the whole
// table block (table_units 16-byte units) from there into the workspace for
// the kernels that follow. TI is the input's element type, T the workspace's
// (fp32 workspaces of bf16 inputs hold the exact values; the sums of squares
// come out bit-identical to the bf16 workspace's).
// The per-call tables, pinned host memory -> the workspace head, for calls
// whose tables are large (the input-staging kernel then reads them from device
// memory instead of each workgroup reading its descriptors over the bus).
__global__ __launch_bounds__(256) void ns_table_copy_kernel(const i32x4 *__restrict__ src, i32x4 *__restrict__ dst,
                                                           int32_t units) {
    for (int u = blockIdx.x * 256 + threadIdx.x; u < units; u += gridDim.x * 256) dst[u] = src[u];
}

// Fixed-order sum over the workgroup (kPrepThreads threads): a butterfly within
// each wavefront, then the wavefronts' sums in wave order. Ends with a barrier.
__device__ __forceinline__ float block_sum_fixed(float v, float *red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kPrepThreads / 64; ++w) t += red[w];
    return t;
}

template <typename TI, typename T = TI>
__global__ __launch_bounds__(kPrepThreads) void ns_prepare_kernel(const NsProb *__restrict__ probs,
                                                                 const StageRun *__restrict__ runs, int32_t count,
                                                                 const i32x4 *__restrict__ table_src,
                                                                 i32x4 *__restrict__ table_dst,
                                                                 int32_t table_units,
                                                                 const RowPiece *__restrict__ pieces) {
    constexpr int ES = sizeof(T), EI = sizeof(TI), E = 16 / EI, TE = kPrepTile;
    constexpr int RB = TE * ES, CPR = TE / E;           // staged row bytes, 16-byte input loads per row
    constexpr int UPL = E * ES / 16;                    // 16-byte workspace units per input load
    static_assert(ES >= EI && UPL >= 1, "the workspace type is at least as wide as the input's");
    __shared__ __attribute__((aligned(16))) char lds[TE * RB];
    __shared__ float red[kPrepThreads];
    __shared__ RowPiece band[kPrepTile];   // the pieces holding the run's input rows
    const int bid = blockIdx.x;
    for (int u = bid * kPrepThreads + threadIdx.x; u < table_units; u += gridDim.x * kPrepThreads)
        table_dst[u] = table_src[u];
    if (bid >= count) return;
    const StageRun run = runs[bid];
    const NsProb &pr = probs[run.prob];
    // A run inside one piece (the usual case) reads it straight from the
    // table, in parallel with the descriptor; more pieces go through LDS.
    const RowPiece one = pieces[run.piece];
    const bool multi = run.npiece > 1;
    if (multi) {
        if (threadIdx.x < run.npiece) band[threadIdx.x] = pieces[run.piece + threadIdx.x];
        __syncthreads();
    }
    const bool tall = pr.tall;
    const int rows = tall ? pr.n : pr.m, cols = tall ? pr.m : pr.n;   // input shape
    char *direct = tall ? pr.xt0 : pr.x0;                 // receives the tile as stored
    char *trans = tall ? pr.x0 : pr.xt0;                  // receives its transpose
    const int ld_direct = tall ? pr.ldxt : pr.ldx, ld_trans = tall ? pr.ldx : pr.ldxt;
    const bool do_direct = direct != nullptr, do_trans = trans != nullptr;   // X0^T is absent when kmajor
    const bool vec_in = pr.vec_in;
    // as stored: the run's tiles share input rows r0 .. r0 + TE - 1
    const int r0 = run.band * TE;
    for (int t = 0; t < run.count; ++t) {
        const int q = run.q0 + t;
        const int ti = tall ? q : run.band, tj = tall ? run.band : q;   // the tile in X's staging grid
        const int c0 = q * TE;                                          // its first input column
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < TE * CPR / kPrepThreads; ++k) {
            const int f = threadIdx.x + kPrepThreads * k;
            const int r = f / CPR, u = f % CPR, c = u * E;
            const int64_t gr = r0 + r, gc = c0 + c;
            i32x4 w = {0, 0, 0, 0};
            if (gr < rows) {
                RowPiece pc = one;   // by value: the reads below stay global loads
                if (multi) pc = find_piece(band, run.npiece, gr);
                const char *src = pc.in + ((gr - pc.row0) * pc.ld_in + gc) * EI;
                if (gc + E <= cols) {
                    w = vec_in ? *(const NSQ_GLOBAL i32x4 *)src : load16_unaligned<TI>(src);
                } else {
                    TI vals[E];
#pragma unroll
                    for (int e = 0; e < E; ++e) vals[e] = gc + e < cols ? gp<TI>(src)[e] : TI(0);
                    __builtin_memcpy(&w, vals, 16);
                }
            }
            TI vals[E];
            __builtin_memcpy(vals, &w, 16);
            float fv[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                fv[e] = to_f32<TI>(vals[e]);
                ss = __builtin_fmaf(fv[e], fv[e], ss);
            }
            if constexpr (UPL == 1) {
                if (do_direct) store16<T>(direct, (int64_t)gr * ld_direct + gc, w);
                if (do_trans) *reinterpret_cast<i32x4 *>(lds + r * RB + ((u ^ (2 * (r & 3))) << 4)) = w;
            } else {   // exact widening to the workspace type, 16 bytes at a time
#pragma unroll
                for (int h = 0; h < UPL; ++h) {
                    T wv[16 / ES];
#pragma unroll
                    for (int e = 0; e < 16 / ES; ++e) wv[e] = (T)fv[h * (16 / ES) + e];
                    i32x4 o;
                    __builtin_memcpy(&o, wv, 16);
                    if (do_direct) store16<T>(direct, (int64_t)gr * ld_direct + gc + h * (16 / ES), o);
                    if (do_trans)
                        *reinterpret_cast<i32x4 *>(lds + r * RB + (((u * UPL + h) ^ (2 * (r & 3))) << 4)) = o;
                }
            }
        }
        // fixed-order block sum of the squares
        const float tile_ss = block_sum_fixed(ss, red);
        if (threadIdx.x == 0) pr.partials[ti * (pr.np / TE) + tj] = tile_ss;
        if (do_trans) {
            // transpose: output row c (tile column), 16 bytes = ET consecutive tile rows
            constexpr int ET = 16 / ES;
            auto at = [&](int r, int c) -> const char * {
                const int byte = c * ES;
                return lds + r * RB + (((byte >> 4) ^ (2 * (r & 3))) << 4) + (byte & 15);
            };
            const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tl = lane & 15, g = lane >> 4;
            constexpr int BR = 4 * ET;                         // tile rows per block (4 lane groups x ET)
            constexpr int BLOCKS = (TE / 16) * (TE / BR);
            for (int blk = wave; blk < BLOCKS; blk += kPrepThreads / 64) {
                const int cb = (blk % (TE / 16)) * 16, rb = (blk / (TE / 16)) * BR + ET * g;
                const int c = cb + tl;
                i32x4 w;
                if constexpr (ES == 2) {
                    s16x4 v[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (NSQ_LDS s16x4 *)at(rb + 4 * h + (tl >> 2), cb + 4 * (tl & 3)));
                    w[0] = (int)(uint16_t)v[0][0] | ((int)(uint16_t)v[0][1] << 16);
                    w[1] = (int)(uint16_t)v[0][2] | ((int)(uint16_t)v[0][3] << 16);
                    w[2] = (int)(uint16_t)v[1][0] | ((int)(uint16_t)v[1][1] << 16);
                    w[3] = (int)(uint16_t)v[1][2] | ((int)(uint16_t)v[1][3] << 16);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = *reinterpret_cast<const int *>(at(rb + e, c));
                }
                store16<T>(trans, (int64_t)(c0 + c) * ld_trans + r0 + rb, w);
            }
        }
        // the next tile rewrites the LDS tile and the block-sum slots
        if (t + 1 < run.count) __syncthreads();
    }
}

// steps == 0: the output is the normalised input, out = s G in the input's
// layout, one run of kPrepTile x kPrepTile tiles of the input (as stored) per
// workgroup.
template <typename T>
__global__ __launch_bounds__(kPrepThreads) void ns_scale_out_kernel(const NsProb *__restrict__ probs,
                                                                   const StageRun *__restrict__ runs,
                                                                   int32_t count, float eps,
                                                                   const RowPiece *__restrict__ pieces) {
    __shared__ float red[kScaleSlots];
    const int bid = blockIdx.x;
    if (bid >= count) return;
    const StageRun run = runs[bid];
    const NsProb &pr = probs[run.prob];
    const float sc = norm_scale(pr.partials, pr.nparts, eps, red);
    const bool tall = pr.tall;
    const int rows = tall ? pr.n : pr.m, cols = tall ? pr.m : pr.n;
    const int64_t r0 = (int64_t)run.band * kPrepTile, c0 = (int64_t)run.q0 * kPrepTile;
    const int64_t width = (int64_t)run.count * kPrepTile;
    for (int64_t e = threadIdx.x; e < kPrepTile * width; e += kPrepThreads) {
        const int64_t r = r0 + e / width, c = c0 + e % width;
        if (r < rows && c < cols) {
            const RowPiece pc = find_piece(pieces + run.piece, run.npiece, r);
            gp<T>(pc.out)[(r - pc.row0) * pc.ld_out + c] =
                from_f32<T>(to_f32<T>(gp<T>(pc.in)[(r - pc.row0) * pc.ld_in + c]) * sc);
        }
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
    bool kmajor;       // B X reads X K-major; no X^T arrays
    bool small;        // small size class: one workgroup per matrix (ns_small_kernel)
    int64_t nparts, syrk_tiles, gemm_tiles;
    int64_t sq_tiles;  // full m x m grid (Gram-space products only)
    int64_t npieces;   // row pieces its input / output is split into
    size_t buf_bytes;
};

// Row pieces of every tensor of a call (indexed like the shapes).
using PieceLists = std::vector<std::vector<RowPiece>>;

// Row strides (elements) and array sizes of one matrix's workspace.
inline int64_t ld_x(const MatInfo &mi, int64_t es) { return mi.np + kRowPadBytes / es; }
inline int64_t ld_t(const MatInfo &mi, int64_t es) { return mi.mp + kRowPadBytes / es; }   // m x m arrays
inline size_t x_bytes(const MatInfo &mi, int64_t es) { return align256((size_t)(mi.mp * ld_x(mi, es) * es)); }
inline size_t xt_bytes(const MatInfo &mi, int64_t es) { return align256((size_t)(mi.np * ld_t(mi, es) * es)); }
inline size_t a_bytes(const MatInfo &mi, int64_t es) { return align256((size_t)(mi.mp * ld_t(mi, es) * es)); }

// B X reads X K-major (through LDS transpose reads) when its K is at most
// this; otherwise it reads the rows of a stored X^T, which the input staging
// and every B X but the last then write too. A bf16 call that runs 256-tiles
// (`big`) reads K-major at every K: the 4-wave pinned loop hides the
// transpose reads, and the X^T copies cost more than they save. The
// 128-tile loop and f32 (four 4-byte reads per fragment) keep X^T past
// K = 1024. NS_KMAJOR_MAX overrides (tuning; both ways give the same bits).
// The Gram-space output product always reads X0 K-major.
int64_t kmajor_max_k(bool big) {
    if (const char *env = getenv("NS_KMAJOR_MAX")) return atoll(env);
    return big ? INT64_MAX : 1024;
}

int pick_tile(const std::vector<int32_t> &group, const std::vector<MatInfo> &info, int64_t es);

// Largest m of the small size class; NS_SMALL_MAX=0 sends every matrix down
// the tiled path (tests compare the two, which give the same bits).
int64_t small_max_m() {
    if (const char *env = getenv("NS_SMALL_MAX")) return std::min<int64_t>(atoll(env), kSmallM);
    return kSmallM;
}

// gram: the Gram-space workspace (fp32 X0, G, Q and Q^T ping/pong, Q G, A,
// A^T, B') instead of the NS one (X ping/pong, A, B' in the input's type).
ns_status describe(int32_t n, const ns_shape *shapes, ns_dtype dtype, std::vector<MatInfo> &info,
                   bool gram = false) {
    if (n < 0) return fail(NS_ERR_INVALID_ARG, "n = %d < 0", n);
    if (n > 0 && !shapes) return fail(NS_ERR_INVALID_ARG, "shapes is NULL");
    if (dtype != NS_BF16 && dtype != NS_F32) return fail(NS_ERR_DTYPE, "dtype %d", (int)dtype);
    const int64_t es = gram ? 4 : dtype == NS_BF16 ? 2 : 4;   // workspace element size
    info.assign(n, MatInfo{});
    for (int32_t i = 0; i < n; ++i) {
        MatInfo &mi = info[i];
        ns_status st = matrix_view(shapes[i], i, &mi.rows, &mi.cols);
        if (st) return st;
        mi.active = mi.rows > 0 && mi.cols > 0;
        if (!mi.active) continue;
        mi.tall = mi.rows > mi.cols;
        mi.m = std::min(mi.rows, mi.cols);
        mi.n = std::max(mi.rows, mi.cols);
        // tile indices are 16-bit; byte offsets inside one padded matrix are 32-bit
        if (mi.n > (int64_t)65535 * kPrepTile ||
            round_up(mi.m, kPad) * (round_up(mi.n, kPad) + kRowPadBytes / es) * es >= (1ll << 31) ||
            round_up(mi.n, kPad) * (round_up(mi.m, kPad) + kRowPadBytes / es) * es >= (1ll << 31))
            return fail(NS_ERR_OVERFLOW, "tensor %d: %lld x %lld is too large", i,
                        (long long)mi.rows, (long long)mi.cols);
        mi.small = !gram && mi.m <= small_max_m();
        const int64_t pad = mi.small ? kSmallPad : kPad;
        mi.mp = round_up(mi.m, pad);
        mi.np = round_up(mi.n, pad);
        // table sizing uses the smaller product tile (more tiles)
        const int64_t tm = mi.mp / 128, tn = mi.np / 128;
        mi.syrk_tiles = mi.small ? 0 : tm * (tm + 1) / 2;
        mi.gemm_tiles = tm * tn;   // the small class keeps its B X tiles in a list of their own
        mi.sq_tiles = gram ? tm * tm : 0;
        mi.nparts = (mi.mp / kPrepTile) * (mi.np / kPrepTile);   // one per staging tile
        mi.npieces = 1;
    }
    // B X's operand layout is set per call, from the product tile the whole
    // call would run (a call split into groups keeps it in every group).
    std::vector<int32_t> all(n);
    for (int32_t i = 0; i < n; ++i) all[i] = i;
    const int64_t kmax = kmajor_max_k(!gram && es == 2 && pick_tile(all, info, es) == 256);
    for (MatInfo &mi : info) {
        if (!mi.active) continue;
        mi.kmajor = gram || mi.mp <= kmax;
        mi.buf_bytes = gram ? x_bytes(mi, es) + 9 * a_bytes(mi, es)
                            : 2 * x_bytes(mi, es) + (mi.kmajor ? 0 : 2 * xt_bytes(mi, es)) + 2 * a_bytes(mi, es);
    }
    return NS_OK;
}

// Workspace head: device tables for one group, then fp32 norm partials. The
// staging runs come last, sized for one tile per run; a group uses (and
// uploads) only the runs it has.
struct TableSizes {
    size_t probs, syrk, gemm, sq, smalls, pieces, ptiles, partials, total;
    size_t o_syrk() const { return probs; }
    size_t o_gemm() const { return o_syrk() + syrk; }   // tiled B X tiles, then the small class's
    size_t o_sq() const { return o_gemm() + gemm; }
    size_t o_smalls() const { return o_sq() + sq; }
    size_t o_pieces() const { return o_smalls() + smalls; }
    size_t o_ptiles() const { return o_pieces() + pieces; }
    size_t o_partials() const { return o_ptiles() + ptiles; }
};

TableSizes table_sizes(const std::vector<MatInfo> &info) {
    int64_t np = 0, sy = 0, ge = 0, sq = 0, pa = 0, pc = 0, sm = 0;
    for (const MatInfo &mi : info) {
        if (!mi.active) continue;
        ++np;
        sm += mi.small;
        sy += mi.syrk_tiles;
        ge += mi.gemm_tiles;
        sq += mi.sq_tiles;
        pa += mi.nparts;
        pc += mi.npieces;
    }
    TableSizes t;
    t.probs = align256(np * sizeof(NsProb));
    t.syrk = align256(sy * sizeof(TileRef));
    t.gemm = align256(ge * sizeof(TileRef));
    t.sq = align256(sq * sizeof(TileRef));
    t.ptiles = align256(pa * sizeof(StageRun));
    t.smalls = align256(sm * sizeof(TileRef));
    t.pieces = align256(pc * sizeof(RowPiece));
    t.partials = align256(pa * sizeof(float));
    t.total = t.o_partials() + t.partials;
    return t;
}

// Workspace for running every tensor at once, and the minimum (the largest
// tensor alone).
void workspace_need(const std::vector<MatInfo> &info, size_t *bytes, size_t *min_bytes) {
    const TableSizes t = table_sizes(info);
    size_t all = t.total, biggest = 0;
    for (const MatInfo &mi : info) {
        all += mi.buf_bytes;
        biggest = std::max(biggest, mi.buf_bytes);
    }
    *bytes = all;
    if (min_bytes) *min_bytes = t.total + biggest;
}

// Pieces of `pc` (sorted by row0, pc[0].row0 == 0) overlapping stored rows
// [lo, hi): the first is the one holding row lo (the last piece when lo is past
// the end, i.e. a tile of padding only).
void band_of(const std::vector<RowPiece> &pc, int64_t lo, int64_t hi, int32_t *first, int32_t *count) {
    int32_t f = 0;
    const int32_t np = (int32_t)pc.size();
    while (f + 1 < np && pc[f + 1].row0 <= lo) ++f;
    int32_t e = f + 1;
    while (e < np && pc[e].row0 < hi) ++e;
    *first = f;
    *count = e - f;
}

// Product tile edge for a group: 256 when the big tiles still give the GPU
// enough workgroups, else 128; f32 always uses 128 (its staged 256 x 256 tile
// would not fit the LDS). NS_TILE=128|256 overrides for bf16 (tuning).
int pick_tile(const std::vector<int32_t> &group, const std::vector<MatInfo> &info, int64_t es) {
    if (es == 4) return 128;
    if (const char *env = getenv("NS_TILE")) {
        const int v = atoi(env);
        if (v == 128 || v == 256) return v;
    }
    int64_t big_syrk = 0;
    for (int32_t idx : group) {
        if (info[idx].small) continue;
        const int64_t t = info[idx].mp / 256;
        big_syrk += t * (t + 1) / 2;
    }
    return big_syrk >= 128 ? 256 : 128;
}

// Tiles of a tm x tn grid (upper triangle only if `upper`) in groups of
// kGroupRows x kGroupCols. Consecutive tile ids land on one XCD, whose 32 CUs
// then work on one group at a time: 4 row panels and 8 column panels shared
// through that XCD's L2, instead of 2 row panels and 16 column panels for a
// plain row-major order.
constexpr int kGroupRows = 4, kGroupCols = 8;
void grouped_tiles(int32_t pid, int tm, int tn, bool upper, std::vector<TileRef> &out) {
    for (int bi = 0; bi < tm; bi += kGroupRows)
        for (int bj = 0; bj < tn; bj += kGroupCols)
            for (int ti = bi; ti < std::min(tm, bi + kGroupRows); ++ti)
                for (int tj = bj; tj < std::min(tn, bj + kGroupCols); ++tj)
                    if (!upper || tj >= ti) out.push_back(TileRef{pid, (uint16_t)ti, (uint16_t)tj, 0, 1});
}

#ifndef NSQ_XCD_DEAL
#define NSQ_XCD_DEAL 1
#endif
// A launch's tile list runs in dispatch order: matrices by descending cost,
// each in tile groups. xcd_remap gives XCD x a contiguous range of it, which
// would put every long tile on the first XCDs when the group mixes sizes.
// Deal the list to the XCDs instead, in runs of up to one tile group (which
// shares operand panels through the XCD's L2), round robin, each XCD taking
// exactly the number of ids xcd_remap gives it. Lists of equal tiles that
// fill each XCD with one run keep their order. Only the order changes.
void deal_to_xcds(std::vector<TileRef> &t) {
    const int64_t g = (int64_t)t.size();
    if (!NSQ_XCD_DEAL || g <= kNumXcd) return;
    const int64_t per = g / kNumXcd, rem = g % kNumXcd;
    const int64_t run = std::min<int64_t>(kGroupRows * kGroupCols, (g + kNumXcd - 1) / kNumXcd);
    std::vector<std::vector<TileRef>> q(kNumXcd);
    int64_t i = 0;
    for (int x = 0; i < g; x = (x + 1) % kNumXcd) {
        const int64_t room = per + (x < rem ? 1 : 0) - (int64_t)q[x].size();
        const int64_t n = std::min(std::min(run, room), g - i);
        if (n > 0) {
            q[x].insert(q[x].end(), t.begin() + i, t.begin() + i + n);
            i += n;
        }
    }
    t.clear();
    for (const std::vector<TileRef> &v : q) t.insert(t.end(), v.begin(), v.end());
}

template <typename T, class C>
void launch_product(TimedScope &ts, dim3 grid, hipStream_t st, const NsProb *probs, const TileRef *tiles,
                    int32_t nt, int32_t mode, int32_t cur, bool last, float s_init, float s_final, float s_diag,
                    int32_t do_product, int32_t first, float eps, const RowPiece *pieces) {
    if (mode == kSyrkX)
        ts.launch(ns_product_kernel<T, C, kSyrkX, false>, grid, dim3(C::THREADS), st, probs, tiles, nt, cur, s_init,
                  s_final, s_diag, do_product, first, eps, pieces);
    else if (mode == kSyrkA)
        ts.launch(ns_product_kernel<T, C, kSyrkA, false>, grid, dim3(C::THREADS), st, probs, tiles, nt, cur, s_init,
                  s_final, s_diag, do_product, first, eps, pieces);
    else if (!last)
        ts.launch(ns_product_kernel<T, C, kGemmBX, false>, grid, dim3(C::THREADS), st, probs, tiles, nt, cur, s_init,
                  s_final, s_diag, do_product, first, eps, pieces);
    else
        ts.launch(ns_product_kernel<T, C, kGemmBX, true>, grid, dim3(C::THREADS), st, probs, tiles, nt, cur, s_init,
                  s_final, s_diag, do_product, first, eps, pieces);
}

void launch_pinned(TimedScope &ts, dim3 grid, hipStream_t st, const NsProb *probs, const TileRef *tiles,
                   int32_t nt, int32_t mode, int32_t cur, bool last, float s_init, float s_final, float s_diag,
                   int32_t do_product, int32_t first, float eps, const RowPiece *pieces) {
    const dim3 block(Quad::THREADS);
    if (mode == kSyrkX)
        ts.launch(ns_pinned_kernel<kSyrkX, false>, grid, block, st, probs, tiles, nt, cur, s_init, s_final, s_diag,
                  do_product, first, eps, pieces);
    else if (mode == kSyrkA)
        ts.launch(ns_pinned_kernel<kSyrkA, false>, grid, block, st, probs, tiles, nt, cur, s_init, s_final, s_diag,
                  do_product, first, eps, pieces);
    else if (!last)
        ts.launch(ns_pinned_kernel<kGemmBX, false>, grid, block, st, probs, tiles, nt, cur, s_init, s_final, s_diag,
                  do_product, first, eps, pieces);
    else
        ts.launch(ns_pinned_kernel<kGemmBX, true>, grid, block, st, probs, tiles, nt, cur, s_init, s_final, s_diag,
                  do_product, first, eps, pieces);
}

// The bf16 256-tile products run on the 4-wave kernel with fixed accumulator
// registers; NS_BIG_WAVES=8 selects the 8-wave kernel instead (measuring;
// both give the same bits).
bool big_tiles_pinned() {
    const char *env = getenv("NS_BIG_WAVES");
    return !(env && atoi(env) == 8);
}

template <typename T, class C, int MODE, bool LAST = false, typename TO = T>
void launch_mode(TimedScope &ts, int32_t nt, hipStream_t st, const NsProb *probs, const TileRef *tiles, int32_t cur,
                 float s_init, float s_final, float s_diag, int32_t do_product, int32_t first, float eps,
                 const RowPiece *pieces) {
    ts.launch(ns_product_kernel<T, C, MODE, LAST, TO>, dim3((unsigned)nt), dim3(C::THREADS), st, probs, tiles, nt,
              cur, s_init, s_final, s_diag, do_product, first, eps, pieces);
}

// The device tables of one group of matrices, built on the host, and what its
// launches need. Each group has its own table layout (`tsz`, over its members
// only) at the head of the workspace; the matrices' buffers start after the
// head sized for the whole call.
struct GroupPlan {
    int bm = 256;                 // product tile edge
    TableSizes tsz{};             // this group's table layout
    std::vector<char> tables;     // the tables up to the last staging run, as they go to the device
    int32_t nsyrk = 0, ngemm = 0, nsq = 0, nruns = 0, nsmall = 0;
    double f_syrk_x = 0, f_syrk_a = 0, f_gemm = 0, f_sq = 0, norm_bytes = 0;
    double f_small = 0;           // algorithmic flops of one step of the small class
    size_t staging_off = 0;       // where its tables sit in the call's staging buffer
};

// Builds the tables of one group. TI's size is esi, the workspace type's es.
// gram: the Gram-space workspace layout.
GroupPlan build_group(const std::vector<int32_t> &group, const std::vector<MatInfo> &info,
                      const PieceLists &pieces, float b, float c, bool gram, int64_t es, int64_t esi,
                      char *ws, size_t head_bytes) {
    GroupPlan g;
    g.bm = gram ? 128 : pick_tile(group, info, es);
    const int bm = g.bm;
    std::vector<MatInfo> members;
    members.reserve(group.size());
    for (int32_t idx : group) members.push_back(info[idx]);
    g.tsz = table_sizes(members);
    std::vector<NsProb> probs;
    std::vector<TileRef> syrk, gemm, sq, smalls, sgemm;
    std::vector<StageRun> runs;
    // Staging tiles per workgroup: one for small groups (enough workgroups to
    // fill the GPU), up to 4 for large ones (32768 tiles and more), which cuts
    // the run table (uploaded with every call) to a quarter. Longer runs
    // measured slower on the dense-transformer set (8 tiles: 3 %, 13: 6 %).
    // The tiles and their sums are the same either way; only the grouping
    // changes.
    int64_t group_parts = 0;
    for (int32_t idx : group) group_parts += info[idx].nparts;
    int run_len = (int)std::max<int64_t>(1, std::min<int64_t>(4, group_parts / 32768));
    if (const char *env = getenv("NS_STAGE_RUN")) run_len = std::max(1, std::min(16, atoi(env)));
    std::vector<RowPiece> gpieces;
    char *base = ws + head_bytes;
    float *partials = reinterpret_cast<float *>(ws + g.tsz.o_partials());
    int64_t part_off = 0;
    for (int32_t idx : group) {
        const MatInfo &mi = info[idx];
        NsProb p{};
        const size_t xb = x_bytes(mi, es), xtb = mi.kmajor ? 0 : xt_bytes(mi, es), ab = a_bytes(mi, es);
        if (!gram) {
            p.x0 = base;
            p.x1 = p.x0 + xb;
            if (!mi.kmajor) {
                p.xt0 = p.x1 + xb;
                p.xt1 = p.xt0 + xtb;
            }
            p.a = p.x1 + xb + 2 * xtb;
            p.b = p.a + ab;
        } else {   // X0, G, Q and Q^T ping/pong, Q G, A, A^T, B'
            p.x0 = base;
            p.g = p.x0 + xb;
            p.q0 = p.g + ab;
            p.q1 = p.q0 + ab;
            p.qt0 = p.q1 + ab;
            p.qt1 = p.qt0 + ab;
            p.t = p.qt1 + ab;
            p.a = p.t + ab;
            p.at = p.a + ab;
            p.b = p.at + ab;
        }
        base += mi.buf_bytes;
        const std::vector<RowPiece> &pc = pieces[idx];
        const int32_t pbase = (int32_t)gpieces.size();
        bool vin = true, vout = true;   // 16-byte accesses: aligned bases and row strides
        for (const RowPiece &q : pc) {
            vin = vin && reinterpret_cast<uintptr_t>(q.in) % 16 == 0 && q.ld_in * esi % 16 == 0;
            vout = vout && reinterpret_cast<uintptr_t>(q.out) % 16 == 0 && q.ld_out * esi % 16 == 0;
            gpieces.push_back(q);
        }
        p.vec_in = vin;
        p.vec_out = vout;
        p.partials = partials + part_off;
        part_off += mi.nparts;
        p.m = (int32_t)mi.m;
        p.n = (int32_t)mi.n;
        p.mp = (int32_t)mi.mp;
        p.np = (int32_t)mi.np;
        p.ldx = (int32_t)ld_x(mi, es);
        p.ldt = (int32_t)ld_t(mi, es);
        p.ldxt = (int32_t)ld_t(mi, es);
        p.kmajor = mi.kmajor;
        p.tall = mi.tall;
        p.nparts = (int32_t)mi.nparts;
        const int32_t pid = (int32_t)probs.size();
        probs.push_back(p);
        // Each tile names the pieces holding the stored rows it reads (staging
        // tiles) or writes (B X tiles, whose last launch writes the output):
        // X rows for a wide tensor, X columns for a tall one.
        auto set_band = [&](TileRef &t, int edge) {
            const int64_t lo = (int64_t)(mi.tall ? t.tj : t.ti) * edge;
            band_of(pc, lo, lo + edge, &t.piece, &t.npiece);
            t.piece += pbase;
        };
        if (mi.small) {   // one entry; its B X tiles (0, tj) with their output pieces in sgemm
            const int tn = (int)(mi.np / kSmallPad);
            smalls.push_back(TileRef{pid, 0, 0, (int32_t)sgemm.size(), tn});
            for (int tj = 0; tj < tn; ++tj) {
                sgemm.push_back(TileRef{pid, 0, (uint16_t)tj, 0, 1});
                set_band(sgemm.back(), kSmallPad);
            }
        } else {
            const int tm = (int)(mi.mp / bm), tn = (int)(mi.np / bm);
            const size_t s0 = syrk.size(), g0 = gemm.size();
            grouped_tiles(pid, tm, tm, true, syrk);
            for (size_t k = s0; k < syrk.size(); ++k) syrk[k].piece = pbase;   // unused by the SYRK steps
            grouped_tiles(pid, tm, tn, false, gemm);
            for (size_t k = g0; k < gemm.size(); ++k) set_band(gemm[k], bm);
        }
        if (gram) {
            const int tm = (int)(mi.mp / bm);
            const size_t q0 = sq.size();
            grouped_tiles(pid, tm, tm, false, sq);
            for (size_t k = q0; k < sq.size(); ++k) sq[k].piece = pbase;   // no caller memory touched
        }
        // Staging runs in the input's storage order: row bands of G, each band's
        // tiles left to right in runs of run_len (for a tall G a band of G rows
        // is a column band tj of X), so the workgroups in flight together read
        // and write whole rows. Tile (ti, tj) writes partial ti * pn + tj.
        const int pm = (int)(mi.mp / kPrepTile), pn = (int)(mi.np / kPrepTile);
        const int outer = mi.tall ? pn : pm, inner = mi.tall ? pm : pn;
        for (int o = 0; o < outer; ++o) {
            int32_t bp = 0, bn = 0;
            band_of(pc, (int64_t)o * kPrepTile, (int64_t)(o + 1) * kPrepTile, &bp, &bn);
            for (int q = 0; q < inner; q += run_len)
                runs.push_back(StageRun{pid, (uint16_t)o, (uint16_t)q, pbase + bp, (uint16_t)bn,
                                        (uint16_t)std::min(run_len, inner - q)});
        }
        const double m = (double)mi.m, n = (double)mi.n;
        const double fx = m * (m + 1) * n;                                              // X X^T, or G
        const double fa = (c != 0.f && std::isfinite(b / c)) ? m * m * (m + 1) : 0.0;   // A A (per step)
        const double fb = 2 * m * m * n;                                                // B X, or Q X0
        if (mi.small) {
            g.f_small += fx + fa + fb;
        } else {
            g.f_syrk_x += fx;
            g.f_syrk_a += fa;
            g.f_gemm += fb;
        }
        g.f_sq += 2.0 * m * m * m;                                                // a full m x m product
        // input read, X0 written (padded), and X0^T when it is kept
        g.norm_bytes += m * n * esi + (mi.kmajor ? 1.0 : 2.0) * (double)mi.mp * (double)mi.np * es;
    }
    deal_to_xcds(syrk);
    deal_to_xcds(gemm);
    deal_to_xcds(sq);
    g.nsyrk = (int32_t)syrk.size();
    g.ngemm = (int32_t)gemm.size();
    g.nsmall = (int32_t)smalls.size();
    for (TileRef &t : smalls) t.piece += g.ngemm;   // the small class's B X tiles follow the tiled ones
    gemm.insert(gemm.end(), sgemm.begin(), sgemm.end());
    g.nsq = (int32_t)sq.size();
    g.nruns = (int32_t)runs.size();
    g.tables.assign(g.tsz.o_ptiles() + align256(runs.size() * sizeof(StageRun)), 0);   // a multiple of 256
    auto put = [&](size_t off, const void *src, size_t bytes) {
        if (bytes) std::memcpy(g.tables.data() + off, src, bytes);
    };
    put(0, probs.data(), probs.size() * sizeof(NsProb));
    put(g.tsz.o_syrk(), syrk.data(), syrk.size() * sizeof(TileRef));
    put(g.tsz.o_gemm(), gemm.data(), gemm.size() * sizeof(TileRef));
    put(g.tsz.o_sq(), sq.data(), sq.size() * sizeof(TileRef));
    put(g.tsz.o_ptiles(), runs.data(), runs.size() * sizeof(StageRun));
    put(g.tsz.o_smalls(), smalls.data(), smalls.size() * sizeof(TileRef));
    put(g.tsz.o_pieces(), gpieces.data(), gpieces.size() * sizeof(RowPiece));
    return g;
}

// Enqueues one group: input staging (which reads the group's tables from
// `hdev`, the device's view of its part of the staging buffer, and copies them
// into the workspace head), then the product launches. TI is the input's
// type, T the workspace's. gram: the Gram-space iteration in fp32 (T = float)
// with the trace ridge `ridge`; else NS in TI. Returns NS_ERR_HIP if a launch
// fails.
template <typename TI, typename T>
ns_status launch_group(const GroupPlan &g, int32_t steps, float a, float b, float c, float eps, bool gram,
                       float ridge, char *ws, const char *hdev, hipStream_t st) {
    static_assert(sizeof(T) >= sizeof(TI), "workspace type");
    const TableSizes &tsz = g.tsz;
    const int bm = g.bm;
    const NsProb *d_probs = reinterpret_cast<const NsProb *>(ws);
    const TileRef *d_syrk = reinterpret_cast<const TileRef *>(ws + tsz.o_syrk());
    const TileRef *d_gemm = reinterpret_cast<const TileRef *>(ws + tsz.o_gemm());
    const TileRef *d_sq = reinterpret_cast<const TileRef *>(ws + tsz.o_sq());
    const StageRun *d_runs = reinterpret_cast<const StageRun *>(ws + tsz.o_ptiles());
    const RowPiece *d_pieces = reinterpret_cast<const RowPiece *>(ws + tsz.o_pieces());
    const int32_t npt = g.nruns;
    {
        TimedScope ts(kTimeNorm, g.norm_bytes);
        const int32_t units = (int32_t)(g.tables.size() / 16);
        auto prep = ns_prepare_kernel<TI, T>;
        if (g.tables.size() <= kTablesFromHostMax) {
            // small tables: each staging workgroup reads its descriptors from the
            // pinned staging and together they copy the tables to the workspace
            ts.launch(prep, dim3((unsigned)npt), dim3(kPrepThreads), st, reinterpret_cast<const NsProb *>(hdev),
                      reinterpret_cast<const StageRun *>(hdev + tsz.o_ptiles()), npt,
                      reinterpret_cast<const i32x4 *>(hdev), reinterpret_cast<i32x4 *>(ws), units,
                      reinterpret_cast<const RowPiece *>(hdev + tsz.o_pieces()));
        } else {
            // large tables: one copy first, then staging reads them from device memory
            const unsigned cgrid = (unsigned)std::min<int64_t>((units + 1023) / 1024, 2048);
            ts.launch(ns_table_copy_kernel, dim3(cgrid), dim3(256), st, reinterpret_cast<const i32x4 *>(hdev),
                      reinterpret_cast<i32x4 *>(ws), units);
            ts.launch(prep, dim3((unsigned)npt), dim3(kPrepThreads), st, d_probs, d_runs, npt,
                      static_cast<const i32x4 *>(nullptr), static_cast<i32x4 *>(nullptr), 0, d_pieces);
        }
        NSQ_HIP(hipGetLastError());
        if (steps == 0)
            ts.launch(ns_scale_out_kernel<TI>, dim3((unsigned)npt), dim3(kPrepThreads), st, d_probs, d_runs, npt,
                      eps, d_pieces);
    }
    NSQ_HIP(hipGetLastError());
    // B' = a I + b A + c A A as c (b / c A + A A) + a I: the accumulators of the
    // A A product start at (b / c) A. With c == 0, or b / c out of fp32 range
    // (c A A is then below fp32 resolution of b A), B' = b A + a I and the
    // product is skipped.
    const float ratio = c != 0.f ? b / c : 0.f;
    const bool sa_fused = c != 0.f && std::isfinite(ratio);
    const float sa_init = sa_fused ? ratio : b, sa_final = sa_fused ? c : 1.f;
    const int32_t sa_product = sa_fused ? 1 : 0;
    if (!gram && g.nsmall > 0 && steps > 0) {
        const TileRef *d_small = reinterpret_cast<const TileRef *>(ws + tsz.o_smalls());
        TimedScope ts(kTimeSmall, g.f_small * steps);
        ts.launch(ns_small_kernel<T>, dim3((unsigned)g.nsmall), dim3(Small::THREADS), st, d_probs, d_small, d_gemm,
                  steps, sa_init, sa_final, a, sa_product, eps, d_pieces);
        NSQ_HIP(hipGetLastError());
    }
    if (gram) {
        if constexpr (sizeof(T) == 4) {
            if (steps > 0) {
                const float ratio = c != 0.f ? b / c : 0.f;
                const bool fused = c != 0.f && std::isfinite(ratio);
                const float si = fused ? ratio : b, sf = fused ? c : 1.f;
                const int32_t prod = fused ? 1 : 0;
                const int32_t nsy = g.nsyrk, nge = g.ngemm, nsq = g.nsq;
                const double f_sq = g.f_sq;   // one full m x m product per matrix: 2 m^3
                {
                    TimedScope ts(kTimeSyrkX, g.f_syrk_x);   // G = s^2 X0 X0^T + ridge tr(G)/m I
                    launch_mode<T, Small, kGramG>(ts, nsy, st, d_probs, d_syrk, 0, 1.f, 1.f, ridge, 1, 1, eps, d_pieces);
                }
                {
                    TimedScope ts(kTimeSyrkA, fused ? f_sq : 0.0);   // Q1 = a I + b G + c G G
                    launch_mode<T, Small, kGramB0>(ts, nsq, st, d_probs, d_sq, 0, si, sf, a, prod, 0, eps, d_pieces);
                }
                NSQ_HIP(hipGetLastError());
                int qcur = 1;
                for (int32_t k = 1; k < steps; ++k) {
                    {
                        TimedScope ts(kTimeProduct, 2 * f_sq);   // T = Q G, A = T Q (and A^T)
                        launch_mode<T, Small, kGramQG>(ts, nsq, st, d_probs, d_sq, qcur, 1.f, 1.f, 0.f, 1, 0, eps, d_pieces);
                        launch_mode<T, Small, kGramTQ>(ts, nsq, st, d_probs, d_sq, qcur, 1.f, 1.f, 0.f, 1, 0, eps, d_pieces);
                    }
                    {
                        TimedScope ts(kTimeSyrkA, fused ? f_sq : 0.0);   // B' = a I + b A + c A A
                        launch_mode<T, Small, kGramAA>(ts, nsq, st, d_probs, d_sq, qcur, si, sf, a, prod, 0, eps, d_pieces);
                    }
                    {
                        TimedScope ts(kTimeProduct, f_sq);   // Q' = B' Q (and Q'^T)
                        launch_mode<T, Small, kGramBQ>(ts, nsq, st, d_probs, d_sq, qcur, 1.f, 1.f, 0.f, 1, 0, eps, d_pieces);
                    }
                    NSQ_HIP(hipGetLastError());
                    qcur ^= 1;
                }
                {
                    TimedScope ts(kTimeFinal, g.f_gemm);   // out = s Q X0
                    launch_mode<T, Small, kGramOut, true, TI>(ts, nge, st, d_probs, d_gemm, qcur, 1.f, 1.f, 0.f, 1, 1,
                                                              eps, d_pieces);
                }
                NSQ_HIP(hipGetLastError());
            }
        }
        return NS_OK;
    }
    int cur = 0;
    const double work[3] = {g.f_syrk_x, g.f_syrk_a, g.f_gemm};
    if (g.nsyrk == 0 && g.ngemm == 0) return NS_OK;   // only small matrices
    for (int32_t s = 0; s < steps; ++s) {
        for (int mode = kSyrkX; mode <= kGemmBX; ++mode) {
            const TileRef *d_t = mode == kGemmBX ? d_gemm : d_syrk;
            const int32_t nt = mode == kGemmBX ? g.ngemm : g.nsyrk;
            const bool last = mode == kGemmBX && s == steps - 1;
            const int kind = last ? kTimeFinal : mode == kSyrkX ? kTimeSyrkX : mode == kSyrkA ? kTimeSyrkA
                                                                                  : kTimeProduct;
            TimedScope ts(kind, work[mode]);
            const float s_init = mode == kSyrkA ? sa_init : 1.f;
            const float s_final = mode == kSyrkA ? sa_final : 1.f;
            const float s_diag = mode == kSyrkA ? a : 0.f;
            const int32_t do_product = mode == kSyrkA ? sa_product : 1;
            if constexpr (sizeof(T) == 2) {
                if (bm == 256) {
                    if (big_tiles_pinned())
                        launch_pinned(ts, dim3(nt), st, d_probs, d_t, nt, mode, cur, last, s_init, s_final, s_diag,
                                      do_product, s == 0, eps, d_pieces);
                    else
                        launch_product<T, Big>(ts, dim3(nt), st, d_probs, d_t, nt, mode, cur, last, s_init, s_final,
                                               s_diag, do_product, s == 0, eps, d_pieces);
                    continue;
                }
            }
            launch_product<T, Small>(ts, dim3(nt), st, d_probs, d_t, nt, mode, cur, last, s_init, s_final,
                                     s_diag, do_product, s == 0, eps, d_pieces);
        }
        NSQ_HIP(hipGetLastError());
        cur ^= 1;
    }
    return NS_OK;
}

// A call split into groups: groups[wave_start[w] .. wave_start[w + 1]) make
// wave w (a plain call is one wave).
struct CallPlan {
    std::vector<GroupPlan> groups;
    std::vector<size_t> wave_start{0};
};

// Validates a call and appends its groups (consecutive matrices in dispatch
// order whose buffers fit the workspace together) to `plan` as one wave.
// Nothing is enqueued. gram: Gram-space workspace layout.
ns_status plan_call(const std::vector<MatInfo> &info, const PieceLists &pieces, ns_dtype dtype, int32_t steps,
                    float b, float c, const int32_t *order, void *workspace, size_t workspace_bytes, bool gram,
                    CallPlan &plan) {
    const int32_t n = (int32_t)info.size();
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
    size_t all, need;
    workspace_need(info, &all, &need);
    if (!workspace) return fail(NS_ERR_WORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
        return fail(NS_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
        return fail(NS_ERR_WORKSPACE, "workspace of %zu bytes < minimum %zu", workspace_bytes, need);
    const int64_t es = gram ? 4 : dtype == NS_BF16 ? 2 : 4, esi = dtype == NS_BF16 ? 2 : 4;
    const size_t room = workspace_bytes - tsz.total;
    std::vector<int32_t> group;
    size_t used = 0;
    auto flush = [&]() {
        if (group.empty()) return;
        plan.groups.push_back(build_group(group, info, pieces, b, c, gram, es, esi, static_cast<char *>(workspace),
                                          tsz.total));
        group.clear();
        used = 0;
    };
    for (int32_t i : ord) {
        if (!info[i].active) continue;
        if (used + info[i].buf_bytes > room) flush();
        group.push_back(i);
        used += info[i].buf_bytes;
    }
    flush();
    plan.wave_start.push_back(plan.groups.size());
    return NS_OK;
}

// Enqueues a planned call: every group's tables go into one pinned staging
// buffer, then wave by wave (after its ready event, if any) the groups' launches.
// Only a HIP runtime failure can stop it after the first enqueue.
ns_status launch_call(CallPlan &plan, ns_dtype dtype, int32_t steps, float a, float b, float c, float eps,
                      bool gram, float ridge, void *workspace, void *const *ready_events, hipStream_t hs,
                      bool may_grow = true) {
    if (plan.groups.empty() && !ready_events) return NS_OK;
    size_t total = 0;
    for (GroupPlan &g : plan.groups) {
        g.staging_off = total;
        total += g.tables.size();   // multiples of 256
    }
    int slot = -1;
    void *staging = nullptr, *staging_dev = nullptr;
    if (total) {
        // Under stream capture the tables go to a staging slot kept for good:
        // the graph's replays read them after this call returns.
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        NSQ_HIP(hipStreamIsCapturing(hs, &cap));
        ns_status sst = cap != hipStreamCaptureStatusNone
                            ? staging_acquire_capture(total, &staging, &staging_dev)
                            : staging_acquire(total, &slot, &staging, &staging_dev, may_grow);
        if (sst) return sst;
        for (const GroupPlan &g : plan.groups)
            std::memcpy(static_cast<char *>(staging) + g.staging_off, g.tables.data(), g.tables.size());
    }
    char *ws = static_cast<char *>(workspace);
    ns_status st = NS_OK;
    bool launched = false;
    const size_t waves = plan.wave_start.size() - 1;
    for (size_t w = 0; w < waves && st == NS_OK; ++w) {
        if (ready_events && ready_events[w]) {
            const hipError_t e = hipStreamWaitEvent(hs, reinterpret_cast<hipEvent_t>(ready_events[w]), 0);
            if (e != hipSuccess) {
                st = fail(NS_ERR_HIP, "hipStreamWaitEvent failed: %s", hipGetErrorString(e));
                break;
            }
        }
        for (size_t k = plan.wave_start[w]; k < plan.wave_start[w + 1] && st == NS_OK; ++k) {
            const GroupPlan &g = plan.groups[k];
            const char *hdev = static_cast<const char *>(staging_dev) + g.staging_off;
            launched = true;
            if (gram)
                st = dtype == NS_BF16 ? launch_group<__bf16, float>(g, steps, a, b, c, eps, true, ridge, ws, hdev, hs)
                                      : launch_group<float, float>(g, steps, a, b, c, eps, true, ridge, ws, hdev, hs);
            else
                st = dtype == NS_BF16 ? launch_group<__bf16, __bf16>(g, steps, a, b, c, eps, false, 0.f, ws, hdev, hs)
                                      : launch_group<float, float>(g, steps, a, b, c, eps, false, 0.f, ws, hdev, hs);
        }
    }
    if (slot >= 0) {
        const ns_status rs = staging_release(slot, hs, launched);
        if (st == NS_OK) st = rs;
    }
    return st;
}

// The common path of the entry points: every active tensor's input and output
// rows are given as row pieces. gram: Gram-space iteration (info described
// with the Gram workspace).
// may_grow = false: the table staging must already be large enough (nothing
// is allocated).
ns_status orthogonalize(const std::vector<MatInfo> &info, const PieceLists &pieces, ns_dtype dtype,
                        int32_t steps, float a, float b, float c, float eps, const int32_t *order,
                        void *workspace, size_t workspace_bytes, hipStream_t hs, bool gram = false,
                        float ridge = 0.f, bool may_grow = true) {
    CallPlan plan;
    ns_status st = plan_call(info, pieces, dtype, steps, b, c, order, workspace, workspace_bytes, gram, plan);
    if (st) return st;
    return launch_call(plan, dtype, steps, a, b, c, eps, gram, ridge, workspace, nullptr, hs, may_grow);
}

ns_status check_coefficients(int32_t steps, float a, float b, float c, float eps) {
    if (steps < 0) return fail(NS_ERR_INVALID_ARG, "steps = %d < 0", steps);
    if (!(eps >= 0.f) || !std::isfinite(a) || !std::isfinite(b) || !std::isfinite(c))
        return fail(NS_ERR_INVALID_ARG, "coefficients must be finite and eps >= 0");
    return NS_OK;
}

// Tensors of a route plan, with each tensor's row pieces as described by the
// plan (one per shard holding a nonzero number of its rows).
ns_status describe_routed(const ns_route_plan *plan, ns_dtype dtype, std::vector<MatInfo> &info) {
    if (!plan) return fail(NS_ERR_INVALID_ARG, "plan is NULL");
    ns_status st = describe(plan->n, plan->shapes.data(), dtype, info);
    if (st) return st;
    if ((dtype == NS_BF16 ? 2 : 4) != plan->elem_bytes)
        return fail(NS_ERR_PLAN_MISMATCH, "dtype element size differs from the plan's %d bytes", plan->elem_bytes);
    const int32_t S = plan->num_shards;
    for (int32_t i = 0; i < plan->n; ++i) {
        int64_t k = 0;
        for (int32_t s = 0; s < S; ++s) k += plan->split_rows[(size_t)i * S + s] > 0;
        if (plan->shard_dim[i] != 0 && k > 1 && info[i].active)
            return fail(NS_ERR_PLAN_MISMATCH,
                        "tensor %d is split along dim %d: fused routing reads row shards only (pack first)", i,
                        plan->shard_dim[i]);
        info[i].npieces = std::max<int64_t>(k, 1);
    }
    return NS_OK;
}

// The checks and row pieces of a batched call (contiguous tensors, one piece
// each). n == 0 leaves `pieces` empty.
ns_status batched_args(int32_t n, const ns_shape *shapes, const void *const *in, void *const *out, ns_dtype dtype,
                       int32_t steps, float a, float b, float c, float eps, std::vector<MatInfo> &info,
                       PieceLists &pieces) {
    ns_status st = describe(n, shapes, dtype, info);
    if (st) return st;
    if ((st = check_coefficients(steps, a, b, c, eps))) return st;
    if (n == 0) return NS_OK;
    if (!in || !out) return fail(NS_ERR_INVALID_ARG, "in and out are required");
    const size_t es = dtype == NS_BF16 ? 2 : 4;
    pieces.assign(n, {});
    for (int32_t i = 0; i < n; ++i) {
        if (!info[i].active) continue;
        if (!in[i] || !out[i]) return fail(NS_ERR_INVALID_ARG, "tensor %d: NULL in/out", i);
        if ((reinterpret_cast<uintptr_t>(in[i]) | reinterpret_cast<uintptr_t>(out[i])) % es)
            return fail(NS_ERR_INVALID_ARG, "tensor %d: in/out not %zu-byte aligned", i, es);
        pieces[i].push_back(RowPiece{0, static_cast<const char *>(in[i]), static_cast<char *>(out[i]),
                                     info[i].cols, info[i].cols});
    }
    return NS_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices];   // device address of `scratch`, per device, once set up

}  // namespace

// Scratch for ns_orthogonalize_batched_noalloc: the workspace of callers that
// cannot allocate. Each GPU the library runs on holds its own copy of this
// array for the life of the process. In host code its name is only a
// stand-in: the device address comes from hipGetSymbolAddress, once per
// device (ns_noalloc_init), and only that address is ever used.
static __device__ __attribute__((aligned(256))) char scratch[kNoAllocScratchBytes];

}  // namespace nsq

using namespace nsq;

extern "C" ns_status ns_workspace_bytes(int32_t n, const ns_shape *shapes, ns_dtype dtype,
                                        size_t *bytes, size_t *min_bytes) {
    if (!bytes) return fail(NS_ERR_INVALID_ARG, "bytes is NULL");
    std::vector<MatInfo> info;
    ns_status st = describe(n, shapes, dtype, info);
    if (st) return st;
    workspace_need(info, bytes, min_bytes);
    return NS_OK;
}

extern "C" ns_status ns_noalloc_init(void) {
    int dev = -1;
    NSQ_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(NS_ERR_INVALID_ARG, "device %d out of range", dev);
    {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        if (!g_scratch_dev[dev]) {
            void *p = nullptr;
            NSQ_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
            if (!p || reinterpret_cast<uintptr_t>(p) % 256)
                return fail(NS_ERR_HIP, "scratch array address %p is unusable", p);
            g_scratch_dev[dev] = p;
        }
    }
    const ns_status st = staging_reserve(kNoAllocTableBytes);
    if (st) return st;
    return staging_reserve_capture(kNoAllocTableBytes);
}

extern "C" ns_status ns_orthogonalize_batched_noalloc(int32_t n, const ns_shape *shapes, const void *const *in,
                                                      void *const *out, ns_dtype dtype, int32_t steps, float a,
                                                      float b, float c, float eps, const int32_t *order,
                                                      void *stream) {
    std::vector<MatInfo> info;
    PieceLists pieces;
    ns_status st = batched_args(n, shapes, in, out, dtype, steps, a, b, c, eps, info, pieces);
    if (st || n == 0) return st;
    size_t all, need;
    workspace_need(info, &all, &need);
    if (need > kNoAllocScratchBytes)
        return fail(NS_ERR_WORKSPACE,
                    "the largest tensor needs %zu bytes of scratch; the no-allocation entry point has %zu", need,
                    kNoAllocScratchBytes);
    int dev = -1;
    NSQ_HIP(hipGetDevice(&dev));
    void *ws = nullptr;
    if (dev >= 0 && dev < kMaxDevices) {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        ws = g_scratch_dev[dev];
    }
    if (!ws) return fail(NS_ERR_INVALID_ARG, "ns_noalloc_init has not been called on device %d", dev);
    return orthogonalize(info, pieces, dtype, steps, a, b, c, eps, order, ws, kNoAllocScratchBytes,
                         reinterpret_cast<hipStream_t>(stream), false, 0.f, false);
}

extern "C" ns_status ns_orthogonalize_batched(int32_t n, const ns_shape *shapes,
                                              const void *const *in, void *const *out,
                                              ns_dtype dtype, int32_t steps, float a, float b,
                                              float c, float eps, const int32_t *order,
                                              void *workspace, size_t workspace_bytes,
                                              void *stream) {
    std::vector<MatInfo> info;
    PieceLists pieces;
    ns_status st = batched_args(n, shapes, in, out, dtype, steps, a, b, c, eps, info, pieces);
    if (st || n == 0) return st;
    return orthogonalize(info, pieces, dtype, steps, a, b, c, eps, order, workspace, workspace_bytes,
                         reinterpret_cast<hipStream_t>(stream));
}

extern "C" ns_status ns_orthogonalize_strided(int32_t n, const ns_shape *shapes, const void *const *in,
                                              const int64_t *in_ld, void *const *out, const int64_t *out_ld,
                                              ns_dtype dtype, int32_t steps, float a, float b, float c,
                                              float eps, const int32_t *order, void *workspace,
                                              size_t workspace_bytes, void *stream) {
    std::vector<MatInfo> info;
    ns_status st = describe(n, shapes, dtype, info);
    if (st) return st;
    if ((st = check_coefficients(steps, a, b, c, eps))) return st;
    if (n == 0) return NS_OK;
    if (!in || !out) return fail(NS_ERR_INVALID_ARG, "in and out are required");
    const size_t es = dtype == NS_BF16 ? 2 : 4;
    PieceLists pieces(n);
    for (int32_t i = 0; i < n; ++i) {
        if (!info[i].active) continue;
        const int64_t li = in_ld ? in_ld[i] : info[i].cols, lo = out_ld ? out_ld[i] : info[i].cols;
        if (li < info[i].cols || lo < info[i].cols)
            return fail(NS_ERR_INVALID_ARG, "tensor %d: row stride (%lld, %lld) < cols %lld", i, (long long)li,
                        (long long)lo, (long long)info[i].cols);
        int64_t span;   // elements from a row's start to the last row's end fit in 63 bits
        if (__builtin_mul_overflow(std::max(li, lo), info[i].rows, &span))
            return fail(NS_ERR_OVERFLOW, "tensor %d: strided extent overflows", i);
        if (!in[i] || !out[i]) return fail(NS_ERR_INVALID_ARG, "tensor %d: NULL in/out", i);
        if ((reinterpret_cast<uintptr_t>(in[i]) | reinterpret_cast<uintptr_t>(out[i])) % es)
            return fail(NS_ERR_INVALID_ARG, "tensor %d: in/out not %zu-byte aligned", i, es);
        pieces[i].push_back(RowPiece{0, static_cast<const char *>(in[i]), static_cast<char *>(out[i]), li, lo});
    }
    return orthogonalize(info, pieces, dtype, steps, a, b, c, eps, order, workspace, workspace_bytes,
                         reinterpret_cast<hipStream_t>(stream));
}

extern "C" ns_status ns_routed_workspace_bytes(const ns_route_plan *plan, ns_dtype dtype, size_t *bytes,
                                               size_t *min_bytes) {
    if (!bytes) return fail(NS_ERR_INVALID_ARG, "bytes is NULL");
    std::vector<MatInfo> info;
    ns_status st = describe_routed(plan, dtype, info);
    if (st) return st;
    workspace_need(info, bytes, min_bytes);
    return NS_OK;
}

extern "C" ns_status ns_orthogonalize_routed(const ns_route_plan *plan, const void *const *shard_in,
                                             void *const *shard_out, ns_dtype dtype, int32_t steps,
                                             float a, float b, float c, float eps, const int32_t *order,
                                             void *workspace, size_t workspace_bytes, void *stream) {
    std::vector<MatInfo> info;
    ns_status st = describe_routed(plan, dtype, info);
    if (st) return st;
    if ((st = check_coefficients(steps, a, b, c, eps))) return st;
    if (plan->n == 0) return NS_OK;
    const int32_t S = plan->num_shards, n = plan->n;
    const int64_t es = plan->elem_bytes;
    if (!shard_in || !shard_out) return fail(NS_ERR_INVALID_ARG, "shard_in and shard_out are required");
    for (int32_t s = 0; s < S; ++s) {
        if (plan->shard_elems[s] == 0) continue;
        if (!shard_in[s] || !shard_out[s]) return fail(NS_ERR_INVALID_ARG, "shard %d: NULL buffer", s);
        if ((reinterpret_cast<uintptr_t>(shard_in[s]) | reinterpret_cast<uintptr_t>(shard_out[s])) % es)
            return fail(NS_ERR_INVALID_ARG, "shard %d: buffer not %lld-byte aligned", s, (long long)es);
    }
    PieceLists pieces(n);
    for (int32_t i = 0; i < n; ++i) {
        if (!info[i].active) continue;
        int64_t row0 = 0;
        for (int32_t s = 0; s < S; ++s) {
            const int64_t r = plan->split_rows[(size_t)i * S + s];
            if (r == 0) continue;
            const int64_t off = plan->shard_offset[(size_t)i * S + s] * es;
            pieces[i].push_back(RowPiece{row0, static_cast<const char *>(shard_in[s]) + off,
                                         static_cast<char *>(shard_out[s]) + off, info[i].cols, info[i].cols});
            row0 += r;
        }
    }
    return orthogonalize(info, pieces, dtype, steps, a, b, c, eps, order, workspace, workspace_bytes,
                         reinterpret_cast<hipStream_t>(stream));
}

extern "C" ns_status ns_orthogonalize_waves(int32_t n, const ns_shape *shapes, const void *const *in,
                                            void *const *out, ns_dtype dtype, int32_t steps, float a,
                                            float b, float c, float eps, const int32_t *wave_of,
                                            int32_t num_waves, void *const *ready_events, void *workspace,
                                            size_t workspace_bytes, void *stream) {
    std::vector<MatInfo> info;
    ns_status st = describe(n, shapes, dtype, info);
    if (st) return st;
    if ((st = check_coefficients(steps, a, b, c, eps))) return st;
    if (num_waves < 0) return fail(NS_ERR_INVALID_ARG, "num_waves = %d < 0", num_waves);
    if (n > 0 && !wave_of) return fail(NS_ERR_INVALID_ARG, "wave_of is NULL");
    if (n > 0 && (!in || !out)) return fail(NS_ERR_INVALID_ARG, "in and out are required");
    const size_t es = dtype == NS_BF16 ? 2 : 4;
    PieceLists pieces(n);
    for (int32_t i = 0; i < n; ++i) {
        if (wave_of[i] >= num_waves)
            return fail(NS_ERR_INVALID_ARG, "tensor %d: wave %d >= num_waves %d", i, wave_of[i], num_waves);
        if (!info[i].active || wave_of[i] < 0) continue;
        if (!in[i] || !out[i]) return fail(NS_ERR_INVALID_ARG, "tensor %d: NULL in/out", i);
        if ((reinterpret_cast<uintptr_t>(in[i]) | reinterpret_cast<uintptr_t>(out[i])) % es)
            return fail(NS_ERR_INVALID_ARG, "tensor %d: in/out not %zu-byte aligned", i, es);
        pieces[i].push_back(RowPiece{0, static_cast<const char *>(in[i]), static_cast<char *>(out[i]),
                                     info[i].cols, info[i].cols});
    }
    size_t all, need;
    workspace_need(info, &all, &need);
    if (!workspace || workspace_bytes < need)
        return fail(NS_ERR_WORKSPACE, "workspace of %zu bytes < minimum %zu", workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(NS_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    // Every wave is planned (and every argument checked) before anything is
    // enqueued; then the waves go out in order, each after its event.
    CallPlan plan;
    for (int32_t w = 0; w < num_waves; ++w) {
        std::vector<MatInfo> wi = info;
        for (int32_t i = 0; i < n; ++i) wi[i].active = info[i].active && wave_of[i] == w;
        if ((st = plan_call(wi, pieces, dtype, steps, b, c, nullptr, workspace, workspace_bytes, false, plan)))
            return st;
    }
    return launch_call(plan, dtype, steps, a, b, c, eps, false, 0.f, workspace, ready_events,
                       reinterpret_cast<hipStream_t>(stream));
}

extern "C" ns_status ns_gram_workspace_bytes(int32_t n, const ns_shape *shapes, ns_dtype dtype, size_t *bytes,
                                             size_t *min_bytes) {
    if (!bytes) return fail(NS_ERR_INVALID_ARG, "bytes is NULL");
    std::vector<MatInfo> info;
    ns_status st = describe(n, shapes, dtype, info, true);
    if (st) return st;
    workspace_need(info, bytes, min_bytes);
    return NS_OK;
}

extern "C" ns_status ns_orthogonalize_gram(int32_t n, const ns_shape *shapes, const void *const *in,
                                           void *const *out, ns_dtype dtype, int32_t steps, float a, float b,
                                           float c, float eps, float ridge, const int32_t *order, void *workspace,
                                           size_t workspace_bytes, void *stream) {
    std::vector<MatInfo> info;
    ns_status st = describe(n, shapes, dtype, info, true);
    if (st) return st;
    if ((st = check_coefficients(steps, a, b, c, eps))) return st;
    if (!(ridge >= 0.f) || !std::isfinite(ridge)) return fail(NS_ERR_INVALID_ARG, "ridge must be finite and >= 0");
    if (n == 0) return NS_OK;
    if (!in || !out) return fail(NS_ERR_INVALID_ARG, "in and out are required");
    const size_t es = dtype == NS_BF16 ? 2 : 4;
    PieceLists pieces(n);
    for (int32_t i = 0; i < n; ++i) {
        if (!info[i].active) continue;
        if (!in[i] || !out[i]) return fail(NS_ERR_INVALID_ARG, "tensor %d: NULL in/out", i);
        if ((reinterpret_cast<uintptr_t>(in[i]) | reinterpret_cast<uintptr_t>(out[i])) % es)
            return fail(NS_ERR_INVALID_ARG, "tensor %d: in/out not %zu-byte aligned", i, es);
        pieces[i].push_back(RowPiece{0, static_cast<const char *>(in[i]), static_cast<char *>(out[i]),
                                     info[i].cols, info[i].cols});
    }
    return orthogonalize(info, pieces, dtype, steps, a, b, c, eps, order, workspace, workspace_bytes,
                         reinterpret_cast<hipStream_t>(stream), true, ridge);
}
