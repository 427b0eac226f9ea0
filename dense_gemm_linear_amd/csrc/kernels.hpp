// GEMM kernels for C[M,N] = A[M,K] * B[N,K]^T on gfx950.
//
// Both kernels work in bytes of K so that bf16 and e4m3 share one pipeline:
// a k-tile is 128 bytes of K (64 bf16 or 128 e4m3 values), i.e. two 64-byte
// blocks of the preshuffled B ("GEMM Optimization Guide" page, section 12.1:
// (N/16, K/64, 4, 16, 16 bytes)).  One 1 KiB block holds 16 columns x 64 K
// bytes; lane l of a wave loads its 16 bytes at l*16, which is the MFMA B
// operand of column l % 16 and K group l / 16.
//
// Tiled kernel ("GEMM Optimization Guide" page, sections 1, 2, 3, 4, 6, 7):
//   - 256 threads = 4 waves of 64; the waves split tile_n, every wave covers
//     all tile_m rows (section 1.1), so B needs no LDS and is never shared;
//   - A goes global -> VGPR -> LDS into one of two buffers (ping-pong, section
//     2) with an XOR swizzle on 16-byte columns (section 3), one barrier per
//     k-tile; B goes global -> VGPR straight from the preshuffled layout
//     (section 4.2), one k-tile ahead;
//   - fp32 accumulators stay in registers for the whole K loop;
//   - the epilogue scales (e4m3), rounds to bf16 and stages the tile through
//     LDS so each lane stores 16 contiguous bytes of a C row (section 7.2);
//   - ragged M, N and the K tail are served by buffer descriptors bounded at
//     the real extent plus an out-of-range offset, and a column predicate on
//     the C store (FlyDSL PR #1303 page).
//
// Skinny kernel (small M: decode and short prefill): one workgroup per group
// of 16-column blocks covering all M rows; the 4 waves split K, stream their
// part of B once at full width and read A straight from global (it is small
// and stays in L2); partial sums are reduced in LDS in a fixed order.
#pragma once

#include <type_traits>

#include "device.hpp"

namespace dg {

enum { DT_BF16 = 0, DT_FP8 = 1 };
// Kernel variants: one-pass with a plain bf16 epilogue, split-K (fp32
// partials, the epilogue runs in the reduction), one-pass with the fused
// epilogue.  Separate instances, so that no variant pays for another's code
// in registers.
enum { MODE_PLAIN = 0, MODE_SPLIT = 1, MODE_EPI = 2, MODE_SK = 3 };
// activation codes (the values of gemm_activation)
enum { ACT_NONE = 0, ACT_RELU = 1, ACT_SILU = 2, ACT_GELU_ERF = 3, ACT_GELU_TANH = 4 };

// Fused epilogue, applied per output element in fp32 after the e4m3
// per-tensor scales: v *= scale_m[row]; v *= scale_n[col]; v += bias[col];
// v = act(v); v *= mul[row][col]; then bf16 rounding.  Every part is
// optional (null pointer, ACT_NONE); `on` is set when any part is present.
struct Epilogue {
    const uint16_t* bias;    // bf16 [N]
    const float* scale_m;    // fp32 [M]: per-row (per-token) multiplier
    const float* scale_n;    // fp32 [N]: per-column (per-channel) multiplier
    const uint16_t* mul;     // bf16 [M, ldmul]
    int64_t ldmul;
    int act;
    int on;
    int mul_vec;             // mul and ldmul allow 16-byte row pieces
};

__device__ __forceinline__ float bf16_to_f32(uint16_t h)
{
    return __uint_as_float((uint32_t)h << 16);
}

// Activations from exponentials and reciprocals (the epilogue is unrolled
// over every accumulator element, so the code per element must stay small;
// it runs after the K loop with nothing to hide it, so its VALU count is
// time).  The reciprocals are the hardware's v_rcp_f32 (1 ulp) rather than
// the correctly rounded division, which takes 11 VALU instructions: SiLU
// drops from 16 to 5, bf16 rounding of the result is far coarser than
// either.  SiLU is x * logistic(x); the tanh form of GELU is x * logistic(2u),
// u = sqrt(2/pi) (x + 0.044715 x^3), since (1 + tanh u) / 2 = logistic(2u);
// the erf form is x * Phi(x) with erf from Abramowitz and Stegun, Handbook of
// Mathematical Functions, formula 7.1.26 (absolute error <= 1.5e-7, far below
// bf16 rounding): erf(z) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) e^(-z^2),
// t = 1 / (1 + p z), z >= 0, odd in z.
// Activation classes, so that a launch evaluates only what its activation
// needs (the class is fixed per launch; inside a class the code is
// branch-free, so the unrolled epilogue has no per-element control flow):
//   0: none, ReLU; 1: SiLU, tanh-form GELU (one exponential, one reciprocal);
//   2: erf-form GELU.
__device__ __forceinline__ int act_class(int act)
{
    return act == ACT_GELU_ERF ? 2 : (act == ACT_SILU || act == ACT_GELU_TANH) ? 1 : 0;
}

template <int C>
__device__ __forceinline__ float activate_c(int act, float x)
{
    if constexpr (C == 0) {
        return act == ACT_RELU ? fmaxf(x, 0.f) : x;
    } else if constexpr (C == 1) {
        const float z = act == ACT_GELU_TANH ? 1.5957691216057308f * (x + 0.044715f * x * x * x) : x;
        return x * __builtin_amdgcn_rcpf(1.f + __expf(-z));
    } else {
        const float a = fabsf(x) * 0.70710678118654752f;
        const float t = __builtin_amdgcn_rcpf(1.f + 0.3275911f * a);
        const float poly =
            t * (0.254829592f +
                 t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
        return 0.5f * x * (1.f + copysignf(1.f - poly * __expf(-a * a), x));
    }
}

__device__ __forceinline__ float activate(int act, float x)
{
    switch (act_class(act)) {
    case 1:
        return activate_c<1>(act, x);
    case 2:
        return activate_c<2>(act, x);
    default:
        return activate_c<0>(act, x);
    }
}

// The epilogue of element (row, col); both must lie inside M x N (callers
// clamp the padding elements they compute but never store).
__device__ __forceinline__ float apply_epilogue(const Epilogue& ep, float v, int row, int col)
{
    if (ep.scale_m)
        v *= ep.scale_m[row];
    if (ep.scale_n)
        v *= ep.scale_n[col];
    if (ep.bias)
        v += bf16_to_f32(ep.bias[col]);
    v = activate(ep.act, v);
    if (ep.mul)
        v *= bf16_to_f32(ep.mul[(int64_t)row * ep.ldmul + col]);
    return v;
}

// Tile rows per raster group, and whether workgroups are renumbered per XCD.
#ifndef DG_GROUP_M
#define DG_GROUP_M 4
#endif
#ifndef DG_XCD_REMAP
#define DG_XCD_REMAP 1
#endif

struct GemmArgs {
    const uint8_t* A;     // [M, lda] elements, row-major
    const uint8_t* Bs;    // preshuffled B
    uint16_t* C;          // [M, ldc] bf16
    const float* sa;      // e4m3 dequant scales (device), unused for bf16
    const float* sb;
    int64_t lda_b;        // A row pitch in bytes
    int64_t ldc;          // C row pitch in elements
    int M, N;
    int KA_b;             // valid K bytes per A row (K * element bytes)
    int KB;               // 64-byte K blocks per 16-column block in Bs
    int nkt;              // k-tiles of 128 bytes = ceil(KB / 2)
    int tail;             // last k-tile reaches past K (needs masked loads)
    int tiles_m, tiles_n; // tiled kernel grid
    int nblk;             // ceil(N / 16)
    int c_vec;            // C base 16-byte aligned and ldc % 8 == 0
    // Split-K (tiled kernels): the grid is tiles x splits workgroups; slice s
    // multiplies k-tiles [s kt_per, (s+1) kt_per) and writes its fp32 partial
    // tile to plane s of ws ([splits][M][ldw], ldw = N rounded up to 4)
    // instead of C.  splits == 1: the whole K range, C written directly.
    int splits;
    int kt_per;           // k-tiles per slice, in the kernel's own k-tile size
    int ldw;
    float* ws;
    Epilogue ep;
    // Stream-K (MODE_SK): a persistent grid of G workgroups.  Tiles
    // [0, sk_dp_tiles) run whole, logical workgroup g taking tiles g, g + G,
    // ...; the (tile, k-tile) units of the other tiles are cut into G equal
    // contiguous ranges, one per workgroup.  A tile cut between workgroups
    // is finished by the last of them to arrive (sk_count), from fp32
    // partials in ws: two slots of TM x TN floats per workgroup.
    int sk_dp_tiles;
    int sk_nkt;           // k-tiles per tile, in the kernel's own k-tile size
    uint32_t* sk_count;   // per stream-K tile; zero on entry, left zero on exit
};

// The K range of one workgroup: k-tiles [kt0, kt0 + n) of KTB bytes, and the
// bounds its masked loads test against (the slice end, or K itself for the
// last slice).  last_full is the first k-tile that needs masking.
struct KRange {
    int kt0, n, ka_end, kb_end, last_full;
};

template <int KTB, bool SPLIT>
__device__ __forceinline__ KRange k_range(const GemmArgs& p, int slice)
{
    constexpr int KPK = KTB / 64;
    const int nkt = (p.KB + KPK - 1) / KPK;
    KRange r;
    if constexpr (!SPLIT) {
        r.kt0 = 0;
        r.n = nkt;
        r.ka_end = p.KA_b;
        r.kb_end = p.KB;
        r.last_full = p.KA_b / KTB;
        return r;
    }
    const int per = p.kt_per;
    r.kt0 = slice * per;
    const int kt_end = min(nkt, r.kt0 + per);
    r.n = kt_end - r.kt0;
    r.ka_end = min(p.KA_b, kt_end * KTB);
    r.kb_end = min(p.KB, kt_end * KPK);
    r.last_full = r.ka_end / KTB;
    return r;
}

// Workgroup -> (output tile index, K slice): slices outermost, so the
// workgroups running together share A rows and B columns of one K range.
template <bool SPLIT>
__device__ __forceinline__ int split_slice(const GemmArgs& p, int& wg)
{
    if constexpr (!SPLIT) {
        wg = (int)blockIdx.x;
        return 0;
    }
    const int G = p.tiles_m * p.tiles_n;
    const int slice = (int)blockIdx.x / G;
    wg = (int)blockIdx.x - slice * G;
    return slice;
}

// Workgroup -> output tile.  Workgroups are dispatched round robin over the 8
// XCDs, each with its own L2; renumber so that every XCD receives one
// contiguous run of logical tiles, then walk the logical tiles in groups of
// GROUP_M tile rows, column by column, so tiles that share A rows or B columns
// run at the same time on the same L2.
__device__ __forceinline__ int xcd_remap(int wg, int G)
{
    if (!DG_XCD_REMAP)
        return wg;
    const int x = wg & 7, j = wg >> 3;
    const int q = G >> 3, r = G & 7;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + j;
}

// Logical tile t -> (tile row, tile column), GROUP_M tile rows at a time.
template <int GROUP_M>
__device__ __forceinline__ void tile_raster(int t, int tiles_m, int tiles_n, int& tm, int& tn)
{
    const int per_group = GROUP_M * tiles_n;
    const int grp = t / per_group;
    const int first = grp * GROUP_M;
    const int gm = min(tiles_m - first, GROUP_M);
    const int in = t - grp * per_group;
    tm = first + in % gm;
    tn = in / gm;
}

template <int GROUP_M>
__device__ __forceinline__ void tile_coords(int wg, int tiles_m, int tiles_n, int& tm, int& tn)
{
    const int t = xcd_remap(wg, tiles_m * tiles_n);
    const int per_group = GROUP_M * tiles_n;
    const int grp = t / per_group;
    const int first = grp * GROUP_M;
    const int gm = min(tiles_m - first, GROUP_M);
    const int in = t - grp * per_group;
    tm = first + in % gm;
    tn = in / gm;
}


// ---------------------------------------------------------------------------
// MFMA atoms.  An atom is one R x R block of C computed by one MFMA per K
// step.  A k-tile (128 bytes of K) takes STEPS MFMAs along K, and for each
// one every lane supplies P 16-byte pieces of A and P of B.  Piece p of step
// s holds the same K bytes of the k-tile in the A operand and in the B
// operand, which is all the sum over K needs to pair A[m][k] with B[n][k]:
//   A: row (lane % R) of the atom in the LDS A tile, 16-byte chunk a_chunk;
//   B: column (lane % R) of the atom, in the 64-byte half b_half of the
//      k-tile (one 1 KiB block of the preshuffled B) and lane group b_group.
// Output element e of lane l sits at row out_row(e, l), column l % R.
//
// The 16 x 16 atoms are the pages' choice ("GEMM Optimization Guide" page,
// section 6.1).  On MI355X the 32 x 32 bf16 MFMA sustains the full dense
// rate with its accumulators in ordinary VGPRs, while back-to-back 16 x 16 x
// 32 bf16 MFMAs from one wave accumulating in VGPRs issue at roughly half of
// it (measured).  With two waves per SIMD taking turns, the 16 x 16 atom
// keeps the pipe as busy as the 32 x 32 one in the 8-wave 256 x 256 tile,
// and the board holds a higher clock with it under its power limit, so the
// ladder has both.
template <int DT, int R>
struct Atom;

template <>
struct Atom<DT_BF16, 16> {   // v_mfma_f32_16x16x32_bf16
    static constexpr int R = 16, STEPS = 2, P = 1, NACC = 4;
    using acc_t = f32x4;
    static __device__ __forceinline__ int a_chunk(int s, int l, int) { return 4 * s + (l >> 4); }
    static __device__ __forceinline__ int b_half(int s, int) { return s; }
    static __device__ __forceinline__ int b_group(int, int l, int) { return l >> 4; }
    static __device__ __forceinline__ int out_row(int e, int l) { return 4 * (l >> 4) + e; }
    static __device__ __forceinline__ acc_t mma(const i32x4 (&a)[P], const i32x4 (&b)[P], acc_t c)
    {
        return mfma_bf16(a[0], b[0], c);
    }
};

template <>
struct Atom<DT_BF16, 32> {   // v_mfma_f32_32x32x16_bf16
    static constexpr int R = 32, STEPS = 4, P = 1, NACC = 16;
    using acc_t = f32x16;
    static __device__ __forceinline__ int a_chunk(int s, int l, int) { return 2 * s + (l >> 5); }
    static __device__ __forceinline__ int b_half(int s, int) { return s >> 1; }
    static __device__ __forceinline__ int b_group(int s, int l, int) { return 2 * (s & 1) + (l >> 5); }
    static __device__ __forceinline__ int out_row(int e, int l) { return 8 * (e >> 2) + 4 * (l >> 5) + (e & 3); }
    static __device__ __forceinline__ acc_t mma(const i32x4 (&a)[P], const i32x4 (&b)[P], acc_t c)
    {
        return mfma_bf16_32(a[0], b[0], c);
    }
};

template <>
struct Atom<DT_FP8, 16> {    // v_mfma_scale_f32_16x16x128_f8f6f4
    static constexpr int R = 16, STEPS = 1, P = 2, NACC = 4;
    using acc_t = f32x4;
    static __device__ __forceinline__ int a_chunk(int, int l, int p) { return 4 * p + (l >> 4); }
    static __device__ __forceinline__ int b_half(int, int p) { return p; }
    static __device__ __forceinline__ int b_group(int, int l, int) { return l >> 4; }
    static __device__ __forceinline__ int out_row(int e, int l) { return 4 * (l >> 4) + e; }
    static __device__ __forceinline__ acc_t mma(const i32x4 (&a)[P], const i32x4 (&b)[P], acc_t c)
    {
        return mfma_fp8(cat(a[0], a[1]), cat(b[0], b[1]), c);
    }
};

template <>
struct Atom<DT_FP8, 32> {    // v_mfma_scale_f32_32x32x64_f8f6f4
    static constexpr int R = 32, STEPS = 2, P = 2, NACC = 16;
    using acc_t = f32x16;
    static __device__ __forceinline__ int a_chunk(int s, int l, int p) { return 4 * s + 2 * (l >> 5) + p; }
    static __device__ __forceinline__ int b_half(int s, int) { return s; }
    static __device__ __forceinline__ int b_group(int, int l, int p) { return 2 * (l >> 5) + p; }
    static __device__ __forceinline__ int out_row(int e, int l) { return 8 * (e >> 2) + 4 * (l >> 5) + (e & 3); }
    static __device__ __forceinline__ acc_t mma(const i32x4 (&a)[P], const i32x4 (&b)[P], acc_t c)
    {
        return mfma_fp8_32(cat(a[0], a[1]), cat(b[0], b[1]), c);
    }
};

template <class AT>
__device__ __forceinline__ typename AT::acc_t zero_acc()
{
    typename AT::acc_t z;
#pragma unroll
    for (int e = 0; e < AT::NACC; ++e)
        z[e] = 0.f;
    return z;
}

typedef __attribute__((address_space(3))) void lds_void;

// ---------------------------------------------------------------------------
// The k-tile: KTB bytes of K (64 or 128) per pipeline stage.  A stage of the
// A tile holds TM rows of KTB bytes; 16-byte chunk c of row r is stored at
// slot c ^ key(r), an XOR swizzle at 16-byte granularity ("GEMM Optimization
// Guide" page, section 3).  key depends on bits 1-3 of r only, so rows 16
// apart share it (a fragment read takes it from lane % 16).  Measured on
// MI355X (SQ_LDS_BANK_CONFLICT of the fragment reads alone): for 128-byte
// rows key = (r / 2) % 8 serves the 16 x 16 and 32 x 32 fragments without a
// conflict; for 64-byte rows (r / 4) % 4 doubled every 16 x 16 fragment read
// (lanes 16 i .. 16 i + 15 reading chunk i of 16 rows), while
// ((r / 4) ^ (r / 2)) % 4 is conflict-free for both atoms.  The global -> LDS
// copy is a 16-byte LDS DMA per lane (page section 11: 16 bytes per op on
// gfx950): one wave load fills 1 KiB = 1024 / KTB rows, lane l landing in row
// l / (KTB / 16), slot l % (KTB / 16), so the swizzle is applied to the global
// address.  B arrives as whole 1 KiB blocks
// of the preshuffled layout (16 columns x 64 K bytes), KTB / 64 per 16-column
// block per k-tile.
template <int KTB>
struct KTile {
    static_assert(KTB == 64 || KTB == 128, "k-tile of 64 or 128 bytes");
    static constexpr int CHUNKS = KTB / 16;        // 16-byte chunks per A row
    static constexpr int ROWS_PER_LOAD = 1024 / KTB;
    static constexpr int KPK = KTB / 64;           // Bs blocks per 16 columns per k-tile
    static __host__ __device__ constexpr uint32_t key(uint32_t row)
    {
        return KTB == 64 ? ((row >> 2) ^ (row >> 1)) & 3u : (row >> 1) & 7u;
    }
};

struct ADma {
    uint32_t goff;   // byte offset of this lane's 16 bytes in the A slab (k-tile 0)
    uint32_t col;    // its K byte within the k-tile (for the K-tail mask)
};

template <int KTB>
__device__ __forceinline__ ADma a_dma_lane(int chunk, int lane, int64_t lda_b)
{
    using KT = KTile<KTB>;
    const uint32_t row = KT::ROWS_PER_LOAD * (uint32_t)chunk + (uint32_t)(lane / KT::CHUNKS);
    const uint32_t col = (uint32_t)(lane % KT::CHUNKS) ^ KT::key(row);
    return {row * (uint32_t)lda_b + col * 16, col * 16};
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), expanded
// at compile time.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Orders this wave's LDS accesses for the compiler, with no instruction and
// no wait: a wave's LDS operations execute in issue order, so a lane reading
// what another lane of the same wave wrote needs nothing more.  The epilogue
// stages each wave's block in a region of its own; a workgroup barrier there
// also waited for every C store in flight (s_barrier comes with vmcnt(0)) and
// lengthened the 4096^3 epilogue by about 0.4 us (measured on MI355X).
__device__ __forceinline__ void wave_lds_order()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Epilogue shared by the tiled kernels: scale (e4m3), round to bf16, stage a
// wave's (MR*R) x (NR*R) accumulator block through its private LDS region
// CH atom rows at a time, and store 16-byte row pieces ("GEMM Optimization
// Guide" page, section 7.2).  Rows past M fall outside the C descriptor; the
// column predicate keeps a row's padding and the next row intact.  It ends
// without a workgroup barrier: a caller that goes on to load a further tile
// into LDS must put one first.
//
// C rows need not start on a 16-byte boundary (odd ldc, or an unaligned C):
// a row segment whose first element sits at element phase ph (mod 8) of its
// absolute address is staged ph elements to the right (the row pitch has 8
// elements of slack), so staged 16-byte piece k is the k-th aligned 16-byte
// piece of C that the segment touches.  Pieces 1 .. PPR-1 are whole: one LDS
// read and one aligned store each.  Piece 0 (8 - ph elements at the head) and
// piece PPR (ph at the tail) are shared with the neighbouring segments and
// are written element by element.
template <int DT, class AT, int MR, int NR, int CH, int SROW, int WCOLS, bool EPI>
__device__ __forceinline__ void store_c_tile(const GemmArgs& p,
                                             const typename AT::acc_t (&acc)[MR][NR],
                                             uint8_t* stage, int m0, int rows, int col_w, int row0,
                                             int lane, float scale_a, float scale_b)
{
    constexpr int R = AT::R;
    const rsrc_t rc = make_rsrc(p.C + (int64_t)m0 * p.ldc,
                                (uint32_t)(((int64_t)(rows - 1) * p.ldc + p.N) * 2));
    constexpr int PPR = WCOLS / 8;                 // 16-byte pieces per staged row
    constexpr int PIECES = CH * R * PPR;
    const int lc = lane % R;
    // element phase (mod 8) of this tile's C base
    const uint32_t base_ph =
        (uint32_t)((((uintptr_t)p.C) >> 1) + (uint64_t)m0 * (uint64_t)p.ldc + (uint32_t)col_w) & 7u;
    const uint32_t ldc_ph = (uint32_t)p.ldc & 7u;
    // phase of row `trow` of the tile; 0 on every row when p.c_vec
    auto row_phase = [&](int trow) __attribute__((always_inline)) {
        return (int)((base_ph + (uint32_t)trow * ldc_ph) & 7u);
    };
    // Fused epilogue operands.  A lane's columns are the same for every
    // element of accumulator column j, so the column scale and bias are
    // loaded once per tile; row scales once per accumulator row; the
    // multiplier through LDS, one block per chunk (below).  (Loaded element
    // by element between the LDS staging stores, each load waited for its
    // own round trip.)  Indices past M or N are clamped: those elements are
    // computed but never stored.
    float col_scale[NR], col_bias[NR];
    if constexpr (EPI) {
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            const int col = min(col_w + j * R + lc, p.N - 1);
            col_scale[j] = p.ep.scale_n ? p.ep.scale_n[col] : 1.f;
            col_bias[j] = p.ep.bias ? bf16_to_f32(p.ep.bias[col]) : 0.f;
        }
    }
    // chunks expanded at compile time: with a large epilogue the unroller
    // may keep this loop (it holds a barrier), and a run-time chunk index
    // would put the accumulators in scratch memory
    auto chunks = [&](auto cls_c, auto scl_c) __attribute__((always_inline)) {
        constexpr int CLS = decltype(cls_c)::value;
        constexpr bool SCL = decltype(scl_c)::value;   // row or column scales given
        static_for<MR / CH>([&](auto cc_c) __attribute__((always_inline)) {
            constexpr int cc = decltype(cc_c)::value;
            if constexpr (EPI) {
                // The multiplier block of this chunk, the same [CH R][WCOLS]
                // shape as the staged C chunk, goes into this wave's staging
                // area first, all loads in flight at once; the staging loop
                // then reads each element from LDS and writes the result
                // over it.  Rows past M fall outside the descriptor.
                if (p.ep.mul) {
                    const rsrc_t rm = make_rsrc(
                        p.ep.mul + (int64_t)m0 * p.ep.ldmul,
                        (uint32_t)(((int64_t)(rows - 1) * p.ep.ldmul + p.N) * 2));
                    if (p.ep.mul_vec && p.c_vec) {
                        constexpr int NQ = (PIECES + 63) / 64;
                        i32x4 mv[NQ];
#pragma unroll
                        for (int k = 0; k < NQ; ++k) {
                            const int q = 64 * k + lane;
                            if (PIECES % 64 == 0 || q < PIECES) {
                                const int prow = q / PPR, pc = q % PPR;
                                const uint32_t trow = (uint32_t)(row0 + cc * CH * R + prow);
                                mv[k] = load16(rm, (trow * (uint32_t)p.ep.ldmul + (uint32_t)col_w +
                                                    8u * (uint32_t)pc) * 2u);
                            }
                        }
#pragma unroll
                        for (int k = 0; k < NQ; ++k) {
                            const int q = 64 * k + lane;
                            if (PIECES % 64 == 0 || q < PIECES) {
                                const int prow = q / PPR, pc = q % PPR;
                                *reinterpret_cast<i32x4*>(stage + prow * SROW + pc * 16) = mv[k];
                            }
                        }
                    } else {
                        // staged at the row's phase, as the C values are
                        for (int idx = lane; idx < CH * R * WCOLS; idx += 64) {
                            const int prow = idx / WCOLS, c = idx % WCOLS;
                            const uint32_t trow = (uint32_t)(row0 + cc * CH * R + prow);
                            const int ph = row_phase((int)trow);
                            *reinterpret_cast<uint16_t*>(stage + prow * SROW + (c + ph) * 2) =
                                __builtin_amdgcn_raw_buffer_load_b16(
                                    rm, (int)((trow * (uint32_t)p.ep.ldmul + (uint32_t)(col_w + c)) * 2u),
                                    0, 0);
                        }
                    }
                    __syncthreads();
                }
            }
#pragma unroll
            for (int ml = 0; ml < CH; ++ml) {
                float row_scale[AT::NACC];
                if constexpr (EPI && SCL) {
#pragma unroll
                    for (int e = 0; e < AT::NACC; ++e) {
                        const int grow =
                            min(m0 + row0 + (cc * CH + ml) * R + AT::out_row(e, lane), p.M - 1);
                        row_scale[e] = p.ep.scale_m ? p.ep.scale_m[grow] : 1.f;
                    }
                }
#pragma unroll
                for (int e = 0; e < AT::NACC; ++e) {
                    const int row = ml * R + AT::out_row(e, lane);
                    const int ph = row_phase(row0 + cc * CH * R + row);
#pragma unroll
                    for (int j = 0; j < NR; ++j) {
                        float v = acc[cc * CH + ml][j][e];
                        if constexpr (DT == DT_FP8)
                            v = (v * scale_a) * scale_b;
                        const int col = j * R + lc + ph;
                        uint16_t* sp = reinterpret_cast<uint16_t*>(stage + row * SROW + col * 2);
                        if constexpr (EPI) {
                            if constexpr (SCL) {
                                v = v * row_scale[e];
                                v = v * col_scale[j];
                            }
                            v = v + col_bias[j];
                            v = activate_c<CLS>(p.ep.act, v);
                            if (p.ep.mul)
                                v = v * bf16_to_f32(*sp);
                        }
                        *sp = bf16_rne(v);
                    }
                }
            }
            wave_lds_order();
#pragma unroll
            for (int q0 = 0; q0 < PIECES; q0 += 64) {
                const int q = q0 + lane;
                if (PIECES % 64 == 0 || q < PIECES) {
                    const int prow = q / PPR, pc = q % PPR;
                    const int trow = row0 + cc * CH * R + prow;   // row within the tile
                    const uint32_t row_off = (uint32_t)((int64_t)trow * p.ldc + col_w);  // elements
                    const uint8_t* srow = stage + prow * SROW;
                    const int ph = row_phase(trow);
                    if (ph == 0 || pc < PPR - 1) {
                        const int k = pc + (ph != 0);               // staged piece
                        const i32x4 v = *reinterpret_cast<const i32x4*>(srow + k * 16);
                        const int col = 8 * k - ph;                 // its first column
                        const int gcol = col_w + col;
                        const uint32_t off = (row_off + (uint32_t)col) * 2u;
                        if (gcol + 8 <= p.N) {
                            store16(rc, off, v);
                        } else {
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                if (gcol + e < p.N)
                                    store2(rc, off + 2 * e,
                                           (uint16_t)(((uint32_t)v[e >> 1]) >> (16 * (e & 1))));
                        }
                    }
                }
            }
            if (!p.c_vec) {
                // The shared pieces of every row: head columns [0, 8 - ph),
                // tail columns [WCOLS - ph, WCOLS), one element per lane.
                constexpr int ELEMS = CH * R * 8;
#pragma unroll
                for (int u0 = 0; u0 < ELEMS; u0 += 64) {
                    const int u = u0 + lane;
                    const int prow = u >> 3, e = u & 7;
                    const int trow = row0 + cc * CH * R + prow;
                    const int ph = row_phase(trow);
                    const int col = e < 8 - ph ? e : WCOLS - 8 + e;
                    if (ph != 0 && col_w + col < p.N)
                        store2(rc, ((uint32_t)((int64_t)trow * p.ldc + col_w) + (uint32_t)col) * 2u,
                               *reinterpret_cast<const uint16_t*>(stage + prow * SROW + (col + ph) * 2));
                }
            }
            wave_lds_order();
        });
    };
    // The activation class is chosen once per launch; for the cheapest class
    // (none or ReLU: a bias alone, say) also whether any scale is given, since
    // there the two multiplies by 1 per element are most of the VALU work after
    // the K loop (exact to drop).  The other classes keep one variant each:
    // more copies of the staging loop raised register spills.
    if constexpr (EPI) {
        const int cls = act_class(p.ep.act);
        if (cls == 1)
            chunks(std::integral_constant<int, 1>{}, std::true_type{});
        else if (cls == 2)
            chunks(std::integral_constant<int, 2>{}, std::true_type{});
        else if (p.ep.scale_m || p.ep.scale_n)
            chunks(std::integral_constant<int, 0>{}, std::true_type{});
        else
            chunks(std::integral_constant<int, 0>{}, std::false_type{});
    } else {
        chunks(std::integral_constant<int, 0>{}, std::false_type{});
    }
}

// Largest CH dividing MR whose staging (WAVES regions of CH*R rows) fits in
// `avail` bytes of LDS.
// Split-K: this wave's fp32 accumulators into plane `slice` of the partial
// workspace, row-major with pitch ldw.  For one accumulator element the 64
// lanes write whole runs of R consecutive floats of one or more rows.  Rows
// past M fall outside the descriptor (dropped); columns past N are switched
// off per lane.
template <class AT, int MR, int NR>
__device__ __forceinline__ void store_partial(const GemmArgs& p,
                                              const typename AT::acc_t (&acc)[MR][NR], int slice,
                                              int row_w, int col_w, int lane)
{
    constexpr int R = AT::R;
    const rsrc_t rw = make_rsrc(p.ws + (int64_t)slice * p.M * p.ldw,
                                (uint32_t)((int64_t)p.M * p.ldw * 4));
    const int lc = lane % R;
    const uint32_t pitch = (uint32_t)p.ldw * 4u;
#pragma unroll
    for (int mi = 0; mi < MR; ++mi)
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            const int col = col_w + j * R + lc;
            // byte offset of element 0; a lane past N gets kOOB, which stays
            // past the bound with the row steps below added (they are under
            // 32 rows, and the host keeps (M + 256) * pitch within 2^31).
            // A branch-free select: one base per accumulator, not per element.
            const uint32_t row0 = (uint32_t)(row_w + mi * R + AT::out_row(0, lane));
            const uint32_t inb = 0u - (uint32_t)(col < p.N);
            const uint32_t base = (((row0 * (uint32_t)p.ldw + (uint32_t)col) * 4u) & inb) |
                                  (kOOB & ~inb);
#pragma unroll
            for (int e = 0; e < AT::NACC; ++e) {
                // the rows of one accumulator's elements differ by constants
                const uint32_t step = (uint32_t)(AT::out_row(e, lane) - AT::out_row(0, lane));
                // through a scalar: hipcc's __builtin_bit_cast of a vector
                // element lvalue reads element 0 (seen in the ISA)
                const float v = acc[mi][j][e];
                store4(rw, base + step * pitch, __float_as_uint(v));
            }
        }
}

// s_waitcnt (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8): vector-memory counter at most n, every LDS access of this
// wave complete (lgkmcnt 0; expcnt left at its maximum).
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4); }

// ---------------------------------------------------------------------------
// Stream-K (the TraceLens GEMM analysis page, "Important considerations",
// names Stream-K among what its tile/wave model leaves out).  The U = tiles x
// k-tiles units of the stream-K tiles, in tile order, are cut into G
// contiguous ranges, [sk_start(g), sk_start(g + 1)) for logical workgroup g.

__device__ __forceinline__ int64_t sk_start(int64_t U, int G, int g)
{
    return U * g / G;
}

// The logical workgroup whose range holds unit u.
__device__ __forceinline__ int sk_owner(int64_t U, int G, int64_t u)
{
    int g = (int)(u * G / U);
    while (g + 1 < G && sk_start(U, G, g + 1) <= u)
        ++g;
    while (g > 0 && sk_start(U, G, g) > u)
        --g;
    return g;
}

// A workgroup's fp32 partial tile, in the order its lanes hold it: for
// wave w and atom (mi, j), piece q (accumulator elements 4q .. 4q + 3) of
// all 64 lanes is one contiguous 1 KiB run, lane l at 16 l, so every store
// and load instruction moves whole cache lines (the stores write through
// to memory).  Slot s of logical workgroup g starts at ws + (2 g + s) TM TN
// floats.  sk_lane_off is the byte offset of piece 0 of lane l.
template <class AT, int MR, int NR>
__device__ __forceinline__ uint32_t sk_lane_off(int wave, int mi, int j, int lane)
{
    return (uint32_t)(((wave * MR + mi) * NR + j) * AT::NACC * 256 + lane * 16);
}

template <class AT, int MR, int NR>
__device__ __forceinline__ void sk_store_partial(rsrc_t rs, const typename AT::acc_t (&acc)[MR][NR],
                                                 int wave, int lane)
{
#pragma unroll
    for (int mi = 0; mi < MR; ++mi)
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            const uint32_t o = sk_lane_off<AT, MR, NR>(wave, mi, j, lane);
#pragma unroll
            for (int e = 0; e < AT::NACC; e += 4) {
                i32x4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x = acc[mi][j][e + i];   // through a scalar (see store_partial)
                    v[i] = __float_as_int(x);
                }
                store16_coherent(rs, o + 256u * e, v);   // piece e / 4: 1 KiB further
            }
        }
}

// The fix-up of stream-K tile ts after this workgroup (logical g) wrote its
// partial to slot `slot` (`flag`: one int of the kernel's LDS, free between
// the K loop and the epilogue; a separate LDS variable made the compiler
// guard every LDS read of the K loop with a wait for all LDS DMA loads).
// Fix-up steps:
// partial to slot `slot`: count the segment in; the last segment to arrive
// sums every segment's partial in k order, ((0 + p0) + p1) + ..., into acc
// and returns true (the caller then stores C).  Nothing waits on another
// workgroup, so no grid-wide residency is assumed.  The partials cross XCDs,
// each with its own L2: they are written through to memory and read past
// the caches (kCpolCoherent), every wave waits for its stores to complete
// before the workgroup barrier, and the counter is a system-scope atomic
// (performed past the L2s), so the last arriver reads every partial as
// written.  (Device-scope fences
// instead wrote back and invalidated the whole L2 at every cut tile: the
// LLaMA prefill took 251 us against 61 us without stream-K.)
template <class AT, int MR, int NR, int TM, int TN>
__device__ __forceinline__ bool sk_fixup(const GemmArgs& p, typename AT::acc_t (&acc)[MR][NR],
                                         int* flag, int g, int G, int64_t U, int ts, int slot,
                                         int wave, int lane)
{
    constexpr uint32_t SLOT_BYTES = (uint32_t)TM * TN * 4u;
    const rsrc_t mine = make_rsrc(p.ws + ((size_t)g * 2 + slot) * TM * TN, SLOT_BYTES);
    sk_store_partial<AT, MR, NR>(mine, acc, wave, lane);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));   // this wave's partial stored
    __syncthreads();
    if (threadIdx.x == 0)
        *flag = (int)__hip_atomic_fetch_add(p.sk_count + ts, 1u, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_SYSTEM);
    __syncthreads();
    const int arrived = *flag;
    // the flag lives in the LDS the epilogue stages C through: every wave
    // has read it before any wave goes on
    __syncthreads();
    const int64_t u0 = (int64_t)ts * p.sk_nkt;
    const int g_first = sk_owner(U, G, u0);
    const int nseg = sk_owner(U, G, u0 + p.sk_nkt - 1) - g_first + 1;
    if (arrived != nseg - 1)
        return false;
#pragma unroll
    for (int mi = 0; mi < MR; ++mi)
#pragma unroll
        for (int j = 0; j < NR; ++j)
            acc[mi][j] = zero_acc<AT>();
    for (int k = 0; k < nseg; ++k) {
        const int gk = g_first + k;
        // slot 0: the tile is the first item of gk's range
        const int sk = sk_start(U, G, gk) >= u0 ? 0 : 1;
        const rsrc_t rk = make_rsrc(p.ws + ((size_t)gk * 2 + sk) * TM * TN, SLOT_BYTES);
#pragma unroll
        for (int mi = 0; mi < MR; ++mi)
#pragma unroll
            for (int j = 0; j < NR; ++j) {
                const uint32_t o = sk_lane_off<AT, MR, NR>(wave, mi, j, lane);
#pragma unroll
                for (int e = 0; e < AT::NACC; e += 4) {
                    const i32x4 v = load16_coherent(rk, o + 256u * e);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[mi][j][e + i] += __int_as_float(v[i]);
                    }
                }
            }
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(p.sk_count + ts, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    return true;
}

// Runs item(tile, kb, ke, slot) for this workgroup's work: its whole tiles,
// then its stream-K range cut at tile boundaries (k-tiles [kb, ke) of the
// tile; slot = which of its two partial slots a cut tile uses).
template <class Item>
__device__ __forceinline__ void sk_for_each(const GemmArgs& p, Item& item)
{
    const int G = (int)gridDim.x;
    const int g = xcd_remap((int)blockIdx.x, G);
    const int tiles = p.tiles_m * p.tiles_n;
    for (int t = g; t < p.sk_dp_tiles; t += G)
        item(t, 0, p.sk_nkt, 0);
    const int nkt = p.sk_nkt;
    const int64_t U = (int64_t)(tiles - p.sk_dp_tiles) * nkt;
    const int64_t u0 = sk_start(U, G, g), u1 = sk_start(U, G, g + 1);
    for (int64_t u = u0; u < u1;) {
        const int ts = (int)(u / nkt);
        const int kb = (int)(u - (int64_t)ts * nkt);
        const int ke = (int)min((int64_t)nkt, kb + (u1 - u));
        item(p.sk_dp_tiles + ts, kb, ke, u == u0 ? 0 : 1);
        u += ke - kb;
    }
}

// The K range of k-tiles [kb, ke) of the whole K.
template <int KTB>
__device__ __forceinline__ KRange k_range_of(const GemmArgs& p, int kb, int ke)
{
    constexpr int KPK = KTB / 64;
    KRange r;
    r.kt0 = kb;
    r.n = ke - kb;
    r.ka_end = min(p.KA_b, ke * KTB);
    r.kb_end = min(p.KB, ke * KPK);
    r.last_full = r.ka_end / KTB;
    return r;
}

constexpr int fit_stage_rows(int MR, int WAVES, int R, int SROW, int avail)
{
    int ch = MR;
    while (ch > 1 && (WAVES * ch * R * SROW > avail || MR % ch != 0))
        --ch;
    return ch;
}


// Per-lane base addresses for LDS reads at compile-time offsets below LDS
// bytes.  ds_read's immediate offset holds 16 bits, so a read at offset c
// takes base c >> 16 and immediate c & 0xFFFF.  The bases past the first are
// passed through an empty asm statement, so that the compiler cannot see them
// as the first plus a constant: when it could, it gave every read past 64 KiB
// an address register of its own (16 more VGPRs on the 8-wave 256 x 256
// tile with 16x16 atoms, which then spilled to scratch).
template <int LDS>
struct LdsBases {
    static constexpr int W = (LDS + 65535) / 65536;
    uint32_t b[W];
    __device__ __forceinline__ void init(uint32_t lane_off)
    {
        b[0] = lane_off;
#pragma unroll
        for (int w = 1; w < W; ++w) {
            b[w] = lane_off + (uint32_t)w * 65536u;
            asm volatile("" : "+v"(b[w]));
        }
    }
    __device__ __forceinline__ uint32_t at(uint32_t c) const { return b[c >> 16] + (c & 0xFFFFu); }
};

// End of a k-tile: this wave's LDS reads of the stage are done and its share
// of the next k-tile has landed (at most `vm` newer loads in flight); the
// barrier then makes both true for the whole workgroup.  No workgroup memory
// fence (__syncthreads would drain every outstanding load, prefetches
// included).
#define DG_STAGE_BARRIER(VM)                                     \
    do {                                                         \
        __builtin_amdgcn_sched_barrier(0);                       \
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(VM));        \
        asm volatile("" ::: "memory");                           \
        __builtin_amdgcn_s_barrier();                            \
        asm volatile("" ::: "memory");                           \
        __builtin_amdgcn_sched_barrier(0);                       \
    } while (0)

// Fragment register sets: consecutive K steps alternate between sets, and a
// trip of ST phases of STEPS steps must return to set 0, so the count
// divides ST * STEPS: 2 when that is even, else its smallest odd divisor.
constexpr int frag_sets(int st, int steps)
{
    const int n = st * steps;
    if (n % 2 == 0)
        return 2;
    for (int d = 3; d < n; d += 2)
        if (n % d == 0)
            return d;
    return n;
}

// Groups a K step is cut into: two MFMAs per group where the step has enough
// of them, at most eight groups.
constexpr int step_groups(int mfmas)
{
    return mfmas >= 16 ? 8 : (mfmas >= 2 ? mfmas / 2 : 1);
}

// Runs f(kt + i, integral_constant<i>, tail, nomask) for i in I...: one trip
// of the steady-state loop (ST phases with compile-time stage indices), and
// the tail variant only while kt + i < nkt.  nomask: every load of the trip
// lies inside K, so the loads need no K-tail masking.
template <bool NOMASK, class F, int... I>
__device__ __forceinline__ void run_phases(F& f, int kt, std::integer_sequence<int, I...>)
{
    (f(kt + I, std::integral_constant<int, I>{}, std::false_type{},
       std::integral_constant<bool, NOMASK>{}),
     ...);
}
template <class F, int... I>
__device__ __forceinline__ void run_tail(F& f, int kt, int nkt, std::integer_sequence<int, I...>)
{
    ((kt + I < nkt ? f(kt + I, std::integral_constant<int, I>{}, std::true_type{}, std::false_type{})
                   : void()),
     ...);
}

// The K loop shared by both tiled kernels.  Phase t multiplies k-tile t out
// of stage t % ST while k-tile t + ST - 1 streams into the stage that phase
// t - 1 finished with.  The workgroup barrier of phase t sits before the
// MFMAs of its last K step: after it, the first fragments of k-tile t + 1 are
// read from LDS while those MFMAs run.  Fragment registers alternate between
// NS = frag_sets(ST, STEPS) sets along the global sequence of K steps.
//
// Issue order.  Every K step is cut into G groups, each a slice of the
// step's MFMAs, of the LDS reads of the next fragments and of the k-tile's
// loads, and the groups are fenced with sched_barrier(0), so that the
// compiler keeps this order: one wave per SIMD (the 4-wave 256 x 256 tile)
// has no second wave to hide a burst of loads or reads behind, and when the
// scheduler was only asked to interleave (sched_group_barrier) it put all of
// a k-tile's LDS DMA loads in one run.  Measured on MI355X (bf16 4096^3, K
// loop cycles per k-tile): 1433 -> 1159 for the 4-wave 256 x 256 tile.
//   - With two or more K steps per k-tile the loads go out during the steps
//     before the last, so that none is issued between the last MFMAs before
//     the barrier and the barrier (with one wave per SIMD the MFMA pipe ran
//     dry there).
//   - With one K step and three or more stages they go out after the barrier,
//     into the stage one further from those being read; with one K step and
//     two stages, before the barrier, which then waits for them.
//
// The last nkt % ST phases (the tail) would only load k-tiles past K: they
// issue no loads and wait for every load in flight.  (Their register loads
// would be dead code the compiler removes, and the steady-state wait counts
// assume every phase issues exactly LOADS loads: with loads removed, a count
// of in-flight loads no longer proves the next k-tile has landed.)  Trips
// whose loads all lie before nomask_end (k-tiles of the whole K range) run
// with loads that need no masking, which take their k-tile offset from a
// scalar register.
//   load(kt, stage, part, nparts, nomask)  issue the loads n of k-tile kt with
//                                          n % nparts == part (zeros past K)
//   read(stage, step, set, g, G)           LDS -> fragment registers, group g
//   mma(stage, step, set, g, G)            the MFMAs of group g of one K step
template <int ST, int STEPS, int LOADS, int G, class Load, class Read, class Mma>
__device__ __forceinline__ void k_loop(int nkt, int nomask_end, Load& load, Read& read, Mma& mma)
{
    constexpr int NS = frag_sets(ST, STEPS);
    constexpr bool AFTER = STEPS == 1 && ST >= 3;   // one step: loads after the barrier
    constexpr int NP = STEPS > 1 ? STEPS - 1 : 1;    // steps that issue loads
    constexpr int LPARTS = NP * G;                   // load parts per k-tile
    constexpr int VM = AFTER ? (ST - 3) * LOADS : (ST - 2) * LOADS;
    static_assert(ST >= 2 && (ST - 2) * LOADS <= 63, "pipeline depth vs vmcnt");
#pragma unroll
    for (int t = 0; t < ST - 1; ++t)
        load(t, t, 0, 1, std::false_type{});
    DG_STAGE_BARRIER((ST - 2) * LOADS);
#pragma unroll
    for (int g = 0; g < G; ++g)
        read(0, 0, 0, g, G);
    auto phase = [&](int t, auto sc, auto tail, auto nomask) __attribute__((always_inline)) {
        constexpr int si = decltype(sc)::value;
        constexpr bool TAIL = decltype(tail)::value;
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            const int cur = (si * STEPS + st) % NS;
            const int nxt = (si * STEPS + st + 1) % NS;
            const bool last = st + 1 == STEPS;
            if (last) {
                if constexpr (!TAIL && STEPS == 1 && !AFTER) {
                    // one step and two stages: the loads go out before the
                    // barrier, which waits for them (VM = 0)
#pragma unroll
                    for (int g = 0; g < G; ++g)
                        load(t + ST - 1, (si + ST - 1) % ST, g, G, nomask);
                }
                if constexpr (TAIL)
                    DG_STAGE_BARRIER(0);
                else
                    DG_STAGE_BARRIER(VM);
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (!last)
                    read(si, st + 1, nxt, g, G);
                else
                    read((si + 1) % ST, 0, nxt, g, G);
                mma(si, st, cur, g, G);
                if constexpr (!TAIL) {
                    if (!last || AFTER)
                        load(t + ST - 1, (si + ST - 1) % ST, (AFTER ? 0 : st) * G + g, LPARTS,
                             nomask);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    int kt = 0;
    for (; kt + ST <= nkt && kt + 2 * ST - 2 < nomask_end; kt += ST)
        run_phases<true>(phase, kt, std::make_integer_sequence<int, ST>{});
    for (; kt + ST <= nkt; kt += ST)
        run_phases<false>(phase, kt, std::make_integer_sequence<int, ST>{});
    run_tail(phase, kt, nkt, std::make_integer_sequence<int, ST - 1>{});
    // Loads past nkt (zeros) still target LDS: drain them everywhere before
    // the epilogue reuses it.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Tiled kernel ("GEMM Optimization Guide" page, sections 1, 2, 3, 4, 6, 7):
// WM x 4 waves, the 4 wave columns splitting tile_n (section 1.1); A through
// LDS (ST-stage ring fed by LDS DMA), B straight from the preshuffled layout
// into VGPRs (section 4.2), ST - 1 k-tiles ahead.
template <int TM, int TN, int WM, int ST, int R, int KTB>
struct TiledShape {
    using KT = KTile<KTB>;
    static constexpr int WAVES = 4 * WM;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int MR = TM / WM / R;          // atoms per wave along M
    static constexpr int NR = TN / 4 / R;           // atoms per wave along N
    static constexpr int A_BUF = TM * KTB;          // bytes of one A stage
    static constexpr int A_DMA = A_BUF / 1024 / WAVES;
    static constexpr int B_LOADS = TN * KTB / 4096;  // 16-byte B loads per lane per k-tile
    static constexpr int LOADS = A_DMA + B_LOADS;   // vector-memory ops per wave per k-tile
    static constexpr int WCOLS = TN / 4;            // C columns per wave
    static constexpr int SROW = WCOLS * 2 + 16;     // staging row pitch (padded)
    static constexpr int CH = fit_stage_rows(MR, WAVES, R, SROW, ST * A_BUF);
    static constexpr int LDS = (ST * A_BUF > WAVES * CH * R * SROW) ? ST * A_BUF
                                                                    : WAVES * CH * R * SROW;
    static_assert(MR >= 1 && NR >= 1 && MR * WM * R == TM && NR * 4 * R == TN, "tile shape");
    static_assert(A_DMA >= 1 && A_DMA * 1024 * WAVES == A_BUF, "A DMA split");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <int DT, int TM, int TN, int WM, int ST, int R, int KTB, int MODE>
__global__ __launch_bounds__(64 * 4 * WM, 1) void gemm_tiled_kernel(GemmArgs p)
{
    using S = TiledShape<TM, TN, WM, ST, R, KTB>;
    using KT = KTile<KTB>;
    using AT = Atom<DT, R>;
    using acc_t = typename AT::acc_t;
    constexpr int MR = S::MR, NR = S::NR, A_DMA = S::A_DMA, A_BUF = S::A_BUF;
    constexpr int WAVES = S::WAVES, P = AT::P, KPK = KT::KPK;
    constexpr int STEPS = AT::STEPS * KTB / 128;    // K steps per k-tile
    static_assert(STEPS >= 1 && AT::STEPS * KTB % 128 == 0, "atom does not fit the k-tile");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[S::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform: the LDS addresses of the DMA loads stay in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;     // wave row (M) and column (N)

    ADma ad[A_DMA];
#pragma unroll
    for (int i = 0; i < A_DMA; ++i)
        ad[i] = a_dma_lane<KTB>(wave + WAVES * i, lane, p.lda_b);
    const int lr = lane % R;                       // row / column of this lane in an atom
    const uint32_t swz = KT::key((uint32_t)(lane & 15));
    const uint32_t row0 = (uint32_t)(wm * (TM / WM));   // first A row of this wave
    // 16-column block of this lane's column in atom 0 of this wave
    const uint32_t bblk = (uint32_t)(wn * NR * (R / 16) + (lr >> 4));
    const uint32_t b_lane = bblk * (uint32_t)p.KB * 1024u + (uint32_t)(lane & 15) * 16;
    // A fragment reads: a per-lane part for each (K step, fragment part)
    // plus a compile-time offset (stage, atom row).
    LdsBases<S::LDS> a_at[STEPS][P];
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
#pragma unroll
        for (int q = 0; q < P; ++q)
            a_at[s][q].init((row0 + (uint32_t)lr) * KTB + (((uint32_t)AT::a_chunk(s, lane, q) ^ swz) << 4));

    i32x4 breg[ST][NR][STEPS][P];
    i32x4 af[frag_sets(ST, STEPS)][MR][P];
    acc_t acc[MR][NR];

    // One work item: output tile (tm, tn) over the K range kr (split-K: its
    // slice; stream-K: k-tiles [kb, ke) of stream-K tile sk_tile, whose
    // partial goes to slot sk_slot unless the item covers the whole K).
    auto run = [&](int tm, int tn, const KRange& kr, int slice, int sk_tile, int sk_slot,
                   bool whole) __attribute__((always_inline)) {
    // a stream-K workgroup runs several items: the previous item's epilogue
    // may still be reading its staging area, which this item's first loads
    // overwrite
    if constexpr (MODE == MODE_SK)
        __syncthreads();
    const int m0 = tm * TM;
    const int n0 = tn * TN;
    const int rows = min(TM, p.M - m0);
    // Descriptors rebased at this tile: rows past M and 16-column blocks past
    // ceil(N/16) fall outside and read as zero.
    const rsrc_t ra = make_rsrc(p.A + (int64_t)m0 * p.lda_b,
                                (uint32_t)((int64_t)(rows - 1) * p.lda_b + p.KA_b));
    const int nb0 = n0 >> 4;
    const int nbv = min(TN / 16, p.nblk - nb0);
    const rsrc_t rb = make_rsrc(p.Bs + (int64_t)nb0 * p.KB * 1024,
                                (uint32_t)nbv * (uint32_t)p.KB * 1024u);
#pragma unroll
    for (int mi = 0; mi < MR; ++mi)
#pragma unroll
        for (int j = 0; j < NR; ++j)
            acc[mi][j] = zero_acc<AT>();

    // A k-tile past the end of this workgroup's K range (past K, or past its
    // slice) loads through out-of-range offsets: zeros, and no memory
    // traffic.  Load op n (A DMAs first, then B fragments) belongs to part
    // n % nparts.  Without masking (every k-tile of the trip inside K) the
    // k-tile's offset is a scalar operand of the load.
    auto load = [&](int kt_local, int stage, int part, int nparts, auto nomask_c)
                    __attribute__((always_inline)) {
        constexpr bool NOMASK = decltype(nomask_c)::value;
        const int kt = kr.kt0 + kt_local;
        const bool mask = kt >= kr.last_full;
#pragma unroll
        for (int i = 0; i < A_DMA; ++i) {
            if (i % nparts != part)
                continue;
            uint8_t* dst = lds + stage * A_BUF + (wave + WAVES * i) * 1024;
            if constexpr (NOMASK) {
                dma16(ra, dst, ad[i].goff, (uint32_t)kt * KTB);
            } else {
                uint32_t off = ad[i].goff + (uint32_t)kt * KTB;
                if (mask && (int)((uint32_t)kt * KTB + ad[i].col) >= kr.ka_end)
                    off = kOOB;
                dma16(ra, dst, off, 0);
            }
        }
#pragma unroll
        for (int j = 0; j < NR; ++j)
#pragma unroll
            for (int s = 0; s < STEPS; ++s)
#pragma unroll
                for (int q = 0; q < P; ++q) {
                    if ((A_DMA + (j * STEPS + s) * P + q) % nparts != part)
                        continue;
                    const uint32_t voff = b_lane +
                                          (uint32_t)(j * (R / 16) * p.KB + AT::b_half(s, q)) * 1024u +
                                          ((uint32_t)AT::b_group(s, lane, q) << 8);
                    if constexpr (NOMASK) {
                        breg[stage][j][s][q] = load16_s(rb, voff, (uint32_t)kt * (KPK * 1024u));
                    } else {
                        const int kb = kt * KPK + AT::b_half(s, q);
                        breg[stage][j][s][q] =
                            load16(rb, mask && kb >= kr.kb_end ? kOOB : voff + (uint32_t)kt * (KPK * 1024u));
                    }
                }
    };
    // group g of a K step: A fragment reads and MFMAs (atom a = mi NR + j)
    auto read = [&](int stage, int s, int set, int g, int G) __attribute__((always_inline)) {
#pragma unroll
        for (int f = 0; f < MR * P; ++f) {
            if (f * G / (MR * P) != g)
                continue;
            const int mi = f / P, q = f % P;
            const uint32_t off = a_at[s][q].at((uint32_t)(stage * A_BUF + mi * R * KTB));
            af[set][mi][q] = *reinterpret_cast<const i32x4*>(lds + off);
        }
    };
    auto mma = [&](int stage, int s, int set, int g, int G) __attribute__((always_inline)) {
#pragma unroll
        for (int a = 0; a < MR * NR; ++a) {
            if (a * G / (MR * NR) != g)
                continue;
            const int mi = a / NR, j = a % NR;
            acc[mi][j] = AT::mma(af[set][mi], breg[stage][j][s], acc[mi][j]);
        }
    };
    k_loop<ST, STEPS, S::LOADS, step_groups(MR * NR)>(kr.n, min(kr.n, kr.last_full - kr.kt0), load,
                                                      read, mma);

    if constexpr (MODE == MODE_SPLIT) {
        store_partial<AT, MR, NR>(p, acc, slice, m0 + (int)row0, n0 + wn * S::WCOLS, lane);
        return;
    }
    if constexpr (MODE == MODE_SK) {
        if (!whole &&
            !sk_fixup<AT, MR, NR, TM, TN>(p, acc, reinterpret_cast<int*>(lds), xcd_remap((int)blockIdx.x, (int)gridDim.x),
                                          (int)gridDim.x,
                                          (int64_t)(p.tiles_m * p.tiles_n - p.sk_dp_tiles) * p.sk_nkt,
                                          sk_tile, sk_slot, wave, lane))
            return;
    }
    float scale_a = 1.f, scale_b = 1.f;
    if constexpr (DT == DT_FP8) {
        scale_a = *p.sa;
        scale_b = *p.sb;
    }
    store_c_tile<DT, AT, MR, NR, S::CH, S::SROW, S::WCOLS, MODE == MODE_EPI>(
        p, acc, lds + wave * (S::CH * R * S::SROW), m0, rows, n0 + wn * S::WCOLS, (int)row0, lane,
        scale_a, scale_b);
    };

    if constexpr (MODE == MODE_SK) {
        auto item = [&](int t, int kb, int ke, int slot) __attribute__((always_inline)) {
            int tm, tn;
            tile_raster<DG_GROUP_M>(t, p.tiles_m, p.tiles_n, tm, tn);
            run(tm, tn, k_range_of<KTB>(p, kb, ke), 0, t - p.sk_dp_tiles, slot,
                kb == 0 && ke == p.sk_nkt);
        };
        sk_for_each(p, item);
    } else {
        int wg, tm, tn;
        const int slice = split_slice<MODE == MODE_SPLIT>(p, wg);
        tile_coords<DG_GROUP_M>(wg, p.tiles_m, p.tiles_n, tm, tn);
        run(tm, tn, k_range<KTB, MODE == MODE_SPLIT>(p, slice), slice, 0, 0, true);
    }
}

// ---------------------------------------------------------------------------
// Tiled kernel with A and B both staged in LDS ("AB" kernel).
//
// Loading a B fragment straight into the registers of every wave that needs
// it (the kernel above) moves it from L2 once per wave row; measured on
// MI355X, the L2 -> CU path, not the MFMA, bounds that kernel once the tile
// is large.  Here each k-tile of A *and* B enters the workgroup once, by
// 16-byte LDS DMA, and the WM x WN waves read their fragments from LDS.  The
// preshuffled B blocks land in LDS unchanged, so a B fragment read is a run
// of 256 contiguous bytes per 16 lanes.  Per stage: [A: TM rows x KTB bytes,
// swizzled][B: TN/16 blocks x KTB/64 x 1 KiB].
template <int TM, int TN, int WM, int WN, int ST, int R, int KTB>
struct ABShape {
    using KT = KTile<KTB>;
    static constexpr int WAVES = WM * WN;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int MR = TM / WM / R;          // atoms per wave along M
    static constexpr int NR = TN / WN / R;          // atoms per wave along N
    static constexpr int A_BUF = TM * KTB;
    static constexpr int B_BUF = TN * KTB;
    static constexpr int STAGE = A_BUF + B_BUF;
    static constexpr int A_DMA = A_BUF / 1024 / WAVES;  // 1 KiB A loads per wave per k-tile
    static constexpr int B_DMA = B_BUF / 1024 / WAVES;  // 1 KiB B loads per wave per k-tile
    static constexpr int LOADS = A_DMA + B_DMA;
    static constexpr int WCOLS = TN / WN;           // C columns per wave
    static constexpr int SROW = WCOLS * 2 + 16;     // staging row pitch (padded)
    static constexpr int CH = fit_stage_rows(MR, WAVES, R, SROW, ST * STAGE);
    static constexpr int LDS = (ST * STAGE > WAVES * CH * R * SROW) ? ST * STAGE
                                                                    : WAVES * CH * R * SROW;
    static_assert(MR >= 1 && NR >= 1 && MR * WM * R == TM && NR * WN * R == TN, "tile shape");
    static_assert(A_DMA >= 1 && B_DMA >= 1 && A_DMA * 1024 * WAVES == A_BUF &&
                      B_DMA * 1024 * WAVES == B_BUF,
                  "DMA split");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <int DT, int TM, int TN, int WM, int WN, int ST, int R, int KTB, int MODE>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_ab_kernel(GemmArgs p)
{
    using S = ABShape<TM, TN, WM, WN, ST, R, KTB>;
    using KT = KTile<KTB>;
    using AT = Atom<DT, R>;
    using acc_t = typename AT::acc_t;
    constexpr int MR = S::MR, NR = S::NR, A_BUF = S::A_BUF, STAGE = S::STAGE;
    constexpr int WAVES = S::WAVES, A_DMA = S::A_DMA, B_DMA = S::B_DMA;
    constexpr int P = AT::P, KPK = KT::KPK;
    constexpr int STEPS = AT::STEPS * KTB / 128;
    static_assert(STEPS >= 1 && AT::STEPS * KTB % 128 == 0, "atom does not fit the k-tile");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[S::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform: the LDS addresses of the DMA loads stay in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // A chunk w + WAVES*i: rows (1024/KTB) c ...  B chunk b = w + WAVES*i:
    // 16-column block b / KPK, 64-byte block b % KPK of the k-tile.
    ADma ad[A_DMA];
    uint32_t b_goff[B_DMA], b_half[B_DMA];
#pragma unroll
    for (int i = 0; i < A_DMA; ++i)
        ad[i] = a_dma_lane<KTB>(wave + WAVES * i, lane, p.lda_b);
#pragma unroll
    for (int i = 0; i < B_DMA; ++i) {
        const uint32_t b = wave + WAVES * i;
        b_goff[i] = ((b / KPK) * (uint32_t)p.KB + (b % KPK)) * 1024u + lane * 16;
        b_half[i] = b % KPK;
    }
    const int lr = lane % R;
    const uint32_t swz = KT::key((uint32_t)(lane & 15));
    const uint32_t row0 = (uint32_t)(wm * (TM / WM));
    // LDS byte offset (within a stage's B region) of this lane's column in
    // atom 0 of this wave, group 0, 64-byte block 0.
    const uint32_t b_lds =
        (uint32_t)((wn * NR * (R / 16) + (lr >> 4)) * KPK * 1024 + (lane & 15) * 16);
    // Fragment reads: a per-lane part for each (K step, fragment part) plus
    // a compile-time offset (stage, atom row or column block, 1 KiB block).
    LdsBases<S::LDS> a_at[STEPS][P], b_at[STEPS][P];
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
#pragma unroll
        for (int q = 0; q < P; ++q) {
            a_at[s][q].init((row0 + (uint32_t)lr) * KTB +
                            (((uint32_t)AT::a_chunk(s, lane, q) ^ swz) << 4));
            b_at[s][q].init(b_lds + ((uint32_t)AT::b_group(s, lane, q) << 8));
        }

    i32x4 af[frag_sets(ST, STEPS)][MR][P], bf[frag_sets(ST, STEPS)][NR][P];
    acc_t acc[MR][NR];

    // One work item: output tile (tm, tn) over the K range kr (split-K: its
    // slice; stream-K: k-tiles [kb, ke) of stream-K tile sk_tile, whose
    // partial goes to slot sk_slot unless the item covers the whole K).
    auto run = [&](int tm, int tn, const KRange& kr, int slice, int sk_tile, int sk_slot,
                   bool whole) __attribute__((always_inline)) {
    // a stream-K workgroup runs several items: the previous item's epilogue
    // may still be reading its staging area, which this item's first loads
    // overwrite
    if constexpr (MODE == MODE_SK)
        __syncthreads();
    const int m0 = tm * TM;
    const int n0 = tn * TN;
    const int rows = min(TM, p.M - m0);
    const rsrc_t ra = make_rsrc(p.A + (int64_t)m0 * p.lda_b,
                                (uint32_t)((int64_t)(rows - 1) * p.lda_b + p.KA_b));
    const int nb0 = n0 >> 4;
    const int nbv = min(TN / 16, p.nblk - nb0);
    const rsrc_t rb = make_rsrc(p.Bs + (int64_t)nb0 * p.KB * 1024,
                                (uint32_t)nbv * (uint32_t)p.KB * 1024u);
#pragma unroll
    for (int mi = 0; mi < MR; ++mi)
#pragma unroll
        for (int j = 0; j < NR; ++j)
            acc[mi][j] = zero_acc<AT>();

    // Load op n (A DMAs first, then B DMAs) belongs to part n % nparts.
    // Without masking (every k-tile of the trip inside K) the k-tile's offset
    // is a scalar operand of the load.
    auto load = [&](int kt_local, int stage, int part, int nparts, auto nomask_c)
                    __attribute__((always_inline)) {
        constexpr bool NOMASK = decltype(nomask_c)::value;
        const int kt = kr.kt0 + kt_local;
        const bool mask = kt >= kr.last_full;
        uint8_t* base = lds + stage * STAGE;
#pragma unroll
        for (int i = 0; i < A_DMA; ++i) {
            if (i % nparts != part)
                continue;
            uint8_t* dst = base + (wave + WAVES * i) * 1024;
            if constexpr (NOMASK) {
                dma16(ra, dst, ad[i].goff, (uint32_t)kt * KTB);
            } else {
                uint32_t off = ad[i].goff + (uint32_t)kt * KTB;
                if (mask && (int)((uint32_t)kt * KTB + ad[i].col) >= kr.ka_end)
                    off = kOOB;
                dma16(ra, dst, off, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < B_DMA; ++i) {
            if ((A_DMA + i) % nparts != part)
                continue;
            uint8_t* dst = base + A_BUF + (wave + WAVES * i) * 1024;
            if constexpr (NOMASK) {
                dma16(rb, dst, b_goff[i], (uint32_t)kt * (KPK * 1024u));
            } else {
                uint32_t off = b_goff[i] + (uint32_t)kt * (KPK * 1024u);
                if (mask && kt * KPK + (int)b_half[i] >= kr.kb_end)
                    off = kOOB;
                dma16(rb, dst, off, 0);
            }
        }
    };
    // group g of a K step: fragment f (B fragments first, then A) and atom
    // a = mi NR + j
    auto read = [&](int stage, int s, int set, int g, int G) __attribute__((always_inline)) {
        constexpr int NF = (MR + NR) * P;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            if (f * G / NF != g)
                continue;
            if (f < NR * P) {
                const int j = f / P, q = f % P;
                const uint32_t off = b_at[s][q].at((uint32_t)(stage * STAGE + A_BUF +
                                                              j * (R / 16) * KPK * 1024 +
                                                              (AT::b_half(s, q) << 10)));
                bf[set][j][q] = *reinterpret_cast<const i32x4*>(lds + off);
            } else {
                const int mi = (f - NR * P) / P, q = (f - NR * P) % P;
                const uint32_t off = a_at[s][q].at((uint32_t)(stage * STAGE + mi * R * KTB));
                af[set][mi][q] = *reinterpret_cast<const i32x4*>(lds + off);
            }
        }
    };
    auto mma = [&](int, int, int set, int g, int G) __attribute__((always_inline)) {
#pragma unroll
        for (int a = 0; a < MR * NR; ++a) {
            if (a * G / (MR * NR) != g)
                continue;
            const int mi = a / NR, j = a % NR;
            acc[mi][j] = AT::mma(af[set][mi], bf[set][j], acc[mi][j]);
        }
    };
    k_loop<ST, STEPS, S::LOADS, step_groups(MR * NR)>(kr.n, min(kr.n, kr.last_full - kr.kt0), load,
                                                      read, mma);

    if constexpr (MODE == MODE_SPLIT) {
        store_partial<AT, MR, NR>(p, acc, slice, m0 + (int)row0, n0 + wn * S::WCOLS, lane);
        return;
    }
    if constexpr (MODE == MODE_SK) {
        if (!whole &&
            !sk_fixup<AT, MR, NR, TM, TN>(p, acc, reinterpret_cast<int*>(lds), xcd_remap((int)blockIdx.x, (int)gridDim.x),
                                          (int)gridDim.x,
                                          (int64_t)(p.tiles_m * p.tiles_n - p.sk_dp_tiles) * p.sk_nkt,
                                          sk_tile, sk_slot, wave, lane))
            return;
    }
    float scale_a = 1.f, scale_b = 1.f;
    if constexpr (DT == DT_FP8) {
        scale_a = *p.sa;
        scale_b = *p.sb;
    }
    store_c_tile<DT, AT, MR, NR, S::CH, S::SROW, S::WCOLS, MODE == MODE_EPI>(
        p, acc, lds + wave * (S::CH * R * S::SROW), m0, rows, n0 + wn * S::WCOLS, (int)row0, lane,
        scale_a, scale_b);
    };

    if constexpr (MODE == MODE_SK) {
        auto item = [&](int t, int kb, int ke, int slot) __attribute__((always_inline)) {
            int tm, tn;
            tile_raster<DG_GROUP_M>(t, p.tiles_m, p.tiles_n, tm, tn);
            run(tm, tn, k_range_of<KTB>(p, kb, ke), 0, t - p.sk_dp_tiles, slot,
                kb == 0 && ke == p.sk_nkt);
        };
        sk_for_each(p, item);
    } else {
        int wg, tm, tn;
        const int slice = split_slice<MODE == MODE_SPLIT>(p, wg);
        tile_coords<DG_GROUP_M>(wg, p.tiles_m, p.tiles_n, tm, tn);
        run(tm, tn, k_range<KTB, MODE == MODE_SPLIT>(p, slice), slice, 0, 0, true);
    }
}

// ---------------------------------------------------------------------------
// A+B kernel with whole-line A loads ("AB-line" kernel), 256 x 256 tiles with
// one K step per 64-byte k-tile (e4m3 32 x 32 atoms).  The A+B kernel above
// loads each k-tile of A as 16 rows x 64 bytes per LDS-DMA instruction: half
// of every 128-byte line, the other half a k-tile later.  Here A is loaded in
// k-tile pairs, 8 rows x 128 bytes (whole lines) per instruction, into NA = 3
// pair stages of 128-byte rows (swizzled as the 128-byte k-tiles are); B keeps
// its ST = 4 stages of 64-byte k-tiles.  Measured on MI355X, the operand
// stream alone (no MFMAs) is 17 % faster this way for the e4m3 4096^3 tile
// grid.  LDS: B stages [0, 64 KiB), A pair stages [64, 160 KiB).
//
// Phase t multiplies k-tile t and reads the fragments of k-tile t + 1, as in
// k_loop, and issues half t % 2 of A pair t / 2 + 2 and all of B k-tile t + 3:
// the same number of loads per wave and phase as the 64-byte kernel (NAL / 2 +
// NBL), so the same wait counts hold.  Pair q's stage last held pair q - 3,
// whose k-tile 2q - 5 was read in phase 2q - 6 and is past the barrier of
// phase 2q - 5; pair q's loads go out after the barriers of phases 2q - 4 and
// 2q - 3 and have landed at the barrier of phase 2q - 1, which reads k-tile
// 2q (one phase of loads, NAL / 2 + NBL, may still be in flight).  Plain and
// fused-epilogue launches only (split-K and stream-K use the A+B kernel).
template <int DT, int R, int WM, int WN, bool EPI>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_ab_line_kernel(GemmArgs p)
{
    constexpr int TM = 256, TN = 256, ST = 4, NA = 3, KTB = 64;
    using AT = Atom<DT, R>;
    using acc_t = typename AT::acc_t;
    constexpr int WAVES = WM * WN, MR = TM / WM / R, NR = TN / WN / R, P = AT::P;
    constexpr int NAL = 32 / WAVES;                   // A loads per wave and pair
    constexpr int NBL = 16 / WAVES;                   // B loads per wave and k-tile
    constexpr int LOADS = NAL / 2 + NBL;              // loads per wave and phase
    constexpr int B_STAGE = TN * KTB;                 // 16 KiB
    constexpr int A_BASE = ST * B_STAGE;              // 64 KiB
    constexpr int A_PSTAGE = TM * 128;                // 32 KiB
    constexpr int LDS = A_BASE + NA * A_PSTAGE;       // 160 KiB
    constexpr int WCOLS = TN / WN, SROW = WCOLS * 2 + 16;
    constexpr int CH = fit_stage_rows(MR, WAVES, R, SROW, LDS);
    constexpr int G = step_groups(MR * NR);
    static_assert(AT::STEPS * KTB / 128 == 1, "one K step per 64-byte k-tile");
    static_assert(WAVES % 2 == 0 && 32 % WAVES == 0 && NAL % 2 == 0, "A pair split");
    static_assert(LDS <= 160 * 1024 && WAVES * CH * R * SROW <= LDS, "LDS budget");
    static_assert(2 * LOADS <= 63, "pipeline depth vs vmcnt");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    int wg, tm, tn;
    split_slice<false>(p, wg);
    tile_coords<DG_GROUP_M>(wg, p.tiles_m, p.tiles_n, tm, tn);
    const KRange kr = k_range<KTB, false>(p, 0);
    const int m0 = tm * TM, n0 = tn * TN;
    const int rows = min(TM, p.M - m0);
    const rsrc_t ra = make_rsrc(p.A + (int64_t)m0 * p.lda_b,
                                (uint32_t)((int64_t)(rows - 1) * p.lda_b + p.KA_b));
    const int nb0 = n0 >> 4;
    const int nbv = min(TN / 16, p.nblk - nb0);
    const rsrc_t rb = make_rsrc(p.Bs + (int64_t)nb0 * p.KB * 1024,
                                (uint32_t)nbv * (uint32_t)p.KB * 1024u);

    // A pair chunk c = wave + WAVES i: rows 8c .. 8c + 7, 128 bytes each.  The
    // swizzle key of row 8c + lane / 8 depends on c only through c % 2 = wave
    // % 2, so chunk i sits 8 WAVES i rows below chunk 0.  The row goes in the
    // per-lane offset, which the descriptor's range check sees (rows past M
    // read zeros); the pair's K offset is scalar and stays inside the row
    // unless the K-tail mask replaces the offset.
    const ADma ad0 = a_dma_lane<128>(wave, lane, p.lda_b);
    const uint32_t a_rows = 8u * WAVES * (uint32_t)p.lda_b;
    const uint32_t b_goff0 = (uint32_t)wave * (uint32_t)p.KB * 1024u + lane * 16;
    const uint32_t b_blocks = (uint32_t)WAVES * (uint32_t)p.KB * 1024u;

    const int lr = lane % R;
    const uint32_t swz = KTile<128>::key((uint32_t)(lane & 15));
    const uint32_t row0 = (uint32_t)(wm * (TM / WM));
    const uint32_t b_lds = (uint32_t)((wn * NR * (R / 16) + (lr >> 4)) * 1024 + (lane & 15) * 16);
    // A fragment offsets for the first half of a 128-byte row; the second
    // half reads chunk c + 4 where the first reads c < 4, i.e. the same
    // offset with bit 6 flipped
    uint32_t a_lane[P], b_lane[P], a_cur[P];
#pragma unroll
    for (int q = 0; q < P; ++q) {
        a_lane[q] = (uint32_t)A_BASE + (row0 + (uint32_t)lr) * 128u +
                    (((uint32_t)AT::a_chunk(0, lane, q) ^ swz) << 4);
        b_lane[q] = b_lds + ((uint32_t)AT::b_group(0, lane, q) << 8);
    }

    i32x4 af[2][MR][P], bf[2][NR][P];
    acc_t acc[MR][NR];
#pragma unroll
    for (int mi = 0; mi < MR; ++mi)
#pragma unroll
        for (int j = 0; j < NR; ++j)
            acc[mi][j] = zero_acc<AT>();

    // A loads of pair q, chunks [i0, i0 + n): op i - i0 + op0 of the phase
    auto load_a = [&](int q, int i0, int n, int part, int nparts, int op0)
                      __attribute__((always_inline)) {
        uint8_t* base = lds + A_BASE + (q % NA) * A_PSTAGE;
        const bool mask = 2 * q + 1 >= kr.last_full;
#pragma unroll
        for (int i = 0; i < NAL; ++i) {
            if (i < i0 || i >= i0 + n || (op0 + i - i0) % nparts != part)
                continue;
            uint32_t off = ad0.goff + (uint32_t)i * a_rows;
            if (mask && (int)((uint32_t)q * 128u + ad0.col) >= kr.ka_end)
                off = kOOB;
            dma16(ra, base + (wave + WAVES * i) * 1024, off, (uint32_t)q * 128u);
        }
    };
    // B loads of k-tile kt into its stage: ops op0 ..
    auto load_b = [&](int kt, int part, int nparts, int op0) __attribute__((always_inline)) {
        const bool mask = kt >= kr.last_full;
        uint8_t* base = lds + (kt % ST) * B_STAGE;
#pragma unroll
        for (int i = 0; i < NBL; ++i) {
            if ((op0 + i) % nparts != part)
                continue;
            uint32_t off = b_goff0 + (uint32_t)i * b_blocks;
            if (mask && kt >= kr.kb_end)
                off = kOOB;
            dma16(rb, base + (wave + WAVES * i) * 1024, off, (uint32_t)kt * 1024u);
        }
    };
    // A read bases of k-tile kt, whose parity H is a constant here (trips of
    // ST phases start at multiples of ST)
    auto set_a = [&](int kt, auto hc) __attribute__((always_inline)) {
        constexpr int H = decltype(hc)::value;
        const uint32_t d = (uint32_t)((kt / 2) % NA) * A_PSTAGE;
#pragma unroll
        for (int q = 0; q < P; ++q)
            a_cur[q] = (a_lane[q] ^ (uint32_t)(H * 64)) + d;
    };
    // group g of the fragment reads of the k-tile in B stage bstage (A from a_cur)
    auto read = [&](int bstage, int set, int g) __attribute__((always_inline)) {
        constexpr int NF = (MR + NR) * P;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            if (f * G / NF != g)
                continue;
            if (f < NR * P) {
                const int j = f / P, q = f % P;
                bf[set][j][q] = *reinterpret_cast<const i32x4*>(
                    lds + b_lane[q] + (uint32_t)(bstage * B_STAGE + j * (R / 16) * 1024));
            } else {
                const int mi = (f - NR * P) / P, q = (f - NR * P) % P;
                af[set][mi][q] =
                    *reinterpret_cast<const i32x4*>(lds + a_cur[q] + (uint32_t)(mi * R * 128));
            }
        }
    };
    auto mma = [&](int set, int g) __attribute__((always_inline)) {
#pragma unroll
        for (int a = 0; a < MR * NR; ++a) {
            if (a * G / (MR * NR) != g)
                continue;
            const int mi = a / NR, j = a % NR;
            acc[mi][j] = AT::mma(af[set][mi], bf[set][j], acc[mi][j]);
        }
    };

    // prologue: A pairs 0 and 1, B k-tiles 0, 1, 2; the first group (pair 0,
    // k-tile 0) has landed once at most the later 2 LOADS are in flight
    load_a(0, 0, NAL, 0, 1, 0);
    load_b(0, 0, 1, 0);
    load_b(1, 0, 1, 0);
    load_a(1, 0, NAL, 0, 1, 0);
    load_b(2, 0, 1, 0);
    DG_STAGE_BARRIER(2 * LOADS);
    set_a(0, std::integral_constant<int, 0>{});
#pragma unroll
    for (int g = 0; g < G; ++g)
        read(0, 0, g);
    auto phase = [&](int t, auto sc, auto tail) __attribute__((always_inline)) {
        constexpr int si = decltype(sc)::value;
        constexpr bool TAIL = decltype(tail)::value;
        if constexpr (TAIL)
            DG_STAGE_BARRIER(0);
        else
            DG_STAGE_BARRIER(LOADS);
        set_a(t + 1, std::integral_constant<int, (si + 1) & 1>{});
#pragma unroll
        for (int g = 0; g < G; ++g) {
            read((si + 1) % ST, (si + 1) & 1, g);
            mma(si & 1, g);
            if constexpr (!TAIL) {
                load_a(t / 2 + 2, (NAL / 2) * (t & 1), NAL / 2, g, G, 0);
                load_b(t + ST - 1, g, G, NAL / 2);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    const int nkt = kr.n;
    int kt = 0;
    for (; kt + ST <= nkt; kt += ST) {
        phase(kt, std::integral_constant<int, 0>{}, std::false_type{});
        phase(kt + 1, std::integral_constant<int, 1>{}, std::false_type{});
        phase(kt + 2, std::integral_constant<int, 2>{}, std::false_type{});
        phase(kt + 3, std::integral_constant<int, 3>{}, std::false_type{});
    }
    // the last nkt % ST phases only ever load k-tiles past K: no loads
    if (kt < nkt)
        phase(kt, std::integral_constant<int, 0>{}, std::true_type{});
    if (kt + 1 < nkt)
        phase(kt + 1, std::integral_constant<int, 1>{}, std::true_type{});
    if (kt + 2 < nkt)
        phase(kt + 2, std::integral_constant<int, 2>{}, std::true_type{});
    // loads past nkt (zeros) still target LDS: drain them before the epilogue
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    __syncthreads();

    float scale_a = 1.f, scale_b = 1.f;
    if constexpr (DT == DT_FP8) {
        scale_a = *p.sa;
        scale_b = *p.sb;
    }
    store_c_tile<DT, AT, MR, NR, CH, SROW, WCOLS, EPI>(p, acc, lds + wave * (CH * R * SROW), m0,
                                                      rows, n0 + wn * WCOLS, (int)row0, lane,
                                                      scale_a, scale_b);
}

// ---------------------------------------------------------------------------
// A+B kernel with ping-pong wave groups ("PP" kernel).
//
// 8 waves in two groups of four; a workgroup's waves are spread round robin
// over the 4 SIMDs, so SIMD i runs wave i of group 0 and wave i of group 1.
// Group g owns rows [g TM/2, (g+1) TM/2) of the tile; within a group the 4
// waves split tile_n.  The K loop runs in half-periods separated by
// workgroup barriers.  In every half one group issues all MFMAs of a k-tile
// from fragments already in its registers while the other group issues its
// share of the LDS DMA and reads the fragments of its next k-tile from LDS,
// so each SIMD's MFMA pipe is fed by one wave while its other wave moves
// data:
//   half 2t:     group 0 loads k-tile t, group 1 multiplies k-tile t - 1
//   half 2t + 1: group 1 loads k-tile t, group 0 multiplies k-tile t
// Stage t % ST is read in halves 2t and 2t + 1 and refilled, with k-tile
// t + ST, in half 2t + 2 (group 0's share) and 2t + 3 (group 1's share).
// Waits at the end of each half: before half 2t both groups' shares of
// k-tile t must have landed (each wave: at most (ST-2) x LOADS of its loads
// still in flight); at the end of half 2t only group 1 needs that much (its
// next read is k-tile t, already complete), group 0 none.
template <int DT, int TM, int TN, int ST, int R, int KTB, int MODE>
__global__ __launch_bounds__(512, 1) void gemm_pp_kernel(GemmArgs p)
{
    using S = ABShape<TM, TN, 2, 4, ST, R, KTB>;
    using KT = KTile<KTB>;
    using AT = Atom<DT, R>;
    using acc_t = typename AT::acc_t;
    constexpr int MR = S::MR, NR = S::NR, A_BUF = S::A_BUF, STAGE = S::STAGE;
    constexpr int WAVES = 8, A_DMA = S::A_DMA, B_DMA = S::B_DMA, LOADS = S::LOADS;
    constexpr int P = AT::P, KPK = KT::KPK;
    constexpr int STEPS = AT::STEPS * KTB / 128;
    static_assert(STEPS >= 1 && AT::STEPS * KTB % 128 == 0, "atom does not fit the k-tile");
    static_assert(ST >= 2 && (ST - 1) * LOADS <= 63, "pipeline depth vs vmcnt");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[S::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;     // wm = the group
    const bool g0 = wm == 0;
    int wg, tm, tn;
    const int slice = split_slice<MODE == MODE_SPLIT>(p, wg);
    tile_coords<DG_GROUP_M>(wg, p.tiles_m, p.tiles_n, tm, tn);
    const int m0 = tm * TM;
    const int n0 = tn * TN;
    const int rows = min(TM, p.M - m0);
    const KRange kr = k_range<KTB, MODE == MODE_SPLIT>(p, slice);
    const rsrc_t ra = make_rsrc(p.A + (int64_t)m0 * p.lda_b,
                                (uint32_t)((int64_t)(rows - 1) * p.lda_b + p.KA_b));
    const int nb0 = n0 >> 4;
    const int nbv = min(TN / 16, p.nblk - nb0);
    const rsrc_t rb = make_rsrc(p.Bs + (int64_t)nb0 * p.KB * 1024,
                                (uint32_t)nbv * (uint32_t)p.KB * 1024u);

    ADma ad[A_DMA];
    uint32_t b_goff[B_DMA], b_half[B_DMA];
#pragma unroll
    for (int i = 0; i < A_DMA; ++i)
        ad[i] = a_dma_lane<KTB>(wave + WAVES * i, lane, p.lda_b);
#pragma unroll
    for (int i = 0; i < B_DMA; ++i) {
        const uint32_t b = wave + WAVES * i;
        b_goff[i] = ((b / KPK) * (uint32_t)p.KB + (b % KPK)) * 1024u + lane * 16;
        b_half[i] = b % KPK;
    }
    const int lr = lane % R;
    const uint32_t swz = KT::key((uint32_t)(lane & 15));
    const uint32_t row0 = (uint32_t)(wm * (TM / 2));
    const uint32_t b_lds =
        (uint32_t)((wn * NR * (R / 16) + (lr >> 4)) * KPK * 1024 + (lane & 15) * 16);

    i32x4 af[STEPS][MR][P], bf[STEPS][NR][P];
    acc_t acc[MR][NR];
#pragma unroll
    for (int mi = 0; mi < MR; ++mi)
#pragma unroll
        for (int j = 0; j < NR; ++j)
            acc[mi][j] = zero_acc<AT>();

    // A k-tile past this workgroup's K range loads through out-of-range
    // offsets: zeros, no traffic.
    auto load = [&](int kt_local, int stage) __attribute__((always_inline)) {
        const int kt = kr.kt0 + kt_local;
        const bool mask = kt >= kr.last_full;
        uint8_t* base = lds + stage * STAGE;
#pragma unroll
        for (int i = 0; i < A_DMA; ++i) {
            uint32_t off = ad[i].goff + (uint32_t)kt * KTB;
            if (mask && (int)((uint32_t)kt * KTB + ad[i].col) >= kr.ka_end)
                off = kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (lds_void*)(base + (wave + WAVES * i) * 1024), 16, off, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < B_DMA; ++i) {
            uint32_t off = b_goff[i] + (uint32_t)kt * (KPK * 1024u);
            if (mask && kt * KPK + (int)b_half[i] >= kr.kb_end)
                off = kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (lds_void*)(base + A_BUF + (wave + WAVES * i) * 1024), 16, off, 0, 0, 0);
        }
    };
    // all fragments of one k-tile
    auto read = [&](int stage) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
#pragma unroll
            for (int j = 0; j < NR; ++j)
#pragma unroll
                for (int q = 0; q < P; ++q) {
                    const uint32_t off = (uint32_t)(stage * STAGE + A_BUF) + b_lds +
                                         (uint32_t)(j * (R / 16) * KPK * 1024) +
                                         ((uint32_t)AT::b_half(s, q) << 10) +
                                         ((uint32_t)AT::b_group(s, lane, q) << 8);
                    bf[s][j][q] = *reinterpret_cast<const i32x4*>(lds + off);
                }
#pragma unroll
            for (int mi = 0; mi < MR; ++mi)
#pragma unroll
                for (int q = 0; q < P; ++q) {
                    const uint32_t row = row0 + (uint32_t)(mi * R + lr);
                    const uint32_t off = (uint32_t)(stage * STAGE) + row * KTB +
                                         (((uint32_t)AT::a_chunk(s, lane, q) ^ swz) << 4);
                    af[s][mi][q] = *reinterpret_cast<const i32x4*>(lds + off);
                }
        }
    };
    auto mma = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s = 0; s < STEPS; ++s)
#pragma unroll
            for (int mi = 0; mi < MR; ++mi)
#pragma unroll
                for (int j = 0; j < NR; ++j)
                    acc[mi][j] = AT::mma(af[s][mi], bf[s][j], acc[mi][j]);
        __builtin_amdgcn_s_setprio(0);
    };

#pragma unroll
    for (int t = 0; t < ST - 1; ++t)
        load(t, t);
    DG_STAGE_BARRIER((ST - 2) * LOADS);
    int stage = 0;           // = t % ST
    int pre = ST - 1;        // = (t + ST - 1) % ST
    for (int t = 0; t < kr.n; ++t) {
        // half 2t
        if (g0) {
            load(t + ST - 1, pre);
            read(stage);
            DG_STAGE_BARRIER((ST - 1) * LOADS);
        } else {
            if (t > 0)
                mma();
            DG_STAGE_BARRIER((ST - 2) * LOADS);
        }
        // half 2t + 1
        if (!g0) {
            load(t + ST - 1, pre);
            read(stage);
        } else {
            mma();
        }
        DG_STAGE_BARRIER((ST - 2) * LOADS);
        stage = stage + 1 == ST ? 0 : stage + 1;
        pre = pre + 1 == ST ? 0 : pre + 1;
    }
    if (!g0)
        mma();
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    __syncthreads();

    if constexpr (MODE == MODE_SPLIT) {
        store_partial<AT, MR, NR>(p, acc, slice, m0 + (int)row0, n0 + wn * S::WCOLS, lane);
        return;
    }
    float scale_a = 1.f, scale_b = 1.f;
    if constexpr (DT == DT_FP8) {
        scale_a = *p.sa;
        scale_b = *p.sb;
    }
    store_c_tile<DT, AT, MR, NR, S::CH, S::SROW, S::WCOLS, MODE == MODE_EPI>(
        p, acc, lds + wave * (S::CH * R * S::SROW), m0, rows, n0 + wn * S::WCOLS, (int)row0, lane,
        scale_a, scale_b);
}

// Skinny kernel (small M: decode and short prefill): one workgroup per NB
// 16-column blocks of B covering all M rows (MR 16-row MFMA blocks).  Its W
// waves split K; each streams its K range of the preshuffled B once, with two
// batches of U k-tiles of loads in flight (the next batch is issued before
// the current one is consumed, so the HBM latency is paid once per wave, not
// once per batch; B with the non-temporal hint, as no other workgroup reads
// it), and reads A straight from global (small; it stays in L2).
// Partial sums are reduced in LDS in a fixed order: deterministic, no
// workspace.
template <int DT, int MR, int NB, int W, bool EPI>
__global__ __launch_bounds__(64 * W) void gemm_skinny_kernel(GemmArgs p)
{
    // k-tiles per batch; 16 waves of 1024 threads have 128 VGPRs each, which
    // two batches of 4 k-tiles of fragments would exceed
    constexpr int U = W >= 16 ? (MR == 1 ? 2 : 1) : (MR == 1 ? 4 : (MR == 2 ? 2 : 1));
    __shared__ f32x4 red[W][MR * NB][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int nb0 = blockIdx.x * NB;
    const int nbv = min(NB, p.nblk - nb0);
    const rsrc_t rb = make_rsrc(p.Bs + (int64_t)nb0 * p.KB * 1024,
                                (uint32_t)nbv * (uint32_t)p.KB * 1024u);
    const rsrc_t ra = make_rsrc(p.A, (uint32_t)((int64_t)(p.M - 1) * p.lda_b + p.KA_b));

    const int per = (p.nkt + W - 1) / W;
    const int kt0 = wave * per;
    const int kt1 = min(p.nkt, kt0 + per);

    f32x4 acc[MR][NB];
#pragma unroll
    for (int mi = 0; mi < MR; ++mi)
#pragma unroll
        for (int j = 0; j < NB; ++j)
            acc[mi][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    i32x4 bv[2][U][NB][2], av[2][U][MR][2];
    // k-tiles at or past kt1 (and the K tail) load through out-of-range
    // offsets: zeros, no memory traffic.
    auto load = [&](int set, int kt) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = kt + u;
            const bool kv = k < kt1;
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int kb = 2 * k + c;
                    uint32_t off = (uint32_t)(j * p.KB + kb) * 1024u + lane * 16;
                    if (!kv || kb >= p.KB)
                        off = kOOB;
                    bv[set][u][j][c] = load16_nt(rb, off);   // each B byte is read once
                }
#pragma unroll
            for (int mi = 0; mi < MR; ++mi)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int byte = k * 128 + h * 64 + g4 * 16;
                    uint32_t off = (uint32_t)(mi * 16 + r16) * (uint32_t)p.lda_b + (uint32_t)byte;
                    if (!kv || byte >= p.KA_b)
                        off = kOOB;
                    av[set][u][mi][h] = load16(ra, off);
                }
        }
    };
    auto comp = [&](int set) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (DT == DT_BF16) {
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int mi = 0; mi < MR; ++mi)
#pragma unroll
                        for (int j = 0; j < NB; ++j)
                            acc[mi][j] = mfma_bf16(av[set][u][mi][s], bv[set][u][j][s], acc[mi][j]);
            } else {
#pragma unroll
                for (int mi = 0; mi < MR; ++mi)
#pragma unroll
                    for (int j = 0; j < NB; ++j)
                        acc[mi][j] = mfma_fp8(cat(av[set][u][mi][0], av[set][u][mi][1]),
                                              cat(bv[set][u][j][0], bv[set][u][j][1]), acc[mi][j]);
            }
        }
    };
    if (kt0 < kt1) {
        load(0, kt0);
        for (int kt = kt0; kt < kt1; kt += 2 * U) {
            load(1, kt + U);
            comp(0);
            if (kt + 2 * U < kt1)
                load(0, kt + 2 * U);
            comp(1);
        }
    }

#pragma unroll
    for (int mi = 0; mi < MR; ++mi)
#pragma unroll
        for (int j = 0; j < NB; ++j)
            red[wave][mi * NB + j][lane] = acc[mi][j];
    __syncthreads();

    float scale_a = 1.f, scale_b = 1.f;
    if constexpr (DT == DT_FP8) {
        scale_a = *p.sa;
        scale_b = *p.sb;
    }
    for (int a = wave; a < MR * NB; a += W) {
        f32x4 s = red[0][a][lane];
#pragma unroll
        for (int w = 1; w < W; ++w)
            s = s + red[w][a][lane];
        const int mi = a / NB, j = a % NB;
        const int col = (nb0 + j) * 16 + r16;
        if (col < p.N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = mi * 16 + 4 * g4 + i;
                if (row < p.M) {
                    float v = s[i];
                    if constexpr (DT == DT_FP8)
                        v = (v * scale_a) * scale_b;
                    if constexpr (EPI)
                        v = apply_epilogue(p.ep, v, row, col);
                    p.C[(int64_t)row * p.ldc + col] = bf16_rne(v);
                }
            }
        }
    }
}

}  // namespace dg
