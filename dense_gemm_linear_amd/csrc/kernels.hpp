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

// Depth of the tiled kernel's load pipeline (k-tiles in LDS / registers):
// 3 for 4-wave tiles (one wave per SIMD hides its own latency), 2 for 8-wave
// tiles (two waves per SIMD share 512 registers and hide each other's).
#ifndef DG_STAGES_4WAVE
#define DG_STAGES_4WAVE 3
#endif
#ifndef DG_STAGES_8WAVE
#define DG_STAGES_8WAVE 2
#endif
// Tile rows per raster group, and whether workgroups are renumbered per XCD.
#ifndef DG_GROUP_M
#define DG_GROUP_M 4
#endif
// A fragments read from LDS ahead of the MFMAs that consume them.
#ifndef DG_LDS_AHEAD
#define DG_LDS_AHEAD 2
#endif
#ifndef DG_XCD_REMAP
#define DG_XCD_REMAP 1
#endif
constexpr int tiled_stages(int waves) { return waves == 8 ? DG_STAGES_8WAVE : DG_STAGES_4WAVE; }

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
};

// Workgroup -> output tile.  Workgroups are dispatched round robin over the 8
// XCDs, each with its own L2; renumber so that every XCD receives one
// contiguous run of logical tiles, then walk the logical tiles in groups of
// GROUP_M tile rows, column by column, so tiles that share A rows or B columns
// run at the same time on the same L2.
template <int GROUP_M>
__device__ __forceinline__ void tile_coords(int wg, int tiles_m, int tiles_n, int& tm, int& tn)
{
    const int G = tiles_m * tiles_n;
    int t = wg;
    if (DG_XCD_REMAP) {
        const int x = wg & 7, j = wg >> 3;
        const int q = G >> 3, r = G & 7;
        t = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + j;
    }
    const int per_group = GROUP_M * tiles_n;
    const int grp = t / per_group;
    const int first = grp * GROUP_M;
    const int gm = min(tiles_m - first, GROUP_M);
    const int in = t - grp * per_group;
    tm = first + in % gm;
    tn = in / gm;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at maximum).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

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
// 32 bf16 MFMAs accumulating in VGPRs issue at roughly half of it (measured),
// so the large tiles use 32 x 32 atoms.
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

// The A tile of one k-tile in LDS: TM rows of 128 bytes, the 16-byte chunk c
// of row r stored at slot c ^ ((r >> 1) & 7) ("GEMM Optimization Guide"
// page, section 3: an XOR swizzle at 16-byte granularity, applied on both
// the write and the read side).  The global -> LDS copy is a 16-byte LDS DMA
// per lane (page section 11: 16 bytes per op on gfx950): one wave load fills
// one 1 KiB chunk = 8 rows, lane l landing at row l / 8, slot l % 8, so the
// swizzle is applied to the global address instead.
struct ADma {
    uint32_t goff;   // byte offset of this lane's 16 bytes in the A slab (k-tile 0)
    uint32_t col;    // its K byte within the k-tile (for the K-tail mask)
};

__device__ __forceinline__ ADma a_dma_lane(int chunk, int lane, int64_t lda_b)
{
    const uint32_t row = 8 * (uint32_t)chunk + (uint32_t)(lane >> 3);
    const uint32_t col = (uint32_t)(lane & 7) ^ ((row >> 1) & 7);
    return {row * (uint32_t)lda_b + col * 16, col * 16};
}

// Epilogue shared by the tiled kernels: scale (e4m3), round to bf16, stage a
// wave's (MR*R) x (NR*R) accumulator block through its private LDS region
// CH atom rows at a time, and store 16-byte row pieces ("GEMM Optimization
// Guide" page, section 7.2).  Rows past M fall outside the C descriptor; the
// column predicate keeps a row's padding and the next row intact, and odd
// leading dimensions or an unaligned C take 2-byte stores.
template <int DT, class AT, int MR, int NR, int CH, int SROW, int WCOLS>
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
#pragma unroll
    for (int cc = 0; cc < MR / CH; ++cc) {
#pragma unroll
        for (int ml = 0; ml < CH; ++ml)
#pragma unroll
            for (int j = 0; j < NR; ++j)
#pragma unroll
                for (int e = 0; e < AT::NACC; ++e) {
                    float v = acc[cc * CH + ml][j][e];
                    if constexpr (DT == DT_FP8)
                        v = (v * scale_a) * scale_b;
                    const int row = ml * R + AT::out_row(e, lane);
                    const int col = j * R + lc;
                    *reinterpret_cast<uint16_t*>(stage + row * SROW + col * 2) = bf16_rne(v);
                }
        __syncthreads();
#pragma unroll
        for (int q0 = 0; q0 < PIECES; q0 += 64) {
            const int q = q0 + lane;
            if (PIECES % 64 == 0 || q < PIECES) {
                const int prow = q / PPR, pc = q % PPR;
                const i32x4 v = *reinterpret_cast<const i32x4*>(stage + prow * SROW + pc * 16);
                const int trow = row0 + cc * CH * R + prow;   // row within the tile
                const int gcol = col_w + pc * 8;
                const uint32_t off = (uint32_t)(((int64_t)trow * p.ldc + gcol) * 2);
                if (p.c_vec && gcol + 8 <= p.N) {
                    store16(rc, off, v);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (gcol + e < p.N)
                            store2(rc, off + 2 * e, (uint16_t)(((uint32_t)v[e >> 1]) >> (16 * (e & 1))));
                }
            }
        }
        __syncthreads();
    }
}

// Largest CH dividing MR whose staging (WAVES regions of CH*R rows) fits in
// `avail` bytes of LDS.
constexpr int fit_stage_rows(int MR, int WAVES, int R, int SROW, int avail)
{
    int ch = MR;
    while (ch > 1 && (WAVES * ch * R * SROW > avail || MR % ch != 0))
        --ch;
    return ch;
}

// Barrier without the workgroup memory fence of __syncthreads (which would
// drain every outstanding load, prefetches included); an explicit vmcnt wait
// before it is what makes the next stage visible.
__device__ __forceinline__ void stage_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Issue order of one k-tile's LDS reads and MFMAs: the reads of step 0, then
// the MFMAs of each step with the next step's reads spread between them, so
// that reads are in flight while MFMAs issue.
template <int STEPS, int MF, int RD>
__device__ __forceinline__ void schedule_ktile()
{
    __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        if (s + 1 < STEPS) {
#pragma unroll
            for (int i = 0; i < MF; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i < RD)
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            if (RD > MF)
                __builtin_amdgcn_sched_group_barrier(0x100, RD > MF ? RD - MF : 1, 0);
        } else {
            __builtin_amdgcn_sched_group_barrier(0x008, MF, 0);
        }
    }
}

// ---------------------------------------------------------------------------
// Tiled kernel ("GEMM Optimization Guide" page, sections 1, 2, 3, 4, 6, 7):
// WM x 4 waves, the 4 wave columns splitting tile_n (section 1.1); A through
// LDS (ST-stage ring fed by LDS DMA), B straight from the preshuffled layout
// into VGPRs (section 4.2), ST - 1 k-tiles ahead.
template <int TM, int TN, int WM, int ST, int R>
struct TiledShape {
    static constexpr int WAVES = 4 * WM;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int MR = TM / WM / R;        // atoms per wave along M
    static constexpr int NR = TN / 4 / R;         // atoms per wave along N
    static constexpr int A_DMA = TM / 8 / WAVES;  // 1 KiB A loads per wave per k-tile
    static constexpr int A_BUF = TM * 128;        // bytes of one A stage
    static constexpr int B_LOADS = TN / 32;       // 16-byte B loads per lane per k-tile
    static constexpr int LOADS = A_DMA + B_LOADS; // vector-memory ops per wave per k-tile
    static constexpr int WCOLS = TN / 4;          // C columns per wave
    static constexpr int SROW = WCOLS * 2 + 16;   // staging row pitch (padded)
    static constexpr int CH = fit_stage_rows(MR, WAVES, R, SROW, ST * A_BUF);
    static constexpr int LDS = (ST * A_BUF > WAVES * CH * R * SROW) ? ST * A_BUF
                                                                    : WAVES * CH * R * SROW;
    static_assert(MR >= 1 && NR >= 1 && MR * WM * R == TM && NR * 4 * R == TN, "tile shape");
    static_assert(A_DMA >= 1 && A_DMA * 8 * WAVES == TM, "A DMA split");
    static_assert(ST >= 2 && ST <= 4 && (ST - 2) * LOADS <= 63, "pipeline depth");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <int DT, int TM, int TN, int WM, int ST, int R>
__global__ __launch_bounds__(64 * 4 * WM, 1) void gemm_tiled_kernel(GemmArgs p)
{
    using S = TiledShape<TM, TN, WM, ST, R>;
    using AT = Atom<DT, R>;
    using acc_t = typename AT::acc_t;
    constexpr int MR = S::MR, NR = S::NR, A_DMA = S::A_DMA, A_BUF = S::A_BUF;
    constexpr int WAVES = S::WAVES, STEPS = AT::STEPS, P = AT::P;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[S::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;     // wave row (M) and column (N)
    int tm, tn;
    tile_coords<DG_GROUP_M>(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
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

    ADma ad[A_DMA];
#pragma unroll
    for (int i = 0; i < A_DMA; ++i)
        ad[i] = a_dma_lane(wave + WAVES * i, lane, p.lda_b);
    const int lr = lane % R;                       // row / column of this lane in an atom
    const uint32_t swz = (uint32_t)((lane & 15) >> 1) & 7;
    const uint32_t row0 = (uint32_t)(wm * (TM / WM));   // first A row of this wave
    // 16-column block of this lane's column in atom 0 of this wave
    const uint32_t bblk = (uint32_t)(wn * NR * (R / 16) + (lr >> 4));
    const uint32_t b_lane = bblk * (uint32_t)p.KB * 1024u + (uint32_t)(lane & 15) * 16;

    i32x4 breg[ST][NR][STEPS][P];
    acc_t acc[MR][NR];
#pragma unroll
    for (int mi = 0; mi < MR; ++mi)
#pragma unroll
        for (int j = 0; j < NR; ++j)
            acc[mi][j] = zero_acc<AT>();

    // A k-tile past the real K (kt >= nkt, or the K tail of the last one)
    // loads through out-of-range offsets: zeros, and no memory traffic.
    const int last_full = p.tail ? p.nkt - 1 : p.nkt;   // first k-tile that needs masking
    auto load_a = [&](int kt, int stage) __attribute__((always_inline)) {
        const bool mask = kt >= last_full;
#pragma unroll
        for (int i = 0; i < A_DMA; ++i) {
            uint32_t off = ad[i].goff + (uint32_t)kt * 128;
            if (mask && (int)((uint32_t)kt * 128 + ad[i].col) >= p.KA_b)
                off = kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (lds_void*)(lds + stage * A_BUF + (wave + WAVES * i) * 1024), 16, off, 0, 0, 0);
        }
    };
    auto load_b = [&](i32x4 (&dst)[NR][STEPS][P], int kt) __attribute__((always_inline)) {
        const bool mask = kt >= last_full;
#pragma unroll
        for (int j = 0; j < NR; ++j)
#pragma unroll
            for (int s = 0; s < STEPS; ++s)
#pragma unroll
                for (int q = 0; q < P; ++q) {
                    const int kb = kt * 2 + AT::b_half(s, q);
                    uint32_t off = b_lane + (uint32_t)(j * (R / 16) * p.KB + kb) * 1024u +
                                   ((uint32_t)AT::b_group(s, lane, q) << 8);
                    if (mask && kb >= p.KB)
                        off = kOOB;
                    dst[j][s][q] = load16(rb, off);
                }
    };
    auto read_a = [&](int stage, int s, i32x4 (&dst)[MR][P]) __attribute__((always_inline)) {
#pragma unroll
        for (int mi = 0; mi < MR; ++mi)
#pragma unroll
            for (int q = 0; q < P; ++q) {
                const uint32_t row = row0 + (uint32_t)(mi * R + lr);
                const uint32_t off = (uint32_t)(stage * A_BUF) + row * 128 +
                                     (((uint32_t)AT::a_chunk(s, lane, q) ^ swz) << 4);
                dst[mi][q] = *reinterpret_cast<const i32x4*>(lds + off);
            }
    };
    auto compute = [&](int stage, const i32x4 (&b)[NR][STEPS][P]) __attribute__((always_inline)) {
        i32x4 af[2][MR][P];
        read_a(stage, 0, af[0]);
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            if (s + 1 < STEPS)
                read_a(stage, s + 1, af[(s + 1) & 1]);
#pragma unroll
            for (int mi = 0; mi < MR; ++mi)
#pragma unroll
                for (int j = 0; j < NR; ++j)
                    acc[mi][j] = AT::mma(af[s & 1][mi], b[j][s], acc[mi][j]);
        }
        schedule_ktile<STEPS, MR * NR, MR * P>();
    };

    // Prologue: k-tiles 0 .. ST-2 in flight, wait for k-tile 0.
#pragma unroll
    for (int t = 0; t < ST - 1; ++t) {
        load_a(t, t);
        load_b(breg[t], t);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((ST - 2) * S::LOADS));
    stage_barrier();

    // Phase t multiplies k-tile t out of stage t % ST while k-tile t + ST - 1
    // streams into the stage that phase t - 1 just finished with.  At the end
    // of the phase, k-tile t + 1 must have landed: at most the ST - 2 newer
    // k-tiles' loads may still be in flight.  Loads past nkt read zeros.
    auto phase = [&](int t, auto sc) __attribute__((always_inline)) {
        constexpr int s = decltype(sc)::value;
        constexpr int pre = (s + ST - 1) % ST;
        load_a(t + ST - 1, pre);
        load_b(breg[pre], t + ST - 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(s, breg[s]);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm((ST - 2) * S::LOADS));
        stage_barrier();
    };
    // Steady state: ST unconditional phases per trip (no control-flow merges
    // inside the loop, so the accumulators keep their registers); the last
    // nkt % ST k-tiles run after it.
    int kt = 0;
    for (; kt + ST <= p.nkt; kt += ST) {
        phase(kt, std::integral_constant<int, 0>{});
        phase(kt + 1, std::integral_constant<int, 1>{});
        if constexpr (ST > 2)
            phase(kt + 2, std::integral_constant<int, 2>{});
        if constexpr (ST > 3)
            phase(kt + 3, std::integral_constant<int, 3>{});
    }
    if (kt < p.nkt)
        phase(kt, std::integral_constant<int, 0>{});
    if constexpr (ST > 2) {
        if (kt + 1 < p.nkt)
            phase(kt + 1, std::integral_constant<int, 1>{});
    }
    if constexpr (ST > 3) {
        if (kt + 2 < p.nkt)
            phase(kt + 2, std::integral_constant<int, 2>{});
    }
    // The zero prefetches past nkt still target LDS: drain them everywhere
    // before the epilogue reuses it.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();

    float scale_a = 1.f, scale_b = 1.f;
    if constexpr (DT == DT_FP8) {
        scale_a = *p.sa;
        scale_b = *p.sb;
    }
    store_c_tile<DT, AT, MR, NR, S::CH, S::SROW, S::WCOLS>(
        p, acc, lds + wave * (S::CH * R * S::SROW), m0, rows, n0 + wn * S::WCOLS, (int)row0, lane,
        scale_a, scale_b);
}

// ---------------------------------------------------------------------------
// Tiled kernel with A and B both staged in LDS ("AB" kernel).
//
// Loading a B fragment straight into the registers of every wave that needs
// it (the kernel above) moves it from L2 once per wave row; measured on
// MI355X, the L2 -> CU path, not the MFMA, bounds that kernel once the tile
// is large.  Here each k-tile of A *and* B enters the workgroup once, by
// 16-byte LDS DMA, and the WM x WN waves read their fragments from LDS.  The
// preshuffled B blocks (1 KiB = 16 columns x 64 K bytes) land in LDS
// unchanged, so a B fragment read is a run of 256 contiguous bytes per 16
// lanes.  Per stage: [A: TM rows x 128 B, XOR-swizzled][B: TN/16 blocks x 2
// halves x 1 KiB].
template <int TM, int TN, int WM, int WN, int ST, int R>
struct ABShape {
    static constexpr int WAVES = WM * WN;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int MR = TM / WM / R;        // atoms per wave along M
    static constexpr int NR = TN / WN / R;        // atoms per wave along N
    static constexpr int A_BUF = TM * 128;
    static constexpr int B_BUF = TN * 128;
    static constexpr int STAGE = A_BUF + B_BUF;
    static constexpr int A_DMA = TM / 8 / WAVES;  // 1 KiB A loads per wave per k-tile
    static constexpr int B_DMA = TN / 8 / WAVES;  // 1 KiB B loads per wave per k-tile
    static constexpr int LOADS = A_DMA + B_DMA;
    static constexpr int WCOLS = TN / WN;         // C columns per wave
    static constexpr int SROW = WCOLS * 2 + 16;   // staging row pitch (padded)
    static constexpr int CH = fit_stage_rows(MR, WAVES, R, SROW, ST * STAGE);
    static constexpr int LDS = (ST * STAGE > WAVES * CH * R * SROW) ? ST * STAGE
                                                                    : WAVES * CH * R * SROW;
    static_assert(MR >= 1 && NR >= 1 && MR * WM * R == TM && NR * WN * R == TN, "tile shape");
    static_assert(A_DMA >= 1 && B_DMA >= 1 && A_DMA * 8 * WAVES == TM && B_DMA * 8 * WAVES == TN,
                  "DMA split");
    static_assert(ST >= 2 && ST <= 4 && (ST - 2) * LOADS <= 63, "pipeline depth");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <int DT, int TM, int TN, int WM, int WN, int ST, int R>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_ab_kernel(GemmArgs p)
{
    using S = ABShape<TM, TN, WM, WN, ST, R>;
    using AT = Atom<DT, R>;
    using acc_t = typename AT::acc_t;
    constexpr int MR = S::MR, NR = S::NR, A_BUF = S::A_BUF, STAGE = S::STAGE;
    constexpr int WAVES = S::WAVES, A_DMA = S::A_DMA, B_DMA = S::B_DMA;
    constexpr int STEPS = AT::STEPS, P = AT::P;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[S::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    int tm, tn;
    tile_coords<DG_GROUP_M>(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
    const int m0 = tm * TM;
    const int n0 = tn * TN;
    const int rows = min(TM, p.M - m0);
    const rsrc_t ra = make_rsrc(p.A + (int64_t)m0 * p.lda_b,
                                (uint32_t)((int64_t)(rows - 1) * p.lda_b + p.KA_b));
    const int nb0 = n0 >> 4;
    const int nbv = min(TN / 16, p.nblk - nb0);
    const rsrc_t rb = make_rsrc(p.Bs + (int64_t)nb0 * p.KB * 1024,
                                (uint32_t)nbv * (uint32_t)p.KB * 1024u);

    // A chunk w + WAVES*i: rows 8c .. 8c+7.  B chunk w + WAVES*i: 16-column
    // block b / 2, 64-byte half b % 2 of the k-tile.
    ADma ad[A_DMA];
    uint32_t b_goff[B_DMA], b_half[B_DMA];
#pragma unroll
    for (int i = 0; i < A_DMA; ++i)
        ad[i] = a_dma_lane(wave + WAVES * i, lane, p.lda_b);
#pragma unroll
    for (int i = 0; i < B_DMA; ++i) {
        const uint32_t b = wave + WAVES * i;
        b_goff[i] = ((b >> 1) * (uint32_t)p.KB + (b & 1)) * 1024u + lane * 16;
        b_half[i] = b & 1;
    }
    const int lr = lane % R;
    const uint32_t swz = (uint32_t)((lane & 15) >> 1) & 7;
    const uint32_t row0 = (uint32_t)(wm * (TM / WM));
    // LDS byte offset (within a stage's B region) of this lane's column in
    // atom 0 of this wave, group 0, half 0.
    const uint32_t b_lds = (uint32_t)((wn * NR * (R / 16) + (lr >> 4)) * 2048 + (lane & 15) * 16);

    acc_t acc[MR][NR];
#pragma unroll
    for (int mi = 0; mi < MR; ++mi)
#pragma unroll
        for (int j = 0; j < NR; ++j)
            acc[mi][j] = zero_acc<AT>();

    const int last_full = p.tail ? p.nkt - 1 : p.nkt;
    auto load = [&](int kt, int stage) __attribute__((always_inline)) {
        const bool mask = kt >= last_full;
        uint8_t* base = lds + stage * STAGE;
#pragma unroll
        for (int i = 0; i < A_DMA; ++i) {
            uint32_t off = ad[i].goff + (uint32_t)kt * 128;
            if (mask && (int)((uint32_t)kt * 128 + ad[i].col) >= p.KA_b)
                off = kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (lds_void*)(base + (wave + WAVES * i) * 1024), 16, off, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < B_DMA; ++i) {
            uint32_t off = b_goff[i] + (uint32_t)kt * 2048u;
            if (mask && kt * 2 + (int)b_half[i] >= p.KB)
                off = kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (lds_void*)(base + A_BUF + (wave + WAVES * i) * 1024), 16, off, 0, 0, 0);
        }
    };
    auto read_frags = [&](int stage, int s, i32x4 (&af)[MR][P], i32x4 (&bf)[NR][P])
                          __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NR; ++j)
#pragma unroll
            for (int q = 0; q < P; ++q) {
                const uint32_t off = (uint32_t)(stage * STAGE + A_BUF) + b_lds +
                                     (uint32_t)(j * (R / 16) * 2048) +
                                     ((uint32_t)AT::b_half(s, q) << 10) +
                                     ((uint32_t)AT::b_group(s, lane, q) << 8);
                bf[j][q] = *reinterpret_cast<const i32x4*>(lds + off);
            }
#pragma unroll
        for (int mi = 0; mi < MR; ++mi)
#pragma unroll
            for (int q = 0; q < P; ++q) {
                const uint32_t row = row0 + (uint32_t)(mi * R + lr);
                const uint32_t off = (uint32_t)(stage * STAGE) + row * 128 +
                                     (((uint32_t)AT::a_chunk(s, lane, q) ^ swz) << 4);
                af[mi][q] = *reinterpret_cast<const i32x4*>(lds + off);
            }
    };
    auto compute = [&](int stage) __attribute__((always_inline)) {
        i32x4 af[2][MR][P], bf[2][NR][P];
        read_frags(stage, 0, af[0], bf[0]);
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            if (s + 1 < STEPS)
                read_frags(stage, s + 1, af[(s + 1) & 1], bf[(s + 1) & 1]);
#pragma unroll
            for (int mi = 0; mi < MR; ++mi)
#pragma unroll
                for (int j = 0; j < NR; ++j)
                    acc[mi][j] = AT::mma(af[s & 1][mi], bf[s & 1][j], acc[mi][j]);
        }
        schedule_ktile<STEPS, MR * NR, (MR + NR) * P>();
    };
    auto phase = [&](int t, auto sc) __attribute__((always_inline)) {
        constexpr int s = decltype(sc)::value;
        constexpr int pre = (s + ST - 1) % ST;
        load(t + ST - 1, pre);
        __builtin_amdgcn_sched_barrier(0);
        compute(s);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm((ST - 2) * S::LOADS));
        stage_barrier();
    };

#pragma unroll
    for (int t = 0; t < ST - 1; ++t)
        load(t, t);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((ST - 2) * S::LOADS));
    stage_barrier();

    int kt = 0;
    for (; kt + ST <= p.nkt; kt += ST) {
        phase(kt, std::integral_constant<int, 0>{});
        phase(kt + 1, std::integral_constant<int, 1>{});
        if constexpr (ST > 2)
            phase(kt + 2, std::integral_constant<int, 2>{});
        if constexpr (ST > 3)
            phase(kt + 3, std::integral_constant<int, 3>{});
    }
    if (kt < p.nkt)
        phase(kt, std::integral_constant<int, 0>{});
    if constexpr (ST > 2) {
        if (kt + 1 < p.nkt)
            phase(kt + 1, std::integral_constant<int, 1>{});
    }
    if constexpr (ST > 3) {
        if (kt + 2 < p.nkt)
            phase(kt + 2, std::integral_constant<int, 2>{});
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();

    float scale_a = 1.f, scale_b = 1.f;
    if constexpr (DT == DT_FP8) {
        scale_a = *p.sa;
        scale_b = *p.sb;
    }
    store_c_tile<DT, AT, MR, NR, S::CH, S::SROW, S::WCOLS>(
        p, acc, lds + wave * (S::CH * R * S::SROW), m0, rows, n0 + wn * S::WCOLS, (int)row0, lane,
        scale_a, scale_b);
}

// Skinny kernel: NB 16-column blocks per workgroup, MR 16-row blocks cover M.
template <int DT, int MR, int NB>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs p)
{
    constexpr int U = 4;   // k-tiles in flight per wave
    __shared__ f32x4 red[4][MR * NB][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int nb0 = blockIdx.x * NB;
    const int nbv = min(NB, p.nblk - nb0);
    const rsrc_t rb = make_rsrc(p.Bs + (int64_t)nb0 * p.KB * 1024,
                                (uint32_t)nbv * (uint32_t)p.KB * 1024u);
    const rsrc_t ra = make_rsrc(p.A, (uint32_t)((int64_t)(p.M - 1) * p.lda_b + p.KA_b));

    const int per = (p.nkt + 3) >> 2;
    const int kt0 = wave * per;
    const int kt1 = min(p.nkt, kt0 + per);

    f32x4 acc[MR][NB];
#pragma unroll
    for (int mi = 0; mi < MR; ++mi)
#pragma unroll
        for (int j = 0; j < NB; ++j)
            acc[mi][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kt = kt0; kt < kt1; kt += U) {
        i32x4 bv[U][NB][2], av[U][MR][2];
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
                    bv[u][j][c] = load16(rb, off);
                }
#pragma unroll
            for (int mi = 0; mi < MR; ++mi)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int byte = k * 128 + h * 64 + g4 * 16;
                    uint32_t off = (uint32_t)(mi * 16 + r16) * (uint32_t)p.lda_b + (uint32_t)byte;
                    if (!kv || byte >= p.KA_b)
                        off = kOOB;
                    av[u][mi][h] = load16(ra, off);
                }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (DT == DT_BF16) {
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int mi = 0; mi < MR; ++mi)
#pragma unroll
                        for (int j = 0; j < NB; ++j)
                            acc[mi][j] = mfma_bf16(av[u][mi][s], bv[u][j][s], acc[mi][j]);
            } else {
#pragma unroll
                for (int mi = 0; mi < MR; ++mi)
#pragma unroll
                    for (int j = 0; j < NB; ++j)
                        acc[mi][j] = mfma_fp8(cat(av[u][mi][0], av[u][mi][1]),
                                              cat(bv[u][j][0], bv[u][j][1]), acc[mi][j]);
            }
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
    for (int a = wave; a < MR * NB; a += 4) {
        f32x4 s = red[0][a][lane];
        s = s + red[1][a][lane];
        s = s + red[2][a][lane];
        s = s + red[3][a][lane];
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
                    p.C[(int64_t)row * p.ldc + col] = bf16_rne(v);
                }
            }
        }
    }
}

}  // namespace dg
