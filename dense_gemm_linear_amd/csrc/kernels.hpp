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

#include "device.hpp"

namespace dg {

enum { DT_BF16 = 0, DT_FP8 = 1 };

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
    const int x = wg & 7, j = wg >> 3;
    const int q = G >> 3, r = G & 7;
    const int t = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + j;
    const int per_group = GROUP_M * tiles_n;
    const int grp = t / per_group;
    const int first = grp * GROUP_M;
    const int gm = min(tiles_m - first, GROUP_M);
    const int in = t - grp * per_group;
    tm = first + in % gm;
    tn = in / gm;
}

template <int TM, int TN>
struct TiledShape {
    static constexpr int MR = TM / 16;            // 16-row MFMA blocks per wave
    static constexpr int NR = TN / 64;            // 16-column blocks per wave
    static constexpr int A_LOADS = TM * 8 / 256;  // 16-byte A chunks per thread per k-tile
    static constexpr int A_BUF = TM * 128;        // bytes of one A buffer
    static constexpr int WCOLS = TN / 4;          // C columns per wave
    static constexpr int SROW = WCOLS * 2 + 16;   // staging row pitch (padded)
    static constexpr int fit_ch()
    {
        int ch = MR;
        while (ch > 1 && (4 * ch * 16 * SROW > 2 * A_BUF || MR % ch != 0))
            --ch;
        return ch;
    }
    static constexpr int CH = fit_ch();           // 16-row blocks per epilogue pass
    static constexpr int LDS = (2 * A_BUF > 4 * CH * 16 * SROW) ? 2 * A_BUF : 4 * CH * 16 * SROW;
    static_assert(TM % 32 == 0 && TN % 64 == 0, "tile shape");
};

template <int DT, int TM, int TN>
__global__ __launch_bounds__(256, 1) void gemm_tiled_kernel(GemmArgs p)
{
    using S = TiledShape<TM, TN>;
    constexpr int MR = S::MR, NR = S::NR, A_LOADS = S::A_LOADS, A_BUF = S::A_BUF;
    __shared__ __attribute__((aligned(16))) uint8_t lds[S::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    int tm, tn;
    tile_coords<4>(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
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

    // A chunk c of a k-tile: row c / 8, 16-byte column c % 8.
    uint32_t a_goff[A_LOADS], a_soff[A_LOADS], a_col[A_LOADS];
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
        const uint32_t c = tid + 256 * i;
        const uint32_t row = c >> 3, col = c & 7;
        a_goff[i] = row * (uint32_t)p.lda_b + col * 16;
        a_soff[i] = row * 128 + ((col ^ ((row >> 1) & 7)) << 4);
        a_col[i] = col * 16;
    }
    const uint32_t b_base = (uint32_t)(wave * NR) * (uint32_t)p.KB * 1024u + lane * 16;
    const int r16 = lane & 15, g4 = lane >> 4;
    const uint32_t swz = (r16 >> 1) & 7;

    i32x4 areg[A_LOADS];
    i32x4 bcur[NR][2], bnext[NR][2];
    f32x4 acc[MR][NR];
#pragma unroll
    for (int mi = 0; mi < MR; ++mi)
#pragma unroll
        for (int j = 0; j < NR; ++j)
            acc[mi][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto load_a = [&](int kt, bool mask) {
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) {
            uint32_t off = a_goff[i] + (uint32_t)kt * 128;
            if (mask && (int)((uint32_t)kt * 128 + a_col[i]) >= p.KA_b)
                off = kOOB;
            areg[i] = load16(ra, off);
        }
    };
    auto load_b = [&](i32x4 (&dst)[NR][2], int kt, bool mask) {
#pragma unroll
        for (int j = 0; j < NR; ++j)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int kb = kt * 2 + c;
                uint32_t off = b_base + (uint32_t)(j * p.KB + kb) * 1024u;
                if (mask && kb >= p.KB)
                    off = kOOB;
                dst[j][c] = load16(rb, off);
            }
    };
    auto store_a = [&](uint8_t* buf) {
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i)
            *reinterpret_cast<i32x4*>(buf + a_soff[i]) = areg[i];
    };
    auto lds_a = [&](const uint8_t* buf, int mi, int col16) -> i32x4 {
        const uint32_t off = (uint32_t)(mi * 16 + r16) * 128 + (((uint32_t)col16 ^ swz) << 4);
        return *reinterpret_cast<const i32x4*>(buf + off);
    };
    auto compute = [&](const uint8_t* buf) {
        if constexpr (DT == DT_BF16) {
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int mi = 0; mi < MR; ++mi) {
                    const i32x4 a = lds_a(buf, mi, 4 * s + g4);
#pragma unroll
                    for (int j = 0; j < NR; ++j)
                        acc[mi][j] = mfma_bf16(a, bcur[j][s], acc[mi][j]);
                }
        } else {
#pragma unroll
            for (int mi = 0; mi < MR; ++mi) {
                const i32x8 a = cat(lds_a(buf, mi, g4), lds_a(buf, mi, 4 + g4));
#pragma unroll
                for (int j = 0; j < NR; ++j)
                    acc[mi][j] = mfma_fp8(a, cat(bcur[j][0], bcur[j][1]), acc[mi][j]);
            }
        }
    };

    // Prologue: k-tile 0 into buffer 0 and registers.
    {
        const bool m = p.tail && p.nkt == 1;
        load_a(0, m);
        load_b(bcur, 0, m);
        store_a(lds);
    }
    __syncthreads();

    for (int kt = 0; kt < p.nkt; ++kt) {
        uint8_t* cur = lds + (kt & 1) * A_BUF;
        uint8_t* nxt = lds + ((kt & 1) ^ 1) * A_BUF;
        const bool has_next = kt + 1 < p.nkt;
        if (has_next) {
            const bool m = p.tail && kt + 2 == p.nkt;
            load_a(kt + 1, m);
            load_b(bnext, kt + 1, m);
        }
        compute(cur);
        if (has_next)
            store_a(nxt);
        __syncthreads();
        if (has_next) {
#pragma unroll
            for (int j = 0; j < NR; ++j) {
                bcur[j][0] = bnext[j][0];
                bcur[j][1] = bnext[j][1];
            }
        }
    }

    // Epilogue: scale, round, stage through LDS, store 16-byte row pieces.
    float scale_a = 1.f, scale_b = 1.f;
    if constexpr (DT == DT_FP8) {
        scale_a = *p.sa;
        scale_b = *p.sb;
    }
    const rsrc_t rc = make_rsrc(p.C + (int64_t)m0 * p.ldc,
                                (uint32_t)(((int64_t)(rows - 1) * p.ldc + p.N) * 2));
    constexpr int CH = S::CH, SROW = S::SROW, WCOLS = S::WCOLS;
    constexpr int PPR = WCOLS / 8;                 // 16-byte pieces per staged row
    constexpr int PIECES = CH * 16 * PPR;
    uint8_t* stage = lds + wave * (CH * 16 * SROW);
    const int col_w = n0 + wave * WCOLS;           // first C column of this wave
#pragma unroll
    for (int cc = 0; cc < MR / CH; ++cc) {
#pragma unroll
        for (int ml = 0; ml < CH; ++ml)
#pragma unroll
            for (int j = 0; j < NR; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v = acc[cc * CH + ml][j][i];
                    if constexpr (DT == DT_FP8)
                        v = (v * scale_a) * scale_b;
                    const int row = ml * 16 + 4 * g4 + i;
                    const int col = j * 16 + r16;
                    *reinterpret_cast<uint16_t*>(stage + row * SROW + col * 2) = bf16_rne(v);
                }
        __syncthreads();
#pragma unroll
        for (int q0 = 0; q0 < PIECES; q0 += 64) {
            const int q = q0 + lane;
            if (PIECES % 64 == 0 || q < PIECES) {
                const int prow = q / PPR, pc = q % PPR;
                const i32x4 v = *reinterpret_cast<const i32x4*>(stage + prow * SROW + pc * 16);
                const int trow = cc * CH * 16 + prow;       // row within the tile
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
