// Host-side declarations shared by the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/densegemm.h"
#include "kernels.hpp"

namespace dg {

// Tiled ladder: (tile_m, tile_n, waves, stages, atom, k-tile bytes).
// X(M, N, W, ST, R, KTB) is applied to every rung.  8-wave rungs arrange the
// waves 2 (M) x 4 (N).
#define DG_TILED_LADDER(X)                                                                  \
    X(256, 128, 8, 2, 16, 128) X(128, 256, 8, 2, 16, 128) X(128, 128, 8, 2, 16, 128)       \
    X(256, 128, 4, 3, 16, 128) X(256, 64, 4, 3, 16, 128)                                   \
    X(128, 256, 4, 3, 16, 128) X(128, 128, 4, 3, 16, 128) X(128, 64, 4, 3, 16, 128)        \
    X(64, 256, 4, 3, 16, 128) X(64, 128, 4, 3, 16, 128) X(64, 64, 4, 3, 16, 128)           \
    X(32, 256, 4, 3, 16, 128) X(32, 128, 4, 3, 16, 128) X(32, 64, 4, 3, 16, 128)           \
    X(256, 256, 8, 2, 32, 128) X(256, 128, 8, 2, 32, 128) X(128, 256, 8, 2, 32, 128)       \
    X(128, 128, 8, 2, 32, 128) X(256, 128, 4, 3, 32, 128) X(128, 256, 4, 3, 32, 128)       \
    X(128, 128, 4, 3, 32, 128) X(64, 256, 4, 3, 32, 128) X(64, 128, 4, 3, 32, 128)         \
    X(128, 256, 4, 4, 32, 64) X(128, 128, 4, 4, 32, 64) X(256, 128, 4, 4, 32, 64)

// A+B-in-LDS ladder: (tile_m, tile_n, wave rows, wave columns, stages, atom,
// k-tile bytes).
#define DG_AB_LADDER(X)                                                                     \
    X(256, 128, 2, 2, 3, 16, 128) X(128, 256, 2, 2, 3, 16, 128)                            \
    X(128, 128, 2, 2, 3, 16, 128)                                                          \
    X(256, 256, 2, 4, 2, 32, 128) X(256, 256, 2, 2, 2, 32, 128)                            \
    X(256, 128, 2, 4, 3, 32, 128) X(256, 128, 2, 2, 3, 32, 128)                            \
    X(128, 256, 2, 2, 3, 32, 128) X(128, 128, 2, 2, 3, 32, 128)                            \
    X(256, 256, 2, 4, 4, 32, 64) X(256, 256, 2, 2, 4, 32, 64)                            \
    X(256, 128, 2, 4, 6, 32, 64) X(128, 256, 2, 2, 6, 32, 64)                            \
    X(256, 256, 2, 4, 4, 16, 64)

// Ping-pong A+B ladder (8 waves, 2 groups x 4): (tile_m, tile_n, stages, atom,
// k-tile bytes).  Narrower tiles halve each wave's MFMAs per k-tile while its
// loads stay the same, and 128-byte k-tiles exceed 256 VGPRs.
#define DG_PP_LADDER(X) X(256, 256, 4, 32, 64)

struct PPRung {
    int tm, tn, st, atom, ktb;
};
constexpr PPRung kPPLadder[] = {
#define DG_PPR(M_, N_, ST_, R_, KTB_) {M_, N_, ST_, R_, KTB_},
    DG_PP_LADDER(DG_PPR)
#undef DG_PPR
};

struct ABRung {
    int tm, tn, wm, wn, st, atom, ktb;
};
constexpr ABRung kABLadder[] = {
#define DG_ABR(M_, N_, WM_, WN_, ST_, R_, KTB_) {M_, N_, WM_, WN_, ST_, R_, KTB_},
    DG_AB_LADDER(DG_ABR)
#undef DG_ABR
};

struct TiledRung {
    int tm, tn, waves, st, atom, ktb;
};
constexpr TiledRung kTiledLadder[] = {
#define DG_RUNG(M_, N_, W_, ST_, R_, KTB_) {M_, N_, W_, ST_, R_, KTB_},
    DG_TILED_LADDER(DG_RUNG)
#undef DG_RUNG
};

// A rung matches a request when every field agrees; a requested stage count
// or k-tile size of 0 matches any (the first such rung in ladder order).
#define DG_MATCH(ST_, KTB_) ((st == 0 || st == (ST_)) && (ktb == 0 || ktb == (KTB_)))
// Skinny ladder: (tile_m, tile_n, waves splitting K).
#define DG_SKINNY_LADDER(X)                                                   \
    X(16, 16, 4) X(16, 32, 4) X(16, 64, 4) X(32, 16, 4) X(32, 32, 4) X(32, 64, 4) \
    X(48, 16, 4) X(48, 32, 4) X(48, 64, 4) X(64, 16, 4) X(64, 32, 4) X(64, 64, 4) \
    X(16, 16, 8) X(16, 32, 8) X(32, 16, 8) X(32, 32, 8) X(16, 16, 16) X(32, 16, 16)

struct SkinnyRung {
    int tm, tn, waves;
};
constexpr SkinnyRung kSkinnyLadder[] = {
#define DG_SR(M_, N_, W_) {M_, N_, W_},
    DG_SKINNY_LADDER(DG_SR)
#undef DG_SR
};

// Index of the ladder rung a request names, or -1 (st, ktb: 0 = any).
int tiled_rung(int tm, int tn, int waves, int atom, int st, int ktb);
int ab_rung(int tm, int tn, int waves, int atom, int st, int ktb);
int pp_rung(int tm, int tn, int waves, int atom, int st, int ktb);
bool skinny_supported(int tm, int tn, int waves);

// Launchers: return hipSuccess or the launch error.  Grids are computed from
// the arguments; shapes are validated by the caller.
// Launch rung `idx` of the tiled / AB ladder.
// Tiled-kernel launchers, one per (element type, MODE_*, family) instance
// file (tiled_inst.hip): family 0 is the tiled ladder, 1 the A+B and
// ping-pong ladders (`kernel` picks which); idx is the rung's index.
#define DG_DECL_INST(D, M, F) \
    hipError_t launch_inst_##D##_##M##_##F(int kernel, int idx, const GemmArgs& a, hipStream_t s);
DG_DECL_INST(0, 0, 0) DG_DECL_INST(0, 0, 1) DG_DECL_INST(0, 1, 0) DG_DECL_INST(0, 1, 1)
DG_DECL_INST(0, 2, 0) DG_DECL_INST(0, 2, 1) DG_DECL_INST(1, 0, 0) DG_DECL_INST(1, 0, 1)
DG_DECL_INST(1, 1, 0) DG_DECL_INST(1, 1, 1) DG_DECL_INST(1, 2, 0) DG_DECL_INST(1, 2, 1)
DG_DECL_INST(0, 3, 0) DG_DECL_INST(0, 3, 1) DG_DECL_INST(1, 3, 0) DG_DECL_INST(1, 3, 1)
#undef DG_DECL_INST
// rung idx of `kernel` (tiled, A+B or ping-pong) for element type dt, in the
// variant the arguments ask for (split-K, fused epilogue, or plain)
hipError_t launch_tiled_rung(int kernel, int dt, int idx, const GemmArgs& a, hipStream_t s);
hipError_t launch_skinny(int dt, int tm, int tn, int waves, const GemmArgs& a, hipStream_t s);
hipError_t launch_transpose(const void* src, int64_t ld_src, void* dst, int64_t ld_dst,
                            int64_t rows, int64_t cols, int elem_bytes, hipStream_t s);
hipError_t launch_shuffle_bt(const void* Bt, int64_t ldbt, uint8_t* Bs, int64_t N, int64_t K,
                             int elem_bytes, hipStream_t s);
hipError_t launch_zero_c(uint16_t* C, int64_t ldc, int64_t M, int64_t N, Epilogue ep, hipStream_t s);
hipError_t launch_shuffle_b(const uint8_t* B, int64_t ldb_b, uint8_t* Bs, int64_t N, int64_t K_b,
                            int64_t KB, int aligned, hipStream_t s);

// Launch a __global__ function taking one GemmArgs by value; returns the
// launch status of this call (not an earlier sticky error).
template <typename F>
inline hipError_t launch_args(F* kernel, dim3 grid, dim3 block, const GemmArgs& a, hipStream_t s)
{
    GemmArgs copy = a;
    void* args[] = {&copy};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, s);
}

// Resource model of the tiled kernel (used by select_tile's feasibility check).
// Resource model of rung `idx` (used by select_tile's feasibility check).
int tiled_lds_bytes(int idx);
int ab_lds_bytes(int idx);
int pp_lds_bytes(int idx);
int tiled_vgpr_estimate(const TiledRung& r);

// Split-K plan of a tiled rung with k-tiles of ktb bytes asked for k_split
// slices: S slices of kt_per k-tiles each (S <= k_split; no slice is empty),
// and the fp32 partial workspace S * M * ldw * 4 bytes, ldw = N rounded up
// to 4.  S == 1 needs no workspace.
struct SplitPlan {
    int S, kt_per, ldw;
    int64_t ws_bytes;
};
SplitPlan split_plan(int64_t M, int64_t N, int64_t K, int e, int ktb, int k_split);
// k-tile bytes of a resolved tiled / A+B / ping-pong rung
int rung_ktb(int kernel, int idx);
void choose_tile(int64_t M, int64_t N, int64_t K, int dt, int cus, size_t ws_bytes,
                 gemm_tile* out);
hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t s);
hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* out, int grid, hipStream_t s);
// Stream-K plan of a resolved tiled / A+B rung (see gemm_workspace_bytes):
// grid G, whole tiles [0, dp_tiles), k-tiles per tile nkt (the rung's k-tile
// size), the partial slots' bytes and the whole workspace.  ok = false when
// the rung has no stream-K instance or the shape has fewer units than G.
struct SkPlan {
    bool ok;
    int grid, dp_tiles, nkt;
    int64_t tiles, slot_bytes, ws_bytes;
};
// stream-K instances: outputs of 128 x 128 to 128 x 256
// An atom whose MFMA takes more K bytes than a k-tile holds has no instance
// (the e4m3 16 x 16 x 128 MFMA needs 128-byte k-tiles).
template <int DT, int R, int KTB>
constexpr bool atom_fits()
{
    return !(DT == DT_FP8 && R == 16 && KTB != 128);
}
constexpr bool atom_fits_rt(int dt, int atom, int ktb)
{
    return !(dt == DT_FP8 && atom == 16 && ktb != 128);
}

constexpr bool sk_rung(int tm, int tn) { return tm * tn >= 128 * 128 && tm * tn <= 128 * 256; }
SkPlan sk_plan(int kernel, int idx, int tm, int tn, int64_t M, int64_t N, int64_t K, int e, int grid);
hipError_t launch_splitk_reduce(const float* ws, int splits, int M, int N, int ldw, uint16_t* C,
                                int64_t ldc, const float* sa, const float* sb, Epilogue ep,
                                hipStream_t s);
// Split-K addresses a partial plane with 32-bit byte offsets, also for the
// up to 256 rows a tile reaches past M (their stores are dropped by the
// buffer bound): (M + 256) * ldw * 4 must stay within 2 GiB.
constexpr int64_t kMaxPartialPlaneBytes = INT64_C(1) << 31;
inline bool partial_plane_fits(int64_t M, int64_t ldw)
{
    return (M + 256) * ldw * 4 <= kMaxPartialPlaneBytes;
}

}  // namespace dg
