// Host-side declarations shared by the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/densegemm.h"
#include "kernels.hpp"

namespace dg {

// Tiled ladder: (tile_m, tile_n, waves).  X(M, N, W) is applied to every rung.
#define DG_TILED_LADDER(X)                                                              \
    X(256, 256, 8) X(256, 128, 8) X(128, 256, 8) X(128, 128, 8)                        \
    X(256, 128, 4) X(256, 64, 4)                                                       \
    X(128, 256, 4) X(128, 128, 4) X(128, 64, 4)                                        \
    X(64, 256, 4) X(64, 128, 4) X(64, 64, 4)                                           \
    X(32, 256, 4) X(32, 128, 4) X(32, 64, 4)

// A+B-in-LDS ladder: (tile_m, tile_n, wave rows, wave columns, stages).
#define DG_AB_LADDER(X)                                                                 \
    X(256, 256, 2, 4, 2) X(256, 256, 2, 2, 2) X(256, 128, 2, 2, 3) X(128, 256, 2, 2, 3)  \
    X(128, 128, 2, 2, 3)

struct ABRung {
    int tm, tn, wm, wn, st;
};
constexpr ABRung kABLadder[] = {
#define DG_ABR(M_, N_, WM_, WN_, ST_) {M_, N_, WM_, WN_, ST_},
    DG_AB_LADDER(DG_ABR)
#undef DG_ABR
};

struct TiledRung {
    int tm, tn, waves;
};
constexpr TiledRung kTiledLadder[] = {
#define DG_RUNG(M_, N_, W_) {M_, N_, W_},
    DG_TILED_LADDER(DG_RUNG)
#undef DG_RUNG
};
constexpr int kSkinnyTM[] = {16, 32, 48, 64};
constexpr int kSkinnyTN[] = {16, 32, 64};

bool tiled_supported(int tm, int tn, int waves);
bool ab_supported(int tm, int tn, int waves);
bool skinny_supported(int tm, int tn);

// Launchers: return hipSuccess or the launch error.  Grids are computed from
// the arguments; shapes are validated by the caller.
hipError_t launch_tiled(int dt, int tm, int tn, int waves, const GemmArgs& a, hipStream_t s);
hipError_t launch_tiled_bf16(int tm, int tn, int waves, const GemmArgs& a, hipStream_t s);
hipError_t launch_tiled_fp8(int tm, int tn, int waves, const GemmArgs& a, hipStream_t s);
hipError_t launch_ab(int dt, int tm, int tn, int waves, const GemmArgs& a, hipStream_t s);
hipError_t launch_ab_bf16(int tm, int tn, int waves, const GemmArgs& a, hipStream_t s);
hipError_t launch_ab_fp8(int tm, int tn, int waves, const GemmArgs& a, hipStream_t s);
hipError_t launch_skinny(int dt, int tm, int tn, const GemmArgs& a, hipStream_t s);
hipError_t launch_zero_c(uint16_t* C, int64_t ldc, int64_t M, int64_t N, hipStream_t s);
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
int tiled_lds_bytes(int tm, int tn, int waves);
int ab_lds_bytes(int tm, int tn, int waves);
int tiled_vgpr_estimate(int tm, int tn, int waves);

}  // namespace dg
