// Host-side declarations shared by the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/densegemm.h"
#include "kernels.hpp"

namespace dg {

// Tile ladders the kernels are instantiated for.
constexpr int kTiledTM[] = {256, 128, 64, 32};
constexpr int kTiledTN[] = {256, 128, 64};
constexpr int kSkinnyTM[] = {16, 32, 48, 64};
constexpr int kSkinnyTN[] = {16, 32, 64};

bool tiled_supported(int tm, int tn);
bool skinny_supported(int tm, int tn);

// Launchers: return hipSuccess or the launch error.  Grids are computed from
// the arguments; shapes are validated by the caller.
hipError_t launch_tiled(int dt, int tm, int tn, const GemmArgs& a, hipStream_t s);
hipError_t launch_tiled_bf16(int tm, int tn, const GemmArgs& a, hipStream_t s);
hipError_t launch_tiled_fp8(int tm, int tn, const GemmArgs& a, hipStream_t s);
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
int tiled_lds_bytes(int tm, int tn);
int tiled_vgpr_estimate(int tm, int tn);

}  // namespace dg
