// Memory-bound helpers: the B preshuffle and the K == 0 fill.
#include "internal.hpp"

namespace dg {

// One thread per 16-byte unit u of the output, in output order:
//   u = ((n0 * KB + k0) * 4 + g) * 16 + nl
// holds row 16*n0 + nl, K bytes [64*k0 + 16*g, +16) of B, or zeros past N or
// past K ("GEMM Optimization Guide" page, section 12.1, read in bytes).
// Consecutive threads write consecutive 16 bytes.
__global__ __launch_bounds__(256) void shuffle_b_kernel(const uint8_t* B, int64_t ldb_b, uint8_t* Bs,
                                                        int64_t N, int64_t K_b, int64_t KB,
                                                        int64_t units, int aligned)
{
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= units)
        return;
    const int64_t nl = u & 15;
    const int64_t g = (u >> 4) & 3;
    const int64_t rest = u >> 6;
    const int64_t k0 = rest % KB;
    const int64_t n0 = rest / KB;
    const int64_t n = n0 * 16 + nl;
    const int64_t kbyte = k0 * 64 + g * 16;
    i32x4 v = {0, 0, 0, 0};
    if (n < N && kbyte < K_b) {
        const uint8_t* src = B + n * ldb_b + kbyte;
        if (aligned) {
            v = *reinterpret_cast<const i32x4*>(src);
        } else {
            uint8_t tmp[16];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                tmp[i] = src[i];
            v = __builtin_bit_cast(i32x4, tmp);
        }
    }
    *reinterpret_cast<i32x4*>(Bs + u * 16) = v;
}

__global__ __launch_bounds__(256) void zero_c_kernel(uint16_t* C, int64_t ldc, int64_t M, int64_t N)
{
    const int64_t total = M * N;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256)
        C[(i / N) * ldc + (i % N)] = 0;
}

hipError_t launch_shuffle_b(const uint8_t* B, int64_t ldb_b, uint8_t* Bs, int64_t N, int64_t K_b,
                            int64_t KB, int aligned, hipStream_t s)
{
    const int64_t units = (N + 15) / 16 * KB * 64;
    const int64_t blocks = (units + 255) / 256;
    void* args[] = {&B, &ldb_b, &Bs, &N, &K_b, &KB, (void*)&units, &aligned};
    return hipLaunchKernel(reinterpret_cast<const void*>(&shuffle_b_kernel), dim3((unsigned)blocks),
                           dim3(256), args, 0, s);
}

hipError_t launch_zero_c(uint16_t* C, int64_t ldc, int64_t M, int64_t N, hipStream_t s)
{
    int64_t blocks = (M * N + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    void* args[] = {&C, &ldc, &M, &N};
    return hipLaunchKernel(reinterpret_cast<const void*>(&zero_c_kernel), dim3((unsigned)blocks),
                           dim3(256), args, 0, s);
}

int ab_lds_bytes(int idx)
{
    int i = 0;
#define DG_CASE(M_, N_, WM_, WN_, ST_, R_, KTB_) \
    if (idx == i++) return ABShape<M_, N_, WM_, WN_, ST_, R_, KTB_>::LDS;
    DG_AB_LADDER(DG_CASE)
#undef DG_CASE
    return -1;
}

int pp_lds_bytes(int idx)
{
    int i = 0;
#define DG_CASE(M_, N_, ST_, R_, KTB_) \
    if (idx == i++) return ABShape<M_, N_, 2, 4, ST_, R_, KTB_>::LDS;
    DG_PP_LADDER(DG_CASE)
#undef DG_CASE
    return -1;
}

int tiled_lds_bytes(int idx)
{
    int i = 0;
#define DG_CASE(M_, N_, W_, ST_, R_, KTB_) \
    if (idx == i++) return TiledShape<M_, N_, W_ / 4, ST_, R_, KTB_>::LDS;
    DG_TILED_LADDER(DG_CASE)
#undef DG_CASE
    return -1;
}

}  // namespace dg
