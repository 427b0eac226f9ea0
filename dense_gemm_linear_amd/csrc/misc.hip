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

// K == 0: the empty sum is 0; with an epilogue, C = bf16(epilogue(0)).
__global__ __launch_bounds__(256) void zero_c_kernel(uint16_t* C, int64_t ldc, int64_t M, int64_t N,
                                                     Epilogue ep)
{
    const int64_t total = M * N;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t row = i / N, col = i % N;
        C[row * ldc + col] = ep.on ? bf16_rne(apply_epilogue(ep, 0.f, (int)row, (int)col)) : 0;
    }
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

hipError_t launch_zero_c(uint16_t* C, int64_t ldc, int64_t M, int64_t N, Epilogue ep, hipStream_t s)
{
    int64_t blocks = (M * N + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    void* args[] = {&C, &ldc, &M, &N, &ep};
    return hipLaunchKernel(reinterpret_cast<const void*>(&zero_c_kernel), dim3((unsigned)blocks),
                           dim3(256), args, 0, s);
}

// Split-K reduction.  ws holds `splits` fp32 partial planes [M][ldw]; the
// output is C[m][n] = bf16_rne(sum over s of ws[s][m][n]) with the planes
// added in increasing s, a fixed order, so the result does not depend on
// which workgroup of the GEMM finished first; e4m3 products are then scaled
// as (x * sa) * sb, as in the one-pass epilogue.  One thread per 4
// consecutive columns of one row; planes are read with 16-byte loads.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* ws, int splits, int M,
                                                            int N, int ldw, uint16_t* C,
                                                            int64_t ldc, const float* sa,
                                                            const float* sb, Epilogue ep)
{
    const int q = ldw >> 2;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (int64_t)M * q)
        return;
    const int row = (int)(t / q);
    const int c0 = (int)(t - (int64_t)row * q) * 4;
    const int64_t plane = (int64_t)M * ldw;
    const float* src = ws + (int64_t)row * ldw + c0;
    f32x4 acc = *reinterpret_cast<const f32x4*>(src);
    for (int s = 1; s < splits; ++s) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(src + s * plane);
        acc[0] += v[0];
        acc[1] += v[1];
        acc[2] += v[2];
        acc[3] += v[3];
    }
    float scale_a = 1.f, scale_b = 1.f;
    if (sa) {
        scale_a = *sa;
        scale_b = *sb;
    }
    uint16_t h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float v = acc[e];
        if (sa)
            v = (v * scale_a) * scale_b;
        if (ep.on)
            v = apply_epilogue(ep, v, row, min(c0 + e, N - 1));
        h[e] = bf16_rne(v);
    }
    uint16_t* dst = C + (int64_t)row * ldc + c0;
    if (c0 + 4 <= N && ((uintptr_t)dst & 7u) == 0) {
        const uint2 w = {(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
        *reinterpret_cast<uint2*>(dst) = w;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (c0 + e < N)
                dst[e] = h[e];
    }
}

hipError_t launch_splitk_reduce(const float* ws, int splits, int M, int N, int ldw, uint16_t* C,
                                int64_t ldc, const float* sa, const float* sb, Epilogue ep,
                                hipStream_t s)
{
    const int64_t threads = (int64_t)M * (ldw / 4);
    const int64_t blocks = (threads + 255) / 256;
    void* args[] = {&ws, &splits, &M, &N, &ldw, &C, &ldc, &sa, &sb, &ep};
    return hipLaunchKernel(reinterpret_cast<const void*>(&splitk_reduce_kernel),
                           dim3((unsigned)blocks), dim3(256), args, 0, s);
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
