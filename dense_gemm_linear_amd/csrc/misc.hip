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

// ---------------------------------------------------------------------------
// Transposes through LDS, for the backward GEMMs: dX = dY W needs B = W^T
// preshuffled (shuffle_b_t), dW = dY^T X needs A = dY^T (transpose_2d) and
// B = X^T preshuffled (shuffle_b_t).  A workgroup of 256 threads moves one
// 64 x 64 tile: it reads 64 source rows along their contiguous axis
// (consecutive lanes, consecutive elements), writes them into LDS with the
// axes swapped (rows padded by one element so a column walk spreads over the
// banks), and writes out along the other axis.  Elements past the source
// edges read as zero.
// vec: the source base and row pitch are 16-byte aligned; a tile wholly
// inside the source then moves in 16-byte pieces (two or one per thread),
// all issued before any is used, others element by element.
template <typename T>
__device__ __forceinline__ void load_tile_swapped(const T* src, int64_t ld, int64_t rows,
                                                  int64_t cols, int64_t r0, int64_t c0,
                                                  T (*t)[65], bool vec)
{
    const int tid = threadIdx.x;
    constexpr int CH = 16 / (int)sizeof(T);          // elements per 16-byte piece
    constexpr int PER = 64 * 64 / CH / 256;          // pieces per thread
    if (vec && r0 + 64 <= rows && c0 + 64 <= cols) {
        i32x4 v[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int q = tid + 256 * k;
            const int r = q / (64 / CH), cp = q % (64 / CH);
            v[k] = *reinterpret_cast<const i32x4*>(src + (r0 + r) * ld + c0 + cp * CH);
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int q = tid + 256 * k;
            const int r = q / (64 / CH), cp = q % (64 / CH);
            T e[CH];
            __builtin_memcpy(e, &v[k], 16);
#pragma unroll
            for (int j = 0; j < CH; ++j)
                t[cp * CH + j][r] = e[j];                    // t[col][row]
        }
    } else {
        const int c = tid & 63;
        for (int i = tid >> 6; i < 64; i += 4) {
            const int64_t r = r0 + i, cc = c0 + c;
            t[c][i] = (r < rows && cc < cols) ? src[r * ld + cc] : T(0);   // t[col][row]
        }
    }
    __syncthreads();
}

// dst[c][r] = src[r][c]; grid (col tiles, row tiles).
// vec_src / vec_dst: base and pitch 16-byte aligned (see load_tile_swapped).
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* src, int64_t ld_src, T* dst,
                                                        int64_t ld_dst, int64_t rows, int64_t cols,
                                                        int vec_src, int vec_dst)
{
    __shared__ T t[64][65];
    const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
    load_tile_swapped(src, ld_src, rows, cols, r0, c0, t, vec_src != 0);
    const int tid = threadIdx.x;
    constexpr int CH = 16 / (int)sizeof(T);
    constexpr int PER = 64 * 64 / CH / 256;
    if (vec_dst && r0 + 64 <= rows && c0 + 64 <= cols) {
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int q = tid + 256 * k;
            const int c = q / (64 / CH), rp = q % (64 / CH);   // dst row c0 + c
            T e[CH];
#pragma unroll
            for (int j = 0; j < CH; ++j)
                e[j] = t[c][rp * CH + j];
            *reinterpret_cast<i32x4*>(dst + (c0 + c) * ld_dst + r0 + rp * CH) =
                __builtin_bit_cast(i32x4, e);
        }
        return;
    }
    const int x = tid & 63;
    for (int i = tid >> 6; i < 64; i += 4) {
        const int64_t dr = c0 + i, dc = r0 + x;     // dst row = src column
        if (dr < cols && dc < rows)
            dst[dr * ld_dst + dc] = t[i][x];
    }
}

// shuffle_b of B [N, K] given its transpose Bt [K, N] (Bt[k][n] = B[n][k]):
// the tile of Bt at (k0e, n0e) holds B[n0e + n][k0e + k] at t[n][k] after the
// swap, and each thread writes whole 16-byte units of the preshuffled
// layout (the same units, in the same order within a 1 KiB block, as
// shuffle_b_kernel).  Grid (tiles over the 16-padded N, tiles over the
// 64-byte-padded K).
template <typename T>
__global__ __launch_bounds__(256) void shuffle_bt_kernel(const T* Bt, int64_t ldbt, uint8_t* Bs,
                                                         int64_t N, int64_t K, int64_t KB, int vec)
{
    __shared__ T t[64][65];
    constexpr int E = (int)sizeof(T);
    constexpr int KP = 16 / E;                 // elements per 16-byte unit
    const int64_t n0e = (int64_t)blockIdx.x * 64, k0e = (int64_t)blockIdx.y * 64;
    load_tile_swapped(Bt, ldbt, K, N, k0e, n0e, t, vec != 0);
    const int64_t nrows = (N + 15) / 16 * 16;
    constexpr int UNITS = 64 * 64 * E / 16;    // 16-byte units in the tile
    for (int q = threadIdx.x; q < UNITS; q += 256) {
        const int nl = q & 15, g = (q >> 4) & 3, rest = q >> 6;
        const int n_local = (rest & 3) * 16 + nl;
        const int k_local = (rest >> 2) * (64 / E) + g * KP;
        const int64_t n = n0e + n_local;
        const int64_t kbyte = (k0e + k_local) * E;
        if (n >= nrows || kbyte >= KB * 64)
            continue;
        T v[KP];
#pragma unroll
        for (int j = 0; j < KP; ++j)
            v[j] = t[n_local][k_local + j];
        const int64_t u = (((n >> 4) * KB + (kbyte >> 6)) * 4 + ((kbyte >> 4) & 3)) * 16 + (n & 15);
        *reinterpret_cast<i32x4*>(Bs + u * 16) = __builtin_bit_cast(i32x4, v);
    }
}

hipError_t launch_transpose(const void* src, int64_t ld_src, void* dst, int64_t ld_dst,
                            int64_t rows, int64_t cols, int elem_bytes, hipStream_t s)
{
    const dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64));
    int vs = ((uintptr_t)src % 16 == 0) && (ld_src * elem_bytes) % 16 == 0;
    int vd = ((uintptr_t)dst % 16 == 0) && (ld_dst * elem_bytes) % 16 == 0;
    if (elem_bytes == 2) {
        const uint16_t* a = static_cast<const uint16_t*>(src);
        uint16_t* b = static_cast<uint16_t*>(dst);
        void* args[] = {&a, &ld_src, &b, &ld_dst, &rows, &cols, &vs, &vd};
        return hipLaunchKernel(reinterpret_cast<const void*>(&transpose_kernel<uint16_t>), grid,
                               dim3(256), args, 0, s);
    }
    const uint8_t* a = static_cast<const uint8_t*>(src);
    uint8_t* b = static_cast<uint8_t*>(dst);
    void* args[] = {&a, &ld_src, &b, &ld_dst, &rows, &cols, &vs, &vd};
    return hipLaunchKernel(reinterpret_cast<const void*>(&transpose_kernel<uint8_t>), grid,
                           dim3(256), args, 0, s);
}

hipError_t launch_shuffle_bt(const void* Bt, int64_t ldbt, uint8_t* Bs, int64_t N, int64_t K,
                             int elem_bytes, hipStream_t s)
{
    const int64_t KB = (K * elem_bytes + 63) / 64;
    const int64_t nrows = (N + 15) / 16 * 16;
    const dim3 grid((unsigned)((nrows + 63) / 64), (unsigned)((KB * 64 / elem_bytes + 63) / 64));
    int vec = ((uintptr_t)Bt % 16 == 0) && (ldbt * elem_bytes) % 16 == 0;
    if (elem_bytes == 2) {
        const uint16_t* a = static_cast<const uint16_t*>(Bt);
        void* args[] = {&a, &ldbt, &Bs, &N, &K, (void*)&KB, &vec};
        return hipLaunchKernel(reinterpret_cast<const void*>(&shuffle_bt_kernel<uint16_t>), grid,
                               dim3(256), args, 0, s);
    }
    const uint8_t* a = static_cast<const uint8_t*>(Bt);
    void* args[] = {&a, &ldbt, &Bs, &N, &K, (void*)&KB, &vec};
    return hipLaunchKernel(reinterpret_cast<const void*>(&shuffle_bt_kernel<uint8_t>), grid,
                           dim3(256), args, 0, s);
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

// Zeroes n 32-bit words (the stream-K tile counters) with vector stores; a
// kernel rather than hipMemsetAsync, so that a graph capturing the launch
// holds no memset node.
__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* p, int n)
{
    const int i = (int)(blockIdx.x * 256 + threadIdx.x);
    if (i < n)
        p[i] = 0u;
}

// Streaming-read probe (a measurement aid, not part of any GEMM): workgroup
// g XORs the 32-bit words of its contiguous share of the buffer, every lane
// keeping D 16-byte non-temporal loads in flight (the access pattern of the
// skinny kernel's weight stream, without its arithmetic), and each wave
// writes its XOR to its own slot.  No workgroup barrier and no LDS: a wave
// that is done leaves at once and frees its slot for the next workgroup's
// waves (measured on MI355X, 90 MB: a barrier before one store per
// workgroup cost 2.7 us, a shuffle reduction through LDS 2.3 us).  Its time
// is the floor under a kernel that must read the same bytes once.
template <int D>
__global__ __launch_bounds__(1024) void read_probe_kernel(const i32x4* buf, int64_t n16,
                                                         int64_t per16, uint32_t* out)
{
    const int64_t base = (int64_t)blockIdx.x * per16;
    const int64_t end = base + per16 < n16 ? base + per16 : n16;
    const int nt = (int)blockDim.x;
    i32x4 acc = {0, 0, 0, 0};
    for (int64_t i = base + threadIdx.x; i < end; i += (int64_t)nt * D) {
        i32x4 v[D];
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int64_t j = i + (int64_t)d * nt;
            v[d] = j < end ? __builtin_nontemporal_load(buf + j) : i32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int d = 0; d < D; ++d)
            acc ^= v[d];
    }
    // XOR over the wave: DPP moves within each row of 16 lanes (quad
    // permutations, then the half-row and row mirrors), then the four row
    // results read into scalars -- no LDS round trips on the way out
    int x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    x ^= __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
    x ^= __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
    x ^= __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);   // row_half_mirror
    x ^= __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false);   // row_mirror
    x = __builtin_amdgcn_readlane(x, 0) ^ __builtin_amdgcn_readlane(x, 16) ^
        __builtin_amdgcn_readlane(x, 32) ^ __builtin_amdgcn_readlane(x, 48);
    // 16 slots per workgroup whatever its size: wave w owns 16 / waves of
    // them, its XOR in the first and zeros in the others
    const int per = 16 / (nt / 64);
    const int lane = (int)threadIdx.x & 63;
    if (lane < per)
        out[(int64_t)blockIdx.x * 16 + (threadIdx.x >> 6) * per + lane] = lane == 0 ? (uint32_t)x : 0u;
}

// grid workgroups; out holds grid * 16 slots, all of them written.
hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* out, int grid, hipStream_t s)
{
    int64_t n16 = bytes / 16;
    int64_t per16 = (n16 + grid - 1) / grid;
    const i32x4* b = static_cast<const i32x4*>(buf);
    void* args[] = {&b, &n16, &per16, &out};
    // measured on MI355X: 256 threads with 4 loads each in flight up to a
    // few tens of MB, 1024 threads with 8 each beyond
    if (bytes >= (64ll << 20))
        return hipLaunchKernel(reinterpret_cast<const void*>(&read_probe_kernel<8>), dim3((unsigned)grid),
                               dim3(1024), args, 0, s);
    return hipLaunchKernel(reinterpret_cast<const void*>(&read_probe_kernel<4>), dim3((unsigned)grid),
                           dim3(256), args, 0, s);
}

hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t s)
{
    if (n <= 0)
        return hipSuccess;
    void* args[] = {&p, &n};
    return hipLaunchKernel(reinterpret_cast<const void*>(&zero_u32_kernel),
                           dim3((unsigned)((n + 255) / 256)), dim3(256), args, 0, s);
}

// Split-K reduction.  ws holds `splits` fp32 partial planes [M][ldw]; the
// output is C[m][n] = bf16_rne(sum over s of ws[s][m][n]) with the planes
// added in increasing s, a fixed order, so the result does not depend on
// which workgroup of the GEMM finished first; e4m3 products are then scaled
// as (x * sa) * sb, as in the one-pass epilogue.  One thread per 4
// consecutive columns of one row; planes are read with 16-byte loads, eight
// at a time in flight before any is added (48 x 4096 x 4096 in six slices,
// measured on MI355X: 14.0-14.2 -> 13.6 us for the whole GEMM).
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
    float scale_a = 1.f, scale_b = 1.f;
    if (sa) {
        scale_a = *sa;
        scale_b = *sb;
    }
    constexpr int B = 8;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < splits; s0 += B) {
        f32x4 v[B];
#pragma unroll
        for (int j = 0; j < B; ++j)
            if (s0 + j < splits)
                v[j] = *reinterpret_cast<const f32x4*>(src + (int64_t)(s0 + j) * plane);
        // plane 0 starts the sum (so a -0 partial stays -0), the others are
        // added in increasing order
#pragma unroll
        for (int j = 0; j < B; ++j) {
            if (s0 + j >= splits)
                break;
            if (s0 + j == 0) {
                acc = v[0];
            } else {
                acc[0] += v[j][0];
                acc[1] += v[j][1];
                acc[2] += v[j][2];
                acc[3] += v[j][3];
            }
        }
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
