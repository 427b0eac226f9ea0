// Device primitives for gfx950 (CDNA4): buffer resources, 16-byte buffer
// loads/stores, MFMA wrappers and the bf16 rounding used by the epilogues.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Word 3 of a gfx9-family buffer resource: untyped 32-bit data, no swizzle,
// offset ("raw") addressing.  A load whose offset lies at or past num_records
// returns zero and a store there is dropped: this is how rows past M, blocks
// past N and the K tail read as zeros without a branch in the loop (FlyDSL
// PR #1303 page: the A and C descriptors are bounded at the real row count).
constexpr int kRsrcWord3 = 0x00020000;
// An offset that is out of range for every descriptor built here (all of
// them are smaller than 2^31 bytes).
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t num_bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes,
                                             kRsrcWord3);
}

__device__ __forceinline__ i32x4 load16(rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// The same with a scalar (wave-uniform) byte offset added to the per-lane
// one, for loads whose k-tile offset is the same in every lane.
__device__ __forceinline__ i32x4 load16_s(rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
}

// Cache policy of a buffer access that must be coherent across XCDs
// without whole-cache maintenance: sc0 | sc1 (gfx940-family bits 0 and 4),
// i.e. system scope -- stores write through the L2 to memory, loads miss in
// the L1 and L2.  For data handed between workgroups on different XCDs
// inside one kernel (the stream-K partials).
constexpr int kCpolCoherent = 0x11;

__device__ __forceinline__ void store16_coherent(rsrc_t r, uint32_t off, i32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kCpolCoherent);
}

__device__ __forceinline__ i32x4 load16_coherent(rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCpolCoherent);
}

// A 16-byte LDS DMA (global -> LDS, no register round trip): lane l's 16
// bytes land at lds_base + 16 l; m0 holds the wave-uniform lds_base.
__device__ __forceinline__ void dma16(rsrc_t r, void* lds_base, uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)lds_base, 16, (int)voff, (int)soff, 0, 0);
}

// The same with the non-temporal cache hint (bit 1 of the cache-policy
// operand, `nt` on gfx950), for data read exactly once: a decode weight
// streamed from HBM.  Measured on MI355X with cold operands, the skinny
// kernel's weight stream is 4-12 % faster with it.
__device__ __forceinline__ i32x4 load16_nt(rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2);
}

__device__ __forceinline__ void store16(rsrc_t r, uint32_t off, i32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}

__device__ __forceinline__ void store4(rsrc_t r, uint32_t off, uint32_t v)
{
    __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 0);
}

__device__ __forceinline__ void store2(rsrc_t r, uint32_t off, uint16_t v)
{
    __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)off, 0, 0);
}

// fp32 -> bf16 bits, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t bf16_rne(float f)
{
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] * B[32x16].  Lane l holds
// row (A) / column (B) l % 16 and the (l / 16)-th group of 8 K values; the
// result lane l holds column l % 16, rows 4*(l/16) .. 4*(l/16)+3.
__device__ __forceinline__ f32x4 mfma_bf16(i32x4 a, i32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// v_mfma_f32_16x16x128_f8f6f4 with both operands in e4m3 (format 0) and no
// block scales: D[16x16] += A[16x128] * B[128x16], 32 K bytes per lane.
__device__ __forceinline__ f32x4 mfma_fp8(i32x8 a, i32x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// v_mfma_f32_32x32x16_bf16: D[32x32] += A[32x16] * B[16x32].  Lane l holds
// row (A) / column (B) l % 32 and the (l / 32)-th group of 8 K values; the
// result lane l holds column l % 32 and, in element e, row
// 8*(e/4) + 4*(l/32) + e%4.
__device__ __forceinline__ f32x16 mfma_bf16_32(i32x4 a, i32x4 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// v_mfma_scale_f32_32x32x64_f8f6f4, e4m3 operands, no block scales:
// D[32x32] += A[32x64] * B[64x32], 32 K bytes per lane, lanes 32..63 holding
// the second half of K.  Output layout as for mfma_bf16_32.
__device__ __forceinline__ f32x16 mfma_fp8_32(i32x8 a, i32x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8 cat(i32x4 lo, i32x4 hi)
{
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

}  // namespace dg
