/*
 * densegemm -- dense linear-layer GEMM for AMD Instinct MI355X (gfx950).
 *
 * The operation is the forward GEMM of an LLM linear layer: Y = X * W^T with
 * the input flattened to X [M = batch * seq_len, K = d_model] and the weight
 * W [N = d_ff, K] in nn.Linear (row-major [out, in]) layout, so that
 *     C[m][n] = sum_k A[m][k] * B[n][k]
 * (TraceLens GEMM analysis page, "Linear layers in LLMs", "Flattening for
 * GEMM" and "Prefill versus decode": M = B*L for prefill, M = B for decode).
 * In BLAS terms this is the (T, N) call on (W, X) of that page's "Linear
 * layer" section; no BLAS is called here.
 *
 * Conventions shared by every entry point:
 *   - Pointers marked "device" must point to device memory of the current
 *     HIP device; the library never dereferences them on the host.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it and the call returns without synchronising.
 *     Faults inside a kernel surface at the caller's next synchronisation.
 *   - The caller owns every buffer.  The library allocates no device memory,
 *     keeps no per-call state and is safe to call from several host threads.
 *   - Errors are reported by return value; nothing throws across this ABI.
 *     Argument checks run before any HIP call, so invalid arguments are
 *     rejected without touching the device.
 *   - Matrices are row-major with unit stride in the last dimension; the
 *     leading dimension (lda, ldb, ldc) is in elements.  A non-unit inner
 *     stride is not representable: callers pass contiguous rows, and nothing
 *     is copied behind their back (TraceLens page, "Edge cases").
 */
#ifndef DENSEGEMM_H
#define DENSEGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_VALUE = 1, /* null pointer, negative size, bad leading dim, misalignment */
    GEMM_ERR_UNSUPPORTED = 2,   /* K granularity, forced tile infeasible, device not gfx950 */
    GEMM_ERR_HIP = 3            /* a HIP runtime call or kernel launch failed */
} gemm_status;

typedef enum {
    GEMM_BF16 = 0,     /* bfloat16 A and B, fp32 accumulation, bf16 C             */
    GEMM_FP8_E4M3 = 1  /* OCP e4m3 (max 448) A and B, fp32 accumulation, bf16 C  */
} gemm_dtype;

typedef enum {
    GEMM_KERNEL_TILED = 0,    /* block tiles, A pipelined through LDS, B straight to VGPRs */
    GEMM_KERNEL_SKINNY = 1,   /* M <= 64: B streamed once, waves split K, LDS reduction    */
    GEMM_KERNEL_TILED_AB = 2, /* block tiles, A and B both pipelined through LDS           */
    GEMM_KERNEL_TILED_PP = 3  /* A+B in LDS, 8 waves in two groups taking turns: one group  */
                              /* multiplies while the other moves the next k-tile           */
} gemm_kernel;

/*
 * One launch configuration.  Inputs to the kernels: kernel, tile_m, tile_n,
 * waves, atom, tile_k and lds_stages (and for the skinny kernel the rows and
 * columns only).  tile_eff, wq_eff and predicted_us are reported by
 * select_tile for information and ignored when a tile is forced.
 *
 * A forced tiled or A+B tile names one rung of a ladder by its fields; atom 0
 * means 16, and tile_k 0 or lds_stages 0 match the first rung that agrees
 * on the other fields.
 *
 *   tiled (A through LDS, B from the preshuffled layout straight into
 *   registers; waves 4 split tile_n, waves 8 form 2 x 4):
 *     16 x 16 atoms, 128-byte k-tiles: 256x128, 128x256, 128x128 with 8 waves
 *       and 2 stages; 256x128, 256x64, 128x256, 128x128, 128x64, 64x256,
 *       64x128, 64x64, 32x256, 32x128, 32x64 with 4 waves and 3 stages
 *       ("GEMM Optimization Guide" page, sections 1.1 and 1.4);
 *     32 x 32 atoms, 128-byte k-tiles: 256x256, 256x128, 128x256, 128x128
 *       with 8 waves and 2 stages; 256x128, 128x256, 128x128, 64x256, 64x128
 *       with 4 waves and 3 stages;
 *     32 x 32 atoms, 64-byte k-tiles, 4 waves, 4 stages: 128x256, 128x128,
 *       256x128.
 *   tiled_ab (A and B both through LDS; waves form 2 x waves/2):
 *     16 x 16, 128-byte k-tiles, 4 waves, 3 stages: 256x128, 128x256, 128x128;
 *     32 x 32, 128-byte k-tiles: 256x256 (8 or 4 waves, 2 stages), 256x128
 *       (8 or 4 waves, 3 stages), 128x256 and 128x128 (4 waves, 3 stages);
 *     32 x 32, 64-byte k-tiles: 256x256 with 8 or 4 waves and 4 stages, 256x128 with 8 waves and 6 stages, 128x256 with
 *       4 waves and 6 stages;
 *     16 x 16, 64-byte k-tiles (bf16 only): 256x256 with 8 waves and 4 stages.
 *   tiled_pp (8 waves; group g owns tile rows [g tile_m/2, (g+1) tile_m/2)):
 *     32 x 32: 256x256 with 4 stages of 64-byte k-tiles.
 *   16 x 16 e4m3 atoms need 128-byte k-tiles.
 *   skinny: tile_m in {16, 32, 48, 64} (rows of 16-row MFMA blocks covering
 *     M), tile_n in {16, 32, 64} (16-column blocks per workgroup), k_split
 *     = waves that split K in one workgroup: 4 for every (tile_m, tile_n),
 *     8 for tile_m, tile_n in {16, 32}, 16 for tile_m in {16, 32} with
 *     tile_n 16; k_split 0 means 4.
 *   split-K (tiled, tiled_ab, tiled_pp with k_split = S > 1): the grid is
 *     tiles x S workgroups; slice s multiplies k-tiles [s P, (s+1) P) with
 *     P = ceil(k-tiles / S), so S is lowered to ceil(k-tiles / P) when
 *     slices would be empty.  Each workgroup writes an fp32 partial tile to
 *     a caller workspace, and a second kernel adds the slices in increasing
 *     s (a fixed order: the result is the same on every run), scales (e4m3)
 *     and rounds to bf16.  It needs the *_ws entry points.
 */
/* Activation of the fused epilogue (see gemm_epilogue). */
typedef enum {
    GEMM_ACT_NONE = 0,
    GEMM_ACT_RELU = 1,       /* max(x, 0) */
    GEMM_ACT_SILU = 2,       /* x / (1 + exp(-x)) */
    GEMM_ACT_GELU_ERF = 3,   /* x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)) */
    GEMM_ACT_GELU_TANH = 4   /* x/2 * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3))) */
} gemm_activation;

/*
 * gemm_epilogue -- work fused into the GEMM's output stage (optional parts;
 * NULL / GEMM_ACT_NONE leave a part out).  For output element (m, n), after
 * the fp32 sum (and, for e4m3, its per-tensor scales sa, sb):
 *     v = v * scale_m[m]            per-row (per-token) fp32 multiplier
 *     v = v * scale_n[n]            per-column (per-channel) fp32 multiplier
 *     v = v + bias[n]               bf16 bias
 *     v = act(v)                    activation
 *     v = v * mul[m][n]             bf16 elementwise multiplier, e.g. the "up"
 *                                   projection for SiLU(gate) * up
 *     C[m][n] = bf16 round-to-nearest-even of v
 * all in fp32.  The Funlib GEMM page lists fused bias and activation as the
 * way to cut intermediate memory traffic (its feed-forward block applies
 * GELU between two GEMMs); the "GEMM Optimization Guide" page counts
 * per-token fp32 scales for M and N in its fp8 byte model (section 8.2); the
 * TraceLens GEMM page's GPT-3-XL table has an addmm with bias.
 *
 *   bias     device bf16 [N], 2-byte aligned
 *   scale_m  device fp32 [M], 4-byte aligned
 *   scale_n  device fp32 [N], 4-byte aligned
 *   mul      device bf16 [M, ld_mul], ld_mul >= N, 2-byte aligned; it may be
 *            C itself (same pointer and ld_mul == ldc: C = act(...) * C in
 *            place); any other overlap with C is undefined
 *   activation  a gemm_activation
 * All are read-only for the call and owned by the caller.
 */
typedef struct {
    const uint16_t* bias;
    const float* scale_m;
    const float* scale_n;
    const uint16_t* mul;
    int64_t ld_mul;
    int32_t activation;
} gemm_epilogue;

typedef struct {
    int32_t kernel;      /* gemm_kernel */
    int32_t tile_m;
    int32_t tile_n;
    int32_t tile_k;      /* elements of K per pipeline stage (k-tile); 0 = any */
    int32_t atom;        /* MFMA block edge: 16 or 32 (0 = 16) */
    int32_t waves;       /* waves per workgroup */
    int32_t k_split;     /* skinny: waves splitting K (0 = 4); tiled kernels: K slices
                            across workgroups (split-K, 0 or 1 = none, at most 64) */
    int32_t lds_stages;  /* k-tiles in the LDS ring (2 = ping-pong); 0 = any */
    float tile_eff;      /* M*N / (M_pad*N_pad) for the chosen tile */
    float wq_eff;        /* tiles / (ceil(tiles / CUs) * CUs) */
    float predicted_us;  /* cost model estimate (informational) */
    int32_t stream_k;    /* tiled / A+B rungs of 128 x 128 to 128 x 256 outputs, k_split <= 1:
                            1 = stream-K launch (see gemm_workspace_bytes); 0 = none */
} gemm_tile;

/*
 * select_tile -- choose a launch configuration for an M x N x K GEMM.
 *
 * Pure host function: deterministic, no device access unless num_cus == 0,
 * in which case the current device's compute-unit count is queried.  Weighs
 * tile quantization (padding) and wave quantization (last-round fill) as the
 * TraceLens page defines them ("GEMM dimension efficiency"), drops tiles that
 * pad the output past 1.25x its real area unless nothing else fits (FlyDSL
 * PR #1303 page, autotuner changes), checks the LDS and register budget
 * ("GEMM Optimization Guide" page, sections 2.4 and 10), and routes small M
 * to the skinny kernel.  Ties are broken by a fixed order.  The choice is
 * kept per (M, N, K, dtype, CU count, workspace bytes) in a table shared by
 * all threads (mutex-guarded, at most 4096 shapes, emptied when full), so a
 * repeated shape costs a lookup instead of pricing the ladder.
 *
 * Returns GEMM_ERR_INVALID_VALUE for out == NULL or negative sizes,
 * GEMM_ERR_HIP when num_cus == 0 and the device query fails.
 */
gemm_status select_tile(int64_t M, int64_t N, int64_t K, gemm_dtype dtype, int32_t num_cus,
                        gemm_tile* out);

/*
 * select_tile_ws -- select_tile, also weighing split-K variants of the tiled
 * rungs whose fp32 partials fit in workspace_bytes (0: none, the same choice
 * as select_tile).  Split-K is considered only when the output has fewer
 * tiles than the device has CUs: the TraceLens page leaves Split-K and
 * Stream-K out of its dimension-efficiency model ("Important
 * considerations"), and the FlyDSL PR #1303 page routes shapes that cannot
 * keep the CUs busy to a separate fallback; here the K slices fill the idle
 * CUs.  Errors as for select_tile.
 */
gemm_status select_tile_ws(int64_t M, int64_t N, int64_t K, gemm_dtype dtype, int32_t num_cus,
                           size_t workspace_bytes, gemm_tile* out);

/*
 * gemm_workspace_bytes -- device workspace the *_ws entry points need to run
 * `tile` on M x N x K: S * M * ldw * 4 bytes for a split-K tile (S slices
 * after lowering, ldw = N rounded up to 4); for a stream-K tile
 * (tile->stream_k = 1) two fp32 partial tiles per workgroup of a grid of at
 * most GEMM_STREAM_K_MAX_GRID workgroups plus one 32-bit counter per
 * stream-K tile (rounded up to 256 bytes); 0 for any other tile.  Returns 0
 * for tile == NULL, sizes <= 0, a tile that names no rung, or a stream-K
 * tile the shape cannot use (fewer k-tile units than workgroups).  Host only.
 *
 * Stream-K (the TraceLens GEMM analysis page lists Stream-K among what its
 * tile/wave-quantization model leaves out): a persistent grid of one
 * workgroup per CU (at most GEMM_STREAM_K_MAX_GRID).  When the tiles fill
 * two or more rounds, all but the last full round and the stray one run as
 * whole tiles, workgroup g taking every G-th; the (tile, k-tile) units of the
 * remaining tiles are cut into G equal contiguous ranges.  A tile cut
 * between workgroups is finished by the last of them to arrive, which adds
 * the fp32 partials in k order -- results are bitwise repeatable -- and
 * applies the epilogue.  No workgroup waits on another.  The fused epilogue
 * (gemm_epilogue) is not offered with stream-K.
 */
#define GEMM_STREAM_K_MAX_GRID 256
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, gemm_dtype dtype,
                            const gemm_tile* tile);

/*
 * shuffle_b_bytes -- size in bytes of the preshuffled weight for N x K.
 *
 * Layout ("GEMM Optimization Guide" page, sections 1.4 and 12.1, read in
 * bytes): [ceil(N/16)][Kp/kb][4][16][kp] elements, kp = 16 / element_bytes
 * (16 bytes, one 16-byte load per lane), kb = 4 * kp (64 bytes of K), Kp = K
 * rounded up to kb.  For e4m3 this is exactly (N/16, K/64, 4, 16, 16); for
 * bf16 (N/16, K/32, 4, 16, 8).  Returns 0 for negative sizes.
 */
size_t shuffle_b_bytes(int64_t N, int64_t K, gemm_dtype dtype);

/*
 * shuffle_b -- rewrite a row-major weight B [N, ldb] (device, bf16 bits or
 * e4m3 codes) into the preshuffled layout Bs (device, shuffle_b_bytes(N, K)
 * bytes, 16-byte aligned):
 *     Bs[n0][k0][g][nl][j] = B[16*n0 + nl][kb*k0 + kp*g + j]
 * with zero in every position whose row is >= N or whose column is >= K.
 * One memory-bound kernel; done once per weight and reused by every GEMM call
 * (page section 12.2).  The "16" index is the MFMA column a lane holds and
 * the "4" index the lane group, so a 64-lane wave reads one contiguous 1 KiB
 * block per load.
 *
 * Errors: INVALID_VALUE for null pointers with N, K > 0, negative sizes,
 * ldb < K, Bs not 16-byte aligned; UNSUPPORTED when K is not a multiple of 16
 * (bf16) or 64 (e4m3); HIP on launch failure.  N == 0 or K == 0: no work.
 */
gemm_status shuffle_b(const void* B, int64_t ldb, void* Bs, int64_t N, int64_t K, gemm_dtype dtype,
                      void* stream);

/*
 * shuffle_b_t -- shuffle_b of B [N, K] given its transpose: Bt is row-major
 * [K, ldbt] (device, ldbt >= N, element-aligned), element (k, n) being
 * B[n][k].  Writes exactly the Bs that shuffle_b(B) writes.  It serves the
 * backward GEMMs of a linear layer Y = X W^T ("TraceLens GEMM analysis"
 * page, backward pass and the GPT-3-XL table): dX = dY W is C = A B^T with
 * A = dY and B = W^T, so Bs = shuffle_b_t(W); dW = dY^T X takes B = X^T,
 * Bs = shuffle_b_t(X) (with A = dY^T from transpose_2d).  One memory-bound
 * kernel that transposes 64 x 64 tiles through LDS.
 *
 * Errors as for shuffle_b, with ldbt < N -> INVALID_VALUE.
 */
gemm_status shuffle_b_t(const void* Bt, int64_t ldbt, void* Bs, int64_t N, int64_t K,
                        gemm_dtype dtype, void* stream);

/*
 * transpose_2d -- dst[c][r] = src[r][c] for r < rows, c < cols: src row-major
 * [rows, ld_src], dst row-major [cols, ld_dst] (device, element-aligned,
 * ld_src >= cols, ld_dst >= rows, not overlapping); elem_bytes 1 (e4m3) or 2
 * (bf16).  The weight-gradient GEMM dW = dY^T X contracts over tokens, the
 * strided dimension of both dY and X; the A operand must have K contiguous,
 * so dY is transposed first.  Memory-bound, 64 x 64 tiles through LDS.
 *
 * Errors: INVALID_VALUE (negative sizes, null pointers with work, pitches,
 * misalignment, elem_bytes), UNSUPPORTED (more than 65535 x 64 rows), HIP.
 * rows == 0 or cols == 0: no work.
 */
gemm_status transpose_2d(const void* src, int64_t ld_src, void* dst, int64_t ld_dst, int64_t rows,
                         int64_t cols, int32_t elem_bytes, void* stream);

/*
 * gemm_bf16 -- C[m][n] = bf16( sum_k A[m][k] * B[n][k] ), fp32 accumulation,
 * C overwritten (no alpha/beta, no bias).
 *
 *   A   device, bf16 bits, row-major [M, lda], lda >= K, base 16-byte aligned,
 *       lda * 2 a multiple of 16 bytes.
 *   Bs  device, the weight B [N, K] preshuffled by shuffle_b(..., GEMM_BF16).
 *   C   device, bf16 bits, row-major [M, ldc], ldc >= N, 2-byte aligned; only
 *       the M x N region is written (columns N..ldc-1 are untouched).
 *   tile  NULL = select_tile(M, N, K, GEMM_BF16, <device CUs>), or the two
 *         launches over column or row ranges gemm_plan describes when that tile
 *         would leave a nearly empty last round; otherwise a forced
 *         configuration, validated against the shape (always one launch).
 *
 * The fp32 sum is rounded to bf16 to nearest, ties to even ("GEMM
 * Optimization Guide" page, section 7.1, direct-store epilogue: the
 * accumulator is truncated to the output type).  Ragged M and N are served by
 * buffer descriptors bounded at the real rows (loads past them read zero,
 * stores past them are dropped) and a column predicate on the C store
 * (FlyDSL PR #1303 page).
 *
 * Errors: INVALID_VALUE (null pointer with M, N > 0; negative size; lda < K;
 * ldc < N; misalignment), UNSUPPORTED (K % 16 != 0; infeasible forced tile;
 * device is not gfx950; a row offset that does not fit 31 bits), HIP.
 * M == 0 or N == 0: GEMM_OK, no launch.  K == 0: C := 0 (empty sum); A and
 * Bs are not read then and may be NULL (no alignment or lda requirement).
 */
gemm_status gemm_bf16(const uint16_t* A, int64_t lda, const void* Bs, uint16_t* C, int64_t ldc,
                      int64_t M, int64_t N, int64_t K, const gemm_tile* tile, void* stream);

/*
 * gemm_fp8_scaled -- C[m][n] = bf16( (sum_k a[m][k] * b[n][k]) * sa * sb ).
 *
 * a, b are OCP e4m3 codes; sa, sb the per-tensor fp32 dequant multipliers,
 * each one float in device memory (so a graph can replay with new scales).
 * The epilogue multiplies the fp32 accumulator by sa, then by sb, in fp32,
 * and rounds to bf16 to nearest even ("GEMM Optimization Guide" page,
 * section 7.1).
 *
 *   A   device, e4m3 [M, lda], lda >= K, base 16-byte aligned, lda % 16 == 0.
 *   Bs  device, shuffle_b(..., GEMM_FP8_E4M3) of B [N, K]: (N/16, K/64, 4, 16, 16).
 *   C   as for gemm_bf16.
 *
 * Errors as for gemm_bf16 with K % 64 != 0 -> UNSUPPORTED and null scale
 * pointers (K > 0) -> INVALID_VALUE.
 */
gemm_status gemm_fp8_scaled(const uint8_t* A, int64_t lda, const void* Bs, const float* scale_a,
                            const float* scale_b, uint16_t* C, int64_t ldc, int64_t M, int64_t N,
                            int64_t K, const gemm_tile* tile, void* stream);

/*
 * gemm_bf16_ws / gemm_fp8_scaled_ws -- gemm_bf16 / gemm_fp8_scaled with a
 * caller-owned device workspace for split-K (see gemm_tile).
 *
 *   workspace        device, 16-byte aligned, workspace_bytes long; NULL
 *                    allowed with workspace_bytes == 0.  Its contents on
 *                    entry are ignored and on return are unspecified; calls
 *                    that share one workspace must not overlap in time.
 *   tile             NULL = select_tile_ws(..., workspace_bytes, ...) (or
 *                    gemm_plan's two launches, as for gemm_bf16); forced
 *                    split-K tiles need gemm_workspace_bytes(tile).
 *
 * The product is the same as without split-K up to fp32 summation order:
 * slice partials are fp32 and are added in a fixed order, so a given tile
 * gives bitwise identical results on every run.  Two kernels are launched
 * on `stream` (the GEMM, then the reduction); the library allocates nothing.
 *
 * Errors as for gemm_bf16 / gemm_fp8_scaled, plus INVALID_VALUE when
 * workspace_bytes > 0 and workspace is NULL or not 16-byte aligned, or a
 * forced split-K tile needs more than workspace_bytes (> 0); UNSUPPORTED when
 * it needs a workspace and workspace_bytes == 0 (as the plain entry points
 *  answer for such a tile) or (M + 256) * ldw * 4 bytes exceed 2 GiB.
 */
gemm_status gemm_bf16_ws(const uint16_t* A, int64_t lda, const void* Bs, uint16_t* C, int64_t ldc,
                         int64_t M, int64_t N, int64_t K, const gemm_tile* tile, void* workspace,
                         size_t workspace_bytes, void* stream);
gemm_status gemm_fp8_scaled_ws(const uint8_t* A, int64_t lda, const void* Bs,
                               const float* scale_a, const float* scale_b, uint16_t* C,
                               int64_t ldc, int64_t M, int64_t N, int64_t K,
                               const gemm_tile* tile, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * gemm_bf16_ex / gemm_fp8_scaled_ex -- the *_ws entry points with a fused
 * epilogue (gemm_epilogue; NULL = none, the same as *_ws).  K == 0 gives
 * C = bf16(epilogue(0)).
 *
 * Errors as for *_ws, plus INVALID_VALUE for an activation outside
 * gemm_activation, misaligned epilogue pointers, mul with ld_mul < N or a row
 * pitch above 4 MiB.
 */
gemm_status gemm_bf16_ex(const uint16_t* A, int64_t lda, const void* Bs, uint16_t* C, int64_t ldc,
                         int64_t M, int64_t N, int64_t K, const gemm_tile* tile,
                         const gemm_epilogue* epilogue, void* workspace, size_t workspace_bytes,
                         void* stream);
gemm_status gemm_fp8_scaled_ex(const uint8_t* A, int64_t lda, const void* Bs,
                               const float* scale_a, const float* scale_b, uint16_t* C,
                               int64_t ldc, int64_t M, int64_t N, int64_t K,
                               const gemm_tile* tile, const gemm_epilogue* epilogue,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * gemm_bf16_noalloc -- gemm_bf16_ws for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The split-K workspace is a fixed array of
 * GEMM_NOALLOC_SCRATCH_BYTES bytes inside the library (one per GPU, held
 * until the process ends); the call allocates nothing and calls no
 * allocating routine.
 *
 *   Arguments as for gemm_bf16; tile NULL = select_tile_ws(...,
 *   GEMM_NOALLOC_SCRATCH_BYTES, ...) (or gemm_plan's two launches).
 *
 * Every call on one GPU shares that GPU's array, and the array keeps the
 * last call's contents (nothing in it needs to start at zero: every split-K
 * slice writes its whole partial plane before the reduction reads it).
 * Calls that overlap in time on one GPU -- concurrent streams, or several
 * host threads -- race on it and must be serialised by the caller.  The
 * first call on a device looks up that device's copy of the array
 * (hipGetSymbolAddress); make it outside graph capture.
 *
 * Errors as for gemm_bf16_ws, with INVALID_VALUE when a forced split-K tile
 * needs more than GEMM_NOALLOC_SCRATCH_BYTES (gemm_workspace_bytes), and
 * GEMM_ERR_HIP when the array's address cannot be obtained.
 */
#define GEMM_NOALLOC_SCRATCH_BYTES (32u << 20)
gemm_status gemm_bf16_noalloc(const uint16_t* A, int64_t lda, const void* Bs, uint16_t* C,
                              int64_t ldc, int64_t M, int64_t N, int64_t K, const gemm_tile* tile,
                              void* stream);

/*
 * gemm_plan -- the launches gemm_bf16 / gemm_fp8_scaled (and their _ws / _ex
 * forms with `workspace_bytes`) make for an M x N x K GEMM when the caller
 * passes tile == NULL, on a device with num_cus compute units.  Pure host
 * function, no device access.
 *
 * Usually one launch: *first = select_tile_ws(...), *first_columns = N,
 * *first_rows = M and *second zeroed.  When the chosen one-pass tiled tile
 * would run two or more
 * full rounds of tiles over the CUs and then a last round that fills at most
 * a quarter of them (wave quantization, TraceLens GEMM analysis page), the
 * columns [0, *first_columns) that fill whole rounds run with *first and the
 * rest as a second GEMM with *second, chosen for that narrower shape -- if
 * its cost, at least about 6 us, is below 40 % of one round's, what such a
 * stray round measured on MI355X.  Both launches are enqueued on the caller's
 * stream, in that order; the outputs they write are disjoint.
 *
 * Otherwise, when a 256 x 256, 256 x 128 or 128 x 256 tile's column count
 * divides the CUs and the rows [0, *first_rows) make whole rounds of such
 * tiles, those rows may run with *first (that tile, chosen for them) and the
 * rows [*first_rows, M) as a second GEMM with *second, if the model prices
 * the pair, plus 3 us for the second launch's start, below 95 % of the single
 * launch.  Measured on MI355X for the GPT-3-XL input gradient 10240 x 2048 x
 * 8192: 302 us as one launch, 270 us as 8192 + 2048 rows.  At most one of
 * *first_columns < N and *first_rows < M.
 *
 * When the chosen one-pass tile (a stream-K rung) fills less than one round
 * of the CUs and the workspace holds its stream-K partials, *first is its
 * stream-K form (stream_k = 1) if the model prices that below 95 % of the
 * one-pass launch: the one-pass time scaled by tiles / CUs and by 1.45 (a
 * stream-K unit measured that much slower than a one-pass one), plus about
 * 20 us for the fix-up of the cut tiles.  The launch with a fused epilogue
 * (gemm_*_ex with any part set) keeps the one-pass form.  It also runs on the
 * 8-wave rung of the same tile when *first would be the 4-wave e4m3
 * 256 x 256 rung with 32 x 32 atoms and four 64-byte stages, whose fused
 * instance spills registers (measured on MI355X, e4m3 4096^3 with per-row
 * and per-column scales: 66-69 us against 58-60 us).
 *
 * GEMM_ERR_INVALID_VALUE for a NULL output, M, N or K <= 0, num_cus <= 0 or
 * an unknown dtype.
 */
gemm_status gemm_plan(int64_t M, int64_t N, int64_t K, gemm_dtype dtype, int32_t num_cus,
                      size_t workspace_bytes, gemm_tile* first, gemm_tile* second,
                      int64_t* first_columns, int64_t* first_rows);

/*
 * gemm_tile_check -- would `tile`, forced on gemm_bf16 (dtype GEMM_BF16) or
 * gemm_fp8_scaled (GEMM_FP8_E4M3) with M rows, name a rung the library has?
 * Pure host function, no device access.  GEMM_OK if so, GEMM_ERR_UNSUPPORTED
 * if not, GEMM_ERR_INVALID_VALUE for tile == NULL, M < 0 or an unknown dtype.
 */
gemm_status gemm_tile_check(const gemm_tile* tile, int64_t M, gemm_dtype dtype);

/*
 * gemm_read_probe -- a measurement aid, not a step of the GEMM: reads the
 * `bytes` bytes of device memory at `buf` once, the way the skinny kernel
 * streams a decode weight (16-byte non-temporal loads, several in flight per
 * lane, no arithmetic but an XOR), so that its duration is the floor under
 * any kernel that reads those bytes on this device (the HBM-bound rows of
 * the "TraceLens GEMM analysis" page, "Prefill versus decode": a decode GEMM
 * is a weight read).  Every wave writes the XOR of the 32-bit words it read
 * to a slot of its own and zeros to the slots no wave owns, so the XOR of
 * all GEMM_READ_PROBE_SLOTS values of out is the XOR of every word of the
 * buffer.
 *   buf    device memory, 16-byte aligned; not written
 *   bytes  a positive multiple of 16, at most 2^40
 *   out    device memory for GEMM_READ_PROBE_SLOTS uint32 values (written)
 * GEMM_ERR_INVALID_VALUE for a null pointer, a misaligned buf or a bad size;
 * GEMM_ERR_HIP if the launch fails.  Asynchronous on `stream`.
 */
#define GEMM_READ_PROBE_SLOTS 32768
gemm_status gemm_read_probe(const void* buf, uint64_t bytes, uint32_t* out, void* stream);

/* Static, human-readable name of a status code ("GEMM_OK", ...). */
const char* gemm_status_string(gemm_status status);

#ifdef __cplusplus
}
#endif

#endif /* DENSEGEMM_H */
