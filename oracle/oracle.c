/*
 * Plain CPU oracle for the dense linear-layer GEMM C[M,N] = A[M,K] * B[N,K]^T.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library may link, call or
 * include this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or constant
 * with the GPU path.
 *
 * Every function is the plain definition of what it computes, written for a
 * reader to check by eye:
 *   - the GEMM is a triple loop with fp64 accumulation in ascending k
 *     ("TraceLens GEMM analysis" page, "Linear layers in LLMs" and "Flattening
 *     for GEMM": Y = X_flat * W^T with M = B*L, N = d_ff, K = d_model);
 *   - the fp8 variant multiplies the fp64 sum by the two per-tensor dequant
 *     scales ("GEMM Optimization Guide" page, section 7.1, where the epilogue
 *     value is the accumulator times scale_a times scale_b);
 *   - bf16 output rounding is round-to-nearest-even (section 7.1 truncates the
 *     fp32 value to the output type; the conversion is read as IEEE RNE);
 *   - the B preshuffle follows section 12.1 of the same page, read in bytes:
 *     (N/16, K/kpack, 4, 16, kpack) with kpack = 16 bytes, padded rows zero;
 *   - the fused epilogue (per-row / per-column scales, bias, activation,
 *     elementwise multiplier) is applied to the fp64 product in that order;
 *   - tile_eff / wq_eff / dim_eff follow the TraceLens page, "Tile quantization
 *     efficiency", "Wave quantization efficiency" and "How it's calculated".
 *
 * Built with -O2 -fno-fast-math -ffp-contract=off so that the fp64 loop is
 * evaluated exactly as written (no reassociation, no fused multiply-add).
 */
#ifndef M_PI
#define M_PI 3.14159265358979323846
#endif
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ codecs */

/* bf16 bits -> value.  A bf16 number is the upper half of an IEEE binary32. */
double orc_bf16_to_f64(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* value -> bf16 bits, round to nearest, ties to even, straight from fp64
 * (no intermediate rounding to binary32).  bf16 keeps 8 significant bits and
 * the binary32 exponent range: normal numbers have quantum 2^(E-7) for
 * 2^E <= |x| < 2^(E+1), subnormals share the quantum 2^-133.  Overflow after
 * rounding gives infinity; NaN gives the quiet NaN 0x7FC0 with the sign kept. */
uint16_t orc_bf16_from_f64(double x)
{
    uint32_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(x);
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0)
        return (uint16_t)sign;
    int ex;
    frexp(a, &ex);            /* a = f * 2^ex with f in [0.5, 1) */
    int E = ex - 1;           /* a = 1.m * 2^E                    */
    if (E < -126)
        E = -126;             /* subnormal range                  */
    double q = ldexp(1.0, E - 7);
    double r = nearbyint(a / q);   /* default rounding mode: ties to even */
    double v = r * q;
    if (v >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80u);
    float f = (float)v;            /* exact: v has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFFu));
}

/* OCP 8-bit float E4M3 ("FN": finite only): 1 sign, 4 exponent bits with bias
 * 7, 3 mantissa bits.  Exponent field 0 is subnormal (m/8 * 2^-6).  S.1111.111
 * is NaN, there is no infinity, so the largest finite value is 1.75 * 2^8 = 448. */
double orc_e4m3_to_f64(uint8_t c)
{
    int s = (c >> 7) & 1;
    int e = (c >> 3) & 0xF;
    int m = c & 7;
    double v;
    if (e == 0xF && m == 7)
        return s ? -NAN : NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* value -> E4M3 bits: round to nearest even, saturate to +-448, NaN -> 0x7F. */
uint8_t orc_e4m3_from_f64(double x)
{
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    if (isnan(x))
        return 0x7F;
    double a = fabs(x);
    if (a == 0.0)
        return sign;
    int ex;
    frexp(a, &ex);
    int E = ex - 1;
    if (E < -6)
        E = -6;                       /* subnormal quantum 2^-9 */
    double q = ldexp(1.0, E - 3);
    double v = nearbyint(a / q) * q;
    if (v > 448.0)
        v = 448.0;                    /* saturating conversion */
    /* encode the representable value v */
    if (v == 0.0)
        return sign;
    frexp(v, &ex);
    E = ex - 1;
    uint8_t code;
    if (E < -6) {                     /* subnormal: v = m/8 * 2^-6 */
        int m = (int)(v / ldexp(1.0, -9));
        code = (uint8_t)m;
    } else {
        int m = (int)((v / ldexp(1.0, E) - 1.0) * 8.0);
        code = (uint8_t)(((E + 7) << 3) | m);
    }
    return (uint8_t)(sign | code);
}

void orc_bf16_encode_array(const double *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_bf16_from_f64(x[i]);
}

void orc_bf16_decode_array(const uint16_t *h, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_bf16_to_f64(h[i]);
}

void orc_e4m3_encode_array(const double *x, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_e4m3_from_f64(x[i]);
}

void orc_e4m3_decode_array(const uint8_t *c, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_e4m3_to_f64(c[i]);
}

/* ------------------------------------------------------------------- GEMM */

enum { ORC_BF16 = 0, ORC_E4M3 = 1 };

typedef struct {
    int dtype;
    const void *A;
    int64_t lda;
    const void *B;
    int64_t ldb;
    int64_t M, N, K;
    double scale;          /* product of the two dequant scales (1 for bf16) */
    double *C;
    int64_t ldc;
    int64_t row0, row1;    /* this worker's rows of C */
    int64_t macs;          /* multiply-adds this worker performed */
} orc_job;

static double elem(int dtype, const void *p, int64_t i)
{
    if (dtype == ORC_BF16)
        return orc_bf16_to_f64(((const uint16_t *)p)[i]);
    return orc_e4m3_to_f64(((const uint8_t *)p)[i]);
}

/* C[m][n] = scale * sum_{k ascending} A[m][k] * B[n][k], all in fp64.
 * A is row-major [M, lda], B is the row-major weight [N, ldb] (nn.Linear
 * layout), so C = A * B^T. */
static void *gemm_rows(void *arg)
{
    orc_job *j = (orc_job *)arg;
    int64_t macs = 0;
    for (int64_t m = j->row0; m < j->row1; m++) {
        for (int64_t n = 0; n < j->N; n++) {
            double acc = 0.0;
            for (int64_t k = 0; k < j->K; k++) {
                double a = elem(j->dtype, j->A, m * j->lda + k);
                double b = elem(j->dtype, j->B, n * j->ldb + k);
                acc += a * b;
                macs++;
            }
            j->C[m * j->ldc + n] = acc * j->scale;
        }
    }
    j->macs = macs;
    return NULL;
}

/* Runs the row blocks on `threads` POSIX threads; returns the number of
 * multiply-adds performed (M*N*K when every row ran). */
static int64_t gemm_threads(orc_job base, int threads)
{
    if (threads < 1)
        threads = 1;
    if (threads > 256)
        threads = 256;
    if (base.M < threads)
        threads = base.M > 0 ? (int)base.M : 1;
    pthread_t tid[256];
    int spawned[256];
    orc_job jobs[256];
    int64_t per = (base.M + threads - 1) / threads;
    int started = 0;
    for (int t = 0; t < threads; t++) {
        jobs[t] = base;
        jobs[t].row0 = (int64_t)t * per;
        jobs[t].row1 = jobs[t].row0 + per < base.M ? jobs[t].row0 + per : base.M;
        if (jobs[t].row0 >= jobs[t].row1)
            break;
        spawned[t] = threads > 1 && pthread_create(&tid[t], NULL, gemm_rows, &jobs[t]) == 0;
        if (!spawned[t])
            gemm_rows(&jobs[t]);
        started++;
    }
    int64_t macs = 0;
    for (int t = 0; t < started; t++) {
        if (spawned[t])
            pthread_join(tid[t], NULL);
        macs += jobs[t].macs;
    }
    return macs;
}

/* bf16 inputs, fp64 result (unrounded).  Returns the multiply-add count. */
int64_t orc_gemm_bf16(const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                      int64_t M, int64_t N, int64_t K, double *C, int64_t ldc, int threads)
{
    orc_job j = {ORC_BF16, A, lda, B, ldb, M, N, K, 1.0, C, ldc, 0, M, 0};
    return gemm_threads(j, threads);
}

/* e4m3 inputs, per-tensor dequant scales, fp64 result (unrounded):
 * C = (sum a*b) * sa * sb. */
int64_t orc_gemm_e4m3(const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                      int64_t M, int64_t N, int64_t K, float sa, float sb,
                      double *C, int64_t ldc, int threads)
{
    orc_job j = {ORC_E4M3, A, lda, B, ldb, M, N, K, (double)sa * (double)sb, C, ldc, 0, M, 0};
    return gemm_threads(j, threads);
}

/* Selected outputs only: out[i] = scale * sum_k A[ms[i]][k] * B[ns[i]][k].
 * Used to check full-size GEMMs on a sample of positions. */
void orc_gemm_points(int dtype, const void *A, int64_t lda, const void *B, int64_t ldb,
                     int64_t K, double scale, const int64_t *ms, const int64_t *ns,
                     int64_t npts, double *out)
{
    for (int64_t i = 0; i < npts; i++) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; k++)
            acc += elem(dtype, A, ms[i] * lda + k) * elem(dtype, B, ns[i] * ldb + k);
        out[i] = acc * scale;
    }
}

/* --------------------------------------------------------------- transposes */

/* dst[c][r] = src[r][c] for r < rows, c < cols (elements of elem_bytes bytes;
 * row pitches in elements).  Used for the backward GEMMs of a linear layer
 * ("TraceLens GEMM analysis" page, backward pass): dW = dY^T X has to see dY
 * with the token dimension contiguous. */
void orc_transpose(const uint8_t *src, int64_t ld_src, int64_t rows, int64_t cols, int elem_bytes,
                   uint8_t *dst, int64_t ld_dst)
{
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++)
            memcpy(dst + (c * ld_dst + r) * elem_bytes, src + (r * ld_src + c) * elem_bytes,
                   (size_t)elem_bytes);
}

/* ---------------------------------------------------------- fused epilogue */

/* Activations, each its textbook definition in fp64 (libm exp, erf, tanh):
 *   0 none; 1 ReLU max(x, 0); 2 SiLU x * logistic(x) = x / (1 + e^-x);
 *   3 GELU x * Phi(x) = x/2 (1 + erf(x / sqrt 2)), Phi the standard normal CDF
 *     (the GELU of the Funlib GEMM page's feed-forward block, read as the
 *     exact form);
 *   4 its tanh approximation x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))). */
double orc_activation(int act, double x)
{
    switch (act) {
    case 1:
        return x > 0.0 ? x : 0.0;
    case 2:
        return x / (1.0 + exp(-x));
    case 3:
        return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
    case 4:
        return 0.5 * x * (1.0 + tanh(sqrt(2.0 / M_PI) * (x + 0.044715 * x * x * x)));
    default:
        return x;
    }
}

/* The fused epilogue on an fp64 product C [M, N] (row-major, already times
 * the per-tensor e4m3 scales), in place, element by element in this order:
 *   v = C[m][n]; v *= scale_m[m]; v *= scale_n[n]; v += bias[n];
 *   v = act(v); v *= mul[m][n]
 * Every part is optional (NULL).  bias and mul are bf16 bits.  Readings: the
 * Funlib GEMM page names fused bias and activation; the "GEMM Optimization
 * Guide" page (section 8.2) counts fp32 per-token scales for both M and N;
 * the TraceLens GEMM page's addmm adds a bias per output column. */
void orc_epilogue(double *C, int64_t M, int64_t N, const float *scale_m, const float *scale_n,
                  const uint16_t *bias, int act, const uint16_t *mul, int64_t ld_mul)
{
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            double v = C[m * N + n];
            if (scale_m)
                v *= (double)scale_m[m];
            if (scale_n)
                v *= (double)scale_n[n];
            if (bias)
                v += orc_bf16_to_f64(bias[n]);
            v = orc_activation(act, v);
            if (mul)
                v *= orc_bf16_to_f64(mul[m * ld_mul + n]);
            C[m * N + n] = v;
        }
}

/* ------------------------------------------------------- B preshuffle layout */

/* Byte reading of the preshuffle layout: kpack = 16 bytes per lane (one
 * 16-byte load), "16" = the 16 columns of one MFMA block = lane % 16, "4" =
 * lane / 16, K block = 4 * kpack.  With e bytes per element, kp = 16/e
 * elements and kb = 4*kp elements per K block:
 *   Bs[n0][k0][g][nl][j] = B[16*n0 + nl][kb*k0 + kp*g + j]
 * K is padded up to a multiple of kb and N up to a multiple of 16; padded
 * positions hold zero. */
int64_t orc_shuffle_b_bytes(int64_t N, int64_t K, int elem_bytes)
{
    int64_t kb = 4 * (16 / elem_bytes);
    int64_t nblk = (N + 15) / 16;
    int64_t kpad = (K + kb - 1) / kb * kb;
    return nblk * 16 * kpad * elem_bytes;
}

void orc_shuffle_b(const uint8_t *B, int64_t ldb, int64_t N, int64_t K, int elem_bytes,
                   uint8_t *Bs)
{
    int64_t kp = 16 / elem_bytes;
    int64_t kb = 4 * kp;
    int64_t nblk = (N + 15) / 16;
    int64_t kblk = (K + kb - 1) / kb;
    int64_t e = elem_bytes;
    for (int64_t n0 = 0; n0 < nblk; n0++)
        for (int64_t k0 = 0; k0 < kblk; k0++)
            for (int64_t g = 0; g < 4; g++)
                for (int64_t nl = 0; nl < 16; nl++)
                    for (int64_t j = 0; j < kp; j++) {
                        int64_t dst = ((((n0 * kblk + k0) * 4 + g) * 16 + nl) * kp + j) * e;
                        int64_t n = 16 * n0 + nl;
                        int64_t k = kb * k0 + kp * g + j;
                        if (n < N && k < K)
                            memcpy(Bs + dst, B + (n * ldb + k) * e, (size_t)e);
                        else
                            memset(Bs + dst, 0, (size_t)e);
                    }
}

/* Inverse: recover row-major B [N, ldb] (only the first K columns written). */
void orc_unshuffle_b(const uint8_t *Bs, int64_t N, int64_t K, int elem_bytes,
                     uint8_t *B, int64_t ldb)
{
    int64_t kp = 16 / elem_bytes;
    int64_t kb = 4 * kp;
    int64_t kblk = (K + kb - 1) / kb;
    int64_t e = elem_bytes;
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) {
            int64_t n0 = n / 16, nl = n % 16;
            int64_t k0 = k / kb, g = (k % kb) / kp, j = k % kp;
            int64_t src = ((((n0 * kblk + k0) * 4 + g) * 16 + nl) * kp + j) * e;
            memcpy(B + (n * ldb + k) * e, Bs + src, (size_t)e);
        }
}

/* ------------------------------------------------- dimension efficiency */

/* Tile quantization: pad M and N up to whole tiles;
 *   tile_eff = M*N / (M_pad*N_pad).
 * Wave quantization: tiles run in rounds of num_cus;
 *   wq_eff = tiles / (ceil(tiles/num_cus) * num_cus).
 * dim_eff = tile_eff * wq_eff. */
void orc_dim_eff(int64_t M, int64_t N, int64_t mt_m, int64_t mt_n, int64_t num_cus,
                 int64_t *num_tiles, double *tile_eff, double *wq_eff, double *dim_eff)
{
    int64_t tiles_m = (M + mt_m - 1) / mt_m;
    int64_t tiles_n = (N + mt_n - 1) / mt_n;
    int64_t tiles = tiles_m * tiles_n;
    double te = ((double)M * (double)N) / ((double)(tiles_m * mt_m) * (double)(tiles_n * mt_n));
    int64_t rounds = (tiles + num_cus - 1) / num_cus;
    double we = (double)tiles / ((double)rounds * (double)num_cus);
    *num_tiles = tiles;
    *tile_eff = te;
    *wq_eff = we;
    *dim_eff = te * we;
}
