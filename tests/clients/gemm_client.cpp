// A host program that runs the GEMM through the C ABI alone: it allocates
// device memory with the HIP runtime, preshuffles B with shuffle_b and calls
// gemm_bf16 (library-chosen tile) on the null stream -- no PyTorch, no Python.
// Inputs and output are raw bf16 bit files, so the test that drives it takes
// the inputs from the seeded generators and the expected values from the
// oracle.
//
//   gemm_client M N K A.bin B.bin C.bin      (A [M,K], B [N,K], C [M,N] row-major)
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "densegemm.h"

#define HIP_OK(x)                                                                           \
    do {                                                                                    \
        hipError_t e_ = (x);                                                                \
        if (e_ != hipSuccess) {                                                             \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            return 2;                                                                       \
        }                                                                                   \
    } while (0)

#define GEMM_OK_(x)                                                                      \
    do {                                                                                 \
        gemm_status s_ = (x);                                                            \
        if (s_ != GEMM_OK) {                                                             \
            fprintf(stderr, "%s at line %d\n", gemm_status_string(s_), __LINE__);       \
            return 3;                                                                    \
        }                                                                                \
    } while (0)

static int read_file(const char* path, void* dst, size_t bytes)
{
    FILE* f = fopen(path, "rb");
    if (!f)
        return 0;
    const size_t n = fread(dst, 1, bytes, f);
    fclose(f);
    return n == bytes;
}

int main(int argc, char** argv)
{
    if (argc != 7) {
        fprintf(stderr, "usage: %s M N K A.bin B.bin C.bin\n", argv[0]);
        return 1;
    }
    const int64_t M = atoll(argv[1]), N = atoll(argv[2]), K = atoll(argv[3]);
    if (M <= 0 || N <= 0 || K <= 0 || M * K > (1 << 26) || N * K > (1 << 26) || M * N > (1 << 26)) {
        fprintf(stderr, "sizes out of range\n");
        return 1;
    }
    const size_t a_bytes = (size_t)(M * K) * 2, b_bytes = (size_t)(N * K) * 2,
                 c_bytes = (size_t)(M * N) * 2;
    const size_t bs_bytes = shuffle_b_bytes(N, K, GEMM_BF16);
    uint16_t* hA = (uint16_t*)malloc(a_bytes);
    uint16_t* hB = (uint16_t*)malloc(b_bytes);
    uint16_t* hC = (uint16_t*)malloc(c_bytes);
    if (!hA || !hB || !hC || !read_file(argv[4], hA, a_bytes) || !read_file(argv[5], hB, b_bytes)) {
        fprintf(stderr, "cannot read inputs\n");
        return 1;
    }
    void *dA, *dB, *dBs, *dC;
    HIP_OK(hipMalloc(&dA, a_bytes));
    HIP_OK(hipMalloc(&dB, b_bytes));
    HIP_OK(hipMalloc(&dBs, bs_bytes));
    HIP_OK(hipMalloc(&dC, c_bytes));
    HIP_OK(hipMemcpy(dA, hA, a_bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dB, hB, b_bytes, hipMemcpyHostToDevice));
    GEMM_OK_(shuffle_b(dB, K, dBs, N, K, GEMM_BF16, NULL));
    GEMM_OK_(gemm_bf16((const uint16_t*)dA, K, dBs, (uint16_t*)dC, N, M, N, K, NULL, NULL));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(hC, dC, c_bytes, hipMemcpyDeviceToHost));
    FILE* f = fopen(argv[6], "wb");
    if (!f || fwrite(hC, 1, c_bytes, f) != c_bytes) {
        fprintf(stderr, "cannot write output\n");
        return 1;
    }
    fclose(f);
    HIP_OK(hipFree(dA));
    HIP_OK(hipFree(dB));
    HIP_OK(hipFree(dBs));
    HIP_OK(hipFree(dC));
    free(hA);
    free(hB);
    free(hC);
    printf("gemm_client ok %lld x %lld x %lld\n", (long long)M, (long long)N, (long long)K);
    return 0;
}
