/* A plain C client of libdensegemm: includes only include/densegemm.h and
 * calls host-side entry points (no device needed).  Prints one line per query
 * for tests/test_c_client.py to compare with the Python binding. */
#include <stdio.h>
#include <stdint.h>

#include "densegemm.h"

static void show(const char* what, const gemm_tile* t)
{
    printf("%s kernel=%d tile_m=%d tile_n=%d tile_k=%d atom=%d waves=%d k_split=%d stages=%d\n",
           what, t->kernel, t->tile_m, t->tile_n, t->tile_k, t->atom, t->waves, t->k_split,
           t->lds_stages);
}

int main(void)
{
    gemm_tile t, t2;
    int64_t n1 = 0, m1 = 0;
    if (select_tile(4096, 4096, 4096, GEMM_BF16, 256, &t) != GEMM_OK)
        return 1;
    show("select_4096", &t);
    if (select_tile(1, 11008, 4096, GEMM_BF16, 256, &t) != GEMM_OK)
        return 1;
    show("select_decode", &t);
    if (select_tile_ws(48, 4096, 4096, GEMM_BF16, 256, (size_t)64 << 20, &t) != GEMM_OK)
        return 1;
    show("select_ws_48", &t);
    printf("workspace_48 %zu\n", gemm_workspace_bytes(48, 4096, 4096, GEMM_BF16, &t));
    if (gemm_plan(1024, 50257, 512, GEMM_BF16, 256, 0, &t, &t2, &n1, &m1) != GEMM_OK)
        return 1;
    show("plan_first", &t);
    show("plan_second", &t2);
    printf("plan_columns %lld\n", (long long)n1);
    printf("plan_rows %lld\n", (long long)m1);
    printf("shuffle_bytes %zu %zu\n", shuffle_b_bytes(11008, 4096, GEMM_BF16),
           shuffle_b_bytes(4096, 4096, GEMM_FP8_E4M3));
    printf("tile_check %d %d\n", (int)gemm_tile_check(&t, 1024, GEMM_BF16),
           (int)gemm_tile_check(&t, -1, GEMM_BF16));
    /* argument errors come back before any HIP call */
    printf("errors %s %s %s\n",
           gemm_status_string(gemm_bf16(NULL, 64, NULL, NULL, 64, 16, 16, 64, NULL, NULL)),
           gemm_status_string(gemm_bf16(NULL, 64, NULL, NULL, 64, -1, 16, 64, NULL, NULL)),
           gemm_status_string(select_tile(1, 1, 1, GEMM_BF16, 0, NULL)));
    printf("ok\n");
    return 0;
}
