/* A C99 caller of the library's host-only entry points (no GPU needed): the
 * plan of a few shapes for every sync mode and stage count, printed one per
 * line as "M N K bt stages sync rc bm bn bk stages grid tiles k_splits
 * tail_tiles tail_splits mfma_block workspace_bytes pipelines", and the text of every
 * status code.  Built with -std=c99 -pedantic -Werror against include/ only. */
#include <stdio.h>
#include <stdint.h>

#include "gemm_bf16.h"

int main(void)
{
    static const int64_t shapes[][3] = {{8192, 8192, 8192}, {4352, 4352, 4096}, {1000, 1032, 8192}, {300, 264, 200}};
    static const int modes[][2] = {{GEMM_SYNC_BARRIER, 0}, {GEMM_SYNC_BARRIER, 2}, {GEMM_SYNC_BARRIER, 3},
                                   {GEMM_SYNC_BARRIER, 4}, {GEMM_SYNC_BARRIER, GEMM_STAGES_WINDOWS},
                                   {GEMM_SYNC_FLAGS, 2}, {GEMM_SYNC_FLAGS, 3}, {GEMM_SYNC_FLAGS, 4},
                                   {GEMM_SYNC_WAVESPEC, 2}, {GEMM_SYNC_WAVESPEC, 3}, {GEMM_SYNC_WAVESPEC, 4},
                                   {GEMM_SYNC_PINGPONG, 2}, {GEMM_SYNC_PINGPONG, 3}, {GEMM_SYNC_PINGPONG, 4}};
    size_t s, m;
    int bt, code;
    for (s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
        for (m = 0; m < sizeof modes / sizeof modes[0]; ++m)
            for (bt = 0; bt < 2; ++bt) {
                gemm_bf16_plan_t p;
                const int rc = gemm_bf16_plan_cus(shapes[s][0], shapes[s][1], shapes[s][2], bt, modes[m][1],
                                                  modes[m][0], 256, &p);
                printf("%lld %lld %lld %d %d %d %d", (long long)shapes[s][0], (long long)shapes[s][1],
                       (long long)shapes[s][2], bt, modes[m][1], modes[m][0], rc);
                if (rc == GEMM_OK)
                    printf(" %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld", (long long)p.bm,
                           (long long)p.bn, (long long)p.bk, (long long)p.stages, (long long)p.grid,
                           (long long)p.tiles, (long long)p.k_splits, (long long)p.tail_tiles,
                           (long long)p.tail_splits, (long long)p.mfma_block, (long long)p.workspace_bytes,
                           (long long)p.pipelines);
                printf("\n");
            }
    for (code = -9; code <= 0; ++code)
        printf("status %d %s\n", code, gemm_bf16_strerror(code));
    return 0;
}
