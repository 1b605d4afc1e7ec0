/* A C99 caller of the library on the GPU: operands in device memory from
 * the HIP runtime API, gemm_bf16 and gemm_bf16_bt in every sync mode on a
 * ragged shape, and the results checked against direct sums.  The entries
 * are -1, 0 or 1 and K = 200, so every sum is an integer of magnitude at
 * most 200: exact in fp32 accumulation and in bf16, whatever the order of
 * the additions.  Prints "ok" and returns 0 on success. */
#include <stdio.h>
#include <stdint.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "gemm_bf16.h"

enum { M = 300, N = 264, K = 200 };

static uint16_t A[M * K], B[K * N], BT[N * K], C[M * N];

/* bf16 bit patterns of -1, 0 and 1 (the upper half of the binary32 word). */
static uint16_t small(int v)
{
    return v == 0 ? 0x0000u : (v > 0 ? 0x3F80u : 0xBF80u);
}

/* The value of a bf16 bit pattern that holds an integer of magnitude at most
 * 256 (sign, exponent, 7 fraction bits), or -1000 for anything else. */
static int int_of(uint16_t b)
{
    const int sign = (b >> 15) ? -1 : 1;
    const int e = (b >> 7) & 0xFF, f = b & 0x7F;
    int v, shift;
    if (e == 0)
        return f == 0 ? 0 : -1000;
    shift = e - 127 - 7;                 /* value = (128 + f) * 2^shift */
    if (shift < -7 || shift > 1)
        return -1000;
    v = shift >= 0 ? (128 + f) << shift : (128 + f) >> -shift;
    if (shift < 0 && (((128 + f) & ((1 << -shift) - 1)) != 0))
        return -1000;                    /* not an integer */
    return sign * v;
}

static int check(const char* what)
{
    int i, j, k, bad = 0;
    for (i = 0; i < M; ++i)
        for (j = 0; j < N; ++j) {
            int want = 0;
            for (k = 0; k < K; ++k) {
                const int a = ((i * 7 + k * 3) % 3) - 1, b = ((k * 5 + j) % 3) - 1;
                want += a * b;
            }
            if (int_of(C[i * N + j]) != want) {
                if (bad < 3)
                    fprintf(stderr, "%s: C[%d][%d] = 0x%04x, want %d\n", what, i, j, C[i * N + j], want);
                ++bad;
            }
        }
    return bad;
}

int main(void)
{
    static const int syncs[] = {GEMM_SYNC_BARRIER, GEMM_SYNC_FLAGS, GEMM_SYNC_WAVESPEC, GEMM_SYNC_PINGPONG};
    void *dA = NULL, *dB = NULL, *dBT = NULL, *dC = NULL;
    int i, j, k, s, bad = 0;
    for (i = 0; i < M; ++i)
        for (k = 0; k < K; ++k)
            A[i * K + k] = small(((i * 7 + k * 3) % 3) - 1);
    for (k = 0; k < K; ++k)
        for (j = 0; j < N; ++j) {
            B[k * N + j] = small(((k * 5 + j) % 3) - 1);
            BT[j * K + k] = B[k * N + j];
        }
    if (hipMalloc(&dA, sizeof A) != hipSuccess || hipMalloc(&dB, sizeof B) != hipSuccess ||
        hipMalloc(&dBT, sizeof BT) != hipSuccess || hipMalloc(&dC, sizeof C) != hipSuccess ||
        hipMemcpy(dA, A, sizeof A, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(dB, B, sizeof B, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(dBT, BT, sizeof BT, hipMemcpyHostToDevice) != hipSuccess) {
        fprintf(stderr, "HIP allocation or copy failed\n");
        return 3;
    }
    for (s = 0; s < 4; ++s) {
        for (j = 0; j < 2; ++j) {
            char what[64];
            int rc;
            memset(C, 0xFF, sizeof C);
            if (hipMemcpy(dC, C, sizeof C, hipMemcpyHostToDevice) != hipSuccess)
                return 3;
            rc = j ? gemm_bf16_bt(M, N, K, dA, K, dBT, K, dC, N, 0, syncs[s], NULL)
                   : gemm_bf16(M, N, K, dA, K, dB, N, dC, N, 0, syncs[s], NULL);
            if (rc != GEMM_OK) {
                fprintf(stderr, "sync %d: %s\n", syncs[s], gemm_bf16_strerror(rc));
                return 2;
            }
            if (hipDeviceSynchronize() != hipSuccess || hipMemcpy(C, dC, sizeof C, hipMemcpyDeviceToHost) != hipSuccess)
                return 3;
            snprintf(what, sizeof what, "%s sync %d", j ? "gemm_bf16_bt" : "gemm_bf16", syncs[s]);
            bad += check(what);
        }
    }
    hipFree(dA);
    hipFree(dB);
    hipFree(dBT);
    hipFree(dC);
    if (bad) {
        fprintf(stderr, "%d wrong elements\n", bad);
        return 1;
    }
    printf("ok\n");
    return 0;
}
