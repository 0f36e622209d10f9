/*
 * Plain-C use of the library's C ABI (include/mxq.h) with the HIP runtime
 * API: device buffers from hipMalloc, the stream as a void pointer, no C++
 * and no torch.  Each call's output is copied back and compared byte for
 * byte with the CPU oracle (oracle/oracle.c, test infrastructure), linked
 * into this test program only.  Exit status 0 when every comparison holds.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mxq.h"

/* oracle entry points (oracle/oracle.c) */
int oracle_quantize_jagged_rowwise(const uint16_t *x, int64_t rows, int64_t cols, int64_t sx_r,
                                   int64_t sx_c, const int32_t *offs, int32_t G, uint8_t *q,
                                   int64_t sq_r, int64_t sq_c, float *scales, int64_t ss_r,
                                   int64_t ss_g);
int oracle_relayout_mx_scales_grouped(const uint8_t *scales, int64_t rows, int64_t ss_r,
                                      int64_t ss_b, const int32_t *offs, int32_t G, uint8_t *out,
                                      int32_t *tile_starts);
int oracle_quantize_mx_3d_colwise(const uint16_t *w, int64_t E, int64_t N, int64_t K, int64_t sw_e,
                                  int64_t sw_n, int64_t sw_k, uint8_t *q, int64_t sq_e,
                                  int64_t sq_n, int64_t sq_k, uint8_t *scales, int64_t ss_e,
                                  int64_t ss_nb, int64_t ss_k, int mode);

#define CHECK_HIP(call)                                                              \
    do {                                                                             \
        hipError_t e_ = (call);                                                      \
        if (e_ != hipSuccess) {                                                      \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));        \
            return 2;                                                                \
        }                                                                            \
    } while (0)

/* xorshift bits of a finite bf16: sign, exponent in [100, 150], mantissa */
static uint16_t next_bf16(uint32_t *st)
{
    uint32_t v = *st;
    v ^= v << 13;
    v ^= v >> 17;
    v ^= v << 5;
    *st = v;
    uint16_t sign = (uint16_t)((v >> 31) << 15);
    uint16_t expo = (uint16_t)(100u + (v >> 8) % 51u);
    return (uint16_t)(sign | (expo << 7) | (v & 0x7Fu));
}

static int same(const void *a, const void *b, size_t n, const char *what)
{
    if (memcmp(a, b, n) != 0) {
        fprintf(stderr, "%s differs from the oracle\n", what);
        return 0;
    }
    return 1;
}

int main(void)
{
    if (mxq_abi_version() != MXQ_ABI_VERSION) {
        fprintf(stderr, "ABI version mismatch\n");
        return 1;
    }
    int ok = 1;
    uint32_t st = 12345u;

    /* jagged rowwise: (rows, cols) row-major, 3 groups along the columns
       (rows 16-byte aligned in and out, as the row-major layout requires) */
    {
        const int64_t rows = 96, cols = 1024;
        const int32_t offs[3] = {250, 250, 1021};
        const size_t n = (size_t)(rows * cols);
        uint16_t *hx = malloc(n * sizeof(uint16_t));
        uint8_t *hq = malloc(n), *oq = malloc(n);
        float *hs = malloc(rows * 3 * sizeof(float)), *os = malloc(rows * 3 * sizeof(float));
        for (size_t i = 0; i < n; ++i)
            hx[i] = next_bf16(&st);
        void *dx, *dq, *ds, *doffs;
        CHECK_HIP(hipMalloc(&dx, n * sizeof(uint16_t)));
        CHECK_HIP(hipMalloc(&dq, n));
        CHECK_HIP(hipMalloc(&ds, rows * 3 * sizeof(float)));
        CHECK_HIP(hipMalloc(&doffs, sizeof offs));
        CHECK_HIP(hipMemcpy(dx, hx, n * sizeof(uint16_t), hipMemcpyHostToDevice));
        CHECK_HIP(hipMemcpy(doffs, offs, sizeof offs, hipMemcpyHostToDevice));
        hipStream_t s;
        CHECK_HIP(hipStreamCreate(&s));
        mxq_status r = mxq_quantize_jagged_rowwise(dx, rows, cols, cols, 1, doffs, 3, dq, cols, 1,
                                                   ds, 3, 1, (void *)s);
        if (r != MXQ_OK) {
            fprintf(stderr, "jagged rowwise: %s\n", mxq_status_string(r));
            return 1;
        }
        CHECK_HIP(hipStreamSynchronize(s));
        CHECK_HIP(hipMemcpy(hq, dq, n, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(hs, ds, rows * 3 * sizeof(float), hipMemcpyDeviceToHost));
        oracle_quantize_jagged_rowwise(hx, rows, cols, cols, 1, offs, 3, oq, cols, 1, os, 3, 1);
        ok &= same(hq, oq, n, "jagged rowwise q");
        ok &= same(hs, os, rows * 3 * sizeof(float), "jagged rowwise scales");
        CHECK_HIP(hipStreamDestroy(s));
        CHECK_HIP(hipFree(dx));
        CHECK_HIP(hipFree(dq));
        CHECK_HIP(hipFree(ds));
        CHECK_HIP(hipFree(doffs));
        free(hx);
        free(hq);
        free(oq);
        free(hs);
        free(os);
    }

    /* MX 3D colwise, rceil: (E, N, K) -> per-expert column-major, null stream */
    {
        const int64_t E = 2, N = 128, K = 64;
        const size_t n = (size_t)(E * N * K), ns = (size_t)(E * (N / 32) * K);
        uint16_t *hw = malloc(n * sizeof(uint16_t));
        uint8_t *hq = malloc(n), *oq = malloc(n), *hs = malloc(ns), *os = malloc(ns);
        for (size_t i = 0; i < n; ++i)
            hw[i] = next_bf16(&st);
        void *dw, *dq, *ds;
        CHECK_HIP(hipMalloc(&dw, n * sizeof(uint16_t)));
        CHECK_HIP(hipMalloc(&dq, n));
        CHECK_HIP(hipMalloc(&ds, ns));
        CHECK_HIP(hipMemcpy(dw, hw, n * sizeof(uint16_t), hipMemcpyHostToDevice));
        mxq_status r = mxq_quantize_mx_3d_colwise(dw, E, N, K, N * K, K, 1, dq, N * K, 1, N, ds,
                                                  (N / 32) * K, K, 1, MXQ_SCALE_RCEIL, NULL);
        if (r != MXQ_OK) {
            fprintf(stderr, "mx 3d colwise: %s\n", mxq_status_string(r));
            return 1;
        }
        CHECK_HIP(hipDeviceSynchronize());
        CHECK_HIP(hipMemcpy(hq, dq, n, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(hs, ds, ns, hipMemcpyDeviceToHost));
        oracle_quantize_mx_3d_colwise(hw, E, N, K, N * K, K, 1, oq, N * K, 1, N, os, (N / 32) * K,
                                      K, 1, 1);
        ok &= same(hq, oq, n, "mx 3d q");
        ok &= same(hs, os, ns, "mx 3d scales");
        CHECK_HIP(hipFree(dw));
        CHECK_HIP(hipFree(dq));
        CHECK_HIP(hipFree(ds));
        free(hw);
        free(hq);
        free(oq);
        free(hs);
        free(os);
    }

    /* scale re-layout: (rows, blocks) e8m0 bytes, 3 groups over 5000 tokens */
    {
        const int64_t rows = 40, extent = 5000, G = 3;
        const int32_t offs[3] = {1700, 1700, 4990};
        const int64_t nbcap = (extent + 31) / 32 + G - 1;
        const size_t ns = (size_t)(rows * nbcap);
        const size_t cap = (size_t)(256 * ((rows + 15) / 16) * ((extent + 511) / 512 + G - 1));
        uint8_t *hs = malloc(ns), *ht = malloc(cap), *ot = malloc(cap);
        int32_t hst[4], ost[4];
        for (size_t i = 0; i < ns; ++i)
            hs[i] = (uint8_t)(next_bf16(&st) % 255u);
        void *ds, *dt, *dst, *doffs;
        CHECK_HIP(hipMalloc(&ds, ns));
        CHECK_HIP(hipMalloc(&dt, cap));
        CHECK_HIP(hipMalloc(&dst, sizeof hst));
        CHECK_HIP(hipMalloc(&doffs, sizeof offs));
        CHECK_HIP(hipMemcpy(ds, hs, ns, hipMemcpyHostToDevice));
        CHECK_HIP(hipMemcpy(doffs, offs, sizeof offs, hipMemcpyHostToDevice));
        CHECK_HIP(hipMemset(dt, 0xA5, cap));
        mxq_status r = mxq_relayout_mx_scales_grouped(ds, rows, nbcap, 1, doffs, (int32_t)G, extent,
                                                      dt, dst, NULL);
        if (r != MXQ_OK) {
            fprintf(stderr, "relayout: %s\n", mxq_status_string(r));
            return 1;
        }
        CHECK_HIP(hipDeviceSynchronize());
        CHECK_HIP(hipMemcpy(ht, dt, cap, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(hst, dst, sizeof hst, hipMemcpyDeviceToHost));
        memset(ot, 0xA5, cap);
        oracle_relayout_mx_scales_grouped(hs, rows, nbcap, 1, offs, (int32_t)G, ot, ost);
        ok &= same(hst, ost, sizeof hst, "relayout tile starts");
        ok &= same(ht, ot, cap, "relayout tiles");
        CHECK_HIP(hipFree(ds));
        CHECK_HIP(hipFree(dt));
        CHECK_HIP(hipFree(dst));
        CHECK_HIP(hipFree(doffs));
        free(hs);
        free(ht);
        free(ot);
    }

    /* host-side validation: a bad argument returns before any launch */
    if (mxq_quantize_blockwise(NULL, -1, 128, 128, 1, 1, 128, NULL, 128, 1, NULL, 1, 1, NULL) !=
        MXQ_ERR_INVALID_ARG) {
        fprintf(stderr, "a negative extent was accepted\n");
        ok = 0;
    }

    printf(ok ? "c abi check: ok\n" : "c abi check: FAILED\n");
    return ok ? 0 : 1;
}
