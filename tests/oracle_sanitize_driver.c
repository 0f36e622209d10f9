/*
 * Runs one oracle function on inputs read from a file and writes its outputs
 * to another, so that a build of oracle/oracle.c with AddressSanitizer and
 * UndefinedBehaviorSanitizer can be checked against the normal build
 * (tests/test_oracle_sanitize.py writes the cases and compares the bytes).
 *
 *   driver <op> <in> <out> <int64 arguments...>
 *
 * Every buffer is allocated at exactly the size the call may touch, so an
 * access past it is reported.  Output buffers start filled with 0xA5.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint8_t oracle_e4m3_encode(double y);
void oracle_e4m3_encode_array(const float *y, int64_t n, uint8_t *out);
float oracle_fp32_scale(float amax);
uint8_t oracle_e8m0_floor(float amax);
uint8_t oracle_e8m0_rceil(float amax);
int oracle_quantize_jagged_rowwise(const uint16_t *, int64_t, int64_t, int64_t, int64_t,
                                   const int32_t *, int32_t, uint8_t *, int64_t, int64_t, float *,
                                   int64_t, int64_t);
int oracle_quantize_jagged_colwise(const uint16_t *, int64_t, int64_t, int64_t, int64_t,
                                   const int32_t *, int32_t, uint8_t *, int64_t, int64_t, float *,
                                   int64_t, int64_t);
int oracle_quantize_mx_3d_colwise(const uint16_t *, int64_t, int64_t, int64_t, int64_t, int64_t,
                                  int64_t, uint8_t *, int64_t, int64_t, int64_t, uint8_t *, int64_t,
                                  int64_t, int64_t, int);
int oracle_quantize_mx_rowwise(const uint16_t *, int64_t, int64_t, int64_t, int64_t, uint8_t *,
                               int64_t, int64_t, uint8_t *, int64_t, int64_t, int);
int oracle_quantize_jagged_mx_rowwise(const uint16_t *, int64_t, int64_t, int64_t, int64_t,
                                      const int32_t *, int32_t, uint8_t *, int64_t, int64_t,
                                      uint8_t *, int64_t, int64_t, int);
int oracle_quantize_jagged_mx_colwise(const uint16_t *, int64_t, int64_t, int64_t, int64_t,
                                      const int32_t *, int32_t, uint8_t *, int64_t, int64_t,
                                      uint8_t *, int64_t, int64_t, int);
int oracle_relayout_mx_scales_grouped(const uint8_t *, int64_t, int64_t, int64_t, const int32_t *,
                                      int32_t, uint8_t *, int32_t *);
int oracle_quantize_blockwise(const uint16_t *, int64_t, int64_t, int64_t, int64_t, int32_t,
                              int32_t, uint8_t *, int64_t, int64_t, float *, int64_t, int64_t);

static void *xalloc(size_t n, int fill)
{
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    memset(p, fill, n ? n : 1);
    return p;
}

/* the next n bytes of the input file, in a buffer of exactly n bytes */
static void *take(FILE *f, size_t n)
{
    void *p = xalloc(n, 0);
    if (n && fread(p, 1, n, f) != n) {
        fprintf(stderr, "short input\n");
        exit(2);
    }
    return p;
}

static void put(FILE *f, const void *p, size_t n)
{
    if (n && fwrite(p, 1, n, f) != n) {
        fprintf(stderr, "short write\n");
        exit(2);
    }
}

int main(int argc, char **argv)
{
    if (argc < 4)
        return 2;
    const char *op = argv[1];
    int64_t a[16] = {0};
    for (int i = 4; i < argc && i - 4 < 16; ++i)
        a[i - 4] = strtoll(argv[i], NULL, 10);
    FILE *in = fopen(argv[2], "rb");
    FILE *out = fopen(argv[3], "wb");
    if (!in || !out)
        return 2;
    int rc = 0;

    if (!strcmp(op, "jagged_rowwise") || !strcmp(op, "jagged_colwise")) {
        /* rows cols sx_r sx_c G xsize */
        int64_t rows = a[0], cols = a[1], G = a[4];
        uint16_t *x = take(in, (size_t)a[5] * 2);
        int32_t *offs = take(in, (size_t)G * 4);
        uint8_t *q = xalloc((size_t)(rows * cols), 0xA5);
        int row = !strcmp(op, "jagged_rowwise");
        size_t ns = (size_t)(row ? rows * G : G * cols);
        float *s = xalloc(ns * 4, 0xA5);
        rc = row ? oracle_quantize_jagged_rowwise(x, rows, cols, a[2], a[3], offs, (int32_t)G, q, cols,
                                                  1, s, G, 1)
                 : oracle_quantize_jagged_colwise(x, rows, cols, a[2], a[3], offs, (int32_t)G, q, cols,
                                                  1, s, cols, 1);
        put(out, q, (size_t)(rows * cols));
        put(out, s, ns * 4);
    } else if (!strcmp(op, "jagged_mx_rowwise") || !strcmp(op, "jagged_mx_colwise")) {
        /* rows cols sx_r sx_c G xsize mode */
        int64_t rows = a[0], cols = a[1], G = a[4];
        uint16_t *x = take(in, (size_t)a[5] * 2);
        int32_t *offs = take(in, (size_t)G * 4);
        uint8_t *q = xalloc((size_t)(rows * cols), 0xA5);
        int row = !strcmp(op, "jagged_mx_rowwise");
        int64_t cap = ((row ? cols : rows) + 31) / 32 + G - 1;
        size_t ns = (size_t)(row ? rows * cap : cap * cols);
        uint8_t *s = xalloc(ns, 0xA5);
        rc = row ? oracle_quantize_jagged_mx_rowwise(x, rows, cols, a[2], a[3], offs, (int32_t)G, q,
                                                     cols, 1, s, cap, 1, (int)a[6])
                 : oracle_quantize_jagged_mx_colwise(x, rows, cols, a[2], a[3], offs, (int32_t)G, q,
                                                     cols, 1, s, cols, 1, (int)a[6]);
        put(out, q, (size_t)(rows * cols));
        put(out, s, ns);
    } else if (!strcmp(op, "mx3d")) {
        /* E N K sw_e sw_n sw_k wsize mode */
        int64_t E = a[0], N = a[1], K = a[2];
        uint16_t *w = take(in, (size_t)a[6] * 2);
        uint8_t *q = xalloc((size_t)(E * N * K), 0xA5);
        uint8_t *s = xalloc((size_t)(E * (N / 32) * K), 0xA5);
        rc = oracle_quantize_mx_3d_colwise(w, E, N, K, a[3], a[4], a[5], q, N * K, K, 1, s,
                                           (N / 32) * K, K, 1, (int)a[7]);
        put(out, q, (size_t)(E * N * K));
        put(out, s, (size_t)(E * (N / 32) * K));
    } else if (!strcmp(op, "mx_rowwise")) {
        /* rows cols sx_r sx_c xsize mode */
        int64_t rows = a[0], cols = a[1];
        uint16_t *x = take(in, (size_t)a[4] * 2);
        uint8_t *q = xalloc((size_t)(rows * cols), 0xA5);
        uint8_t *s = xalloc((size_t)(rows * (cols / 32)), 0xA5);
        rc = oracle_quantize_mx_rowwise(x, rows, cols, a[2], a[3], q, cols, 1, s, cols / 32, 1,
                                        (int)a[5]);
        put(out, q, (size_t)(rows * cols));
        put(out, s, (size_t)(rows * (cols / 32)));
    } else if (!strcmp(op, "blockwise")) {
        /* rows cols sx_r sx_c br bc xsize */
        int64_t rows = a[0], cols = a[1], br = a[4], bc = a[5];
        uint16_t *x = take(in, (size_t)a[6] * 2);
        uint8_t *q = xalloc((size_t)(rows * cols), 0xA5);
        size_t ns = (size_t)((rows / br) * (cols / bc));
        float *s = xalloc(ns * 4, 0xA5);
        rc = oracle_quantize_blockwise(x, rows, cols, a[2], a[3], (int32_t)br, (int32_t)bc, q, cols, 1,
                                       s, cols / bc, 1);
        put(out, q, (size_t)(rows * cols));
        put(out, s, ns * 4);
    } else if (!strcmp(op, "relayout")) {
        /* rows ss_r ss_b G extent ssize: tiles of capacity 256 * ceil(rows/16) *
         * (ceil(extent/512) + G - 1) bytes */
        int64_t rows = a[0], G = a[3], extent = a[4];
        uint8_t *sc = take(in, (size_t)a[5]);
        int32_t *offs = take(in, (size_t)G * 4);
        size_t cap = (size_t)(256 * ((rows + 15) / 16) * ((extent + 511) / 512 + G - 1));
        uint8_t *tiles = xalloc(cap, 0xA5);
        int32_t *starts = xalloc((size_t)(G + 1) * 4, 0xA5);
        rc = oracle_relayout_mx_scales_grouped(sc, rows, a[1], a[2], offs, (int32_t)G, tiles, starts);
        put(out, tiles, cap);
        put(out, starts, (size_t)(G + 1) * 4);
    } else if (!strcmp(op, "encode")) {
        /* n */
        float *y = take(in, (size_t)a[0] * 4);
        uint8_t *o = xalloc((size_t)a[0], 0xA5);
        oracle_e4m3_encode_array(y, a[0], o);
        put(out, o, (size_t)a[0]);
    } else if (!strcmp(op, "scales")) {
        /* every bf16 pattern with a finite value: fp32 multiplier, e8m0 floor, e8m0 rceil */
        for (uint32_t b = 0; b < 0x8000u; ++b) {
            if (((b >> 7) & 0xFFu) == 0xFFu)
                continue;
            uint32_t u = b << 16;
            float amax;
            memcpy(&amax, &u, 4);
            float s = oracle_fp32_scale(amax);
            uint8_t f = oracle_e8m0_floor(amax), r = oracle_e8m0_rceil(amax);
            put(out, &s, 4);
            put(out, &f, 1);
            put(out, &r, 1);
        }
    } else {
        fprintf(stderr, "unknown op %s\n", op);
        return 2;
    }
    fclose(in);
    fclose(out);
    if (rc != 0) {
        fprintf(stderr, "%s returned %d\n", op, rc);
        return 3;
    }
    return 0;
}
