/*
 * Plain single-threaded CPU oracle for dynamic float8 quantization of MoE
 * grouped-GEMM operands.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant
 * generator with the HIP library.
 *
 * What it computes, and where the pages say so:
 *   - "[scaled grouped mm] add triton kernels for float8 rowwise quantization
 *     with per-group/jagged scales", Motivation and Summary: one scale per
 *     (row, group) for the row-major left operand and one scale per
 *     (group, column) for the column-major right operand, groups given by
 *     cumulative token offsets that the host never reads.  The CPU loop over
 *     offsets that this page replaces is exactly the loop written here.
 *   - "[scaled grouped mm] integrate triton kernels into differentiable scaled
 *     grouped mm", Summary: that per-group CPU loop is kept as the accuracy
 *     reference.
 *   - "[fp8 blockwise] load 2d chunks for groupwise quant ...", body: fixed
 *     1 x blocksize and blocksize x blocksize blocks with one scale each.
 *   - "[mxfp8 moe training] add CUDA kernel to quantize 3d tensor colwise",
 *     Summary and the author's comment: 3D expert weights (E,N,K) scaled along
 *     N in 32-element blocks and written column-major per expert; the "floor"
 *     scale-calculation mode.
 *   - "[mxfp8 moe training] add CUDA kernel for per-group conversion of scale
 *     factors to blocked layout", stacked PR list: MX scales of token groups
 *     along the GEMM's K dimension.  Jagged MX blocks restart at each group
 *     start (reading: the pages fix no padding of groups to 32; a block never
 *     spans two groups, a group's last block may be short, and scale entries
 *     are numbered group after group).
 *
 *   - "[mxfp8 moe training] add CUDA kernel for per-group conversion of scale
 *     factors to blocked layout", title and stacked PR list: after jagged MX
 *     quantization with groups along K, each group's e8m0 scales are re-laid
 *     out for the consumer grouped GEMM.  The page does not print the target
 *     layout (it is another vendor's MMA layout); the layout written here is
 *     the scale operand order of the gfx950 scaled MFMA with 16 rows and 128
 *     K values per instruction (AMD CDNA4 ISA, V_MFMA_SCALE_F32_16X16X128_
 *     F8F6F4), as stated at oracle_relayout_mx_scales_grouped.
 *
 * Numeric readings (the pages name the formats but print no formula):
 *   - fp8 is OCP E4M3FN: bias 7, 3 mantissa bits, no infinities, max 448,
 *     codes 0x7F/0xFF are NaN.  Encoding is round-to-nearest-even with
 *     saturation to +-448 applied before rounding; a negative value that
 *     rounds to zero encodes as 0x80.
 *   - fp32 scales: s = RN32(448 / max(amax, RN32(1e-12))), the quantize
 *     multiplier.  Each element becomes enc(sat(RN32(x * s))).
 *   - e8m0 scales ("floor" mode, OCP Microscaling Formats v1.0 shared-exponent
 *     rule with emax(E4M3) = 8): se = clamp(floor(log2(amax)) - 8, -127, 127),
 *     code = se + 127; amax = 0 gives code 0.  Each element becomes
 *     enc(sat(RN32(x * 2^-se))).  "rceil" mode (named by the 3D colwise
 *     page, not defined there): the smallest se with amax <= 448 * 2^se.
 *
 * Arithmetic is done in double precision, where every product and quotient
 * below is either exact or rounded exactly once to binary32 by an explicit
 * (float) conversion, so no compiler contraction or evaluation-order choice
 * can change a result.  Build without -ffast-math and with -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1

/* ---------------------------------------------------------------- formats */

/* bf16 bit pattern -> its exact value (bf16 is the top half of binary32). */
static double bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest binary32 value (ties to even). */
static double round_to_fp32(double v)
{
    volatile float f = (float)v;
    return (double)f;
}

/* Magnitude of the E4M3FN code c in [0x00, 0x7E]: exponent field E = c >> 3,
 * mantissa field M = c & 7; subnormal (E = 0): M * 2^-9, else
 * (1 + M/8) * 2^(E-7). */
static double e4m3_code_magnitude(int c)
{
    int E = c >> 3, M = c & 7;
    if (E == 0)
        return ldexp((double)M, -9);
    return ldexp(8.0 + (double)M, E - 10);
}

static double g_e4m3_table[127];
static int g_table_ready = 0;

static void ensure_table(void)
{
    if (g_table_ready)
        return;
    for (int c = 0; c <= 0x7E; ++c)
        g_e4m3_table[c] = e4m3_code_magnitude(c);
    g_table_ready = 1;
}

/* Saturating round-to-nearest-even encode of y into an E4M3FN byte.
 * y must not be NaN. */
uint8_t oracle_e4m3_encode(double y)
{
    ensure_table();
    if (y > 448.0)
        y = 448.0;
    if (y < -448.0)
        y = -448.0;
    int sign = signbit(y) ? 1 : 0;
    double a = fabs(y);

    /* largest code whose magnitude does not exceed a */
    int i = 0x7E;
    while (g_e4m3_table[i] > a)
        --i;

    int code;
    if (g_e4m3_table[i] == a) {
        code = i;
    } else {
        /* strictly between codes i and i+1 (i < 0x7E since a <= 448);
         * 2a and V(i) + V(i+1) are exact in double */
        double twice = 2.0 * a;
        double mid2 = g_e4m3_table[i] + g_e4m3_table[i + 1];
        if (twice < mid2)
            code = i;
        else if (twice > mid2)
            code = i + 1;
        else
            code = (i % 2 == 0) ? i : i + 1;
    }
    return (uint8_t)((sign << 7) | code);
}

/* Value of an E4M3FN byte; NaN for 0x7F and 0xFF. */
double oracle_e4m3_decode(uint8_t c)
{
    if ((c & 0x7F) == 0x7F)
        return NAN;
    double m = e4m3_code_magnitude(c & 0x7F);
    return (c & 0x80) ? -m : m;
}

void oracle_e4m3_encode_array(const float *y, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3_encode((double)y[i]);
}

/* ----------------------------------------------------------------- scales */

/* fp32 quantize multiplier: RN32(448 / max(amax, RN32(1e-12))).
 * The double quotient rounded once to binary32 equals the correctly rounded
 * binary32 quotient (53 >= 2*24 + 2, so double rounding is innocuous). */
float oracle_fp32_scale(float amax)
{
    double eps = (double)(float)1e-12;
    double a = (double)amax;
    if (a < eps)
        a = eps;
    return (float)(448.0 / a);
}

/* e8m0 "floor" code: clamp(floor(log2(amax)) - 8, -127, 127) + 127.
 * amax = 0 has log2 = -inf and clamps to the minimum code 0. */
uint8_t oracle_e8m0_floor(float amax)
{
    if (amax == 0.0f)
        return 0;
    int e;
    double m = frexp((double)amax, &e); /* amax = m * 2^e, m in [0.5, 1) */
    (void)m;
    int fl = e - 1;                     /* floor(log2(amax)) */
    int se = fl - 8;
    if (se < -127)
        se = -127;
    if (se > 127)
        se = 127;
    return (uint8_t)(se + 127);
}

/* e8m0 "rceil" code.  The pages name an rceil scale-calculation mode next to
 * floor without defining it; the reading taken here: the scale is rounded UP
 * to a power of two, i.e. se is the smallest integer with
 * amax <= 448 * 2^se (so no element saturates), clamped to [-127, 127];
 * amax = 0 gives the minimum code 0. */
uint8_t oracle_e8m0_rceil(float amax)
{
    if (amax == 0.0f)
        return 0;
    double a = (double)amax;
    int e;
    frexp(a / 448.0, &e);            /* a/448 = m * 2^e, m in [0.5, 1) */
    int se = e;                      /* candidate: 448 * 2^e >= a */
    while (448.0 * ldexp(1.0, se - 1) >= a)
        --se;
    while (448.0 * ldexp(1.0, se) < a)
        ++se;
    if (se < -127)
        se = -127;
    if (se > 127)
        se = 127;
    return (uint8_t)(se + 127);
}

static uint8_t e8m0_code(float amax, int mode)
{
    return mode == 1 ? oracle_e8m0_rceil(amax) : oracle_e8m0_floor(amax);
}

/* quantize one bf16 element with an fp32 multiplier */
static uint8_t quant_fp32(uint16_t xbits, float s)
{
    double y = round_to_fp32(bf16_to_double(xbits) * (double)s);
    return oracle_e4m3_encode(y);
}

/* quantize one bf16 element with an e8m0 code (multiplier 2^-(code-127)) */
static uint8_t quant_e8m0(uint16_t xbits, uint8_t code)
{
    int se = (int)code - 127;
    double y = round_to_fp32(ldexp(bf16_to_double(xbits), -se));
    return oracle_e4m3_encode(y);
}

static double bf16_abs(uint16_t bits) { return fabs(bf16_to_double(bits)); }

/* --------------------------------------------------------- jagged (groups) */

/* Group g covers [lo, hi) with lo = offs[g-1] (0 for g = 0), hi = offs[g]. */
static int check_offs_args(int32_t G) { return G > 0 ? ORACLE_OK : ORACLE_BAD_ARG; }

/* Rowwise: x is rows x cols, groups along dim 1 (columns).
 * scales[r * ss_r + g * ss_g] = scale of (row r, group g);
 * q[r * sq_r + c * sq_c] for every c inside a group. */
int oracle_quantize_jagged_rowwise(const uint16_t *x, int64_t rows, int64_t cols, int64_t sx_r,
                                   int64_t sx_c, const int32_t *offs, int32_t G, uint8_t *q,
                                   int64_t sq_r, int64_t sq_c, float *scales, int64_t ss_r,
                                   int64_t ss_g)
{
    if (rows < 0 || cols < 0 || check_offs_args(G) != ORACLE_OK)
        return ORACLE_BAD_ARG;
    for (int32_t g = 0; g < G; ++g) {
        int64_t lo = g == 0 ? 0 : offs[g - 1];
        int64_t hi = offs[g];
        for (int64_t r = 0; r < rows; ++r) {
            double amax = 0.0;
            for (int64_t c = lo; c < hi; ++c) {
                double a = bf16_abs(x[r * sx_r + c * sx_c]);
                if (a > amax)
                    amax = a;
            }
            float s = oracle_fp32_scale((float)amax);
            scales[r * ss_r + g * ss_g] = s;
            for (int64_t c = lo; c < hi; ++c)
                q[r * sq_r + c * sq_c] = quant_fp32(x[r * sx_r + c * sx_c], s);
        }
    }
    return ORACLE_OK;
}

/* Colwise: x is rows x cols, groups along dim 0 (rows).
 * scales[g * ss_g + c * ss_c] = scale of (group g, column c). */
int oracle_quantize_jagged_colwise(const uint16_t *x, int64_t rows, int64_t cols, int64_t sx_r,
                                   int64_t sx_c, const int32_t *offs, int32_t G, uint8_t *q,
                                   int64_t sq_r, int64_t sq_c, float *scales, int64_t ss_g,
                                   int64_t ss_c)
{
    if (rows < 0 || cols < 0 || check_offs_args(G) != ORACLE_OK)
        return ORACLE_BAD_ARG;
    for (int32_t g = 0; g < G; ++g) {
        int64_t lo = g == 0 ? 0 : offs[g - 1];
        int64_t hi = offs[g];
        for (int64_t c = 0; c < cols; ++c) {
            double amax = 0.0;
            for (int64_t r = lo; r < hi; ++r) {
                double a = bf16_abs(x[r * sx_r + c * sx_c]);
                if (a > amax)
                    amax = a;
            }
            float s = oracle_fp32_scale((float)amax);
            scales[g * ss_g + c * ss_c] = s;
            for (int64_t r = lo; r < hi; ++r)
                q[r * sq_r + c * sq_c] = quant_fp32(x[r * sx_r + c * sx_c], s);
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------- MX (e8m0) */

/* 3D expert weights W (E, N, K): blocks of 32 consecutive n at fixed (e, k).
 * scales[e * ss_e + nb * ss_nb + k * ss_k] is the e8m0 code of block
 * (e, nb, k); q[e * sq_e + n * sq_n + k * sq_k]. */
int oracle_quantize_mx_3d_colwise(const uint16_t *w, int64_t E, int64_t N, int64_t K, int64_t sw_e,
                                  int64_t sw_n, int64_t sw_k, uint8_t *q, int64_t sq_e,
                                  int64_t sq_n, int64_t sq_k, uint8_t *scales, int64_t ss_e,
                                  int64_t ss_nb, int64_t ss_k, int mode)
{
    if (E < 0 || N < 0 || K < 0 || N % 32 != 0 || (mode != 0 && mode != 1))
        return ORACLE_BAD_ARG;
    for (int64_t e = 0; e < E; ++e)
        for (int64_t nb = 0; nb < N / 32; ++nb)
            for (int64_t k = 0; k < K; ++k) {
                double amax = 0.0;
                for (int64_t n = 32 * nb; n < 32 * nb + 32; ++n) {
                    double a = bf16_abs(w[e * sw_e + n * sw_n + k * sw_k]);
                    if (a > amax)
                        amax = a;
                }
                uint8_t code = e8m0_code((float)amax, mode);
                scales[e * ss_e + nb * ss_nb + k * ss_k] = code;
                for (int64_t n = 32 * nb; n < 32 * nb + 32; ++n)
                    q[e * sq_e + n * sq_n + k * sq_k] =
                        quant_e8m0(w[e * sw_e + n * sw_n + k * sw_k], code);
            }
    return ORACLE_OK;
}

/* 2D x (rows, cols): blocks of 32 consecutive columns at fixed row.
 * scales[r * ss_r + b * ss_b] is the e8m0 code of block (r, b). */
int oracle_quantize_mx_rowwise(const uint16_t *x, int64_t rows, int64_t cols, int64_t sx_r,
                               int64_t sx_c, uint8_t *q, int64_t sq_r, int64_t sq_c,
                               uint8_t *scales, int64_t ss_r, int64_t ss_b, int mode)
{
    if (rows < 0 || cols < 0 || cols % 32 != 0 || (mode != 0 && mode != 1))
        return ORACLE_BAD_ARG;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < cols / 32; ++b) {
            double amax = 0.0;
            for (int64_t c = 32 * b; c < 32 * b + 32; ++c) {
                double a = bf16_abs(x[r * sx_r + c * sx_c]);
                if (a > amax)
                    amax = a;
            }
            uint8_t code = e8m0_code((float)amax, mode);
            scales[r * ss_r + b * ss_b] = code;
            for (int64_t c = 32 * b; c < 32 * b + 32; ++c)
                q[r * sq_r + c * sq_c] = quant_e8m0(x[r * sx_r + c * sx_c], code);
        }
    return ORACLE_OK;
}

/* ----------------------------------------------------------- jagged MX */

/* Jagged MXFP8: 32-element blocks that restart at every group start, so no
 * block mixes two groups; a group of n elements has ceil(n / 32) blocks and
 * its last block holds n mod 32 elements when that is not zero.  Blocks are
 * numbered group after group: block k of group g has scale index B_g + k,
 * B_g = sum over j < g of ceil(n_j / 32).  Scale entries past the last block
 * are not written. */

/* Rowwise: groups along dim 1; scales[r * ss_r + b * ss_b]. */
int oracle_quantize_jagged_mx_rowwise(const uint16_t *x, int64_t rows, int64_t cols,
                                      int64_t sx_r, int64_t sx_c, const int32_t *offs,
                                      int32_t G, uint8_t *q, int64_t sq_r, int64_t sq_c,
                                      uint8_t *scales, int64_t ss_r, int64_t ss_b, int mode)
{
    if (rows < 0 || cols < 0 || check_offs_args(G) != ORACLE_OK || (mode != 0 && mode != 1))
        return ORACLE_BAD_ARG;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t b = 0;   /* running block index */
        for (int32_t g = 0; g < G; ++g) {
            int64_t lo = g == 0 ? 0 : offs[g - 1];
            int64_t hi = offs[g];
            for (int64_t c0 = lo; c0 < hi; c0 += 32, ++b) {
                int64_t c1 = c0 + 32 < hi ? c0 + 32 : hi;
                double amax = 0.0;
                for (int64_t c = c0; c < c1; ++c) {
                    double a = bf16_abs(x[r * sx_r + c * sx_c]);
                    if (a > amax)
                        amax = a;
                }
                uint8_t code = e8m0_code((float)amax, mode);
                scales[r * ss_r + b * ss_b] = code;
                for (int64_t c = c0; c < c1; ++c)
                    q[r * sq_r + c * sq_c] = quant_e8m0(x[r * sx_r + c * sx_c], code);
            }
        }
    }
    return ORACLE_OK;
}

/* Colwise: groups along dim 0; scales[b * ss_b + c * ss_c]. */
int oracle_quantize_jagged_mx_colwise(const uint16_t *x, int64_t rows, int64_t cols,
                                      int64_t sx_r, int64_t sx_c, const int32_t *offs,
                                      int32_t G, uint8_t *q, int64_t sq_r, int64_t sq_c,
                                      uint8_t *scales, int64_t ss_b, int64_t ss_c, int mode)
{
    if (rows < 0 || cols < 0 || check_offs_args(G) != ORACLE_OK || (mode != 0 && mode != 1))
        return ORACLE_BAD_ARG;
    for (int64_t c = 0; c < cols; ++c) {
        int64_t b = 0;
        for (int32_t g = 0; g < G; ++g) {
            int64_t lo = g == 0 ? 0 : offs[g - 1];
            int64_t hi = offs[g];
            for (int64_t r0 = lo; r0 < hi; r0 += 32, ++b) {
                int64_t r1 = r0 + 32 < hi ? r0 + 32 : hi;
                double amax = 0.0;
                for (int64_t r = r0; r < r1; ++r) {
                    double a = bf16_abs(x[r * sx_r + c * sx_c]);
                    if (a > amax)
                        amax = a;
                }
                uint8_t code = e8m0_code((float)amax, mode);
                scales[b * ss_b + c * ss_c] = code;
                for (int64_t r = r0; r < r1; ++r)
                    q[r * sq_r + c * sq_c] = quant_e8m0(x[r * sx_r + c * sx_c], code);
            }
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------ MX scales -> scaled-MFMA scale tiles */

/* Per-group re-layout of jagged MX scales (groups along K) into tiles that a
 * gfx950 scaled-MFMA grouped GEMM loads as its scale operand.
 *
 * The consumer instruction multiplies a 16-row x 128-K operand tile; lane
 * 16j + i of the wave supplies, in one 32-bit register, the e8m0 scale of row
 * i and K block j (32 K values) of that tile, and the instruction's op_sel
 * picks one byte of the register.  Four consecutive K steps therefore share
 * one register per lane, byte u for step u: a tile here is 16 rows x 16
 * blocks (512 K values) stored as 64 lane words of 4 bytes, 256 bytes:
 *
 *   byte 4 * lane + u of a tile = scale of row i = lane % 16 and block
 *   4 * u + lane / 16 of the tile (u = 0..3).
 *
 * Group g (token range from offs, n_g tokens, nb_g = ceil(n_g / 32) blocks
 * numbered from B_g as the jagged MX functions number them) gets
 * RB = ceil(rows / 16) x KT_g = ceil(nb_g / 16) tiles, row-block-major:
 * tile (rb, kt) is tile number T_g + rb * KT_g + kt, T_g = RB * sum over h < g
 * of KT_h.  Entries past the last row or past the group's last block are 0.
 * tile_starts[g] = T_g for g = 0..G (tile_starts[G] = total tiles).
 *
 * scales[r * ss_r + b * ss_b] is the scale of row r and block b; for the
 * colwise operand the "rows" are its columns. */
int oracle_relayout_mx_scales_grouped(const uint8_t *scales, int64_t rows, int64_t ss_r,
                                      int64_t ss_b, const int32_t *offs, int32_t G,
                                      uint8_t *out, int32_t *tile_starts)
{
    if (rows < 0 || check_offs_args(G) != ORACLE_OK)
        return ORACLE_BAD_ARG;
    const int64_t RB = (rows + 15) / 16;
    int64_t b0 = 0; /* B_g */
    int64_t t0 = 0; /* T_g */
    for (int32_t g = 0; g < G; ++g) {
        int64_t lo = g == 0 ? 0 : offs[g - 1];
        int64_t n = offs[g] - lo;
        if (n < 0)
            n = 0;
        const int64_t nb = (n + 31) / 32;
        const int64_t KT = (nb + 15) / 16;
        tile_starts[g] = (int32_t)t0;
        for (int64_t rb = 0; rb < RB; ++rb)
            for (int64_t kt = 0; kt < KT; ++kt) {
                uint8_t *tile = out + (t0 + rb * KT + kt) * 256;
                for (int lane = 0; lane < 64; ++lane)
                    for (int u = 0; u < 4; ++u) {
                        const int64_t r = rb * 16 + lane % 16;
                        const int64_t blk = kt * 16 + 4 * u + lane / 16;
                        tile[4 * lane + u] =
                            (r < rows && blk < nb) ? scales[r * ss_r + (b0 + blk) * ss_b] : 0;
                    }
            }
        b0 += nb;
        t0 += RB * KT;
    }
    tile_starts[G] = (int32_t)t0;
    return ORACLE_OK;
}

/* -------------------------------------------------------------- blockwise */

/* Fixed block_r x block_c blocks with one fp32 multiplier each.
 * scales[rb * ss_rb + cb * ss_cb] for block (rb, cb). */
int oracle_quantize_blockwise(const uint16_t *x, int64_t rows, int64_t cols, int64_t sx_r,
                              int64_t sx_c, int32_t block_r, int32_t block_c, uint8_t *q,
                              int64_t sq_r, int64_t sq_c, float *scales, int64_t ss_rb,
                              int64_t ss_cb)
{
    if (rows < 0 || cols < 0 || block_r <= 0 || block_c <= 0 || rows % block_r != 0 ||
        cols % block_c != 0)
        return ORACLE_BAD_ARG;
    for (int64_t rb = 0; rb < rows / block_r; ++rb)
        for (int64_t cb = 0; cb < cols / block_c; ++cb) {
            double amax = 0.0;
            for (int64_t r = rb * block_r; r < (rb + 1) * block_r; ++r)
                for (int64_t c = cb * block_c; c < (cb + 1) * block_c; ++c) {
                    double a = bf16_abs(x[r * sx_r + c * sx_c]);
                    if (a > amax)
                        amax = a;
                }
            float s = oracle_fp32_scale((float)amax);
            scales[rb * ss_rb + cb * ss_cb] = s;
            for (int64_t r = rb * block_r; r < (rb + 1) * block_r; ++r)
                for (int64_t c = cb * block_c; c < (cb + 1) * block_c; ++c)
                    q[r * sq_r + c * sq_c] = quant_fp32(x[r * sx_r + c * sx_c], s);
        }
    return ORACLE_OK;
}
