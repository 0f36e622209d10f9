// Test-only consumer of the scaled-MFMA scale tiles: a plain grouped GEMM
// C_g = A_g B_g^T over token groups along K, one wave per (group, 16-row
// block of A, 16-row block of B), built on the gfx950 scaled MFMA with fp8
// (E4M3) operands, 16 x 16 x 128 per instruction.  It exists to show that the
// re-laid-out scales are what the instruction reads; it is not tuned.
//
// Operand order of the instruction (CDNA4 ISA, V_MFMA_SCALE_F32_16X16X128_
// F8F6F4): lane 16q + i holds row i of A (of B), bytes 0..15 = K values
// 16q..16q+15 and bytes 16..31 = K values 64+16q..64+16q+15 of the step;
// lane 16kb + i supplies the scale of row i for K block kb (32 values) in the
// byte of its scale register that op_sel selects; lane l, element r of the
// result is C[4*(l/16) + r][l % 16].
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

namespace {

// 32 operand bytes of one lane: row `row` of q (token-contiguous, row pitch
// ld), tokens of the K step starting at k0, zero at or past `hi` or past the
// last row
__device__ v8i lane_operand(const uint8_t *q, int64_t ld, int row, int nrows, int k0, int hi,
                            int grp)
{
    uint32_t w[8];
    for (int d = 0; d < 8; ++d) {
        uint32_t v = 0;
        for (int e = 0; e < 4; ++e) {
            const int j = 4 * d + e;
            const int k = k0 + (j < 16 ? 16 * grp + j : 64 + 16 * grp + (j - 16));
            if (row < nrows && k < hi)
                v |= (uint32_t)q[(int64_t)row * ld + k] << (8 * e);
        }
        w[d] = v;
    }
    v8i r;
    for (int d = 0; d < 8; ++d)
        r[d] = (int)w[d];
    return r;
}

__device__ int tile_word(const uint8_t *tiles, int64_t tile, int lane)
{
    return *reinterpret_cast<const int *>(tiles + tile * 256 + 4 * lane);
}

__global__ __launch_bounds__(64) void grouped_gemm_kernel(
    const uint8_t *qa, int64_t lda, int rows, const uint8_t *qb, int64_t ldb, int cols,
    const uint8_t *ta, const int32_t *sta, const uint8_t *tb, const int32_t *stb,
    const int32_t *offs, float *out, int ra0, int rb0)
{
    const int g = blockIdx.z, lane = threadIdx.x;
    const int ra = ra0 + (int)blockIdx.y, rb = rb0 + (int)blockIdx.x;
    const int orows = 16 * (int)gridDim.y, ocols = 16 * (int)gridDim.x;
    const int lo = g ? offs[g - 1] : 0;
    const int hi = offs[g];
    const int n = hi > lo ? hi - lo : 0;
    const int kt = (n + 511) / 512;
    const int grp = lane / 16, i = lane % 16;
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    for (int step = 0; step < (n + 127) / 128; ++step) {
        const int k0 = lo + 128 * step;
        const v8i a = lane_operand(qa, lda, 16 * ra + i, rows, k0, hi, grp);
        const v8i b = lane_operand(qb, ldb, 16 * rb + i, cols, k0, hi, grp);
        const int sa = tile_word(ta, (int64_t)sta[g] + (int64_t)ra * kt + step / 4, lane);
        const int sb = tile_word(tb, (int64_t)stb[g] + (int64_t)rb * kt + step / 4, lane);
        switch (step & 3) {
        case 0: acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, sa, 0, sb); break;
        case 1: acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 1, sa, 1, sb); break;
        case 2: acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 2, sa, 2, sb); break;
        default: acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 3, sa, 3, sb); break;
        }
    }
    for (int r = 0; r < 4; ++r) {
        const int row = 16 * ra + 4 * grp + r;
        const int col = 16 * rb + i;
        if (row < rows && col < cols)
            out[((int64_t)g * orows + row - 16 * ra0) * ocols + col - 16 * rb0] = acc[r];
    }
}

}  // namespace

// qa: (rows, tokens) e4m3, row pitch lda; qb: (cols, tokens) e4m3, row pitch
// ldb; ta/tb and sta/stb: the scale tiles and tile starts of A and B.  The
// product is computed for row blocks ra0 .. ra0+nra-1 of A and row blocks
// rb0 .. rb0+nrb-1 of B only; out: (G, 16*nra, 16*nrb) fp32, entries past
// the last row or column untouched.  All device pointers; synchronous.
// Returns 0 on success.
extern "C" int consumer_grouped_gemm(const uint8_t *qa, int64_t lda, int rows, const uint8_t *qb,
                                     int64_t ldb, int cols, const uint8_t *ta, const int32_t *sta,
                                     const uint8_t *tb, const int32_t *stb, const int32_t *offs,
                                     int G, float *out, int ra0, int nra, int rb0, int nrb)
{
    if (rows <= 0 || cols <= 0 || G <= 0 || nra <= 0 || nrb <= 0 || ra0 < 0 || rb0 < 0 ||
        16 * (ra0 + nra) > rows + 15 || 16 * (rb0 + nrb) > cols + 15)
        return 1;
    dim3 grid(nrb, nra, G);
    hipLaunchKernelGGL(grouped_gemm_kernel, grid, dim3(64), 0, 0, qa, lda, rows, qb, ldb, cols, ta,
                       sta, tb, stb, offs, out, ra0, rb0);
    if (hipGetLastError() != hipSuccess)
        return 2;
    return hipDeviceSynchronize() == hipSuccess ? 0 : 3;
}
