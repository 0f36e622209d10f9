// Fixed-block fp8 quantization kernels: MXFP8 (e8m0 scales, 32-element
// blocks) and blockwise (fp32 scales, 1x128 / 128x128 / 128x1 blocks).
//
// block_contig_kernel: blocks of B elements along the unit-stride dim (1xB),
// the layout "[fp8 blockwise] load 2d chunks for groupwise quant ..." uses for
// activations and `to_mx` uses for MX along the last dim.  LPB lanes share a
// block, each loading 16-byte pieces, so one load instruction reads whole
// block rows of consecutive blocks; the block amax is reduced with DPP inside
// the lane group.
//
// block_strided_kernel: blocks that extend BR rows down the strided dim
// (BR x 1 or BR x BC), output column-major — the 3D expert-weight case of
// "[mxfp8 moe training] add CUDA kernel to quantize 3d tensor colwise"
// (32 x 1 along N, written per expert in column-major order) and the 128x128
// weight blocks of the blockwise page.  A workgroup covers 128 rows x 256
// columns (four waves side by side); a lane holds a 16-row x 8-column
// sub-tile, reduces its 8 column maxima over its 16 rows in registers,
// combines them with the lanes holding the other rows of the block, and,
// after scaling, owns 16 consecutive bytes of each of its 8 output columns,
// so the transpose happens in registers and each store is a 16-byte piece of
// a 128-byte column run shared by the 8 lanes of the same column group.
#pragma once

#include "mxq_device.hpp"
#include "wave_ops.hpp"

namespace mxq {

constexpr int kBlockThreads = 256;

// ----------------------------------------------------------------- contig

// x: (rows, cols), row r at x + r*ldx, unit column stride, cols % B == 0.
// q: (rows, cols), row r at q + r*ldq.
// scales: fp32 or e8m0 byte at [r*ss_r + b*ss_b] for block b of row r.
// Each workgroup handles U slots of 256/LPB blocks.
template <int B, int LPB, bool E8M0, int U>
__global__ __launch_bounds__(kBlockThreads) void block_contig_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, int64_t nbpr, int64_t nblocks,
    uint8_t *__restrict__ q, int64_t ldq, void *__restrict__ scales, int64_t ss_r, int64_t ss_b,
    int rceil)
{
    constexpr int L = B / (8 * LPB);           // 16-byte pieces per lane per block
    constexpr int BPW = kBlockThreads / LPB;   // blocks per workgroup slot
    static_assert(L >= 1 && B == 8 * LPB * L, "block must split into 16-byte pieces");

    const int t = threadIdx.x;
    const int j = t % LPB;

    // issue every load of the workgroup's U slots before consuming any
    uint4 v[U][L];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t blk = ((int64_t)blockIdx.x * U + u) * BPW + t / LPB;
        const bool ok = blk < nblocks;
        const int64_t r = ok ? blk / nbpr : 0;
        const int64_t b = ok ? blk % nbpr : 0;
        const uint16_t *xp = x + r * ldx + b * B;
#pragma unroll
        for (int l = 0; l < L; ++l)
            v[u][l] = ok ? ld16_nt(xp + 8 * (j + LPB * l)) : make_uint4(0u, 0u, 0u, 0u);
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t blk = ((int64_t)blockIdx.x * U + u) * BPW + t / LPB;
        const bool ok = blk < nblocks;
        const int64_t r = ok ? blk / nbpr : 0;
        const int64_t b = ok ? blk % nbpr : 0;
        uint8_t *qp = q + r * ldq + b * B;

        uint32_t m = 0u;
#pragma unroll
        for (int l = 0; l < L; ++l)
            m = pkmax(m, absmax_u4(v[u][l]));
        m = group_max<LPB>(fold2(m));

        float s;
        if constexpr (E8M0) {
            const uint32_t code = e8m0_code(m, rceil != 0);
            s = e8m0_multiplier(code);
            if (ok && j == 0)
                reinterpret_cast<uint8_t *>(scales)[r * ss_r + b * ss_b] = (uint8_t)code;
        } else {
            s = fp32_scale(m);
            if (ok && j == 0)
                reinterpret_cast<float *>(scales)[r * ss_r + b * ss_b] = s;
        }
        if (ok) {
#pragma unroll
            for (int l = 0; l < L; ++l)
                st8_nt(qp + 8 * (j + LPB * l), E8M0 ? quant8(v[u][l], s) : quant8_fp32scale(v[u][l], s));
        }
    }
}

// ---------------------------------------------------------------- strided

// Batched over E: x (E, rows, cols), element (e, r, c) at x[e*sxe + r*ldx + c],
// cols % 8 == 0, rows % BR == 0.  q column-major per batch entry:
// (e, r, c) at q[e*sqe + c*ldq + r].  scales (E, rows/BR, cols/BC) at
// [e*sse + rb*ss_rb + cb*ss_cb] (cb = c for BC == 1).
// BR in {32, 128}; BC in {1, 128} (BC == 128 needs BR == 128).
// Grid: E * tiles_r * tiles_c, tile 128 rows x 256 columns.
// nt: nontemporal q stores, for a launch whose 128-row column runs start on
// 128-byte lines (each output line is then one store instruction's); with
// runs off the lines, plain stores let L2 merge the two parts of a line
// before it goes to HBM, where a partial nontemporal write of a line costs a
// read-modify-write of a memory burst.
template <int BR, int BC, bool E8M0>
__global__ __launch_bounds__(kBlockThreads) void block_strided_kernel(
    const uint16_t *__restrict__ x, int64_t sxe, int64_t ldx, int rows, int cols,
    uint8_t *__restrict__ q, int64_t sqe, int64_t ldq, void *__restrict__ scales, int64_t sse,
    int64_t ss_rb, int64_t ss_cb, int tiles_r, int tiles_c, int rceil, int nt)
{
    static_assert(BR == 32 || BR == 128, "BR");
    static_assert(BC == 1 || (BC == 128 && BR == 128), "BC");
    constexpr int QPB = BR / 16;   // lanes (16-row pieces) per block column

    __shared__ uint32_t s_red[4];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = t >> 6;
    const int cg = lane & 7;
    const int qd = lane >> 3;

    const int64_t bid = blockIdx.x;
    const int tc = (int)(bid % tiles_c);
    const int tr = (int)((bid / tiles_c) % tiles_r);
    const int64_t e = bid / ((int64_t)tiles_c * tiles_r);

    const int r0 = tr * 128 + 16 * qd;
    const int c0 = tc * 256 + 64 * w + 8 * cg;
    const bool ok = r0 < rows && c0 < cols;

    const uint16_t *xp = x + e * sxe + (int64_t)r0 * ldx + c0;
    uint4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        v[i] = ok ? ld16_nt(xp + (int64_t)i * ldx) : make_uint4(0u, 0u, 0u, 0u);

    uint32_t mx[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        mx[0] = absmax2(mx[0], v[i].x);
        mx[1] = absmax2(mx[1], v[i].y);
        mx[2] = absmax2(mx[2], v[i].z);
        mx[3] = absmax2(mx[3], v[i].w);
    }
    // combine the QPB lanes (lane bits 3.. of qd) that hold the block's rows
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int msk = 8; msk < 8 * QPB; msk <<= 1)
            mx[d] = pkmax(mx[d], (uint32_t)__shfl_xor((int)mx[d], msk, 64));
    }

    float sc[8];
    uint32_t codes[8];
    if constexpr (BC == 1) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const uint32_t a = (jj & 1) ? (mx[jj >> 1] >> 16) : (mx[jj >> 1] & 0xffffu);
            if constexpr (E8M0) {
                codes[jj] = e8m0_code(a, rceil != 0);
                sc[jj] = e8m0_multiplier(codes[jj]);
            } else {
                sc[jj] = fp32_scale(a);
            }
        }
        if (ok && (qd % QPB) == 0) {
            const int64_t base = e * sse + (int64_t)(r0 / BR) * ss_rb + (int64_t)c0 * ss_cb;
            if constexpr (E8M0) {
                uint8_t *sp = reinterpret_cast<uint8_t *>(scales) + base;
                if (ss_cb == 1 && ((reinterpret_cast<uintptr_t>(sp) & 7u) == 0)) {
                    uint2 pk;
                    pk.x = codes[0] | (codes[1] << 8) | (codes[2] << 16) | (codes[3] << 24);
                    pk.y = codes[4] | (codes[5] << 8) | (codes[6] << 16) | (codes[7] << 24);
                    *reinterpret_cast<uint2 *>(sp) = pk;
                } else {
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj)
                        sp[jj * ss_cb] = (uint8_t)codes[jj];
                }
            } else {
                float *sp = reinterpret_cast<float *>(scales) + base;
#pragma unroll
                for (int jj = 0; jj < 8; ++jj)
                    sp[jj * ss_cb] = sc[jj];
            }
        }
    } else {
        // 128 x 128: one block per pair of waves
        uint32_t a = fold2(pkmax(pkmax(mx[0], mx[1]), pkmax(mx[2], mx[3])));
        a = group_max<8>(a);   // across the 8 column groups (lane bits 0..2)
        if (lane == 0)
            s_red[w] = a;
        __syncthreads();
        a = umax(s_red[w & 2], s_red[(w & 2) + 1]);
        const float s = fp32_scale(a);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            sc[jj] = s;
        if (lane == 0 && (w & 1) == 0 && ok) {
            const int64_t cb = c0 / 128;
            reinterpret_cast<float *>(scales)[e * sse + (int64_t)(r0 / 128) * ss_rb + cb * ss_cb] = s;
        }
    }

    if (!ok)
        return;
    uint8_t *qp = q + e * sqe + (int64_t)c0 * ldq + r0;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
        uint4 o;
        o.x = cvt4_sel<E8M0>(elem8(v[0], jj) * sc[jj], elem8(v[1], jj) * sc[jj], elem8(v[2], jj) * sc[jj],
                   elem8(v[3], jj) * sc[jj]);
        o.y = cvt4_sel<E8M0>(elem8(v[4], jj) * sc[jj], elem8(v[5], jj) * sc[jj], elem8(v[6], jj) * sc[jj],
                   elem8(v[7], jj) * sc[jj]);
        o.z = cvt4_sel<E8M0>(elem8(v[8], jj) * sc[jj], elem8(v[9], jj) * sc[jj], elem8(v[10], jj) * sc[jj],
                   elem8(v[11], jj) * sc[jj]);
        o.w = cvt4_sel<E8M0>(elem8(v[12], jj) * sc[jj], elem8(v[13], jj) * sc[jj], elem8(v[14], jj) * sc[jj],
                   elem8(v[15], jj) * sc[jj]);
        if (nt)
            st16_nt(qp + (int64_t)jj * ldq, o);
        else
            st16(qp + (int64_t)jj * ldq, o);
    }
}

}  // namespace mxq
