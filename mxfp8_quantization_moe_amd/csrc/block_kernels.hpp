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
// (BR x 1 or BR x BC) or 1 x 128 blocks of a tile loaded the same way, output
// column-major or row-major — the 3D expert-weight case of
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
// cols % 8 == 0, rows % 16 == 0 (and rows % BR == 0).  q per batch entry:
// column-major, (e, r, c) at q[e*sqe + c*ldq + r] (QROW false), or row-major,
// at q[e*sqe + r*ldq + c] (QROW true).  scales (E, rows/BR, cols/BC) at
// [e*sse + rb*ss_rb + cb*ss_cb].
// Blocks (BR, BC): (32, 1) and (128, 1) down the rows of one column,
// (128, 128), and (1, 128) along one row.
// Grid: E * tiles_r * tiles_c, tile 128 rows x 256 columns.
// Tile order (a permutation of the grid; any order gives the same output):
// chunk == 0: column tile fastest, then row tile, then batch entry.
// chunk > 0: the dispatcher hands workgroup ids to the 8 XCDs in turn (id
// mod 8), so ids are renumbered for XCD x to take chunks x, x + 8, x + 16, ...
// of `chunk` consecutive tiles, counted in column-pair order (the two column
// tiles of a pair side by side, then down the rows, pair after pair; an odd
// last column tile alone); a partial last round of 8 chunks keeps its ids.
// Each XCD then sweeps a compact 512-column x (chunk/2 x 128)-row region: its
// reads are 1 KB row pieces and its column-major writes run down whole
// columns, which measured faster than the plain order on grids of many
// residency rounds (the 64-expert weights) and no faster on small ones.
// nt: the q stores.  0: plain.  1: nontemporal, for a column-major launch
// whose 128-row column runs start on 128-byte lines; with runs off the
// lines, plain stores let L2 merge the two parts of a line before it goes to
// HBM, where a partial nontemporal write of a line costs a read-modify-write
// of a memory burst.  2: as 1, at device scope through a buffer descriptor
// per batch entry (written through the XCD's L2); the host picks it when
// every q offset of a batch entry fits in 32 bits.  Row-major q is written
// in 64-byte halves of lines by two waves, so it takes plain stores (nt = 0).
template <int BR, int BC, bool E8M0, bool QROW = false>
__global__ __launch_bounds__(kBlockThreads) void block_strided_kernel(
    const uint16_t *__restrict__ x, int64_t sxe, int64_t ldx, int rows, int cols,
    uint8_t *__restrict__ q, int64_t sqe, int64_t ldq, void *__restrict__ scales, int64_t sse,
    int64_t ss_rb, int64_t ss_cb, int tiles_r, int tiles_c, int rceil, int nt, int chunk)
{
    static_assert((BC == 1 && (BR == 32 || BR == 128)) || (BC == 128 && (BR == 128 || BR == 1)),
                  "block shape");
    static_assert(!E8M0 || (BR == 32 && BC == 1), "e8m0 scales come in 32 x 1 blocks");
    constexpr int QPB = BR >= 16 ? BR / 16 : 1;   // lanes (16-row pieces) per block column

    __shared__ uint32_t s_red[4];
    __shared__ uint32_t s_rows[4][128];          // (1, 128): per-wave row maxima

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = t >> 6;
    const int cg = lane & 7;
    const int qd = lane >> 3;

    int tc, tr;
    int64_t e;
    if (chunk > 0) {
        uint32_t bid = blockIdx.x;
        const uint32_t ck = (uint32_t)chunk, span = 8u * ck, full = gridDim.x / span * span;
        if (bid < full) {
            const uint32_t l = bid >> 3;
            bid = ((l / ck) * 8u + (bid & 7u)) * ck + l % ck;
        }
        const uint32_t per_e = (uint32_t)tiles_r * (uint32_t)tiles_c;
        const uint32_t l = bid % per_e, pair_tiles = 2u * (uint32_t)tiles_r;
        const uint32_t paired = (uint32_t)(tiles_c >> 1) * pair_tiles;
        e = bid / per_e;
        if (l < paired) {
            const uint32_t m = l % pair_tiles;
            tc = (int)(2u * (l / pair_tiles) + (m & 1u));
            tr = (int)(m >> 1);
        } else {
            tc = tiles_c - 1;
            tr = (int)(l - paired);
        }
    } else {
        const int64_t bid = blockIdx.x;
        tc = (int)(bid % tiles_c);
        tr = (int)((bid / tiles_c) % tiles_r);
        e = bid / ((int64_t)tiles_c * tiles_r);
    }

    const int r0 = tr * 128 + 16 * qd;
    const int c0 = tc * 256 + 64 * w + 8 * cg;
    const bool ok = r0 < rows && c0 < cols;

    const uint16_t *xp = x + e * sxe + (int64_t)r0 * ldx + c0;
    uint4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        v[i] = ok ? ld16_nt(xp + (int64_t)i * ldx) : make_uint4(0u, 0u, 0u, 0u);

    // multiplier of element (row i, column j) of the lane's sub-tile:
    // sc[j] per column (BC == 1, and BC == 128 with one value), sr[i] per row
    // (BR == 1)
    float sc[8];
    float sr[16];
    if constexpr (BR == 1) {
        // one row of 128 columns: 8 columns in the lane, 8 lanes (lane bits
        // 0..2) across 64 columns, two waves across 128
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            uint32_t m = fold2(absmax_u4(v[i]));
            m = group_max<8>(m);
            if (cg == 0)
                s_rows[w][16 * qd + i] = m;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t a = umax(s_rows[w & 2][16 * qd + i], s_rows[(w & 2) + 1][16 * qd + i]);
            sr[i] = fp32_scale(a);
        }
        if (ok && cg == 0 && (w & 1) == 0) {
            float *sp = reinterpret_cast<float *>(scales) + e * sse + (int64_t)(c0 / 128) * ss_cb;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                sp[(int64_t)(r0 + i) * ss_rb] = sr[i];
        }
    } else {
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
        if constexpr (BC == 1) {
            uint32_t codes[8];
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
    }

    if (!ok)
        return;
    auto mul = [&](int i, int j) __attribute__((always_inline)) {
        if constexpr (BR == 1)
            return elem8(v[i], j) * sr[i];
        else
            return elem8(v[i], j) * sc[j];
    };
    if constexpr (QROW) {
        // row-major q: the lane's 8 columns of each of its 16 rows are 8
        // consecutive bytes; the 8 lanes of a row piece write 64 bytes
        uint8_t *qp = q + e * sqe + (int64_t)r0 * ldq + c0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            uint2 o;
            o.x = cvt4_sel<E8M0>(mul(i, 0), mul(i, 1), mul(i, 2), mul(i, 3));
            o.y = cvt4_sel<E8M0>(mul(i, 4), mul(i, 5), mul(i, 6), mul(i, 7));
            if (nt)
                st8_nt(qp + (int64_t)i * ldq, o);
            else
                st8(qp + (int64_t)i * ldq, o);
        }
    } else {
        // column-major q: the lane owns 16 consecutive bytes of each of its
        // 8 output columns (the transpose happens in registers)
        uint8_t *qp = q + e * sqe + (int64_t)c0 * ldq + r0;
        // nt == 2: offsets from the batch entry's base, below 2^32 (host-checked)
        const auto rq = buffer_rsrc(q + e * sqe, 0xFFFFFFFFu);
        const uint32_t qoff = (uint32_t)c0 * (uint32_t)ldq + (uint32_t)r0;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            uint4 o;
            o.x = cvt4_sel<E8M0>(mul(0, jj), mul(1, jj), mul(2, jj), mul(3, jj));
            o.y = cvt4_sel<E8M0>(mul(4, jj), mul(5, jj), mul(6, jj), mul(7, jj));
            o.z = cvt4_sel<E8M0>(mul(8, jj), mul(9, jj), mul(10, jj), mul(11, jj));
            o.w = cvt4_sel<E8M0>(mul(12, jj), mul(13, jj), mul(14, jj), mul(15, jj));
            if (nt == 2)
                stbuf16_nt_device(rq, qoff + (uint32_t)jj * (uint32_t)ldq, o);
            else if (nt)
                st16_nt(qp + (int64_t)jj * ldq, o);
            else
                st16(qp + (int64_t)jj * ldq, o);
        }
    }
}

}  // namespace mxq
