// Jagged MXFP8: e8m0-scaled e4m3 with 32-element blocks that restart at
// every token-group start, for MX grouped GEMMs whose groups run along K
// ("[mxfp8 moe training] add CUDA kernel for per-group conversion of scale
// factors to blocked layout", stacked PR list: scales of groups along K).
// A group of n elements has ceil(n/32) blocks, the last one short when n is
// not a multiple of 32; blocks are numbered group after group, so block k of
// group g has scale index B_g + k, B_g = sum over j < g of ceil(n_j/32).
//
// Both kernels build, per workgroup, a table of the groups from the device
// offsets (clamped group ends and exclusive prefix counts of blocks or
// tiles), then find their own group by binary search: the host never reads
// the offsets and the grid depends only on the extents and G.
//
//  * jagged_mx_rowwise_kernel — blocks along the unit-stride dim.  Four lanes
//    share a block (8 elements each, one 16-byte load when the block starts
//    on an 8-element boundary), a workgroup covers 64 block slots x RW rows,
//    loads all RW rows before reducing, and reduces each block with a
//    quad-lane DPP max.
//  * jagged_mx_colwise_kernel — blocks across rows, output column-major.  A
//    workgroup covers 128 rows of one group (starting at the group start)
//    x 256 columns; a lane holds 16 rows x 8 columns, two lanes make a
//    32-row block, and the lane writes each of its 8 columns as one 16-byte
//    piece when the group start is a multiple of 16.  Plain stores: a tile
//    that starts off a 128-row boundary writes every output line in two
//    parts, which L2 merges (nontemporal partial writes cost HBM a
//    read-modify-write each: 44.8 against 39.3 us on the MoE x operand).
#pragma once

#include <stdint.h>

#include "group_tables.hpp"
#include "mxq_device.hpp"
#include "wave_ops.hpp"

namespace mxq {

constexpr int kJmxThreads = 256;

// x: (rows, cols), row r at x + r*ldx (ldx % 8 == 0), unit column stride;
// groups along the columns.  q: row-major, ldq % 16 == 0.
// scales[r*ss_r + j*ss_b] for block j of row r.
// Grid: nbt * ceil(rows / RW) with nbt = ceil((ceil(cols/32) + G - 1) / 64).
template <int RW>
__global__ __launch_bounds__(kJmxThreads) void jagged_mx_rowwise_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, int rows, int cols,
    const int32_t *__restrict__ offs, int G, uint8_t *__restrict__ q, int64_t ldq,
    uint8_t *__restrict__ scales, int64_t ss_r, int64_t ss_b, int nbt, int rceil)
{
    // group table, sized for the largest G: the LDS it takes keeps the
    // occupancy at a level measured to stream faster than a table sized by G
    __shared__ int s_end[kMaxTableGroups];
    __shared__ int s_pre[kMaxTableGroups + 1];

    const int t = threadIdx.x;
    const int bj = (int)(blockIdx.x % (unsigned)nbt);
    const int br = (int)(blockIdx.x / (unsigned)nbt);
    const int r0 = br * RW;

    // block table: prefix counts of 32-element blocks per group
    if (G <= 64) {
        if (t < 64)
            wave_group_tables<5, 5>(offs, G, cols, s_end, s_pre, s_pre);
        __syncthreads();
    } else {
        load_group_ends<kJmxThreads>(offs, G, cols, s_end);
        slot_prefix<kJmxThreads>(G, s_pre, [&](int g) { return units_of<5>(group_len(s_end, g)); });
    }
    const int total = s_pre[G];

    const int j = bj * 64 + (t >> 2);
    const int l = t & 3;
    int p0 = 0, pn = 0;
    if (j < total) {
        const int g = find_slot(s_pre, G, j);
        const int lo = g ? s_end[g - 1] : 0;
        const int hi = s_end[g];
        const int start = lo + 32 * (j - s_pre[g]);
        const int end = start + 32 < hi ? start + 32 : hi;
        p0 = start + 8 * l;
        pn = end - p0;
        pn = pn < 0 ? 0 : (pn > 8 ? 8 : pn);
    }
    const bool fast = pn == 8 && (p0 & 7) == 0;

    uint4 v[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        const int r = r0 + i;
        v[i] = (fast && r < rows) ? ld16_nt(x + (int64_t)r * ldx + p0) : make_uint4(0u, 0u, 0u, 0u);
    }
    if (!fast && pn > 0) {
        // a piece that is short or does not start on an 8-element boundary
#pragma unroll
        for (int i = 0; i < RW; ++i) {
            const int r = r0 + i;
            if (r < rows) {
                const uint16_t *xp = x + (int64_t)r * ldx + p0;
                uint32_t wv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (e < pn)
                        wv[e >> 1] |= (uint32_t)xp[e] << (16 * (e & 1));
                v[i] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
            }
        }
    }

#pragma unroll
    for (int i = 0; i < RW; ++i) {
        const int r = r0 + i;
        const uint32_t m = group_max<4>(fold2(absmax_u4(v[i])));
        const uint32_t code = e8m0_code(m, rceil != 0);
        const float s = e8m0_multiplier(code);
        if (r >= rows || pn == 0)
            continue;
        if (l == 0)
            scales[(int64_t)r * ss_r + (int64_t)j * ss_b] = (uint8_t)code;
        const uint2 o = quant8(v[i], s);
        uint8_t *qp = q + (int64_t)r * ldq + p0;
        if (fast) {
            st8_nt(qp, o);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (e < pn)
                    qp[e] = (uint8_t)((e < 4 ? o.x : o.y) >> (8 * (e & 3)));
        }
    }
}

// x: (rows, cols), row r at x + r*ldx (ldx % 8 == 0), unit column stride,
// cols % 8 == 0; groups along the rows.  q column-major: (r, c) at
// q[c*ldq + r], ldq % 16 == 0.  scales[j*ss_b + c*ss_c] for block j.
// Grid: ntr * tiles_c, ntr = ceil(rows/128) + G - 1 (an upper bound of the
// number of 128-row group tiles), tiles_c = ceil(cols/256).
__global__ __launch_bounds__(kJmxThreads) void jagged_mx_colwise_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, int rows, int cols,
    const int32_t *__restrict__ offs, int G, uint8_t *__restrict__ q, int64_t ldq,
    uint8_t *__restrict__ scales, int64_t ss_b, int64_t ss_c, int tiles_c, int rceil)
{
    // group table, sized for the largest G (see the rowwise kernel)
    __shared__ int s_end[kMaxTableGroups];
    __shared__ int s_pt[kMaxTableGroups + 1];   // 128-row tiles
    __shared__ int s_pb[kMaxTableGroups + 1];   // 32-row blocks

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = t >> 6;
    const int cg = lane & 7;
    const int qd = lane >> 3;
    const int tc = (int)(blockIdx.x % (unsigned)tiles_c);
    const int tid = (int)(blockIdx.x / (unsigned)tiles_c);

    if (G <= 64) {
        if (t < 64)
            wave_group_tables<7, 5>(offs, G, rows, s_end, s_pt, s_pb);
        __syncthreads();
    } else {
        load_group_ends<kJmxThreads>(offs, G, rows, s_end);
        slot_prefix2<kJmxThreads>(G, s_pt, s_pb,
                                  [&](int gg) { return units_of<7>(group_len(s_end, gg)); },
                                  [&](int gg) { return units_of<5>(group_len(s_end, gg)); });
    }
    if (tid >= s_pt[G])
        return;
    const int g = find_slot(s_pt, G, tid);
    const int lo = g ? s_end[g - 1] : 0;
    const int hi = s_end[g];
    const int k = tid - s_pt[g];
    const int rt = lo + 128 * k;          // first row of this tile
    const int rb = rt + 16 * qd;          // first row of this lane
    const int c0 = tc * 256 + 64 * w + 8 * cg;
    const bool col_ok = c0 < cols;

    // rows past the group end read row hi-1, which lies in the same 32-row
    // block whenever that block has a row inside the group, so block maxima
    // are unchanged; blocks wholly past the end are not written
    const int cl = col_ok ? c0 : 0;
    uint4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = rb + i < hi ? rb + i : hi - 1;
        v[i] = ld16_nt(x + (int64_t)r * ldx + cl);
    }

    uint32_t mx[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        mx[0] = absmax2(mx[0], v[i].x);
        mx[1] = absmax2(mx[1], v[i].y);
        mx[2] = absmax2(mx[2], v[i].z);
        mx[3] = absmax2(mx[3], v[i].w);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d)
        mx[d] = pkmax(mx[d], (uint32_t)__shfl_xor((int)mx[d], 8, 64));

    float sc[8];
    uint32_t codes[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
        const uint32_t a = (jj & 1) ? (mx[jj >> 1] >> 16) : (mx[jj >> 1] & 0xffffu);
        codes[jj] = e8m0_code(a, rceil != 0);
        sc[jj] = e8m0_multiplier(codes[jj]);
    }

    if (!col_ok || rb >= hi)
        return;
    if ((qd & 1) == 0) {
        // this lane starts a block (rt + 32*(qd/2) < hi, since rb < hi)
        const int64_t jb = (int64_t)s_pb[g] + 4 * k + (qd >> 1);
        uint8_t *sp = scales + jb * ss_b + (int64_t)c0 * ss_c;
        if (ss_c == 1 && ((reinterpret_cast<uintptr_t>(sp) & 7u) == 0)) {
            uint2 pk;
            pk.x = codes[0] | (codes[1] << 8) | (codes[2] << 16) | (codes[3] << 24);
            pk.y = codes[4] | (codes[5] << 8) | (codes[6] << 16) | (codes[7] << 24);
            *reinterpret_cast<uint2 *>(sp) = pk;
        } else {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
                sp[jj * ss_c] = (uint8_t)codes[jj];
        }
    }

    const bool full = (rb & 15) == 0 && rb + 16 <= hi;
    uint8_t *qp = q + (int64_t)c0 * ldq + rb;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
        uint4 o;
        o.x = cvt4(elem8(v[0], jj) * sc[jj], elem8(v[1], jj) * sc[jj], elem8(v[2], jj) * sc[jj],
                   elem8(v[3], jj) * sc[jj]);
        o.y = cvt4(elem8(v[4], jj) * sc[jj], elem8(v[5], jj) * sc[jj], elem8(v[6], jj) * sc[jj],
                   elem8(v[7], jj) * sc[jj]);
        o.z = cvt4(elem8(v[8], jj) * sc[jj], elem8(v[9], jj) * sc[jj], elem8(v[10], jj) * sc[jj],
                   elem8(v[11], jj) * sc[jj]);
        o.w = cvt4(elem8(v[12], jj) * sc[jj], elem8(v[13], jj) * sc[jj], elem8(v[14], jj) * sc[jj],
                   elem8(v[15], jj) * sc[jj]);
        uint8_t *p = qp + (int64_t)jj * ldq;
        if (full) {
            st16(p, o);
        } else {
            const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (rb + i < hi)
                    p[i] = (uint8_t)(ow[i >> 2] >> (8 * (i & 3)));
        }
    }
}

}  // namespace mxq
