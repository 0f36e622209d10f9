// Jagged per-group fp8 quantization kernels (groups from device offsets).
//
// Follows "[scaled grouped mm] add triton kernels for float8 rowwise
// quantization with per-group/jagged scales" (Motivation, Summary): one
// launch covers every group, the group boundaries are read on the device, and
// the scale of a (row, group) or (group, column) is 448 / max(amax, 1e-12).
//
// Two memory patterns cover both operands:
//
//  * jagged_contig_kernel — the reduction runs along the unit-stride dim
//    (rowwise on a row-major tensor).  One workgroup owns one row, so every
//    workgroup does the same work whatever the group sizes; the row is held
//    in registers (up to 16384 elements), amax per group is reduced with DPP
//    per wave and LDS atomics across waves, then the same registers are
//    scaled and stored.  Rows longer than the register window are processed
//    in chunks and re-read for the scaling pass, last chunk first.
//
//  * jagged_strided_kernel — the reduction runs across rows (colwise on a
//    row-major tensor), the output is column-major.  A workgroup owns one
//    (column strip, group).  Each lane holds a 16-row x 8-column sub-tile
//    loaded as sixteen 16-byte row pieces, so a load instruction reads whole
//    row segments and, after the scale is applied per column, the lane owns
//    16 consecutive bytes of each of its 8 output columns: the transpose to
//    column-major happens inside the lane's registers and every store is a
//    16-byte piece of a contiguous column run.  Workgroups are ordered
//    largest group first (computed on the device from the offsets).
#pragma once

#include "mxq_device.hpp"
#include "wave_ops.hpp"

namespace mxq {

constexpr int kThreads = 256;

// smallest g' >= g with e < offs[g'] (G if none); offs non-decreasing and
// offs[g-1] <= e
__device__ __forceinline__ int advance_group(const int32_t *s_offs, int G, int g, int e)
{
#pragma unroll 1
    for (int k = 0; k < 4; ++k) {
        if (g >= G || s_offs[g] > e)
            return g;
        ++g;
    }
    int lo = g, hi = G;
#pragma unroll 1
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (s_offs[mid] <= e)
            lo = mid + 1;
        else
            hi = mid;
    }
    return lo;
}

// 8 bf16 at x[e0 .. e0+8) clipped to [0, n): full 16-byte load when inside
__device__ __forceinline__ uint4 load_seg(const uint16_t *xr, int e0, int n)
{
    if (e0 + 8 <= n)
        return ld16(xr + e0);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (e0 + j < n)
            w[j >> 1] |= (uint32_t)xr[e0 + j] << (16 * (j & 1));
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// ---------------------------------------------------------------- contig

// x row r at x + r*ldx (unit column stride); q row r at q + r*ldq;
// scales[r*ss_r + g*ss_g].  Dynamic LDS: 3*G words.  Grid: rows.
template <int NR>
__global__ __launch_bounds__(kThreads) void jagged_contig_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, int cols, const int32_t *__restrict__ offs, int G,
    uint8_t *__restrict__ q, int64_t ldq, float *__restrict__ scales, int64_t ss_r, int64_t ss_g)
{
    extern __shared__ uint32_t smem[];
    int32_t *s_offs = reinterpret_cast<int32_t *>(smem);
    uint32_t *s_amax = smem + G;
    float *s_scale = reinterpret_cast<float *>(smem + 2 * G);

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int64_t row = blockIdx.x;

    for (int g = t; g < G; g += kThreads) {
        int o = offs[g];
        s_offs[g] = o < 0 ? 0 : (o > cols ? cols : o);
        s_amax[g] = 0u;
    }
    __syncthreads();

    const uint16_t *xr = x + row * ldx;
    uint8_t *qr = q + row * ldq;
    constexpr int kChunk = 8 * kThreads * NR;
    const int nchunks = (cols + kChunk - 1) / kChunk;

    uint4 v[NR];

    // pass 1: amax per group
    for (int c = 0; c < nchunks; ++c) {
        const int cbase = c * kChunk;
        int g = advance_group(s_offs, G, 0, cbase + 8 * t);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int e0 = cbase + 8 * (i * kThreads + t);
            const bool inb = e0 < cols;
            v[i] = inb ? load_seg(xr, e0, cols) : make_uint4(0u, 0u, 0u, 0u);
            g = advance_group(s_offs, G, g, e0);
            const bool fast = inb && g < G && e0 + 8 <= s_offs[g] && e0 + 8 <= cols;
            const uint32_t m = fast ? fold2(absmax_u4(v[i])) : 0u;
            const int gw = __builtin_amdgcn_readfirstlane(g);
            const bool mine = fast && g == gw;
            const uint32_t wm = wave_max(mine ? m : 0u);
            if (lane == 0 && gw < G && wm != 0u)
                atomicMax(&s_amax[gw], wm);
            if (fast && !mine) {
                atomicMax(&s_amax[g], m);
            } else if (inb && !fast) {
                int gj = g;
#pragma unroll 1
                for (int j = 0; j < 8 && e0 + j < cols; ++j) {
                    gj = advance_group(s_offs, G, gj, e0 + j);
                    if (gj < G)
                        atomicMax(&s_amax[gj], elem8_bits(v[i], j) & 0x7fffu);
                }
            }
        }
    }
    __syncthreads();

    for (int g = t; g < G; g += kThreads) {
        const float s = fp32_scale(s_amax[g]);
        s_scale[g] = s;
        scales[row * ss_r + (int64_t)g * ss_g] = s;
    }
    __syncthreads();

    // pass 2: scale and store, last chunk first (it is still in registers)
    for (int c = nchunks - 1; c >= 0; --c) {
        const int cbase = c * kChunk;
        int g = advance_group(s_offs, G, 0, cbase + 8 * t);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int e0 = cbase + 8 * (i * kThreads + t);
            const bool inb = e0 < cols;
            if (c != nchunks - 1 && inb)
                v[i] = load_seg(xr, e0, cols);
            g = advance_group(s_offs, G, g, e0);
            if (!inb)
                continue;
            const bool fast = g < G && e0 + 8 <= s_offs[g] && e0 + 8 <= cols;
            if (fast) {
                st8(qr + e0, quant8(v[i], s_scale[g]));
            } else {
                int gj = g;
#pragma unroll 1
                for (int j = 0; j < 8 && e0 + j < cols; ++j) {
                    gj = advance_group(s_offs, G, gj, e0 + j);
                    if (gj < G)
                        qr[e0 + j] = (uint8_t)cvt1(elem8(v[i], j) * s_scale[gj]);
                }
            }
        }
    }
}

// --------------------------------------------------------------- strided

// x: (rows, cols), row r at x + r*ldx, unit column stride, cols % 8 == 0.
// q: column-major, element (r, c) at q[c*ldq + r].
// scales[g*ss_g + c*ss_c].
// Grid: G * nstrips workgroups; CG column groups of 8 per wave.
template <int CG>
__global__ __launch_bounds__(kThreads) void jagged_strided_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, int rows, int cols,
    const int32_t *__restrict__ offs, int G, uint8_t *__restrict__ q, int64_t ldq,
    float *__restrict__ scales, int64_t ss_g, int64_t ss_c, int nstrips)
{
    constexpr int QD = 64 / CG;       // 16-row blocks per wave
    constexpr int WROWS = 16 * QD;    // rows per wave
    constexpr int TROWS = 4 * WROWS;  // rows per workgroup pass
    constexpr int SW = 8 * CG;        // strip width in columns

    __shared__ int s_group;
    __shared__ uint32_t s_red[4][SW];
    __shared__ float s_scale[SW];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = t >> 6;
    const int cg = lane % CG;
    const int qd = lane / CG;

    const int rank = blockIdx.x / nstrips;
    const int strip = blockIdx.x % nstrips;

    // largest group first (ties by index) when G is small enough to rank here
    if (G <= 64) {
        if (t < G) {
            auto len = [&](int g) {
                int lo = g == 0 ? 0 : offs[g - 1];
                int hi = offs[g];
                lo = lo < 0 ? 0 : (lo > rows ? rows : lo);
                hi = hi < lo ? lo : (hi > rows ? rows : hi);
                return hi - lo;
            };
            const int mine = len(t);
            int r = 0;
            for (int h = 0; h < G; ++h) {
                const int lh = len(h);
                r += (lh > mine) || (lh == mine && h < t);
            }
            if (r == rank)
                s_group = t;
        }
    } else if (t == 0) {
        s_group = rank;
    }
    __syncthreads();
    const int g = s_group;

    int lo = g == 0 ? 0 : offs[g - 1];
    int hi = offs[g];
    lo = lo < 0 ? 0 : (lo > rows ? rows : lo);
    hi = hi < lo ? lo : (hi > rows ? rows : hi);

    const int cbase = strip * SW + 8 * cg;
    const bool col_ok = cbase < cols;
    const int rbeg = lo & ~15;
    const int nit = hi > lo ? (hi - rbeg + TROWS - 1) / TROWS : 0;

    uint4 v[16];
    auto load_tile = [&](int it) {
        const int rb = rbeg + it * TROWS + w * WROWS + 16 * qd;
        const bool full = rb >= lo && rb + 16 <= hi;
        const uint16_t *p = x + (int64_t)rb * ldx + cbase;
        if (col_ok && full) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                v[i] = ld16(p + (int64_t)i * ldx);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = rb + i;
                v[i] = (col_ok && r >= lo && r < hi) ? ld16(p + (int64_t)i * ldx)
                                                      : make_uint4(0u, 0u, 0u, 0u);
            }
        }
    };

    // pass 1: per-column amax over the group's rows
    uint32_t mx[4] = {0u, 0u, 0u, 0u};
    for (int it = 0; it < nit; ++it) {
        load_tile(it);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            mx[0] = absmax2(mx[0], v[i].x);
            mx[1] = absmax2(mx[1], v[i].y);
            mx[2] = absmax2(mx[2], v[i].z);
            mx[3] = absmax2(mx[3], v[i].w);
        }
    }
#pragma unroll
    for (int d = 0; d < 4; ++d)
        mx[d] = strided_pkmax<CG>(mx[d]);
    if (qd == 0) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            s_red[w][8 * cg + 2 * d] = mx[d] & 0xffffu;
            s_red[w][8 * cg + 2 * d + 1] = mx[d] >> 16;
        }
    }
    __syncthreads();
    if (t < SW) {
        const uint32_t a = umax(umax(s_red[0][t], s_red[1][t]), umax(s_red[2][t], s_red[3][t]));
        const float s = fp32_scale(a);
        s_scale[t] = s;
        const int c = strip * SW + t;
        if (c < cols)
            scales[(int64_t)g * ss_g + (int64_t)c * ss_c] = s;
    }
    __syncthreads();

    float sc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        sc[j] = s_scale[8 * cg + j];

    // pass 2: scale, transpose in registers, store 16-byte column pieces;
    // the last pass-1 tile is still in registers
    for (int it = nit - 1; it >= 0; --it) {
        if (it != nit - 1)
            load_tile(it);
        if (!col_ok)
            continue;
        const int rb = rbeg + it * TROWS + w * WROWS + 16 * qd;
        const bool full = rb >= lo && rb + 16 <= hi;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint4 o;
            o.x = cvt4(elem8(v[0], j) * sc[j], elem8(v[1], j) * sc[j], elem8(v[2], j) * sc[j],
                       elem8(v[3], j) * sc[j]);
            o.y = cvt4(elem8(v[4], j) * sc[j], elem8(v[5], j) * sc[j], elem8(v[6], j) * sc[j],
                       elem8(v[7], j) * sc[j]);
            o.z = cvt4(elem8(v[8], j) * sc[j], elem8(v[9], j) * sc[j], elem8(v[10], j) * sc[j],
                       elem8(v[11], j) * sc[j]);
            o.w = cvt4(elem8(v[12], j) * sc[j], elem8(v[13], j) * sc[j], elem8(v[14], j) * sc[j],
                       elem8(v[15], j) * sc[j]);
            uint8_t *p = q + (int64_t)(cbase + j) * ldq + rb;
            if (full) {
                st16(p, o);
            } else {
                const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = rb + i;
                    if (r >= lo && r < hi)
                        p[i] = (uint8_t)(ow[i >> 2] >> (8 * (i & 3)));
                }
            }
        }
    }
}

}  // namespace mxq
