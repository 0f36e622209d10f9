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
//    on an 8-element boundary, else the one or two aligned 16-byte chunks
//    that cover the piece, shifted), a workgroup covers 64 block slots x RW rows,
//    loads all RW rows before reducing, and reduces each block with a
//    quad-lane DPP max.  Pieces off 8-byte boundaries are stored as aligned
//    8-byte words shared with the neighbouring lane's piece.
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

// Elements sh .. sh + pn - 1 of the 16 bf16 values in lo (elements 0..7)
// and hi (8..15), as an 8-element piece whose elements past pn are zero
// (0 <= sh < 8, 1 <= pn <= 8): 64-bit funnel shifts and a mask, no indexed
// register access.
__device__ __forceinline__ uint4 shift_piece(const uint4 &lo, const uint4 &hi, int sh, int pn)
{
    const uint64_t q0 = ((uint64_t)lo.y << 32) | lo.x, q1 = ((uint64_t)lo.w << 32) | lo.z;
    const uint64_t q2 = ((uint64_t)hi.y << 32) | hi.x, q3 = ((uint64_t)hi.w << 32) | hi.z;
    const bool up = sh >= 4;
    const uint64_t a = up ? q1 : q0, b = up ? q2 : q1, c = up ? q3 : q2;
    const int s = 16 * (sh & 3);
    uint64_t o0 = s ? (a >> s) | (b << (64 - s)) : a;
    uint64_t o1 = s ? (b >> s) | (c << (64 - s)) : b;
    o0 &= pn >= 4 ? ~0ull : (1ull << (16 * pn)) - 1;
    o1 &= pn >= 8 ? ~0ull : pn > 4 ? (1ull << (16 * (pn - 4))) - 1 : 0ull;
    return make_uint4((uint32_t)o0, (uint32_t)(o0 >> 32), (uint32_t)o1, (uint32_t)(o1 >> 32));
}

// 16-byte values as two 64-bit halves, moved by whole bytes (0 < s < 16).
// bytes_up: byte j of the result is byte j - s of v (0 below s).
// bytes_down: byte j of the result is byte j + s of v (0 from 16 - s).
__device__ __forceinline__ uint4 bytes_up(const uint4 &v, int s)
{
    const uint64_t a = ((uint64_t)v.y << 32) | v.x, b = ((uint64_t)v.w << 32) | v.z;
    uint64_t ra, rb;
    if (s < 8) {
        ra = a << (8 * s);
        rb = (b << (8 * s)) | (s ? a >> (64 - 8 * s) : 0ull);
    } else {
        ra = 0ull;
        rb = a << (8 * (s - 8));
    }
    return make_uint4((uint32_t)ra, (uint32_t)(ra >> 32), (uint32_t)rb, (uint32_t)(rb >> 32));
}
__device__ __forceinline__ uint4 bytes_down(const uint4 &v, int s)
{
    const uint64_t a = ((uint64_t)v.y << 32) | v.x, b = ((uint64_t)v.w << 32) | v.z;
    uint64_t ra, rb;
    if (s < 8) {
        ra = (a >> (8 * s)) | (s ? b << (64 - 8 * s) : 0ull);
        rb = b >> (8 * s);
    } else {
        ra = b >> (8 * (s - 8));
        rb = 0ull;
    }
    return make_uint4((uint32_t)ra, (uint32_t)(ra >> 32), (uint32_t)rb, (uint32_t)(rb >> 32));
}

// Bytes [from, to) of the 16-byte value v (byte k at base[k], base 16-byte
// aligned), 0 <= from <= to <= 16, as aligned pieces of 1, 2, 4 and 8 bytes
// (at most four stores on each side of the aligned middle).
__device__ __forceinline__ void put16_range(uint8_t *base, const uint4 &v, int from, int to)
{
    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
    int k = from;
    if ((k & 1) && k < to) {
        base[k] = (uint8_t)(wd[k >> 2] >> (8 * (k & 3)));
        k += 1;
    }
    if ((k & 2) && k + 2 <= to) {
        *reinterpret_cast<uint16_t *>(base + k) = (uint16_t)(wd[k >> 2] >> (8 * (k & 3)));
        k += 2;
    }
    if ((k & 4) && k + 4 <= to) {
        *reinterpret_cast<uint32_t *>(base + k) = wd[k >> 2];
        k += 4;
    }
    if (k + 8 <= to) {
        *reinterpret_cast<uint2 *>(base + k) = make_uint2(wd[k >> 2], wd[(k >> 2) + 1]);
        k += 8;
    }
    if (k + 4 <= to) {
        *reinterpret_cast<uint32_t *>(base + k) = wd[k >> 2];
        k += 4;
    }
    if (k + 2 <= to) {
        *reinterpret_cast<uint16_t *>(base + k) = (uint16_t)(wd[k >> 2] >> (8 * (k & 3)));
        k += 2;
    }
    if (k < to)
        base[k] = (uint8_t)(wd[k >> 2] >> (8 * (k & 3)));
}

// Bytes [from, to) of w (byte k of w at base[k]), one byte store each: the
// ends of a run of contiguous pieces.
__device__ __forceinline__ void put_bytes(uint8_t *base, uint64_t w, int from, int to)
{
#pragma unroll
    for (int k = 0; k < 8; ++k)
        if (k >= from && k < to)
            base[k] = (uint8_t)(w >> (8 * k));
}

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
    // other pieces inside the row's whole 8-element chunks: the one or two
    // aligned chunks that cover them, shifted into place (only a piece that
    // reaches into a partial last chunk is read element by element)
    const bool tail = pn > 0 && p0 + pn > (cols & ~7);
    const bool shifted = pn > 0 && !fast && !tail;
    const int a0 = p0 & ~7, sh = p0 & 7;
    // Stores of pieces off 8-byte boundaries.  Within a group the pieces of
    // consecutive lanes are contiguous, so a lane whose piece runs from
    // a0 + sh into the next aligned word [a0 + 8, a0 + 16) writes that whole
    // word, its last sh bytes followed by the next lane's first 8 - sh
    // (`joined`), when the next lane's piece continues it far enough; the
    // next lane then leaves its first word alone.  Bytes at the ends of such
    // runs (group ends, the wave's last lane) go out one by one.
    const int lane = t & 63;
    const int p0n = (int)from_next_lane((uint32_t)p0), pnn = (int)from_next_lane((uint32_t)pn);
    const bool joined = sh > 0 && pn == 8 && lane < 63 && p0n == p0 + 8 && pnn >= 8 - sh;
    const bool prev_joined = __shfl_up(joined ? 1 : 0, 1, 64) != 0 && lane > 0;

    // Loads: every fast or shifted lane reads the aligned chunk at a0 of
    // each row.  A shifted piece that reaches past it (sh + pn > 8) needs the
    // chunk at a0 + 8 too, which the next lane has read when its piece
    // continues this one (its a0 is a0 + 8): taken from it by a lane
    // shuffle, else (group ends, the wave's last lane) read here, issued with
    // the first loads.  The second chunk lies before cols & ~7 as well.
    const bool chunk = fast || shifted;
    const bool chunk_next = from_next_lane(chunk ? 1u : 0u) != 0u;
    const bool need_hi = shifted && sh + pn > 8;
    const bool own_hi = need_hi && !(lane < 63 && chunk_next && (p0n & ~7) == a0 + 8);
    // wave-uniform: waves with no shifted piece (or no joined store) skip
    // the exchanges
    const bool wave_shifted = __ballot(shifted) != 0;
    const bool wave_joined = __ballot(joined) != 0;
    uint4 v[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        const int r = r0 + i;
        v[i] = (chunk && r < rows) ? ld16_nt(x + (int64_t)r * ldx + a0) : make_uint4(0u, 0u, 0u, 0u);
    }
    if (wave_shifted) {
        uint4 h[RW];
#pragma unroll
        for (int i = 0; i < RW; ++i) {
            const int r = r0 + i;
            h[i] = (own_hi && r < rows) ? ld16_nt(x + (int64_t)r * ldx + a0 + 8) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int i = 0; i < RW; ++i) {
            uint4 hi;
            hi.x = from_next_lane(v[i].x);
            hi.y = from_next_lane(v[i].y);
            hi.z = from_next_lane(v[i].z);
            hi.w = from_next_lane(v[i].w);
            if (own_hi)
                hi = h[i];
            if (shifted)
                v[i] = shift_piece(v[i], hi, sh, pn);
        }
    }
    if (tail) {
        // a piece that reaches into the row's partial last chunk
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
        const uint2 o = quant8(v[i], s);
        uint64_t nxt = 0u;
        if (wave_joined)
            nxt = (uint64_t)from_next_lane(o.x) | ((uint64_t)from_next_lane(o.y) << 32);
        if (r >= rows || pn == 0)
            continue;
        if (l == 0)
            scales[(int64_t)r * ss_r + (int64_t)j * ss_b] = (uint8_t)code;
        uint8_t *qr = q + (int64_t)r * ldq;
        if (fast) {
            st8_nt(qr + p0, o);
        } else {
            const uint64_t pw = (uint64_t)o.x | ((uint64_t)o.y << 32);
            // the piece's bytes in the word at a0: positions sh .. sh + pn - 1, up to 7
            if (!prev_joined)
                put_bytes(qr + a0, pw << (8 * sh), sh, sh + pn < 8 ? sh + pn : 8);
            // the rest, in the word at a0 + 8 (positions 0 .. sh + pn - 9; sh > 0 here)
            if (sh + pn > 8) {
                const uint64_t rest = pw >> (64 - 8 * sh);
                if (joined) {
                    const uint64_t wd = rest | (nxt << (8 * sh));
                    st8(qr + a0 + 8, make_uint2((uint32_t)wd, (uint32_t)(wd >> 32)));
                } else
                    put_bytes(qr + a0 + 8, rest, 0, sh + pn - 8);
            }
        }
    }
}

// Column jj of a lane's 16 rows x 8 columns, times s, as 16 e4m3 bytes
// (row i in byte i); SAT as in cvt4_sel
template <bool SAT>
__device__ __forceinline__ uint4 tile_column_bytes(const uint4 (&v)[16], int jj, float s)
{
    uint4 o;
    o.x = cvt4_sel<SAT>(elem8(v[0], jj) * s, elem8(v[1], jj) * s, elem8(v[2], jj) * s, elem8(v[3], jj) * s);
    o.y = cvt4_sel<SAT>(elem8(v[4], jj) * s, elem8(v[5], jj) * s, elem8(v[6], jj) * s, elem8(v[7], jj) * s);
    o.z = cvt4_sel<SAT>(elem8(v[8], jj) * s, elem8(v[9], jj) * s, elem8(v[10], jj) * s, elem8(v[11], jj) * s);
    o.w = cvt4_sel<SAT>(elem8(v[12], jj) * s, elem8(v[13], jj) * s, elem8(v[14], jj) * s,
                        elem8(v[15], jj) * s);
    return o;
}

// Column-major e4m3 stores (q + c * ldq + r) of one lane's 16 rows x 8
// columns of a 128-row tile anchored at a group start: rows rb .. rb + 15
// (rb < hi, the group end), columns c0 .. c0 + 7, each value times its
// column's multiplier sc[j], clamped to +-448 when SAT (e8m0 multipliers)
// and not otherwise (fp32 multipliers, see cvt4_nosat).  The 8 lanes of a
// column (lane bits 3..5, qd) hold the tile's consecutive 16-row pieces;
// every lane of the tile that holds rows of the group calls this.
template <bool SAT>
__device__ __forceinline__ void store_tile_columns(const uint4 (&v)[16], const float (&sc)[8],
                                                   uint8_t *__restrict__ q, int64_t ldq, int c0,
                                                   int rb, int hi, int qd)
{
    // A group start off a 16-row boundary (sh = rb mod 16, the same for
    // every lane of the tile): the 8 lanes of a column (lane bits 3..5) hold
    // consecutive 16-row pieces, so a lane stores the aligned 16-byte word
    // that holds its last sh rows and the next lane's first 16 - sh rows
    // (`joined`, when all of them lie in the group); the first lane's head
    // and the last lane's tail, and pieces at the group's end, go out as
    // aligned parts.
    const int sh = rb & 15;
    if (sh != 0) {
        const int nval = hi - rb;   // this lane's rows inside the group (>= 1)
        const bool joined = qd < 7 && rb + 32 - sh <= hi;
        const bool prev_joined = qd > 0 && rb + 16 - sh <= hi;
        uint8_t *qa = q + (int64_t)c0 * ldq + (rb - sh);   // 16-byte aligned
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const uint4 o = tile_column_bytes<SAT>(v, jj, sc[jj]);
            // the next lane's piece of this column (used only when joined,
            // i.e. when that lane holds rows of the group and is active)
            uint4 nx;
            nx.x = (uint32_t)__shfl_down((int)o.x, 8, 64);
            nx.y = (uint32_t)__shfl_down((int)o.y, 8, 64);
            nx.z = (uint32_t)__shfl_down((int)o.z, 8, 64);
            nx.w = (uint32_t)__shfl_down((int)o.w, 8, 64);
            uint8_t *p = qa + (int64_t)jj * ldq;
            if (!prev_joined)
                put16_range(p, bytes_up(o, sh), sh, sh + nval < 16 ? sh + nval : 16);
            if (nval > 16 - sh) {
                // the word after: this lane's last rows, then the next lane's first
                const uint4 lo = bytes_down(o, 16 - sh), hi2 = bytes_up(nx, sh);
                const uint4 w2 = make_uint4(lo.x | hi2.x, lo.y | hi2.y, lo.z | hi2.z, lo.w | hi2.w);
                if (joined)
                    st16(p + 16, w2);
                else
                    put16_range(p + 16, w2, 0, nval - (16 - sh) < sh ? nval - (16 - sh) : sh);
            }
        }
        return;
    }

    const bool full = rb + 16 <= hi;
    uint8_t *qp = q + (int64_t)c0 * ldq + rb;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
        const uint4 o = tile_column_bytes<SAT>(v, jj, sc[jj]);
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

    // this workgroup's group g (tile tid of the tile count), its first tile
    // pt_g and first 32-row block pb_g, and its rows [lo, hi)
    int g, pt_g, pb_g, lo, hi;
    if (G <= 64) {
        // every wave builds the table in registers (lane l holds group l)
        // and finds g by a ballot: no barrier and no LDS round trip before
        // the loads
        const bool valid = lane < G;
        int e = valid ? offs[lane] : rows;
        e = e < 0 ? 0 : (e > rows ? rows : e);
        int el = __shfl_up(e, 1, 64);
        el = lane == 0 ? 0 : el;
        const int n = valid && e > el ? e - el : 0;
        const int ut = units_of<7>(n), ub = units_of<5>(n);
        int it = ut, ib = ub;   // inclusive prefixes
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int yt = __shfl_up(it, d, 64);
            const int yb = __shfl_up(ib, d, 64);
            if (lane >= d) {
                it += yt;
                ib += yb;
            }
        }
        if (tid >= __builtin_amdgcn_readlane(it, 63))
            return;
        g = (int)__popcll(__ballot(it <= tid));   // groups whose tiles all precede tile tid
        pt_g = __builtin_amdgcn_readlane(it - ut, g);
        pb_g = __builtin_amdgcn_readlane(ib - ub, g);
        lo = __builtin_amdgcn_readlane(el, g);
        hi = __builtin_amdgcn_readlane(e, g);
    } else {
        load_group_ends<kJmxThreads>(offs, G, rows, s_end);
        slot_prefix2<kJmxThreads>(G, s_pt, s_pb,
                                  [&](int gg) { return units_of<7>(group_len(s_end, gg)); },
                                  [&](int gg) { return units_of<5>(group_len(s_end, gg)); });
        if (tid >= s_pt[G])
            return;
        g = find_slot(s_pt, G, tid);
        pt_g = s_pt[g];
        pb_g = s_pb[g];
        lo = g ? s_end[g - 1] : 0;
        hi = s_end[g];
    }
    const int k = tid - pt_g;
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
        const int64_t jb = (int64_t)pb_g + 4 * k + (qd >> 1);
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

    store_tile_columns<true>(v, sc, q, ldq, c0, rb, hi, qd);
}

}  // namespace mxq
