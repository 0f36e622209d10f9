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
//    (column strip, item), an item being one long group or a pack of
//    consecutive short groups.  Each lane holds a 16-row x 8-column sub-tile
//    loaded as sixteen 16-byte row pieces, so a load instruction reads whole
//    row segments and, after the scale is applied per column, the lane owns
//    16 consecutive bytes of each of its 8 output columns: the transpose to
//    column-major happens inside the lane's registers and every store is a
//    16-byte piece of a contiguous column run.  Long groups come first,
//    largest first (ranked on the device from the offsets).
#pragma once

#include "group_tables.hpp"
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

// The groups of NQ elements at once: g[q] = the number of ends s_offs[j]
// <= e[q] (j < G), i.e. the group holding element e[q] for non-decreasing
// ends (G past the last end), always in [0, G].  A fixed-step search
// (powers of two from the largest <= G down to 1) advanced for all queries
// together, so each step's NQ LDS reads are independent and overlap, where
// one search after another would wait on every read in turn.
template <int NQ>
__device__ __forceinline__ void groups_of(const int32_t *s_offs, int G, const int (&e)[NQ], int (&g)[NQ])
{
    int step = 1;
    while (2 * step <= G)
        step *= 2;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
        g[q] = 0;
    for (; step > 0; step >>= 1) {
        int v[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int p = g[q] + step;
            v[q] = s_offs[(p <= G ? p : G) - 1];
        }
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int p = g[q] + step;
            g[q] = (p <= G && v[q] <= e[q]) ? p : g[q];
        }
    }
}

// ---------------------------------------------------------------- contig

// Per-segment group bookkeeping of the contig kernels.  A segment is the
// 8 elements [e0, e0 + 8) one lane loads with one 16-byte access.
struct SegInfo {
    int g;       // group of element e0 (G if e0 is past every group)
    bool inb;    // e0 < cols
    bool fast;   // the whole segment lies inside group g (and inside cols)
};

// the segment [e0, e0 + 8) given g, the group of element e0
__device__ __forceinline__ SegInfo seg_info_at(const int32_t *s_offs, int G, int g, int e0, int cols)
{
    SegInfo si;
    si.inb = e0 < cols;
    si.g = g;
    si.fast = si.inb && si.g < G && e0 + 8 <= s_offs[si.g] && e0 + 8 <= cols;
    return si;
}

__device__ __forceinline__ SegInfo seg_info(const int32_t *s_offs, int G, int g_hint, int e0, int cols)
{
    return seg_info_at(s_offs, G, advance_group(s_offs, G, g_hint, e0), e0, cols);
}

// Element j of a segment that is not wholly inside one group: from the
// segment's registers by a select of one 64-bit half and a shift (no
// indexed register access, so nothing goes to scratch memory), except in a row's partial
// last segment, which the loads return as zeros and which is read again
// from memory.
__device__ __forceinline__ uint32_t seg_elem(const uint16_t *xr, const uint4 &v, int e0, int j,
                                             int cols)
{
    if (e0 + 8 > cols)
        return (uint32_t)xr[e0 + j];
    const uint64_t lo = ((uint64_t)v.y << 32) | v.x, hi = ((uint64_t)v.w << 32) | v.z;
    return (uint32_t)((j < 4 ? lo : hi) >> (16 * (j & 3))) & 0xffffu;
}

// Reduce, element by element, a segment that is not wholly inside one group.
__device__ __forceinline__ void reduce_segment_elementwise(uint32_t *s_amax, const int32_t *s_offs,
                                                           int G, const uint16_t *xr, const uint4 &v,
                                                           const SegInfo &si, int e0, int cols)
{
    int gj = si.g;
#pragma unroll 1
    for (int j = 0; j < 8 && e0 + j < cols; ++j) {
        gj = advance_group(s_offs, G, gj, e0 + j);
        if (gj < G)
            atomicMax(&s_amax[gj], seg_elem(xr, v, e0, j, cols) & 0x7fffu);
    }
}

// A segment with exactly one group boundary inside: elements [0, b) in its
// own group g, [b, 8) in group g2 (or in no group when g2 == G), packed as
// b | 8 | g2 << 4, worked out once per workgroup (the boundaries are the same
// for every row); 0 for any other segment.
__device__ __forceinline__ uint32_t segment_split(const int32_t *s_offs, int G, const SegInfo &si,
                                                  int e0, int cols)
{
    if (!si.inb || si.fast || si.g >= G || e0 + 8 > cols)
        return 0u;
    const int b = s_offs[si.g] - e0;   // group g ends inside the segment
    if (b <= 0 || b >= 8)
        return 0u;
    const int g2 = advance_group(s_offs, G, si.g + 1, e0 + b);
    if (g2 < G && s_offs[g2] < e0 + 8)
        return 0u;   // a second boundary inside: element by element
    return (uint32_t)b | 8u | ((uint32_t)g2 << 4);
}

// The group of every element of a segment that is not wholly inside one
// group, for the many-groups kernel: nibble j = (group of element j) - (group
// of element 0), 0..14 (groups are ordered, so the nibbles never decrease; a
// group index of G or more means no group); worked out once per workgroup.
// 0 for a whole segment or one past every group; kSegByElement for a
// segment reduced and stored element by element (the row's partial last
// segment, or more than 14 groups inside 8 elements).
constexpr uint32_t kSegByElement = 0xFFFFFFFFu;

// A segment_groups word with one boundary inside (two groups): the boundary
// b (its first element of the second group) and the second group's offset
// d; false for more boundaries.  The nibbles never decrease and nibble 0 is
// 0, so b is the lowest nonzero nibble and d the top one.
__device__ __forceinline__ bool one_boundary(uint32_t sg, int &b, int &d)
{
    b = __builtin_ctz(sg) >> 2;
    d = (int)(sg >> 28);
    return sg == (((uint32_t)d * 0x11111111u) << (4 * b));
}
__device__ __forceinline__ uint32_t segment_groups(const int32_t *s_offs, int G, const SegInfo &si,
                                                   int e0, int cols)
{
    if (!si.inb || si.fast || si.g >= G)
        return 0u;
    if (e0 + 8 > cols)
        return kSegByElement;
    // each group end p inside the segment (0 < p < 8) moves elements p..7 on
    // by one group: one LDS read per end, at most 14 ends (no nibble carries)
    uint32_t d = 0u;
    int n = 0;
#pragma unroll 1
    for (int g = si.g; g < G; ++g) {
        const int p = s_offs[g] - e0;
        if (p >= 8)
            break;
        if (++n > 14)
            return kSegByElement;
        d += 0x11111111u << (4 * p);
    }
    return d;
}

// the two maxima of a split segment (sp = segment_split(...) != 0)
__device__ __forceinline__ void reduce_split_inl(uint32_t *s_amax, int G, uint4 v, int g1, uint32_t sp)
{
    const int b = (int)(sp & 7u), g2 = (int)(sp >> 4);
    uint32_t m1 = 0u, m2 = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t a = elem8_bits(v, j) & 0x7fffu;
        if (j < b)
            m1 = a > m1 ? a : m1;
        else
            m2 = a > m2 ? a : m2;
    }
    if (m1 != 0u)
        atomicMax(&s_amax[g1], m1);
    if (g2 < G && m2 != 0u)
        atomicMax(&s_amax[g2], m2);
}

// Scale and store a split segment: each element times its own group's
// multiplier (every element is within its group's amax, so no clamp is
// needed); 8 bytes at once unless the second part lies past the last group.
__device__ __forceinline__ void store_split_inl(uint8_t *qr, const float *s_scale, int G, uint4 v,
                                                int g1, uint32_t sp, int e0)
{
    const int b = (int)(sp & 7u), g2 = (int)(sp >> 4);
    const float s1 = s_scale[g1], s2 = g2 < G ? s_scale[g2] : 0.0f;
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        y[j] = elem8(v, j) * (j < b ? s1 : s2);
    uint2 o;
    o.x = cvt4_nosat(y[0], y[1], y[2], y[3]);
    o.y = cvt4_nosat(y[4], y[5], y[6], y[7]);
    if (g2 < G) {
        st8_nt(qr + e0, o);
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < b)
                qr[e0 + j] = (uint8_t)((j < 4 ? o.x : o.y) >> (8 * (j & 3)));
    }
}

// Out-of-line forms for the few-groups kernels, where inlined they would
// take registers from the common path (128 VGPRs, four waves per SIMD) and
// spill; a call costs the caller a wait for all its outstanding loads, which
// the many-groups kernel, where split segments are common, cannot afford
// (it reduces and stores them inline, in its own form).
__device__ __attribute__((noinline)) void reduce_split(uint32_t *s_amax, int G, uint4 v, int g1,
                                                       uint32_t sp)
{
    reduce_split_inl(s_amax, G, v, g1, sp);
}

__device__ __attribute__((noinline)) void store_split(uint8_t *qr, const float *s_scale, int G,
                                                      uint4 v, int g1, uint32_t sp, int e0)
{
    store_split_inl(qr, s_scale, G, v, g1, sp, e0);
}

// Reduce one segment's |x| max into s_amax for every group it touches.
// `uni`: the caller knows every lane of the wave has a fast segment of the
// same group gw (one wave max, one atomic); otherwise lanes are grouped by a
// ballot loop (lanes hold consecutive segments, so few iterations), and the
// segments that straddle a group boundary take their split or per-element
// atomics.
__device__ __forceinline__ void reduce_segment(uint32_t *s_amax, const int32_t *s_offs, int G,
                                               const uint16_t *xr, const uint4 &v, const SegInfo &si,
                                               int e0, int cols, bool uni, int gw_uni, int lane,
                                               uint32_t sp)
{
    const uint32_t m = si.fast ? fold2(absmax_u4(v)) : 0u;
    if (uni) {
        const uint32_t wm = wave_max(m);
        if (lane == 0 && wm != 0u)
            atomicMax(&s_amax[gw_uni], wm);
        return;
    }
    bool pending = si.fast;
#pragma unroll 1
    while (true) {
        const uint64_t mask = __ballot(pending);
        if (mask == 0)
            break;
        const int first = __ffsll((unsigned long long)mask) - 1;
        const int gw = __builtin_amdgcn_readlane(si.g, first);
        const bool mine = pending && si.g == gw;
        const uint32_t wm = wave_max(mine ? m : 0u);
        if (lane == first && wm != 0u)
            atomicMax(&s_amax[gw], wm);
        pending = pending && !mine;
    }
    if (sp != 0u)
        reduce_split(s_amax, G, v, si.g, sp);
    else if (si.inb && !si.fast && si.g < G)
        reduce_segment_elementwise(s_amax, s_offs, G, xr, v, si, e0, cols);
}

// Scale and store one segment (row-major q row qr) in the few-groups kernel.
__device__ __forceinline__ void store_segment(uint8_t *qr, const float *s_scale, const int32_t *s_offs,
                                              int G, const uint16_t *xr, const uint4 &v,
                                              const SegInfo &si, int e0, int cols, uint32_t sp)
{
    if (!si.inb || si.g >= G)
        return;
    if (si.fast) {
        st8_nt(qr + e0, quant8_fp32scale(v, s_scale[si.g]));
        return;
    }
    if (sp != 0u) {
        store_split(qr, s_scale, G, v, si.g, sp, e0);
        return;
    }
    int gj = si.g;
#pragma unroll 1
    for (int j = 0; j < 8 && e0 + j < cols; ++j) {
        gj = advance_group(s_offs, G, gj, e0 + j);
        if (gj < G)
            qr[e0 + j] = (uint8_t)cvt1(__uint_as_float(seg_elem(xr, v, e0, j, cols) << 16) *
                                       s_scale[gj]);
    }
}

// Scale and store one segment in the many-groups kernel (sg = its
// segment_groups word): whole segments and segments with group boundaries
// inside share one 8-byte store, each element times its own group's
// multiplier, so a wave whose lanes hold both kinds issues one store per
// slot; elements past the last group are left alone (byte stores for such a
// segment), and kSegByElement segments go element by element.
__device__ __forceinline__ void store_segment_seg(uint8_t *qr, const float *s_scale, const int32_t *s_offs,
                                                  int G, const uint16_t *xr, const uint4 &v,
                                                  const SegInfo &si, int e0, int cols, uint32_t sg)
{
    if (!si.inb || si.g >= G)
        return;
    if (sg != kSegByElement) {
        float y[8];
        uint32_t valid = 0u;
        if (si.fast) {
            const float sa = s_scale[si.g];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                y[j] = elem8(v, j) * sa;
            valid = 0xFFu;
        } else {
            int b, d;
            if (one_boundary(sg, b, d)) {
                const float sa = s_scale[si.g];
                const bool second = si.g + d < G;
                const float sb = second ? s_scale[si.g + d] : 0.0f;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    y[j] = elem8(v, j) * (j < b ? sa : sb);
                valid = second ? 0xFFu : (1u << b) - 1u;
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int g = si.g + (int)((sg >> (4 * j)) & 15u);
                    y[j] = g < G ? elem8(v, j) * s_scale[g] : 0.0f;
                    valid |= g < G ? 1u << j : 0u;
                }
            }
        }
        uint2 o;
        o.x = cvt4_nosat(y[0], y[1], y[2], y[3]);
        o.y = cvt4_nosat(y[4], y[5], y[6], y[7]);
        if (valid == 0xFFu) {
            st8_nt(qr + e0, o);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if ((valid >> j) & 1u)
                    qr[e0 + j] = (uint8_t)((j < 4 ? o.x : o.y) >> (8 * (j & 3)));
        }
        return;
    }
    int gj = si.g;
#pragma unroll 1
    for (int j = 0; j < 8 && e0 + j < cols; ++j) {
        gj = advance_group(s_offs, G, gj, e0 + j);
        if (gj < G)
            qr[e0 + j] = (uint8_t)cvt1(__uint_as_float(seg_elem(xr, v, e0, j, cols) << 16) * s_scale[gj]);
    }
}

// x row r at x + r*ldx (unit column stride); q row r at q + r*ldq;
// scales[r*ss_r + g*ss_g].  Dynamic LDS: 3*G words.  cols <= 2048*NR.
//
// Persistent: workgroup b handles rows b, b + gridDim.x, ...  A row is one
// register chunk (NR 16-byte segments per lane, segment i of lane t at
// columns 8*(256*i + t)), so the group of every segment is the same for all
// rows: it is worked out once per workgroup, together with which
// (wave, segment-slot) pairs are uniform.  Two register buffers alternate:
// the loads of the next row are in flight while the current row is reduced,
// scaled and stored.
//
// SEG (many groups, chosen on the host from G): the wave slots that hold
// several groups would take the general reduction; instead every lane
// writes its segment maxima to its wave's part of LDS, and lane l then
// folds NR consecutive entries of its own wave (NR consecutive segments of
// one slot, NR*8 columns) into runs of one group, with one LDS atomic per
// run; a wave's LDS operations complete in order, so this needs no
// workgroup barrier.  A segment with group boundaries inside enters the fold
// with the elements of its first group and sends each later group's
// elements to it by one atomic; its per-element groups (segment_groups) are
// worked out once per workgroup, like the group of each folded segment.
// Dynamic LDS: 3*G words, rounded up to 4, plus NR*256 words of segment
// maxima (SEG) and NR*256 words of per-segment boundary words (SEG:
// segment_groups, else segment_split) for every lane's segments.
template <int NR, bool SEG>
__device__ __forceinline__ void jagged_contig_body(
    const uint16_t *__restrict__ x, int64_t ldx, int rows, int cols,
    const int32_t *__restrict__ offs, int G, uint8_t *__restrict__ q, int64_t ldq,
    float *__restrict__ scales, int64_t ss_r, int64_t ss_g)
{
    extern __shared__ uint32_t smem[];
    int32_t *s_offs = reinterpret_cast<int32_t *>(smem);
    uint32_t *s_amax = smem + G;
    float *s_scale = reinterpret_cast<float *>(smem + 2 * G);
    uint32_t *s_seg = smem + ((3 * G + 3) & ~3);   // SEG: NR*256 segment maxima in column order
    uint32_t *s_split = s_seg + (SEG ? NR * kThreads : 0);   // NR*256 boundary words

    const int t = threadIdx.x;
    const int lane = t & 63;

    // The row is read through a buffer descriptor whose range is the row's
    // whole 8-element segments: a segment past them (the partial last one
    // included) and every segment of a row past the last one (range 0) read
    // as zeros without a memory access, so the loads carry no branch.  Only
    // segments that lie wholly inside one group are used from registers; the
    // others are read again element by element where they are reduced and
    // stored.  With loads under branches the compiler waits for every
    // outstanding load at the first use of any, i.e. for the next row's loads
    // too, and the two buffers would not overlap.
    auto load_row = [&](uint4 (&d)[NR], int r) __attribute__((always_inline)) {
        const bool ok = r < rows;
        const auto rs = buffer_rsrc(x + (int64_t)(ok ? r : 0) * ldx, ok ? 2u * (uint32_t)(cols & ~7) : 0u);
#pragma unroll
        for (int i = 0; i < NR; ++i)
            d[i] = ldbuf16_nt(rs, 16u * (uint32_t)(i * kThreads + t));
    };

    uint4 va[NR], vb[NR];
    int row = blockIdx.x;
    // the offsets are loaded before the first row: loads retire in order, so
    // an offsets load issued after the row would wait for the whole row, and
    // the group bookkeeping below (and with it the next row's loads) with it
    // Threads past the last group store the last group's entry again (the
    // same value): an unconditional use keeps the compiler from sinking the
    // load below the row's loads.
    const int g_first = t < G ? t : G - 1;
    const int o_first = offs[g_first];
    load_row(va, row);   // the grid never exceeds the row count
    s_offs[g_first] = o_first < 0 ? 0 : (o_first > cols ? cols : o_first);
    s_amax[g_first] = 0u;
    for (int g = t + kThreads; g < G; g += kThreads) {
        const int o = offs[g];
        s_offs[g] = o < 0 ? 0 : (o > cols ? cols : o);
        s_amax[g] = 0u;
    }
    __syncthreads();

    // the groups of this lane's segments (and, SEG, of the NR consecutive
    // segments it folds, see fold_seg below), all searched at once
    const int wv = t >> 6;
    const int fold_seg = 256 * ((NR * lane) / 64) + 64 * wv + (NR * lane) % 64;
    constexpr int NQ = SEG ? 2 * NR : NR;
    int gq[NQ];
    {
        int eq[NQ];
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            eq[i] = 8 * (i * kThreads + t);
            if constexpr (SEG)
                eq[NR + i] = 8 * (fold_seg + i);
        }
        groups_of<NQ>(s_offs, G, eq, gq);
    }

    SegInfo si[NR];
    uint32_t uni = 0u;   // bit i: every lane of this wave has a fast segment i of one group
    bool lane_fast = true;  // every segment of this lane is fast
    int gw[NR];
    {
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int e0 = 8 * (i * kThreads + t);
            si[i] = seg_info_at(s_offs, G, gq[i], e0, cols);
            s_split[i * kThreads + t] = SEG ? segment_groups(s_offs, G, si[i], e0, cols)
                                            : segment_split(s_offs, G, si[i], e0, cols);
            gw[i] = __builtin_amdgcn_readfirstlane(si[i].g);
            const bool same = si[i].fast && si[i].g == gw[i];
            if (__ballot(same) == ~0ull)
                uni |= 1u << i;
            lane_fast = lane_fast && si[i].fast;
        }
    }
    // SEG: every lane of the wave has only whole segments
    const bool wave_fast = __ballot(!lane_fast) == 0ull;

    // SEG: groups of this thread's NR consecutive segments (G where a
    // segment is not wholly inside one group: those are reduced element by
    // element by the lane that loads them)
    int sgv[SEG ? NR : 1];
    auto sg = [&](int j) __attribute__((always_inline)) { return sgv[j]; };
    // the folded entries NR*lane + j of this wave: slot (NR*lane + j) / 64,
    // lane (NR*lane + j) % 64 of that slot, i.e. segment fold_seg + j
    if constexpr (SEG) {
#pragma unroll
        for (int j = 0; j < NR; ++j)
            sgv[j] = 8 * (fold_seg + j) < cols ? gq[NR + j] : G;   // the group of the segment's first element
    }

    auto process_row = [&](uint4 (&cur)[NR], uint4 (&nxt)[NR], int r) __attribute__((always_inline)) {
        load_row(nxt, r + (int)gridDim.x);   // range 0 past the last row
        const uint16_t *xr = x + (int64_t)r * ldx;
        if constexpr (SEG) {
            uint32_t *const wseg = s_seg + wv * (NR * 64);   // this wave's entries
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                // a whole segment's max, or the max of the elements in the
                // segment's first group (the fold's group for the entry); the
                // elements of each later group go to it by one atomic per
                // group; kSegByElement segments reduce element by element and
                // contribute 0 here
                uint32_t m = 0u;
                if (si[i].fast) {
                    m = fold2(absmax_u4(cur[i]));
                } else if (si[i].inb && si[i].g < G) {
                    const uint32_t sg = s_split[i * kThreads + t];
                    int b, d;
                    if (sg != kSegByElement && one_boundary(sg, b, d)) {
                        uint32_t m2 = 0u;
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const uint32_t a = elem8_bits(cur[i], j) & 0x7fffu;
                            if (j < b)
                                m = a > m ? a : m;
                            else
                                m2 = a > m2 ? a : m2;
                        }
                        if (si[i].g + d < G && m2 != 0u)
                            atomicMax(&s_amax[si[i].g + d], m2);
                    } else if (sg != kSegByElement) {
                        uint32_t acc = 0u;
                        int run = 0;
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const int dj = (int)((sg >> (4 * j)) & 15u);
                            const uint32_t a = elem8_bits(cur[i], j) & 0x7fffu;
                            if (dj == 0) {
                                m = a > m ? a : m;
                            } else {
                                if (dj != run) {
                                    if (run > 0 && acc != 0u && si[i].g + run < G)
                                        atomicMax(&s_amax[si[i].g + run], acc);
                                    acc = 0u;
                                    run = dj;
                                }
                                acc = a > acc ? a : acc;
                            }
                        }
                        if (run > 0 && acc != 0u && si[i].g + run < G)
                            atomicMax(&s_amax[si[i].g + run], acc);
                    } else {
                        reduce_segment_elementwise(s_amax, s_offs, G, xr, cur[i], si[i],
                                                   8 * (i * kThreads + t), cols);
                    }
                }
                wseg[i * 64 + lane] = m;
            }
            // this wave's writes are done before its reads (LDS operations of
            // a wave complete in order; the wait and the memory clobber keep
            // the compiler from moving the reads above the writes)
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
            __asm__ __volatile__("" ::: "memory");
            uint32_t m[NR];
            if constexpr (NR % 4 == 0) {
#pragma unroll
                for (int j = 0; j < NR; j += 4) {
                    const uint4 w4 = *reinterpret_cast<const uint4 *>(wseg + NR * lane + j);
                    m[j] = w4.x;
                    m[j + 1] = w4.y;
                    m[j + 2] = w4.z;
                    m[j + 3] = w4.w;
                }
            } else {
#pragma unroll
                for (int j = 0; j < NR; ++j)
                    m[j] = wseg[NR * lane + j];
            }
            uint32_t acc = m[0];
#pragma unroll
            for (int j = 1; j < NR; ++j) {
                if (sg(j) == sg(j - 1)) {
                    acc = umax(acc, m[j]);
                } else {
                    if (acc != 0u && sg(j - 1) < G)
                        atomicMax(&s_amax[sg(j - 1)], acc);
                    acc = m[j];
                }
            }
            if (acc != 0u && sg(NR - 1) < G)
                atomicMax(&s_amax[sg(NR - 1)], acc);
        } else if (uni == (1u << NR) - 1u) {
            // every slot uniform: all wave maxima first (independent chains),
            // then one lane merges consecutive slots of the same group and
            // issues one LDS atomic per run
            uint32_t wm[NR];
#pragma unroll
            for (int i = 0; i < NR; ++i)
                wm[i] = wave_max(fold2(absmax_u4(cur[i])));
            if (lane == 0) {
                uint32_t acc = wm[0];
#pragma unroll
                for (int i = 1; i < NR; ++i) {
                    if (gw[i] == gw[i - 1]) {
                        acc = umax(acc, wm[i]);
                    } else {
                        if (acc != 0u)
                            atomicMax(&s_amax[gw[i - 1]], acc);
                        acc = wm[i];
                    }
                }
                if (acc != 0u)
                    atomicMax(&s_amax[gw[NR - 1]], acc);
            }
        } else {
            // a group boundary falls inside this wave's window of some slot:
            // uniform slots keep the single wave max, the others take the
            // general path
#pragma unroll
            for (int i = 0; i < NR; ++i)
                reduce_segment(s_amax, s_offs, G, xr, cur[i], si[i], 8 * (i * kThreads + t), cols,
                               (uni >> i) & 1u, gw[i], lane, si[i].fast ? 0u : s_split[i * kThreads + t]);
        }
        __syncthreads();
        // scales; s_amax is reset for the next row, whose atomics come after
        // the barrier below
        for (int g = t; g < G; g += kThreads) {
            const float s = fp32_scale(s_amax[g]);
            s_amax[g] = 0u;
            s_scale[g] = s;
            scales[(int64_t)r * ss_r + (int64_t)g * ss_g] = s;
        }
        __syncthreads();
        uint8_t *qr = q + (int64_t)r * ldq;
        if (SEG ? wave_fast : lane_fast) {
            float sc[NR];
#pragma unroll
            for (int i = 0; i < NR; ++i)
                sc[i] = s_scale[si[i].g];
#pragma unroll
            for (int i = 0; i < NR; ++i)
                st8_nt(qr + 8 * (i * kThreads + t), quant8_fp32scale(cur[i], sc[i]));
        } else if constexpr (SEG) {
#pragma unroll
            for (int i = 0; i < NR; ++i)
                store_segment_seg(qr, s_scale, s_offs, G, xr, cur[i], si[i], 8 * (i * kThreads + t), cols,
                                  si[i].fast ? 0u : s_split[i * kThreads + t]);
        } else {
#pragma unroll
            for (int i = 0; i < NR; ++i)
                store_segment(qr, s_scale, s_offs, G, xr, cur[i], si[i], 8 * (i * kThreads + t), cols,
                              si[i].fast ? 0u : s_split[i * kThreads + t]);
        }
    };

    while (row < rows) {
        process_row(va, vb, row);
        row += gridDim.x;
        if (row >= rows)
            break;
        process_row(vb, va, row);
        row += gridDim.x;
    }
}

// The few-groups kernel is held to four waves per SIMD (the persistent grid
// runs four workgroups per CU; 128 VGPRs, nothing spilled); the many-groups
// kernel needs more registers and runs three workgroups per CU.
template <int NR>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void jagged_contig_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, int rows, int cols,
    const int32_t *__restrict__ offs, int G, uint8_t *__restrict__ q, int64_t ldq,
    float *__restrict__ scales, int64_t ss_r, int64_t ss_g)
{
    jagged_contig_body<NR, false>(x, ldx, rows, cols, offs, G, q, ldq, scales, ss_r, ss_g);
}

template <int NR>
__global__ __launch_bounds__(kThreads) void jagged_contig_seg_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, int rows, int cols,
    const int32_t *__restrict__ offs, int G, uint8_t *__restrict__ q, int64_t ldq,
    float *__restrict__ scales, int64_t ss_r, int64_t ss_g)
{
    jagged_contig_body<NR, true>(x, ldx, rows, cols, offs, G, q, ldq, scales, ss_r, ss_g);
}

// Rows longer than one register chunk (cols > 2048*NR): one workgroup per
// row; the row is reduced chunk by chunk, then re-read for the scaling pass
// (last chunk first: it is still in registers).
template <int NR>
__global__ __launch_bounds__(kThreads) void jagged_contig_long_kernel(
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
    const uint16_t *xr = x + row * ldx;
    uint8_t *qr = q + row * ldq;
    constexpr int kChunk = 8 * kThreads * NR;
    const int nchunks = (cols + kChunk - 1) / kChunk;

    for (int g = t; g < G; g += kThreads) {
        int o = offs[g];
        s_offs[g] = o < 0 ? 0 : (o > cols ? cols : o);
        s_amax[g] = 0u;
    }
    __syncthreads();

    // chunks read through a descriptor over the row's whole 8-element
    // segments, as in jagged_contig_kernel: no load under a branch, and the
    // partial last segment (never used from registers) reads as zeros
    uint4 v[NR];
    const auto rs = buffer_rsrc(xr, 2u * (uint32_t)(cols & ~7));
    auto load_chunk = [&](int cbase) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NR; ++i)
            v[i] = ldbuf16(rs, 2u * ((uint32_t)cbase + 8u * (uint32_t)(i * kThreads + t)));
    };

    for (int c = 0; c < nchunks; ++c) {
        const int cbase = c * kChunk;
        load_chunk(cbase);
        int g = advance_group(s_offs, G, 0, cbase + 8 * t);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int e0 = cbase + 8 * (i * kThreads + t);
            const SegInfo si = seg_info(s_offs, G, g, e0, cols);
            g = si.g;
            reduce_segment(s_amax, s_offs, G, xr, v[i], si, e0, cols, false, 0, lane, 0u);
        }
    }
    __syncthreads();
    for (int g = t; g < G; g += kThreads) {
        const float s = fp32_scale(s_amax[g]);
        s_scale[g] = s;
        scales[row * ss_r + (int64_t)g * ss_g] = s;
    }
    __syncthreads();
    for (int c = nchunks - 1; c >= 0; --c) {
        const int cbase = c * kChunk;
        if (c != nchunks - 1)
            load_chunk(cbase);
        int g = advance_group(s_offs, G, 0, cbase + 8 * t);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int e0 = cbase + 8 * (i * kThreads + t);
            const SegInfo si = seg_info(s_offs, G, g, e0, cols);
            g = si.g;
            store_segment(qr, s_scale, s_offs, G, xr, v[i], si, e0, cols, 0u);
        }
    }
}

// --------------------------------------------------------------- strided

// Colwise work items, per column strip.  A long group (16-row-aligned span
// over TROWS rows) is one item; its workgroup reads up to T tiles into
// registers and streams the rest.  Short groups (empty ones included) are
// packed: the consecutive short groups whose starts fall in one TROWS-row
// block, at most kPackMax of them, make one item.  A pack spans fewer than
// 2*TROWS rows, so it is read once into registers; each wave reduces its
// rows with shuffles when they all belong to one group and with per-lane
// segments otherwise, merging into per-group column maxima in LDS.  Every
// item owns at least one group, so a strip has at most G items.  Long
// groups come first, largest first when G <= 64 (ranked on the device by
// one wave, lane g holding group g), then the packs in group order.
constexpr int kPackMax = 64;

// Split path (a caller's workspace): a long group's 16-row-aligned span
// [lo & ~15, hi) is cut into nc = ceil(span / CH) chunks of
// csz = round16(ceil(span / nc)) <= CH rows (the last one shorter), each
// chunk an item of its own that holds its rows in registers; the chunks of
// one (group, strip) exchange their column maxima through the workspace, so
// no row is read twice.
__device__ __forceinline__ int chunk_count(int lo, int hi, int ch)
{
    const int span = hi - (lo & ~15);
    return (span + ch - 1) / ch;
}
__device__ __forceinline__ int chunk_rows(int lo, int hi, int nc)
{
    const int span = hi - (lo & ~15);
    return ((span + nc - 1) / nc + 15) & ~15;
}

// Workspace of the split path: one set of kSetWords 32-bit words per
// (long group, column strip), addressed by the group's first item index:
// the strip's column maxima (|bf16| bit patterns, at most 64 words), the
// arrival count (word 64) and the departure count (word 65).  Zero between
// calls: the last chunk to leave a set clears it.
constexpr int kSetWords = 72;
constexpr int kSetArrive = 64;
constexpr int kSetDepart = 65;

// Split path without a workspace: the chunks of a (group, strip) exchange
// each column's maximum through that column's own fp32 scale slot of the
// group, zeroed beforehand by jagged_colwise_clear_kernel.  While the
// exchange runs a slot holds the column maximum (|bf16| bits, bits 0-14),
// the arrival count (bits 15-23) and the departure count (bits 24-31); an
// arrival merges the maximum and counts itself in one compare-and-swap, and
// the last chunk to leave writes the scale over the word.  So a group may
// have at most 255 chunks (the host checks the extent).
constexpr uint32_t kSlotMax = 0x7FFFu;
constexpr uint32_t kSlotArrive = 1u << 15;
constexpr uint32_t kSlotDepart = 1u << 24;
constexpr int kSlotMaxChunks = 255;
__device__ __forceinline__ uint32_t slot_arrivals(uint32_t w) { return (w >> 15) & 0x1FFu; }

// Zeroes the scale slots the workspace-free split path exchanges through:
// every column of each group cut into more than one chunk of ch rows (the
// main kernel's rule: clamped ends, span from the 16-row-aligned start).
// Grid (column blocks, G); 256 threads.
__global__ __launch_bounds__(256) void jagged_colwise_clear_kernel(
    const int32_t *__restrict__ offs, int G, int rows, int cols, float *__restrict__ scales,
    int64_t ss_g, int64_t ss_c, int ch)
{
    const int g = blockIdx.y;
    auto clamp_end = [&](int e) { return e < 0 ? 0 : (e > rows ? rows : e); };
    const int lo = g ? clamp_end(offs[g - 1]) : 0;
    int hi = clamp_end(offs[g]);
    hi = hi < lo ? lo : hi;
    if (chunk_count(lo, hi, ch) <= 1)
        return;
    for (int c = blockIdx.x * 256 + threadIdx.x; c < cols; c += gridDim.x * 256)
        scales[(int64_t)g * ss_g + (int64_t)c * ss_c] = 0.0f;
}

// Workgroup -> (item, column strip).  SPS = 8 / CG strips of 8*CG columns
// (16*CG bytes of a row) make one 128-byte "superstrip"; the SPS workgroups
// of a superstrip get block ids that differ by 8, so with the round-robin
// placement of workgroups on the 8 XCDs they share one XCD (and its L2) and
// are dispatched back to back: their row pieces complete each other's cache
// lines.  Superstrips are numbered item-major.
struct StripMap {
    int item, strip;
    bool valid;
};

template <int SPS>
__device__ __forceinline__ StripMap map_strip(int b, int nsuper, int max_items)
{
    const int x = b & 7;               // XCD slot
    const int k = b >> 3;
    const int sub = k % SPS;           // strip within the superstrip
    const int S = (k / SPS) * 8 + x;   // logical superstrip index
    StripMap m;
    m.item = S / nsuper;
    m.strip = (S % nsuper) * SPS + sub;
    m.valid = m.item < max_items;
    return m;
}

// Per-workgroup item table for G > 64 (NTH threads), all in LDS: s_end
// (clamped group ends), s_lead (1 for a group that starts a pack), s_lpre /
// s_ppre (exclusive prefix counts of long groups / pack leaders by group
// index; long groups then go in index order).  TR = rows per tile.
// In split mode (CH > 0) s_lpre counts a long group's chunks instead of 1.
template <int NTH, int TR, int CH>
__device__ void strided_table(const int32_t *__restrict__ offs, int G, int rows, int *s_end,
                              uint8_t *s_lead, int *s_lpre, int *s_ppre)
{
    load_group_ends<NTH>(offs, G, rows, s_end);
    auto lo_of = [&](int g) { return g ? s_end[g - 1] : 0; };
    auto is_long = [&](int g) {
        const int lo = lo_of(g), hi = s_end[g];
        return hi > lo && hi - (lo & ~15) > TR;
    };
    // run starts: a run of short groups breaks at a long group and where the
    // start moves to another TR-row block; inclusive max-scan of the breaks
    {
        __shared__ int s_wmax[NTH / 64];
        const int t = threadIdx.x, lane = t & 63, w = t >> 6;
        const int ch = (G + NTH - 1) / NTH;
        const int s0 = t * ch;
        auto brk = [&](int g) {
            return (g == 0 || is_long(g) || is_long(g - 1) || lo_of(g) / TR != lo_of(g - 1) / TR)
                       ? g : -1;
        };
        int m = -1;
        for (int k = 0; k < ch; ++k)
            if (s0 + k < G)
                m = max(m, brk(s0 + k));
        int inc = m;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(inc, d, 64);
            if (lane >= d)
                inc = max(inc, y);
        }
        if (lane == 63)
            s_wmax[w] = inc;
        __syncthreads();
        int run = __shfl_up(inc, 1, 64);
        if (lane == 0)
            run = -1;
        for (int ww = 0; ww < w; ++ww)
            run = max(run, s_wmax[ww]);
        for (int k = 0; k < ch; ++k) {
            const int g = s0 + k;
            if (g < G) {
                run = max(run, brk(g));
                s_lead[g] = (!is_long(g) && ((g - run) % kPackMax) == 0) ? 1 : 0;
            }
        }
        __syncthreads();
    }
    slot_prefix2<NTH>(G, s_lpre, s_ppre,
                      [&](int g) {
                          if (!is_long(g))
                              return 0;
                          return CH > 0 ? chunk_count(lo_of(g), s_end[g], CH) : 1;
                      },
                      [&](int g) { return (int)s_lead[g]; });
}

// x: (rows, cols), row r at x + r*ldx, unit column stride, cols % 8 == 0.
// q: column-major, element (r, c) at q[c*ldq + r].
// scales[g*ss_g + c*ss_c].
// Each lane holds a 16-row x 8-column piece; a wave stacks 64/CG pieces
// down the rows and CG across; NW waves stack down the rows, so one
// register tile covers TROWS = NW*16*64/CG rows x 8*CG columns.  Up to T
// tiles stay resident: a long group of at most T*TROWS rows is read from
// HBM once; longer groups stream their tiles beyond the first T-1 through
// the last buffer and re-read them in the scaling pass.
// Grid: 8 * (8/CG) * ceil(G * nsuper / 8) workgroups (see map_strip);
// dynamic LDS (3G + 2) * 4 + G bytes when G > 64, none otherwise.
// q is written with plain stores: a group's column runs start at its first
// row, so a 128-byte output line at a group boundary (or any line, when q
// itself is off the lines) is written in parts by two store instructions;
// L2 merges the parts, where nontemporal partial writes would each cost HBM
// a read-modify-write (55.5 against 52.2 us on the MoE x operand, 72 against
// 52 us with q 16 bytes off the lines).
//
// SPLIT: long groups come as chunks of at most T tiles (see chunk_count),
// so every row is read once; the chunks of one (group, strip) publish their
// column maxima to the workspace `ws` with device-scope atomics, count their
// arrival, wait for the others (at most spin_limit polls; past it, or at
// once for a negative limit, a chunk reduces its group's rows of the strip
// itself, which is always correct),
// and count their departure; the last to leave clears the set.  Chunks of a
// set have consecutive item numbers, and workgroups are dispatched in order,
// so the waits are short.  max_items: the grid's item bound.
template <int CG, int T, int NW, bool SPLIT = false>
__global__ __launch_bounds__(64 * NW) void jagged_strided_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, int rows, int cols,
    const int32_t *__restrict__ offs, int G, uint8_t *__restrict__ q, int64_t ldq,
    float *__restrict__ scales, int64_t ss_g, int64_t ss_c, int nsuper, int max_items,
    uint32_t *__restrict__ ws, int spin_limit)
{
    constexpr int QD = 64 / CG;       // 16-row pieces per wave
    constexpr int WROWS = 16 * QD;    // rows per wave
    constexpr int TROWS = NW * WROWS; // rows per register tile
    constexpr int SW = 8 * CG;        // strip width in columns
    constexpr int NTH = 64 * NW;
    constexpr int CH = SPLIT ? T * TROWS : 0;   // rows per chunk of a long group
    static_assert(T >= 2, "a pack spans up to two tiles");
    static_assert(SW + 2 <= kSetWords, "a strip's maxima and two counters fit a set");
    static_assert(!SPLIT || CG == 8, "split mode numbers workgroups one strip per superstrip");

    // group tables: 64 ends in static LDS; for G > 64 the launch passes
    // (3G + 2) ints and G bytes of dynamic LDS.  Little LDS lets the next
    // workgroup on a CU start while this one's last waves drain.
    __shared__ int s_end64[64];
    extern __shared__ int s_dyn[];
    int *const s_end = G <= 64 ? s_end64 : s_dyn;
    int *const s_lpre = s_dyn + G;
    int *const s_ppre = s_dyn + 2 * G + 1;
    uint8_t *const s_lead = reinterpret_cast<uint8_t *>(s_dyn + 3 * G + 2);
    __shared__ uint32_t s_red[NW][SW];
    __shared__ float s_scale[SW];
    __shared__ uint32_t s_pk[kPackMax][SW];   // pack: column maxima, then multipliers

    const StripMap sm = map_strip<8 / CG>(blockIdx.x, nsuper, max_items);
    if (!sm.valid)
        return;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = t >> 6;
    const int cg = lane % CG;
    const int qd = lane / CG;

    // this workgroup's item: a long group g (in split mode: its chunk k, and
    // the group's first item number, which names its workspace set), or a
    // pack of short groups [g0, g1)
    __shared__ int s_sel[4];
    if (G <= 64) {
        // one wave builds the table with lane g holding group g
        if (w == 0) {
            const bool valid = lane < G;
            int hi = valid ? offs[lane] : rows;
            hi = hi < 0 ? 0 : (hi > rows ? rows : hi);
            int lo = __shfl_up(hi, 1, 64);
            lo = lane == 0 ? 0 : lo;
            if (valid)
                s_end[lane] = hi;
            const int len = hi > lo ? hi - lo : 0;
            const bool lng = valid && hi > lo && hi - (lo & ~15) > TROWS;
            const int blk = lo / TROWS;
            const int pblk = __shfl_up(blk, 1, 64);
            const int plng = __shfl_up(lng ? 1 : 0, 1, 64);
            int run = (valid && (lane == 0 || lng || plng || blk != pblk)) ? lane : -1;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int y = __shfl_up(run, d, 64);
                if (lane >= d)
                    run = max(run, y);
            }
            const bool lead = valid && !lng && ((lane - run) % kPackMax) == 0;
            const uint64_t mlong = __ballot(lng);
            const uint64_t mlead = __ballot(lead);
            // items of each long group: 1, or its chunks in split mode
            const int nch = lng ? (SPLIT ? chunk_count(lo, hi, CH) : 1) : 0;
            int nl = nch;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1)
                nl += __shfl_xor(nl, d, 64);
            const int item = sm.item;
            if (item < nl) {
                // long groups in rank order: longer first, ties by index; the
                // group's first item is the count of items ranked before it
                int first = 0;
                for (int h = 0; h < G; ++h) {
                    const int lh = __builtin_amdgcn_readlane(len, h);
                    const int nh = __builtin_amdgcn_readlane(nch, h);
                    const bool hl = (mlong >> h) & 1ull;
                    first += (hl && ((lh > len) || (lh == len && h < lane))) ? nh : 0;
                }
                if (lng && first <= item && item < first + nch) {
                    s_sel[0] = 0;
                    s_sel[1] = lane;
                    s_sel[2] = item - first;
                    s_sel[3] = first;
                }
            } else if (lane == 0) {
                int k = item - nl;
                uint64_t m = mlead;
                while (k > 0 && m) {
                    m &= m - 1;
                    --k;
                }
                if (!m) {
                    s_sel[0] = 2;   // no such item
                } else {
                    const int g0 = __ffsll((unsigned long long)m) - 1;
                    const uint64_t after = g0 + 1 < 64 ? ~0ull << (g0 + 1) : 0ull;
                    const uint64_t stop = (mlead | mlong) & after;
                    s_sel[0] = 1;
                    s_sel[1] = g0;
                    s_sel[2] = stop ? __ffsll((unsigned long long)stop) - 1 : G;
                }
            }
        }
        __syncthreads();
    } else if (G <= NTH) {
        // one group per thread (thread g holds group g): its flags stay in
        // registers, two scans run across the workgroup, and the thread that
        // owns this workgroup's item writes it (no search)
        __shared__ int s_wmax[NW], s_wa[NW], s_wb[NW], s_wfirst[NW];
        const bool valid = t < G;
        int hi = rows;
        if (valid) {
            const int e = offs[t];
            hi = e < 0 ? 0 : (e > rows ? rows : e);
            s_end[t] = hi;
        }
        __syncthreads();
        const int lo = (valid && t > 0) ? s_end[t - 1] : 0;
        const int lo_prev = (valid && t > 1) ? s_end[t - 2] : 0;   // start of group t - 1
        const bool lng = valid && hi > lo && hi - (lo & ~15) > TROWS;
        const bool lng_prev = valid && t > 0 && lo > lo_prev && lo - (lo_prev & ~15) > TROWS;
        const int brk =
            (valid && (t == 0 || lng || lng_prev || lo / TROWS != lo_prev / TROWS)) ? t : -1;
        // run start of group t: inclusive max-scan of the breaks
        int run = brk;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(run, d, 64);
            if (lane >= d)
                run = max(run, y);
        }
        if (lane == 63)
            s_wmax[w] = run;
        __syncthreads();
        for (int ww = 0; ww < w; ++ww)
            run = max(run, s_wmax[ww]);
        const bool lead = valid && !lng && ((t - run) % kPackMax) == 0;
        const int nch = lng ? (CH > 0 ? chunk_count(lo, hi, CH) : 1) : 0;
        // exclusive prefix counts of long-group items and of packs; the
        // first stop (pack leader or long group) after each group
        int ia = nch, ib = lead ? 1 : 0;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int ya = __shfl_up(ia, d, 64);
            const int yb = __shfl_up(ib, d, 64);
            if (lane >= d) {
                ia += ya;
                ib += yb;
            }
        }
        const uint64_t stops = __ballot(lead || lng);
        if (lane == 63) {
            s_wa[w] = ia;
            s_wb[w] = ib;
        }
        if (lane == 0)
            s_wfirst[w] = stops ? 64 * w + __ffsll((unsigned long long)stops) - 1 : G;
        __syncthreads();
        int ea = ia - nch, eb = ib - (lead ? 1 : 0), nlong = 0, npack = 0;
        for (int ww = 0; ww < NW; ++ww) {
            if (ww < w) {
                ea += s_wa[ww];
                eb += s_wb[ww];
            }
            nlong += s_wa[ww];
            npack += s_wb[ww];
        }
        const uint64_t above = lane < 63 ? stops & (~0ull << (lane + 1)) : 0ull;
        int next = above ? 64 * w + __ffsll((unsigned long long)above) - 1 : G;
        for (int ww = w + 1; ww < NW && !above; ++ww)
            if (s_wfirst[ww] < G) {
                next = s_wfirst[ww];
                break;
            }
        const int item = sm.item;
        if (lng && ea <= item && item < ea + nch) {
            s_sel[0] = 0;
            s_sel[1] = t;
            s_sel[2] = item - ea;
            s_sel[3] = ea;
        }
        if (lead && item == nlong + eb) {
            s_sel[0] = 1;
            s_sel[1] = t;
            s_sel[2] = next;
        }
        if (t == 0 && item >= nlong + npack)
            s_sel[0] = 2;
        __syncthreads();
    } else {
        strided_table<NTH, TROWS, CH>(offs, G, rows, s_end, s_lead, s_lpre, s_ppre);
        if (t == 0) {
            const int nlong = s_lpre[G], npack = s_ppre[G];
            if (sm.item < nlong) {
                const int g = find_slot(s_lpre, G, sm.item);
                s_sel[0] = 0;
                s_sel[1] = g;
                s_sel[2] = sm.item - s_lpre[g];
                s_sel[3] = s_lpre[g];
            } else if (sm.item < nlong + npack) {
                const int pk = sm.item - nlong;
                const int g0 = find_slot(s_ppre, G, pk);
                int g1 = pk + 1 < npack ? find_slot(s_ppre, G, pk + 1) : G;
                if (s_lpre[g0] < nlong) {
                    const int gl = find_slot(s_lpre, G, s_lpre[g0]);   // first long group after g0
                    g1 = gl < g1 ? gl : g1;
                }
                s_sel[0] = 1;
                s_sel[1] = g0;
                s_sel[2] = g1;
            } else {
                s_sel[0] = 2;
            }
        }
        __syncthreads();
    }
    const int kind = s_sel[0];
    if (kind == 2)
        return;

    if (kind == 1) {
        // ---- a pack of short groups [g0, g1)
        const int g0 = s_sel[1];
        const int g1 = s_sel[2];
        const int npk = g1 - g0;
        const int plo = g0 ? s_end[g0 - 1] : 0;
        int phi = s_end[g1 - 1];
        phi = phi < plo ? plo : phi;
        const int prb = plo & ~15;
        int nit = phi > plo ? (phi - prb + TROWS - 1) / TROWS : 0;
        nit = nit < T ? nit : T;
        const int cbase = sm.strip * SW + 8 * cg;
        const bool col_ok = cbase < cols;

        // group of row r inside the pack (rows before plo / at phi and after
        // have none): first g in [g0, g1) whose end is past r
        auto group_of = [&](int r) {
            int a = g0, b = g1;
            while (a < b) {
                const int m = (a + b) >> 1;
                if (s_end[m] <= r)
                    a = m + 1;
                else
                    b = m;
            }
            return a;
        };

        for (int e = t; e < npk * SW; e += NTH)
            s_pk[e / SW][e % SW] = 0u;

        uint4 v[T][16];
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
            if (tt < nit) {
                const int rb = prb + tt * TROWS + w * WROWS + 16 * qd;
                const uint16_t *p = x + (int64_t)rb * ldx + cbase;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = rb + i;
                    v[tt][i] = (col_ok && r >= plo && r < phi) ? ld16_nt(p + (int64_t)i * ldx)
                                                                : make_uint4(0u, 0u, 0u, 0u);
                }
            }
        }
        __syncthreads();   // s_pk cleared

        // reduce: per tile, a wave whose rows all lie in one group uses
        // shuffles; otherwise each lane merges its own row segments
        int ga[T], gb[T];   // group of the lane's first / last row in the pack (g1: none)
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
            ga[tt] = gb[tt] = g1;
            if (tt >= nit)
                continue;
            const int rb = prb + tt * TROWS + w * WROWS + 16 * qd;
            const int r0 = rb < plo ? plo : rb;
            const int r1 = (rb + 16 < phi ? rb + 16 : phi) - 1;
            if (r0 <= r1) {
                ga[tt] = group_of(r0);
                gb[tt] = group_of(r1);
            }
            const uint64_t has = __ballot(ga[tt] < g1);
            if (has == 0)
                continue;
            const int gw = __shfl(ga[tt], __ffsll((unsigned long long)has) - 1, 64);
            const bool uniform = __all(ga[tt] == g1 || (ga[tt] == gb[tt] && ga[tt] == gw));
            if (uniform) {
                uint32_t mx[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    mx[0] = absmax2(mx[0], v[tt][i].x);
                    mx[1] = absmax2(mx[1], v[tt][i].y);
                    mx[2] = absmax2(mx[2], v[tt][i].z);
                    mx[3] = absmax2(mx[3], v[tt][i].w);
                }
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    mx[d] = strided_pkmax<CG>(mx[d]);
                if (qd == 0 && col_ok) {
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        atomicMax(&s_pk[gw - g0][8 * cg + 2 * d], mx[d] & 0xffffu);
                        atomicMax(&s_pk[gw - g0][8 * cg + 2 * d + 1], mx[d] >> 16);
                    }
                }
            } else if (__all(ga[tt] == gb[tt])) {
                // every lane's rows in one group (16-row aligned groups):
                // the lane's column maxima, then a segmented max scan down
                // the wave's row pieces (lanes 8 apart, runs of one group),
                // so the last lane of each run issues its group's atomics
                const int gme = ga[tt];
                uint32_t mx[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    mx[0] = absmax2(mx[0], v[tt][i].x);
                    mx[1] = absmax2(mx[1], v[tt][i].y);
                    mx[2] = absmax2(mx[2], v[tt][i].z);
                    mx[3] = absmax2(mx[3], v[tt][i].w);
                }
                // every shuffle runs on all lanes (a lane shuffle reads 0
                // from a lane that is switched off), the tests after it
#pragma unroll
                for (int k = 1; k < 8; k <<= 1) {
                    const int gprev = __shfl_up(gme, 8 * k, 64);
                    const bool take = qd >= k && gprev == gme;
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const uint32_t pv = (uint32_t)__shfl_up((int)mx[d], 8 * k, 64);
                        mx[d] = take ? pkmax(mx[d], pv) : mx[d];
                    }
                }
                const int gnext = __shfl_down(gme, 8, 64);
                const bool last = qd == 7 || gnext != gme;
                if (last && gme < g1 && col_ok) {
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        atomicMax(&s_pk[gme - g0][8 * cg + 2 * d], mx[d] & 0xffffu);
                        atomicMax(&s_pk[gme - g0][8 * cg + 2 * d + 1], mx[d] >> 16);
                    }
                }
            } else if (ga[tt] < g1 && col_ok) {
                int gc = ga[tt];
                int next = s_end[gc];
                uint32_t acc[4] = {0u, 0u, 0u, 0u};
                auto flush = [&]() {
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        atomicMax(&s_pk[gc - g0][8 * cg + 2 * d], acc[d] & 0xffffu);
                        atomicMax(&s_pk[gc - g0][8 * cg + 2 * d + 1], acc[d] >> 16);
                        acc[d] = 0u;
                    }
                };
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = rb + i;
                    if (r >= plo && r < phi) {
                        if (r >= next) {
                            flush();
                            while (gc < g1 - 1 && s_end[gc] <= r)
                                ++gc;
                            next = s_end[gc];
                        }
                        acc[0] = absmax2(acc[0], v[tt][i].x);
                        acc[1] = absmax2(acc[1], v[tt][i].y);
                        acc[2] = absmax2(acc[2], v[tt][i].z);
                        acc[3] = absmax2(acc[3], v[tt][i].w);
                    }
                }
                flush();
            }
        }
        __syncthreads();
        for (int e = t; e < npk * SW; e += NTH) {
            const int k = e / SW, c = e % SW;
            const float s = fp32_scale(s_pk[k][c]);
            s_pk[k][c] = __float_as_uint(s);
            const int col = sm.strip * SW + c;
            if (col < cols)
                scales[(int64_t)(g0 + k) * ss_g + (int64_t)col * ss_c] = s;
        }
        __syncthreads();
        if (!col_ok)
            return;

#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
            if (tt >= nit || ga[tt] >= g1)
                continue;
            const int rb = prb + tt * TROWS + w * WROWS + 16 * qd;
            if (ga[tt] == gb[tt]) {
                float sc[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    sc[j] = __uint_as_float(s_pk[ga[tt] - g0][8 * cg + j]);
                const bool full = rb >= plo && rb + 16 <= phi;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    uint4 o;
                    o.x = cvt4_nosat(elem8(v[tt][0], j) * sc[j], elem8(v[tt][1], j) * sc[j],
                                     elem8(v[tt][2], j) * sc[j], elem8(v[tt][3], j) * sc[j]);
                    o.y = cvt4_nosat(elem8(v[tt][4], j) * sc[j], elem8(v[tt][5], j) * sc[j],
                                     elem8(v[tt][6], j) * sc[j], elem8(v[tt][7], j) * sc[j]);
                    o.z = cvt4_nosat(elem8(v[tt][8], j) * sc[j], elem8(v[tt][9], j) * sc[j],
                                     elem8(v[tt][10], j) * sc[j], elem8(v[tt][11], j) * sc[j]);
                    o.w = cvt4_nosat(elem8(v[tt][12], j) * sc[j], elem8(v[tt][13], j) * sc[j],
                                     elem8(v[tt][14], j) * sc[j], elem8(v[tt][15], j) * sc[j]);
                    uint8_t *pq = q + (int64_t)(cbase + j) * ldq + rb;
                    if (full) {
                        st16(pq, o);
                    } else {
                        const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
                        for (int i = 0; i < 16; ++i)
                            if (rb + i >= plo && rb + i < phi)
                                pq[i] = (uint8_t)(ow[i >> 2] >> (8 * (i & 3)));
                    }
                }
            } else if (rb >= plo && rb + 16 <= phi && s_end[gb[tt] - 1] == s_end[ga[tt]]) {
                // rows of two groups (any groups between them empty), all
                // inside the pack: the first b rows take group ga's
                // multipliers, the rest gb's; one 16-byte store per column
                const int b = s_end[ga[tt]] - rb;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float sa = __uint_as_float(s_pk[ga[tt] - g0][8 * cg + j]);
                    const float sb = __uint_as_float(s_pk[gb[tt] - g0][8 * cg + j]);
                    float y[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        y[i] = elem8(v[tt][i], j) * (i < b ? sa : sb);
                    uint4 o;
                    o.x = cvt4_nosat(y[0], y[1], y[2], y[3]);
                    o.y = cvt4_nosat(y[4], y[5], y[6], y[7]);
                    o.z = cvt4_nosat(y[8], y[9], y[10], y[11]);
                    o.w = cvt4_nosat(y[12], y[13], y[14], y[15]);
                    st16(q + (int64_t)(cbase + j) * ldq + rb, o);
                }
            } else {
                // rows of more groups, or rows outside the pack: per-row
                // multipliers, byte stores
                int gc = ga[tt];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = rb + i;
                    if (r < plo || r >= phi)
                        continue;
                    while (gc < g1 - 1 && s_end[gc] <= r)
                        ++gc;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float sj = __uint_as_float(s_pk[gc - g0][8 * cg + j]);
                        q[(int64_t)(cbase + j) * ldq + r] = (uint8_t)cvt1(elem8(v[tt][i], j) * sj);
                    }
                }
            }
        }
        return;
    }

    // ---- a long group (in split mode, chunk k of it)
    const int g = s_sel[1];
    const int lo = g ? s_end[g - 1] : 0;
    int hi = s_end[g];
    hi = hi < lo ? lo : hi;

    // rows this workgroup holds: [clo, chi) inside [lo, hi), tiles from rbeg
    int rbeg = lo & ~15, clo = lo, chi = hi, nc = 1, k = 0, strip = sm.strip;
    if constexpr (SPLIT) {
        // a long group's workgroups run strip-major over its chunks, so the
        // chunks of one (group, strip), which wait for each other, have
        // consecutive workgroup numbers (one strip per superstrip here)
        nc = chunk_count(lo, hi, CH);
        const int local = (sm.item - s_sel[3]) * nsuper + sm.strip;
        strip = local / nc;
        k = local % nc;
        const int csz = chunk_rows(lo, hi, nc);
        rbeg = (lo & ~15) + k * csz;
        clo = rbeg > lo ? rbeg : lo;
        chi = rbeg + csz < hi ? rbeg + csz : hi;
    }
    const int nit = chi > clo ? (chi - rbeg + TROWS - 1) / TROWS : 0;
    const int cbase = strip * SW + 8 * cg;
    const bool col_ok = cbase < cols;

    uint4 v[T][16];

    // one register tile: 16 rows x 8 columns per lane; rows outside
    // [clo, chi) are neither read nor counted.  Tiles that will be read
    // again (keep) use ordinary loads, the others the streaming hint.
    auto load_tile = [&](uint4 (&d)[16], int it, bool keep) {
        const int rb = rbeg + it * TROWS + w * WROWS + 16 * qd;
        const bool full = rb >= clo && rb + 16 <= chi;
        const uint16_t *p = x + (int64_t)rb * ldx + cbase;
        if (col_ok && full) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                d[i] = keep ? ld16(p + (int64_t)i * ldx) : ld16_nt(p + (int64_t)i * ldx);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = rb + i;
                d[i] = (col_ok && r >= clo && r < chi) ? ld16(p + (int64_t)i * ldx)
                                                        : make_uint4(0u, 0u, 0u, 0u);
            }
        }
    };
    auto accumulate = [&](uint32_t (&mx)[4], const uint4 (&d)[16]) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            mx[0] = absmax2(mx[0], d[i].x);
            mx[1] = absmax2(mx[1], d[i].y);
            mx[2] = absmax2(mx[2], d[i].z);
            mx[3] = absmax2(mx[3], d[i].w);
        }
    };
    auto store_tile = [&](const uint4 (&d)[16], int it, const float (&sc)[8]) {
        if (!col_ok)
            return;
        const int rb = rbeg + it * TROWS + w * WROWS + 16 * qd;
        const bool full = rb >= clo && rb + 16 <= chi;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint4 o;
            o.x = cvt4_nosat(elem8(d[0], j) * sc[j], elem8(d[1], j) * sc[j], elem8(d[2], j) * sc[j],
                       elem8(d[3], j) * sc[j]);
            o.y = cvt4_nosat(elem8(d[4], j) * sc[j], elem8(d[5], j) * sc[j], elem8(d[6], j) * sc[j],
                       elem8(d[7], j) * sc[j]);
            o.z = cvt4_nosat(elem8(d[8], j) * sc[j], elem8(d[9], j) * sc[j], elem8(d[10], j) * sc[j],
                       elem8(d[11], j) * sc[j]);
            o.w = cvt4_nosat(elem8(d[12], j) * sc[j], elem8(d[13], j) * sc[j], elem8(d[14], j) * sc[j],
                       elem8(d[15], j) * sc[j]);
            uint8_t *p = q + (int64_t)(cbase + j) * ldq + rb;
            if (full) {
                st16(p, o);
            } else {
                const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = rb + i;
                    if (r >= clo && r < chi)
                        p[i] = (uint8_t)(ow[i >> 2] >> (8 * (i & 3)));
                }
            }
        }
    };

    // pass 1: issue the loads of every resident tile, then reduce
    uint32_t mx[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int tt = 0; tt < T; ++tt)
        if (tt < nit)
            load_tile(v[tt], tt, !SPLIT && tt == T - 1 && nit > T);
#pragma unroll
    for (int tt = 0; tt < T; ++tt)
        if (tt < nit)
            accumulate(mx, v[tt]);
    if constexpr (!SPLIT) {
        // tiles beyond the register window stream through the last buffer
        for (int it = T; it < nit; ++it) {
            load_tile(v[T - 1], it, true);
            accumulate(mx, v[T - 1]);
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
    uint32_t acol = 0u;   // column t's maximum (t < SW)
    if (t < SW) {
#pragma unroll
        for (int ww = 0; ww < NW; ++ww)
            acol = umax(acol, s_red[ww][t]);
    }
    // in split mode without a workspace, column t's scale slot of group g
    // carries the exchange (see kSlotMax)
    const bool in_slots = SPLIT && nc > 1 && ws == nullptr;
    uint32_t *const slot =
        reinterpret_cast<uint32_t *>(scales + (int64_t)g * ss_g + (int64_t)(strip * SW + t) * ss_c);
    const bool has_col = t < SW && strip * SW + t < cols;
    if constexpr (SPLIT) {
        if (nc > 1) {
            // Every global access of the exchange hands its result to LDS
            // before the next barrier: a barrier does not wait for a
            // thread's outstanding global operations, only the use of their
            // results does, so this is what orders one thread's atomics
            // before another thread's arrival or departure.
            __shared__ int s_flag;
            __shared__ uint32_t s_col[SW];
            uint32_t *const set =
                ws ? ws + ((int64_t)s_sel[3] * nsuper + strip) * kSetWords : nullptr;
            if (in_slots) {
                static_assert(!SPLIT || SW == 64, "the slot exchange runs on wave 0, one lane per column");
                if (w == 0) {
                    // arrive: merge this chunk's maximum and count it in one
                    // compare-and-swap (each chunk changes a slot at most
                    // twice, so the loop ends), then poll until every chunk
                    // has arrived; a negative limit takes the fallback
                    // without looking, 0 looks once
                    bool done = true;
                    uint32_t cur = 0u;
                    if (has_col) {
                        cur = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        uint32_t want;
                        do {
                            want = ((cur & ~kSlotMax) + kSlotArrive) | umax(cur & kSlotMax, acol);
                        } while (!__hip_atomic_compare_exchange_strong(
                            slot, &cur, want, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_AGENT));
                        cur = want;
                        done = spin_limit >= 0 && slot_arrivals(cur) >= (uint32_t)nc;
                        for (int n = 0; !done && spin_limit >= 0 && n < spin_limit; ++n) {
                            __builtin_amdgcn_s_sleep(2);
                            cur = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            done = slot_arrivals(cur) >= (uint32_t)nc;
                        }
                    }
                    const bool all = __all(done);
                    s_col[t] = cur & kSlotMax;
                    if (t == 0)
                        s_flag = all ? 1 : 0;
                }
            } else {
                if (t < SW)
                    s_col[t] = umax(acol, __hip_atomic_fetch_max(set + t, acol, __ATOMIC_RELAXED,
                                                                 __HIP_MEMORY_SCOPE_AGENT));
                __syncthreads();   // all of this workgroup's maxima are in
                if (t == 0) {
                    __hip_atomic_fetch_add(set + kSetArrive, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    // a negative limit takes the fallback without looking
                    int n = 0;
                    bool all = false;
                    while (spin_limit >= 0 &&
                           !(all = __hip_atomic_load(set + kSetArrive, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT) >= (uint32_t)nc) &&
                           n < spin_limit) {
                        __builtin_amdgcn_s_sleep(2);
                        ++n;
                    }
                    s_flag = all ? 1 : 0;
                }
            }
            __syncthreads();
            if (s_flag) {
                if (!in_slots && t < SW)
                    s_col[t] = __hip_atomic_load(set + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
                // the other chunks did not arrive in time: reduce every row of
                // the group in this strip here (8 lanes per row, 16 bytes each)
                if (t < SW)
                    s_col[t] = 0u;
                __syncthreads();
                uint32_t m[4] = {0u, 0u, 0u, 0u};
                const int pc = t & 7;
                const int c0 = strip * SW + 8 * pc;
                if (c0 < cols) {
                    for (int r = lo + (t >> 3); r < hi; r += NTH / 8) {
                        const uint4 vv = ld16(x + (int64_t)r * ldx + c0);
                        m[0] = absmax2(m[0], vv.x);
                        m[1] = absmax2(m[1], vv.y);
                        m[2] = absmax2(m[2], vv.z);
                        m[3] = absmax2(m[3], vv.w);
                    }
                }
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    atomicMax(&s_col[8 * pc + 2 * d], m[d] & 0xffffu);
                    atomicMax(&s_col[8 * pc + 2 * d + 1], m[d] >> 16);
                }
            }
            __syncthreads();   // every read of the set has returned
            if (!in_slots) {
                if (t == 0) {
                    const uint32_t prev = __hip_atomic_fetch_add(set + kSetDepart, 1u, __ATOMIC_RELAXED,
                                                                 __HIP_MEMORY_SCOPE_AGENT);
                    s_flag = prev == (uint32_t)nc - 1 ? 2 : 0;
                }
                __syncthreads();
                if (s_flag == 2 && t < kSetWords)
                    __hip_atomic_store(set + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            if (t < SW)
                acol = s_col[t];
        }
    }
    if (t < SW) {
        const float s = fp32_scale(acol);
        s_scale[t] = s;
        if (in_slots) {
            // depart (this lane's reads of the slot have returned: their
            // values were used above); the last chunk out writes the scale
            if (has_col) {
                const uint32_t prev = __hip_atomic_fetch_add(slot, kSlotDepart, __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT);
                if ((prev >> 24) == (uint32_t)nc - 1)
                    __hip_atomic_store(slot, __float_as_uint(s), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        } else if (has_col && k == 0) {
            scales[(int64_t)g * ss_g + (int64_t)(strip * SW + t) * ss_c] = s;
        }
    }
    __syncthreads();

    float sc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        sc[j] = s_scale[8 * cg + j];

    // pass 2: scale, transpose in registers, store 16-byte column pieces
#pragma unroll
    for (int tt = 0; tt < T - 1; ++tt)
        if (tt < nit)
            store_tile(v[tt], tt, sc);
    if constexpr (SPLIT) {
        if (T - 1 < nit)
            store_tile(v[T - 1], T - 1, sc);
    } else {
        // the last buffer holds tile nit-1 (or T-1); walk the streamed tiles
        // backwards so the most recently read ones are re-read first
        for (int it = (nit > T ? nit : T) - 1; it >= T - 1; --it) {
            if (it >= nit)
                continue;
            if (it != nit - 1)
                load_tile(v[T - 1], it, true);
            store_tile(v[T - 1], it, sc);
        }
    }
}

}  // namespace mxq
