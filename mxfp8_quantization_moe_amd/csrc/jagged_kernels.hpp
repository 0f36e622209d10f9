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

// ---------------------------------------------------------------- contig

// Per-segment group bookkeeping of the contig kernels.  A segment is the
// 8 elements [e0, e0 + 8) one lane loads with one 16-byte access.
struct SegInfo {
    int g;       // group of element e0 (G if e0 is past every group)
    bool inb;    // e0 < cols
    bool fast;   // the whole segment lies inside group g (and inside cols)
};

__device__ __forceinline__ SegInfo seg_info(const int32_t *s_offs, int G, int g_hint, int e0, int cols)
{
    SegInfo si;
    si.inb = e0 < cols;
    si.g = advance_group(s_offs, G, g_hint, e0);
    si.fast = si.inb && si.g < G && e0 + 8 <= s_offs[si.g] && e0 + 8 <= cols;
    return si;
}

// Reduce one segment's |x| max into s_amax for every group it touches.
// `uni`: the caller knows every lane of the wave has a fast segment of the
// same group gw (one wave max, one atomic); otherwise lanes are grouped by a
// ballot loop (lanes hold consecutive segments, so few iterations), and the
// segments that straddle a group boundary fall back to per-element atomics.
__device__ __forceinline__ void reduce_segment(uint32_t *s_amax, const int32_t *s_offs, int G,
                                               const uint16_t *xr, const uint4 &v, const SegInfo &si,
                                               int e0, int cols, bool uni, int gw_uni, int lane)
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
    if (si.inb && !si.fast) {
        // rare: re-read the elements one by one (the line is in cache) rather
        // than index the segment's registers with a runtime element number
        int gj = si.g;
#pragma unroll 1
        for (int j = 0; j < 8 && e0 + j < cols; ++j) {
            gj = advance_group(s_offs, G, gj, e0 + j);
            if (gj < G)
                atomicMax(&s_amax[gj], (uint32_t)xr[e0 + j] & 0x7fffu);
        }
    }
}

// Scale and store one segment (row-major q row qr).
__device__ __forceinline__ void store_segment(uint8_t *qr, const float *s_scale, const int32_t *s_offs,
                                              int G, const uint16_t *xr, const uint4 &v,
                                              const SegInfo &si, int e0, int cols)
{
    if (!si.inb)
        return;
    if (si.fast) {
        st8_nt(qr + e0, quant8_fp32scale(v, s_scale[si.g]));
        return;
    }
    int gj = si.g;
#pragma unroll 1
    for (int j = 0; j < 8 && e0 + j < cols; ++j) {
        gj = advance_group(s_offs, G, gj, e0 + j);
        if (gj < G)
            qr[e0 + j] = (uint8_t)cvt1(__uint_as_float((uint32_t)xr[e0 + j] << 16) * s_scale[gj]);
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
template <int NR>
__global__ __launch_bounds__(kThreads) void jagged_contig_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, int rows, int cols,
    const int32_t *__restrict__ offs, int G, uint8_t *__restrict__ q, int64_t ldq,
    float *__restrict__ scales, int64_t ss_r, int64_t ss_g)
{
    extern __shared__ uint32_t smem[];
    int32_t *s_offs = reinterpret_cast<int32_t *>(smem);
    uint32_t *s_amax = smem + G;
    float *s_scale = reinterpret_cast<float *>(smem + 2 * G);

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

    SegInfo si[NR];
    uint32_t uni = 0u;   // bit i: every lane of this wave has a fast segment i of one group
    bool lane_fast = true;  // every segment of this lane is fast
    int gw[NR];
    {
        int g = advance_group(s_offs, G, 0, 8 * t);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int e0 = 8 * (i * kThreads + t);
            si[i] = seg_info(s_offs, G, g, e0, cols);
            g = si[i].g;
            gw[i] = __builtin_amdgcn_readfirstlane(si[i].g);
            const bool same = si[i].fast && si[i].g == gw[i];
            if (__ballot(same) == ~0ull)
                uni |= 1u << i;
            lane_fast = lane_fast && si[i].fast;
        }
    }

    auto process_row = [&](uint4 (&cur)[NR], uint4 (&nxt)[NR], int r) __attribute__((always_inline)) {
        load_row(nxt, r + (int)gridDim.x);   // range 0 past the last row
        const uint16_t *xr = x + (int64_t)r * ldx;
        if (uni == (1u << NR) - 1u) {
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
                               (uni >> i) & 1u, gw[i], lane);
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
        if (lane_fast) {
            float sc[NR];
#pragma unroll
            for (int i = 0; i < NR; ++i)
                sc[i] = s_scale[si[i].g];
#pragma unroll
            for (int i = 0; i < NR; ++i)
                st8_nt(qr + 8 * (i * kThreads + t), quant8_fp32scale(cur[i], sc[i]));
        } else {
#pragma unroll
            for (int i = 0; i < NR; ++i)
                store_segment(qr, s_scale, s_offs, G, xr, cur[i], si[i], 8 * (i * kThreads + t), cols);
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
            reduce_segment(s_amax, s_offs, G, xr, v[i], si, e0, cols, false, 0, lane);
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
            store_segment(qr, s_scale, s_offs, G, xr, v[i], si, e0, cols);
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
constexpr int kPackMax = 16;

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
__device__ __forceinline__ StripMap map_strip(int b, int nsuper, int G)
{
    const int x = b & 7;               // XCD slot
    const int k = b >> 3;
    const int sub = k % SPS;           // strip within the superstrip
    const int S = (k / SPS) * 8 + x;   // logical superstrip index
    StripMap m;
    m.item = S / nsuper;
    m.strip = (S % nsuper) * SPS + sub;
    m.valid = m.item < G;
    return m;
}

// Per-workgroup item table for G > 64 (NTH threads), all in LDS: s_end
// (clamped group ends), s_lead (1 for a group that starts a pack), s_lpre /
// s_ppre (exclusive prefix counts of long groups / pack leaders by group
// index; long groups then go in index order).  TR = rows per tile.
template <int NTH, int TR>
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
    slot_prefix2<NTH>(G, s_lpre, s_ppre, [&](int g) { return is_long(g) ? 1 : 0; },
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
template <int CG, int T, int NW>
__global__ __launch_bounds__(64 * NW) void jagged_strided_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, int rows, int cols,
    const int32_t *__restrict__ offs, int G, uint8_t *__restrict__ q, int64_t ldq,
    float *__restrict__ scales, int64_t ss_g, int64_t ss_c, int nsuper)
{
    constexpr int QD = 64 / CG;       // 16-row pieces per wave
    constexpr int WROWS = 16 * QD;    // rows per wave
    constexpr int TROWS = NW * WROWS; // rows per register tile
    constexpr int SW = 8 * CG;        // strip width in columns
    constexpr int NTH = 64 * NW;
    static_assert(T >= 2, "a pack spans up to two tiles");

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

    const StripMap sm = map_strip<8 / CG>(blockIdx.x, nsuper, G);
    if (!sm.valid)
        return;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = t >> 6;
    const int cg = lane % CG;
    const int qd = lane / CG;

    // this workgroup's item: a long group g, or a pack of short groups [g0, g1)
    __shared__ int s_sel[3];
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
            const int nl = __popcll(mlong);
            const int item = sm.item;
            if (item < nl) {
                // rank of a long group: longer first, ties by index
                int r = 0;
                for (int h = 0; h < G; ++h) {
                    const int lh = __builtin_amdgcn_readlane(len, h);
                    const bool hl = (mlong >> h) & 1ull;
                    r += hl && ((lh > len) || (lh == len && h < lane));
                }
                if (lng && r == item) {
                    s_sel[0] = 0;
                    s_sel[1] = lane;
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
    } else {
        strided_table<NTH, TROWS>(offs, G, rows, s_end, s_lead, s_lpre, s_ppre);
        if (t == 0) {
            const int nlong = s_lpre[G], npack = s_ppre[G];
            if (sm.item < nlong) {
                s_sel[0] = 0;
                s_sel[1] = find_slot(s_lpre, G, sm.item);
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
            } else {
                // rows of several groups: per-row multipliers, byte stores
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

    // ---- a long group
    const int g = s_sel[1];
    const int lo = g ? s_end[g - 1] : 0;
    int hi = s_end[g];
    hi = hi < lo ? lo : hi;

    const int cbase = sm.strip * SW + 8 * cg;
    const bool col_ok = cbase < cols;
    const int rbeg = lo & ~15;
    const int nit = hi > lo ? (hi - rbeg + TROWS - 1) / TROWS : 0;

    uint4 v[T][16];

    // one register tile: 16 rows x 8 columns per lane; rows outside [lo, hi)
    // are neither read nor counted.  Tiles that will be read again (keep)
    // use ordinary loads, the others the streaming hint.
    auto load_tile = [&](uint4 (&d)[16], int it, bool keep) {
        const int rb = rbeg + it * TROWS + w * WROWS + 16 * qd;
        const bool full = rb >= lo && rb + 16 <= hi;
        const uint16_t *p = x + (int64_t)rb * ldx + cbase;
        if (col_ok && full) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                d[i] = keep ? ld16(p + (int64_t)i * ldx) : ld16_nt(p + (int64_t)i * ldx);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = rb + i;
                d[i] = (col_ok && r >= lo && r < hi) ? ld16(p + (int64_t)i * ldx)
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
        const bool full = rb >= lo && rb + 16 <= hi;
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
                    if (r >= lo && r < hi)
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
            load_tile(v[tt], tt, tt == T - 1 && nit > T);
#pragma unroll
    for (int tt = 0; tt < T; ++tt)
        if (tt < nit)
            accumulate(mx, v[tt]);
    // tiles beyond the register window stream through the last buffer
    for (int it = T; it < nit; ++it) {
        load_tile(v[T - 1], it, true);
        accumulate(mx, v[T - 1]);
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
        uint32_t a = 0u;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww)
            a = umax(a, s_red[ww][t]);
        const float s = fp32_scale(a);
        s_scale[t] = s;
        const int c = sm.strip * SW + t;
        if (c < cols)
            scales[(int64_t)g * ss_g + (int64_t)c * ss_c] = s;
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

}  // namespace mxq
