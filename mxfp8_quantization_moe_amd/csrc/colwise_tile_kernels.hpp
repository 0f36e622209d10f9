// Jagged colwise with fp32 scales on 128 x 256 tiles: one scale per (token
// group, column), the amax taken over the group's rows of that column
// ("[scaled grouped mm] add triton kernels for float8 rowwise quantization
// with per-group/jagged scales", Summary: per-group column scales for the
// operand whose groups run along the reduction dim; the group offsets stay
// on the device).
//
// A workgroup of four waves side by side covers 256 columns (512 bytes of
// every row it reads) and a chunk of T 128-row tiles of one group, anchored
// at the group start rounded down to 16 rows (the scales are per group, so
// any tiling will do, and 16-row pieces make whole 16-byte column stores); a
// lane holds 16 rows x 8 columns per tile, in registers, so every element is
// read from HBM once.  A group longer than one chunk is cut into nu chunks
// per 256-column tile; the chunks of one (group, column tile) exchange
// their 256 column maxima, either through a
// set of words in a caller's workspace or through the group's own fp32
// scale slots (zeroed first by jagged_colwise_tile_clear_kernel), then each
// quantizes its rows with the group's scales.  Every group, an empty one
// included, has at least one chunk; chunk 0 writes the group's scales, except
// in the slot exchange, where the last chunk to leave writes them over the
// exchange words.
//
// Workgroup numbering: group-major, then column blocks (kTileSpan), so a set
// only waits on workgroups of its own block, at most kTileSpan consecutive
// ids; with in-order dispatch and at least that many workgroups resident, the
// lowest block still running always has all its workgroups on the GPU, so
// every set completes.  The wait is bounded anyway: past the bound a chunk
// reduces the group's rows of its tile itself (correct, slower).
#pragma once

#include <stdint.h>

#include "group_tables.hpp"
#include "jagged_kernels.hpp"
#include "jagged_mx_kernels.hpp"
#include "mxq_device.hpp"
#include "wave_ops.hpp"

namespace mxq {

// largest G of the tile kernel (its group table lives in LDS)
constexpr int kTileMaxGroups = 256;
// one workspace set per (long group, column tile): 256 column maxima
// (|bf16| bit patterns), the arrival count and the departure count, padded
// to 32 bytes; zero between calls (the last chunk to leave clears it)
constexpr int kTileSetWords = 264;
constexpr int kTileSetArrive = 256;
constexpr int kTileSetDepart = 257;

// Workgroups of a group are numbered in column blocks: the chunks of B
// adjacent 256-column tiles, chunk-major, so workgroups dispatched together
// read B * 512 bytes of each row (whole rows when B covers every tile).  B
// is the largest count with B * nu <= kTileSpan (nu chunks per tile), so
// every exchange set lies in a block of at most kTileSpan consecutive
// workgroups, fewer than are resident at once (three per CU).
constexpr int kTileSpan = 512;

// The rows a group's chunks cover: from its start rounded down to 16 rows to
// its end (0 for an empty group), and the chunks of ch rows over them (an
// empty group has one).
__device__ __forceinline__ int tile_span(int lo, int hi) { return hi > lo ? hi - (lo & ~15) : 0; }
__device__ __forceinline__ int tile_chunks(int span, int ch) { return span > ch ? (span + ch - 1) / ch : 1; }

// Zeroes the scale slots the workspace-free exchange runs in: every column
// of each group whose span (tile_span) exceeds one chunk of ch rows (clamped
// ends as in the main kernel).  Grid (column blocks, G); 256 threads.
__global__ __launch_bounds__(256) void jagged_colwise_tile_clear_kernel(
    const int32_t *__restrict__ offs, int G, int rows, int cols, float *__restrict__ scales,
    int64_t ss_g, int64_t ss_c, int ch)
{
    const int g = blockIdx.y;
    auto clamp_end = [&](int e) { return e < 0 ? 0 : (e > rows ? rows : e); };
    const int lo = g ? clamp_end(offs[g - 1]) : 0;
    const int hi = clamp_end(offs[g]);
    if (tile_span(lo, hi) <= ch)
        return;
    for (int c = blockIdx.x * 256 + threadIdx.x; c < cols; c += gridDim.x * 256)
        scales[(int64_t)g * ss_g + (int64_t)c * ss_c] = 0.0f;
}

// x (rows, cols) row-major with row pitch ldx; q column-major with column
// pitch ldq; scales (G, cols) at g * ss_g + c * ss_c.  G <= kTileMaxGroups,
// cols a multiple of 8, tiles_c = ceil(cols / 256); grid at least
// tiles_c * (G + (rows + 14 G) / (128 T)) workgroups of 256 threads (spare
// ones exit).
// ws: the workspace sets (null: exchange in the scale slots, which the
// clear kernel has zeroed; then at most kSlotMaxChunks chunks per group),
// nsets of them per column tile (offsets that break their precondition can
// make more long groups than the host's bound: those chunks take the
// fallback instead of writing past the workspace).
// spin_limit: polls before the fallback (negative: fall back at once).
template <int T>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void jagged_colwise_tile_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, int rows, int cols,
    const int32_t *__restrict__ offs, int G, uint8_t *__restrict__ q, int64_t ldq,
    float *__restrict__ scales, int64_t ss_g, int64_t ss_c, int tiles_c, uint32_t *__restrict__ ws,
    int nsets, int spin_limit)
{
    constexpr int CH = 128 * T;   // rows per chunk
    __shared__ int s_end[kTileMaxGroups];
    __shared__ int s_pu[kTileMaxGroups + 1];   // chunks per group, exclusive prefix
    __shared__ int s_pl[kTileMaxGroups + 1];   // groups of more than one chunk, exclusive prefix
    __shared__ uint32_t s_col[256];            // column maxima, then the scales' bits
    __shared__ int s_flag;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = t >> 6;
    const int cg = lane & 7;
    const int qd = lane >> 3;

    // this workgroup's group g (chunk j of the chunk count), its chunks nu,
    // their first index pu_g, its index among the groups of more than one
    // chunk pl_g, and its rows [lo, hi)
    const int j = (int)(blockIdx.x / (unsigned)tiles_c);
    int g, nu, pu_g, pl_g, lo, hi;
    if (G <= 64) {
        // every wave builds the table in registers (lane l holds group l)
        // and finds g by a ballot: no barrier and no LDS round trip before
        // the loads
        const bool valid = lane < G;
        int e = valid ? offs[lane] : rows;
        e = e < 0 ? 0 : (e > rows ? rows : e);
        int el = __shfl_up(e, 1, 64);
        el = lane == 0 ? 0 : el;
        const int sp = tile_span(el, e);
        const int cu = valid ? tile_chunks(sp, CH) : 0;
        const int lg = valid && sp > CH ? 1 : 0;
        int iu = cu, il = lg;   // inclusive prefixes
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int yu = __shfl_up(iu, d, 64);
            const int yl = __shfl_up(il, d, 64);
            if (lane >= d) {
                iu += yu;
                il += yl;
            }
        }
        if (j >= __builtin_amdgcn_readlane(iu, 63))
            return;
        g = (int)__popcll(__ballot(iu <= j));   // groups whose chunks all precede chunk j
        pu_g = __builtin_amdgcn_readlane(iu - cu, g);
        nu = __builtin_amdgcn_readlane(cu, g);
        pl_g = __builtin_amdgcn_readlane(il - lg, g);
        lo = __builtin_amdgcn_readlane(el, g);
        hi = __builtin_amdgcn_readlane(e, g);
    } else {
        load_group_ends<256>(offs, G, rows, s_end);
        slot_prefix2<256>(
            G, s_pu, s_pl, [&](int gg) { return tile_chunks(tile_span(gg ? s_end[gg - 1] : 0, s_end[gg]), CH); },
            [&](int gg) { return tile_span(gg ? s_end[gg - 1] : 0, s_end[gg]) > CH ? 1 : 0; });
        if (j >= s_pu[G])
            return;
        g = find_slot(s_pu, G, j);
        pu_g = s_pu[g];
        nu = s_pu[g + 1] - pu_g;
        pl_g = s_pl[g];
        lo = g ? s_end[g - 1] : 0;
        hi = s_end[g];
    }
    hi = hi < lo ? lo : hi;
    // column block of B tiles: its chunks, chunk-major (B * nu workgroups,
    // at most kTileSpan, the last block narrower)
    const int local = (int)blockIdx.x - pu_g * tiles_c;
    int B = kTileSpan / nu;
    B = B < 1 ? 1 : (B > tiles_c ? tiles_c : B);
    const int blk = local / (nu * B);
    const int wb = tiles_c - blk * B < B ? tiles_c - blk * B : B;
    const int rr = local - blk * nu * B;
    const int k = rr / wb;
    const int tc = blk * B + (rr - k * wb);
    const int rt = (lo & ~15) + k * CH;      // first row of this chunk
    const int c0 = tc * 256 + 64 * w + 8 * cg;
    const bool col_ok = c0 < cols;
    const int cl = col_ok ? c0 : 0;

    // loads: 16 rows x 8 columns per lane and tile; rows before the group
    // start read row lo, rows past its end row hi - 1 (same group, so the
    // maxima are unchanged); tiles wholly past the end, and every tile of an
    // empty group (whose rounded-down start lies below its end), are not read
    uint4 v[T][16];
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
        const int rb = rt + 128 * tt + 16 * qd;
        if (hi > lo && rt + 128 * tt < hi) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = rb + i < lo ? lo : (rb + i < hi ? rb + i : hi - 1);
                v[tt][i] = ld16_nt(x + (int64_t)r * ldx + cl);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                v[tt][i] = make_uint4(0u, 0u, 0u, 0u);
        }
    }

    // column maxima of the chunk: in-lane over rows, then across the 8 lanes
    // of a column (lane bits 3..5); lane qd = 0 hands them to LDS, thread t
    // then owns column tc * 256 + t
    uint32_t mx[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            mx[0] = absmax2(mx[0], v[tt][i].x);
            mx[1] = absmax2(mx[1], v[tt][i].y);
            mx[2] = absmax2(mx[2], v[tt][i].z);
            mx[3] = absmax2(mx[3], v[tt][i].w);
        }
    }
#pragma unroll
    for (int d = 0; d < 4; ++d)
        mx[d] = strided_pkmax<8>(mx[d]);
    if (qd == 0) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            s_col[64 * w + 8 * cg + 2 * d] = mx[d] & 0xffffu;
            s_col[64 * w + 8 * cg + 2 * d + 1] = mx[d] >> 16;
        }
    }
    __syncthreads();
    uint32_t acol = s_col[t];
    const int col = tc * 256 + t;
    const bool has_col = col < cols;
    float *const slot_f = scales + (int64_t)g * ss_g + (int64_t)col * ss_c;
    uint32_t *const slot = reinterpret_cast<uint32_t *>(slot_f);
    const bool in_slots = nu > 1 && ws == nullptr;
    bool last_out = false;

    if (nu > 1) {
        // Every global access of the exchange hands its result to LDS before
        // the next barrier: a barrier does not wait for a thread's
        // outstanding global operations, only the use of their results does,
        // so this is what orders one thread's atomics before another
        // thread's arrival or departure.
        const bool in_ws = ws != nullptr && pl_g < nsets;
        uint32_t *const set = in_ws ? ws + ((int64_t)pl_g * tiles_c + tc) * kTileSetWords : nullptr;
        bool done = true;   // (thread t alone uses s_col[t] until the fallback)
        // the exchange runs in the scale slots or in a workspace set; a chunk
        // whose set lies past the workspace reduces its group's rows itself
        const bool exch = in_slots || in_ws;
        uint32_t *const count = in_slots ? reinterpret_cast<uint32_t *>(scales + (int64_t)g * ss_g +
                                                                        (int64_t)(tc * 256) * ss_c)
                                         : (in_ws ? set + kTileSetArrive : nullptr);
        if (exch) {
            // A chunk raises a shared maximum only when its own is larger than
            // the value it reads first: the chunks of a set arrive together, and
            // one atomic per chunk and word would queue on the same words.
            uint32_t *const word = in_slots ? slot : set + t;
            uint32_t cur = 0u;
            if (has_col) {
                cur = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (in_slots && t == 0) {
                    // the control word (the tile's first column): raise its
                    // maximum bits by compare-and-swap, leaving the counts
                    while ((cur & kSlotMax) < acol &&
                           !__hip_atomic_compare_exchange_strong(word, &cur, (cur & ~kSlotMax) | acol,
                                                                 __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                                 __HIP_MEMORY_SCOPE_AGENT)) {
                    }
                } else if ((cur & kSlotMax) < acol) {
                    cur = __hip_atomic_fetch_max(word, acol, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            s_col[t] = umax(acol, cur & kSlotMax);
            __syncthreads();   // all of this workgroup's maxima are in
            const uint32_t one = in_slots ? kSlotArrive : 1u;
            if (t == 0) {
                // arrive, then poll until every chunk has; a negative limit takes
                // the fallback without looking, 0 looks once
                uint32_t c = __hip_atomic_fetch_add(count, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + one;
                auto arrived = [&](uint32_t v) {
                    return (in_slots ? slot_arrivals(v) : v) >= (uint32_t)nu;
                };
                bool all = spin_limit >= 0 && arrived(c);
                for (int n = 0; !all && spin_limit >= 0 && n < spin_limit; ++n) {
                    __builtin_amdgcn_s_sleep(2);
                    all = arrived(__hip_atomic_load(count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
                }
                s_flag = all ? 1 : 0;
            }
            __syncthreads();
            done = s_flag != 0;
            if (done && has_col)
                s_col[t] = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kSlotMax;
        } else {
            done = false;
        }
        if (!done) {
            // no exchange, or the other chunks did not arrive in time: reduce
            // every row of the group in this column tile here (32 lanes per
            // row, 16 bytes each)
            __syncthreads();
            s_col[t] = 0u;
            __syncthreads();
            uint32_t m[4] = {0u, 0u, 0u, 0u};
            const int pc = t & 31;
            const int cc = tc * 256 + 8 * pc;
            if (cc < cols) {
                for (int r = lo + (t >> 5); r < hi; r += 8) {
                    const uint4 vv = ld16(x + (int64_t)r * ldx + cc);
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
        __syncthreads();   // every read of the set or slots has returned
        acol = s_col[t];
        if (exch && t == 0) {
            const uint32_t dep = in_slots ? kSlotDepart : 1u;
            uint32_t *const dcount = in_slots ? count : set + kTileSetDepart;
            const uint32_t prev =
                __hip_atomic_fetch_add(dcount, dep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_flag = (in_slots ? prev >> 24 : prev) == (uint32_t)nu - 1 ? 2 : 0;
        }
        __syncthreads();
        last_out = exch && s_flag == 2;
        if (last_out && !in_slots) {
            // the set is zero again for the next call
            __hip_atomic_store(set + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (t < kTileSetWords - 256)
                __hip_atomic_store(set + 256 + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    // the scales: chunk 0 writes them, except in the slot exchange, where
    // the last chunk out writes them over the words (every other chunk has
    // read its slots by then)
    const float s = fp32_scale(acol);
    if (has_col && in_slots && last_out)
        __hip_atomic_store(slot, __float_as_uint(s), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else if (has_col && !in_slots && k == 0)
        *slot_f = s;
    __syncthreads();   // s_col read above by its owner
    s_col[t] = __float_as_uint(s);
    __syncthreads();

    if (!col_ok)
        return;
    float sc[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
        sc[jj] = __uint_as_float(s_col[64 * w + 8 * cg + jj]);
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
        const int rb = rt + 128 * tt + 16 * qd;
        if (hi <= lo || rb >= hi)
            continue;
        // the lane's 16 rows of each column as one 16-byte piece of the column
        // run; the group's first and last pieces hold only the rows in
        // [lo, hi), written as aligned parts
        const int from = lo > rb ? lo - rb : 0, to = hi - rb < 16 ? hi - rb : 16;
        uint8_t *qp = q + (int64_t)c0 * ldq + rb;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const uint4 o = tile_column_bytes<false>(v[tt], jj, sc[jj]);
            if (from == 0 && to == 16)
                st16(qp + (int64_t)jj * ldq, o);
            else
                put16_range(qp + (int64_t)jj * ldq, o, from, to);
        }
    }
}

}  // namespace mxq
