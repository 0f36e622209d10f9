// Per-workgroup tables of token groups built from the device offsets, shared
// by the kernels that map workgroups onto per-group work without the host
// reading the offsets: clamped group ends, a workgroup-wide exclusive scan of
// per-slot work counts, and the binary search from a work index to its slot.
#pragma once

#include <stdint.h>

namespace mxq {

// largest G the tables hold (the C ABI's limit)
constexpr int kMaxTableGroups = 4096;

// units of 2^SH elements in a group of n (n <= 0: none)
template <int SH>
__device__ __forceinline__ int units_of(int n)
{
    return n > 0 ? (n + (1 << SH) - 1) >> SH : 0;
}

// s_end[g] = offs[g] clamped to [0, extent], for every g < G.  Ends with a
// barrier.  Group g then covers [s_end[g-1], s_end[g]) (s_end[-1] = 0); a
// group whose end precedes its start is empty.
template <int NTH>
__device__ __forceinline__ void load_group_ends(const int32_t *__restrict__ offs, int G, int extent,
                                                int *s_end)
{
    for (int g = threadIdx.x; g < G; g += NTH) {
        const int e = offs[g];
        s_end[g] = e < 0 ? 0 : (e > extent ? extent : e);
    }
    __syncthreads();
}

__device__ __forceinline__ int group_len(const int *s_end, int g)
{
    const int n = s_end[g] - (g ? s_end[g - 1] : 0);
    return n > 0 ? n : 0;
}

// Exclusive prefix over slots 0..G-1 of count(slot) (non-negative) into
// s_pre[0..G] (s_pre[G] = total).  Each thread owns a contiguous chunk of
// slots; chunk sums are scanned with shuffles in each wave and across the
// waves through LDS.  Ends with a barrier.
template <int NTH, typename Count>
__device__ void slot_prefix(int G, int *s_pre, Count count)
{
    __shared__ int s_wsum[NTH / 64];
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = t >> 6;
    const int ch = (G + NTH - 1) / NTH;
    const int s0 = t * ch;
    int sum = 0;
    for (int k = 0; k < ch; ++k)
        if (s0 + k < G)
            sum += count(s0 + k);
    int inc = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(inc, d, 64);
        if (lane >= d)
            inc += y;
    }
    if (lane == 63)
        s_wsum[w] = inc;
    __syncthreads();
    int ex = inc - sum;
    for (int ww = 0; ww < w; ++ww)
        ex += s_wsum[ww];
    for (int k = 0; k < ch; ++k)
        if (s0 + k < G) {
            s_pre[s0 + k] = ex;
            ex += count(s0 + k);
        }
    if (t == NTH - 1)
        s_pre[G] = ex;
    __syncthreads();
}

// Two prefixes in one scan: s_pa from count_a and s_pb from count_b (as
// slot_prefix).  Ends with a barrier.
template <int NTH, typename CountA, typename CountB>
__device__ void slot_prefix2(int G, int *s_pa, int *s_pb, CountA count_a, CountB count_b)
{
    __shared__ int s_wa[NTH / 64], s_wb[NTH / 64];
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = t >> 6;
    const int ch = (G + NTH - 1) / NTH;
    const int s0 = t * ch;
    int sa = 0, sb = 0;
    for (int k = 0; k < ch; ++k)
        if (s0 + k < G) {
            sa += count_a(s0 + k);
            sb += count_b(s0 + k);
        }
    int ia = sa, ib = sb;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int ya = __shfl_up(ia, d, 64);
        const int yb = __shfl_up(ib, d, 64);
        if (lane >= d) {
            ia += ya;
            ib += yb;
        }
    }
    if (lane == 63) {
        s_wa[w] = ia;
        s_wb[w] = ib;
    }
    __syncthreads();
    int ea = ia - sa, eb = ib - sb;
    for (int ww = 0; ww < w; ++ww) {
        ea += s_wa[ww];
        eb += s_wb[ww];
    }
    for (int k = 0; k < ch; ++k)
        if (s0 + k < G) {
            s_pa[s0 + k] = ea;
            s_pb[s0 + k] = eb;
            ea += count_a(s0 + k);
            eb += count_b(s0 + k);
        }
    if (t == NTH - 1) {
        s_pa[G] = ea;
        s_pb[G] = eb;
    }
    __syncthreads();
}

// The same tables for G <= 64 built by the calling wave alone (lane g holds
// group g): s_end, and the exclusive prefix counts of units of 2^SHA and
// 2^SHB elements per group into s_pa / s_pb (entry G = total).  One global
// load per lane and shuffle scans; the caller follows with a barrier.
template <int SHA, int SHB>
__device__ __forceinline__ void wave_group_tables(const int32_t *__restrict__ offs, int G,
                                                  int extent, int *s_end, int *s_pa, int *s_pb)
{
    const int lane = threadIdx.x & 63;
    const bool valid = lane < G;
    int hi = valid ? offs[lane] : extent;
    hi = hi < 0 ? 0 : (hi > extent ? extent : hi);
    int lo = __shfl_up(hi, 1, 64);
    lo = lane == 0 ? 0 : lo;
    const int n = valid && hi > lo ? hi - lo : 0;
    const int ua = units_of<SHA>(n), ub = units_of<SHB>(n);
    int ia = ua, ib = ub;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int ya = __shfl_up(ia, d, 64);
        const int yb = __shfl_up(ib, d, 64);
        if (lane >= d) {
            ia += ya;
            ib += yb;
        }
    }
    if (valid) {
        s_end[lane] = hi;
        s_pa[lane] = ia - ua;
        s_pb[lane] = ib - ub;
    }
    if (lane == G - 1) {
        s_pa[G] = ia;
        s_pb[G] = ib;
    }
}

// wave_group_tables with a third prefix: units of 2^SHC elements into s_pc
// (which may alias s_pb when SHC == SHB).  The caller follows with a barrier.
template <int SHA, int SHB, int SHC>
__device__ __forceinline__ void wave_group_tables3(const int32_t *__restrict__ offs, int G,
                                                   int extent, int *s_end, int *s_pa, int *s_pb,
                                                   int *s_pc)
{
    const int lane = threadIdx.x & 63;
    const bool valid = lane < G;
    int hi = valid ? offs[lane] : extent;
    hi = hi < 0 ? 0 : (hi > extent ? extent : hi);
    int lo = __shfl_up(hi, 1, 64);
    lo = lane == 0 ? 0 : lo;
    const int n = valid && hi > lo ? hi - lo : 0;
    const int ua = units_of<SHA>(n), ub = units_of<SHB>(n), uc = units_of<SHC>(n);
    int ia = ua, ib = ub, ic = uc;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int ya = __shfl_up(ia, d, 64);
        const int yb = __shfl_up(ib, d, 64);
        const int yc = __shfl_up(ic, d, 64);
        if (lane >= d) {
            ia += ya;
            ib += yb;
            ic += yc;
        }
    }
    if (valid) {
        s_end[lane] = hi;
        s_pa[lane] = ia - ua;
        s_pb[lane] = ib - ub;
        s_pc[lane] = ic - uc;
    }
    if (lane == G - 1) {
        s_pa[G] = ia;
        s_pb[G] = ib;
        s_pc[G] = ic;
    }
}

// the slot whose work covers index j: s_pre[s] <= j < s_pre[s+1], given
// 0 <= j < s_pre[G] (slots with no work are skipped)
__device__ __forceinline__ int find_slot(const int *s_pre, int G, int j)
{
    int a = 0, b = G;
    while (b - a > 1) {
        const int m = (a + b) >> 1;
        if (s_pre[m] <= j)
            a = m;
        else
            b = m;
    }
    return a;
}

}  // namespace mxq
