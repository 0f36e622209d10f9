// Per-group re-layout of jagged MX e8m0 scales (groups along K) into the
// scale-operand tiles of a gfx950 scaled-MFMA grouped GEMM ("[mxfp8 moe
// training] add CUDA kernel for per-group conversion of scale factors to
// blocked layout": after MX quantization with token groups along K, each
// group's scales are converted to the layout the grouped GEMM reads; the
// layout itself is the consumer's).
//
// Consumer: the scaled MFMA with 16 rows x 128 K values of e4m3 per
// instruction (CDNA4 ISA, V_MFMA_SCALE_F32_16X16X128_F8F6F4).  Lane 16j + i
// supplies the e8m0 scale of row i and 32-value K block j in a 32-bit
// register whose byte is chosen by op_sel, so one register serves four K
// steps.  A tile is 16 rows x 16 blocks = 64 lane words = 256 bytes:
//
//   byte 4*lane + u of a tile = scale of row lane % 16, block 4u + lane / 16.
//
// Group g (n_g tokens, nb_g = ceil(n_g/32) blocks starting at scale column
// B_g, as the jagged MX kernels number them) owns RB = ceil(rows/16) x
// KT_g = ceil(n_g/512) tiles, row-block-major from tile T_g = RB * sum of
// KT_h over h < g.  Entries past the last row or the group's last block are
// zero.
//
// An item of work is 64 tiles staged through LDS: 16 x 1024 bytes of scales,
// each wave reading one 1024-byte row piece per instruction (aligned 16-byte
// loads, shifted into place by the piece's byte offset, bytes outside the
// item's valid span dropped); then each thread assembles 4 lane words (16
// output bytes) per tile from LDS and stores them as one 16-byte piece of a
// tile.
//   LAYOUT 0: scales contiguous along blocks (ss_b == 1, the rowwise
//             operand): an item is 1 row block x 64 K tiles (16 rows x 1024
//             blocks); its 64 output tiles are contiguous.
//   LAYOUT 1: scales contiguous along rows (ss_r == 1, the colwise operand's
//             columns): an item is 64 row blocks x 1 K tile (16 blocks x 1024
//             rows).
//   LAYOUT 2: any strides: LAYOUT 0's item with byte loads.
// Items of 1024 bytes per staged row, rather than 256, 512 or 2048, measured
// fastest: smaller items pay the per-workgroup table build and latency more
// often, larger ones lose occupancy to their LDS.
// The host never reads the offsets: each workgroup builds the group tables
// (prefix counts of blocks, K tiles and items; clamped ends too for G <= 64)
// and finds its group by binary search; spare workgroups of the upper-bound
// grid exit.
#pragma once

#include <stdint.h>

#include "group_tables.hpp"
#include "mxq_device.hpp"
#include "wave_ops.hpp"

namespace mxq {

constexpr int kRelayoutThreads = 256;

__host__ __device__ constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

// SEG 16-byte segments per thread along the contiguous dim: an item is
// 16 x 256*SEG staged bytes (the kernel takes SEG = 4: one wave per staged
// row).
template <int LAYOUT, int SEG>
struct RelayoutShape {
    static constexpr int CR = LAYOUT == 1 ? 16 * SEG : 1;   // row blocks per item
    static constexpr int CK = LAYOUT == 1 ? 1 : 16 * SEG;   // K tiles per item
    // log2 of the tokens an item spans (512 tokens per K tile)
    static constexpr int SHC = 9 + ilog2(CK);
    // LDS pitch in bytes of one staged row (LAYOUT 0/2) or block (LAYOUT 1),
    // chosen so the assembly reads of a wave fall into distinct banks
    static constexpr int PITCH = 256 * SEG + (LAYOUT == 1 ? 64 : 16);
};

// ints of group table before the staged bytes (rounded to 16 bytes).  For
// G <= 64 one wave builds ends and three prefixes (blocks, K tiles, items);
// for larger G the workgroup scans K tiles and items only, reading group
// lengths from the offsets, and sums its own group's block base: the tables
// then take at most 32 KB, so tables and stage stay under 64 KB at G = 4096.
__host__ __device__ constexpr int relayout_table_ints(int G, int layout)
{
    return G <= 64 ? ((G + 3 * (G + 1) + 3) / 4) * 4
                   : (((G + 1) + (layout != 1 ? G + 1 : 0) + 3) / 4) * 4;
}

template <int LAYOUT, int SEG>
__host__ __device__ constexpr int relayout_lds_bytes(int G)
{
    return 4 * relayout_table_ints(G, LAYOUT) + 16 * RelayoutShape<LAYOUT, SEG>::PITCH;
}

// Shifted 16-byte pieces for a wave whose lanes read consecutive pieces p =
// base + 16 * lane (so the byte shift p % 16 is the same for every lane and
// the select on it does not diverge); nvalid bytes of a piece are wanted (up
// to 16), the rest read as zero.  Each lane loads only the aligned 16-byte
// chunk holding p and takes the chunk after it from the next lane by a DPP
// whole-wave shift (a VALU move); lane 63 loads that chunk itself.  A lane
// loads its chunk when it wants bytes of it or when the previous lane's
// wanted bytes run into it (nvalid_prev: the previous lane's count, 0 for
// lane 0).  issue() only loads, so a caller issues the loads of all its
// pieces before the first combine() waits for any; combine() needs all
// lanes of the wave.
// Nontemporal loads: the same speed warm and cold (8192 x 32770 scales: 121 /
// 121 us), where plain loads run 107 us warm from the memory-side cache but
// 147 us cold.
struct ShiftedPiece {
    uint4 c0, c63;
    int sh, nvalid;

    __device__ __forceinline__ void issue(const uint8_t *p, int nv, int nvalid_prev, int lane)
    {
        const uintptr_t a = reinterpret_cast<uintptr_t>(p);
        sh = (int)(a & 15);
        nvalid = nv;
        const uint16_t *c = reinterpret_cast<const uint16_t *>(a & ~uintptr_t(15));
        c0 = make_uint4(0u, 0u, 0u, 0u);
        c63 = make_uint4(0u, 0u, 0u, 0u);
        if (nv > 0 || (sh != 0 && nvalid_prev > 16 - sh))
            c0 = ld16_nt(c);
        if (lane == 63 && nv > 16 - sh)
            c63 = ld16_nt(c + 8);
    }

    __device__ __forceinline__ uint4 combine(int lane) const
    {
        uint4 c1 = make_uint4(from_next_lane(c0.x), from_next_lane(c0.y), from_next_lane(c0.z),
                              from_next_lane(c0.w));
        if (lane == 63)
            c1 = c63;
        if (nvalid <= 0)
            return make_uint4(0u, 0u, 0u, 0u);
        const uint32_t d[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const int q = sh >> 2, b = sh & 3;
        uint32_t o[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t lo = q == 0 ? d[w] : q == 1 ? d[w + 1] : q == 2 ? d[w + 2] : d[w + 3];
            const uint32_t hi = q == 0 ? d[w + 1] : q == 1 ? d[w + 2] : q == 2 ? d[w + 3] : d[w + 4];
            o[w] = (uint32_t)((((uint64_t)hi << 32) | lo) >> (8 * b));
        }
        if (nvalid < 16) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int keep = nvalid - 4 * w;
                const uint32_t mask =
                    keep >= 4 ? 0xFFFFFFFFu : (keep <= 0 ? 0u : ((1u << (8 * keep)) - 1u));
                o[w] &= mask;
            }
        }
        return make_uint4(o[0], o[1], o[2], o[3]);
    }
};

__device__ __forceinline__ uint32_t byte_of(uint32_t v, int k) { return (v >> (8 * k)) & 0xFFu; }

// scales[r*ss_r + b*ss_b]: block b of row r (b counts every group's blocks,
// group after group).  tiles: 256-byte tiles as described above (16-byte
// aligned).  tile_starts (may be null): T_g for g = 0..G, written by
// workgroup 0.  Grid: at least ceil(RB / CR) * nchunk workgroups (nitems),
// nchunk = ceil(extent / 2^SHC) + G - 1 (an upper bound of the items along
// K), a multiple of 8 when XCD is set; dynamic LDS relayout_lds_bytes.
// XCD: workgroup b runs on XCD b % 8, so item b % 8 * (grid / 8) + b / 8 keeps
// the items of one XCD consecutive and the cache line two neighbouring row
// pieces share is fetched into one L2.
template <int LAYOUT, int SEG, bool XCD>
__global__ __launch_bounds__(kRelayoutThreads) void relayout_mx_scales_kernel(
    const uint8_t *__restrict__ scales, int64_t ss_r, int64_t ss_b, int rows, int extent,
    const int32_t *__restrict__ offs, int G, uint8_t *__restrict__ tiles,
    int32_t *__restrict__ tile_starts, int nchunk, int nitems)
{
    using SH = RelayoutShape<LAYOUT, SEG>;
    extern __shared__ __align__(16) int relayout_lds[];
    __shared__ int s_red[kRelayoutThreads / 64];
    const bool small = G <= 64;
    int *s_end = relayout_lds;                               // G <= 64 only
    int *s_pt = relayout_lds + (small ? G : 0);              // K tiles, G + 1
    int *s_pc = LAYOUT == 1 ? s_pt : s_pt + G + 1;           // items along K, G + 1
    int *s_pb = small ? s_pt + 2 * (G + 1) : nullptr;        // blocks, G + 1 (G <= 64)
    uint8_t *stage = reinterpret_cast<uint8_t *>(relayout_lds + relayout_table_ints(G, LAYOUT));

    // group length, clamped as everywhere: from the table for G <= 64, else
    // straight from the offsets
    auto glen = [&](int g) {
        if (small)
            return group_len(s_end, g);
        int hi = offs[g], lo = g ? offs[g - 1] : 0;
        hi = hi < 0 ? 0 : (hi > extent ? extent : hi);
        lo = lo < 0 ? 0 : (lo > extent ? extent : lo);
        return hi > lo ? hi - lo : 0;
    };
    const int t = threadIdx.x;
    if (small) {
        if (t < 64)
            wave_group_tables3<9, SH::SHC, 5>(offs, G, extent, s_end, s_pt, s_pc, s_pb);
        __syncthreads();
    } else {
        if (LAYOUT == 1)
            slot_prefix<kRelayoutThreads>(G, s_pt, [&](int g) { return units_of<9>(glen(g)); });
        else
            slot_prefix2<kRelayoutThreads>(
                G, s_pt, s_pc, [&](int g) { return units_of<9>(glen(g)); },
                [&](int g) { return units_of<SH::SHC>(glen(g)); });
    }
    const int RB = (rows + 15) >> 4;
    if (blockIdx.x == 0 && tile_starts != nullptr)
        for (int g = t; g <= G; g += kRelayoutThreads)
            tile_starts[g] = RB * s_pt[g];

    const int item = XCD ? (int)((blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3))
                         : (int)blockIdx.x;
    if (item >= nitems)
        return;
    const int kc_all = item % nchunk;
    const int rc = item / nchunk;
    if (kc_all >= s_pc[G] || rc * SH::CR >= RB)
        return;
    const int g = find_slot(s_pc, G, kc_all);
    const int kc = kc_all - s_pc[g];
    const int n = glen(g);
    const int nb = units_of<5>(n);
    const int KT = units_of<9>(n);
    int64_t B;
    if (small) {
        B = s_pb[g];
    } else {
        // block base of this workgroup's group: blocks of the groups before it
        int part = 0;
        for (int h = t; h < g; h += kRelayoutThreads)
            part += units_of<5>(glen(h));
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1)
            part += __shfl_xor(part, d, 64);
        if ((t & 63) == 0)
            s_red[t >> 6] = part;
        __syncthreads();
        int sum = 0;
#pragma unroll
        for (int w = 0; w < kRelayoutThreads / 64; ++w)
            sum += s_red[w];
        B = sum;
    }
    const int64_t T = (int64_t)RB * s_pt[g];

    const int hi16 = t >> 4;   // staged row (LAYOUT 0/2) or block (LAYOUT 1)
    const int seg = t & 15;    // 16-byte segment of it (plus 16 * s, s < SEG)

    // ---- stage 16 x 1024 bytes: wave w reads staged rows 4w .. 4w+3, one
    // 1024-byte row piece per instruction (lane = 16-byte segment)
    static_assert(SEG == 4, "one wave covers one 1024-byte staged row");
    const int lane = t & 63;
    const int wv = t >> 6;
    uint4 v[4];
    ShiftedPiece pc[4];   // LAYOUT 0 / 1: every piece's loads, then the combines
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int hr = 4 * wv + it;
        // bytes this lane wants (and the previous lane: 16 more of the same
        // run), clamped to a 16-byte piece
        auto clamp16 = [](int n) { return n < 0 ? 0 : (n > 16 ? 16 : n); };
        if (LAYOUT == 1) {
            const int blk = 16 * kc + hr;                    // block within the group
            const int r0 = 1024 * rc + 16 * lane;
            const bool any = blk < nb;
            const int nv = any ? clamp16(rows - r0) : 0;
            const int nvp = any && lane ? clamp16(rows - r0 + 16) : 0;
            pc[it].issue(scales + (B + blk) * ss_b + r0, nv, nvp, lane);
        } else {
            const int r = 16 * rc + hr;
            const int b0 = 1024 * kc + 16 * lane;            // first block within the group
            const bool any = r < rows;
            const int nv = any ? clamp16(nb - b0) : 0;
            const int nvp = any && lane ? clamp16(nb - b0 + 16) : 0;
            const uint8_t *p = scales + (int64_t)r * ss_r + (B + b0) * ss_b;
            if (LAYOUT == 0) {
                pc[it].issue(p, nv, nvp, lane);
            } else {
                uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (e < nv)
                        o[e >> 2] |= (uint32_t)p[e * ss_b] << (8 * (e & 3));
                v[it] = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
    }
    if (LAYOUT != 2) {
#pragma unroll
        for (int it = 0; it < 4; ++it)
            v[it] = pc[it].combine(lane);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it)
        *reinterpret_cast<uint4 *>(stage + (4 * wv + it) * SH::PITCH + 16 * lane) = v[it];
    __syncthreads();

    // ---- assemble: for each s this thread writes lane words 4*seg .. 4*seg+3
    // of output tile hi16 + 16*s of the item (lane L = 4*seg + m holds row
    // i = 4*(seg&3) + m and block column j = seg>>2)
    const int j = seg >> 2;
#pragma unroll
    for (int s = 0; s < SEG; ++s) {
        const int ti = hi16 + 16 * s;   // tile of the item
        uint32_t o[4];
        if (LAYOUT == 1) {
            // bytes u of the four lanes: block 4u + j, rows 16*ti + 4*(seg&3) + m
            uint32_t d[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                d[u] = *reinterpret_cast<const uint32_t *>(stage + (4 * u + j) * SH::PITCH +
                                                           16 * ti + 4 * (seg & 3));
#pragma unroll
            for (int m = 0; m < 4; ++m)
                o[m] = byte_of(d[0], m) | byte_of(d[1], m) << 8 | byte_of(d[2], m) << 16 |
                       byte_of(d[3], m) << 24;
        } else {
            // lane m: staged row 4*(seg&3) + m, bytes 16*ti + 4u + j for u = 0..3
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const uint4 row = *reinterpret_cast<const uint4 *>(
                    stage + (4 * (seg & 3) + m) * SH::PITCH + 16 * ti);
                o[m] = byte_of(row.x, j) | byte_of(row.y, j) << 8 | byte_of(row.z, j) << 16 |
                       byte_of(row.w, j) << 24;
            }
        }
        int64_t tile;
        if (LAYOUT == 1) {
            const int rb = SH::CR * rc + ti;
            if (rb >= RB)
                continue;
            tile = T + (int64_t)rb * KT + kc;
        } else {
            const int kt = SH::CK * kc + ti;
            if (kt >= KT)
                continue;
            tile = T + (int64_t)rc * KT + kt;
        }
        // 16 lanes write a whole 256-byte tile: nontemporal stores (110 against
        // 129 us on (8192, 32770) scales; nontemporal loads were slower)
        st16_nt(tiles + tile * 256 + 16 * seg, make_uint4(o[0], o[1], o[2], o[3]));
    }
}

}  // namespace mxq
