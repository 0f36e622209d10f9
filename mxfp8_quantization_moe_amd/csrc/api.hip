// C-ABI entry points of libmxq: argument validation, layout dispatch and
// kernel launches.  No allocation, no synchronisation, no read-back.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <utility>

#include "mxq.h"
#include "block_kernels.hpp"
#include "colwise_tile_kernels.hpp"
#include "jagged_kernels.hpp"
#include "jagged_mx_kernels.hpp"
#include "relayout_kernels.hpp"

namespace {

using namespace mxq;

constexpr int kJaggedStridedCG = 8;     // 64-column strips (full 128-byte row pieces)
constexpr int kJaggedStridedTiles = 3;  // register tiles per lane (233 VGPRs, 2 waves per SIMD)
constexpr int kJaggedStridedWaves = 8;  // waves per workgroup: tile = 8*16*64/CG = 1024 rows
// the colwise kernel with a workspace: 4-wave workgroups (two per CU, so one
// workgroup's loads overlap another's exchange and stores), tiles of 512
// rows, chunks of 3 tiles (measured against 8 waves and 2 tiles)
constexpr int kSplitTiles = 3;
constexpr int kSplitWaves = 4;
// the rowwise kernel folds segment maxima through LDS (one atomic per run of
// a group per thread) above this many groups; at most this many (one group:
// no boundary inside a row) it reduces each 512-column wave slot with one
// wave maximum.  With 2-16 groups the fold is as fast or faster wherever
// boundaries fall off the 512-column slots (MoE grad_out^T 40.6 against
// 42.8 us cold, its ends moved off 8 elements 45.3 against 53.8, 16 random
// groups 52.6 against 71.2) and 1-2 us slower on equal groups of 2048 or
// 8192 columns
constexpr int kContigSegGroups = 1;
// tile order of the 128 x 256 tile kernel: grids of at least this many
// workgroups (about 13 rounds of the 1280 that are resident at once) take
// XCD chunks of kTileChunk tiles in column-pair order; smaller grids keep the
// plain order (measured on (E, 8192, 5120) weights: 3 to 7 percent faster for
// E >= 16, within noise at E = 8, slower for a single round)
constexpr int64_t kTileOrderMinBlocks = 16384;
constexpr int kTileChunk = 64;
int tile_chunk(int64_t nblocks) { return nblocks >= kTileOrderMinBlocks ? kTileChunk : 0; }
// polls of a split colwise chunk waiting for the other chunks of its group
// (each a device-scope load and a short sleep, about a microsecond) before
// it reduces the group's rows itself
constexpr int kColwiseSpinLimit = 4000;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// column-major q whose 128-row column runs start on 128-byte lines: base and
// the column (and batch) strides on lines
int line_aligned(const void *q, int64_t ldq, int64_t sqe)
{
    return ((reinterpret_cast<uintptr_t>(q) & 127u) == 0 && ldq % 128 == 0 && sqe % 128 == 0) ? 1 : 0;
}

// q stores of the MX 3D kernel: nontemporal at device scope when q is on
// 128-byte lines and every offset inside one expert fits in 32 bits (the
// last column's run ends at (K - 1) * ldq + N), else as line_aligned says
int mx3d_store_mode(const void *q, int64_t N, int64_t K, int64_t ldq, int64_t sqe)
{
    if (!line_aligned(q, ldq, sqe))
        return 0;
    return (K - 1) * ldq + N <= (int64_t)UINT32_MAX ? 2 : 1;
}

mxq_status launch_status()
{
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? MXQ_OK : MXQ_ERR_LAUNCH;
}

// number of compute units of the device that runs `st` (the calling
// thread's current device for the null stream), queried once per device;
// the cache is atomic so concurrent callers are safe
int device_cu_count(hipStream_t st)
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (st) {
        hipDevice_t d = 0;
        if (hipStreamGetDevice(st, &d) != hipSuccess)
            return 256;
        dev = (int)d;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return 256;
    }
    if (dev < 0 || dev >= 64)
        return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// jagged, reduction along the unit-stride dim of a (nrows, ext) view
mxq_status run_jagged_contig(const uint16_t *x, int64_t nrows, int64_t ext, int64_t ldx,
                             const int32_t *offs, int32_t G, uint8_t *q, int64_t ldq,
                             float *scales, int64_t ss_row, int64_t ss_g, hipStream_t st)
{
    if (nrows == 0)
        return MXQ_OK;
    if (nrows > INT32_MAX)
        return MXQ_ERR_INVALID_ARG;
    // many groups: the segment-fold reduction (slots of 512 columns would
    // otherwise hold several groups and take the general path)
    const bool seg = G > kContigSegGroups;
    // persistent grid: as many workgroups per compute unit as fit (four;
    // three for the segment-fold kernel on long rows, whose 140 VGPRs allow
    // three waves per SIMD), each walking rows
    const int64_t per_cu = (seg && ext > 4096) ? 3 : 4;
    const int64_t nwg = std::min<int64_t>(nrows, per_cu * device_cu_count(st));
    const dim3 grid((unsigned)nwg), block(kThreads);
    const int rows = (int)nrows, cols = (int)ext;
    if (ext > 8 * kThreads * 8) {
        jagged_contig_long_kernel<8><<<dim3((unsigned)nrows), block, (size_t)3 * G * sizeof(uint32_t),
                                       st>>>(x, ldx, cols, offs, G, q, ldq, scales, ss_row, ss_g);
        return launch_status();
    }
#define MXQ_CONTIG(NR)                                                                             \
    do {                                                                                           \
        const size_t lds = ((3 * (size_t)G + 3) & ~(size_t)3) * sizeof(uint32_t) +                \
                           (seg ? 2 : 1) * (size_t)NR * kThreads * sizeof(uint32_t);               \
        if (seg)                                                                                   \
            jagged_contig_seg_kernel<NR><<<grid, block, lds, st>>>(x, ldx, rows, cols, offs, G, q,  \
                                                                   ldq, scales, ss_row, ss_g);     \
        else                                                                                       \
            jagged_contig_kernel<NR><<<grid, block, lds, st>>>(x, ldx, rows, cols, offs, G, q, ldq, \
                                                               scales, ss_row, ss_g);              \
    } while (0)
    if (ext <= 2048)
        MXQ_CONTIG(1);
    else if (ext <= 4096)
        MXQ_CONTIG(2);
    else if (ext <= 8192)
        MXQ_CONTIG(4);
    else
        MXQ_CONTIG(8);
#undef MXQ_CONTIG
    return launch_status();
}

// Grid and workspace of the colwise (strided) kernel on an (ext, ncols)
// view with G groups.  Items per strip (long groups and packs of short
// groups; only the device knows which) are bounded from the extent and G
// alone: a long group spans more than TROWS - 15 rows, so there are at most
// ext / (TROWS - 14) of them; a run of short groups starts at group 0 or
// where a group start enters another TROWS-row block (which includes every
// group after a long one), so there are at most ext / TROWS + 1 runs, each
// packed kPackMax groups at a time; and every item owns a group.  In split
// mode a long group of span n (rows from its 16-row-aligned start) makes
// ceil(n / CH) items, i.e. fewer than n / CH more than one, and the spans of
// at most min(G, ext / (TROWS - 14)) long groups add up to at most the
// extent plus 15 rows each.  Workgroups past the items exit after building
// the table, which costs about a microsecond per CU each.
struct ColwisePlan {
    int64_t nsuper, items, nblocks, ws_bytes;
};

// The split kernel's 4-wave workgroups build the group table one group per
// thread up to this many groups; beyond it every workgroup scans the whole
// table, and the 8-wave kernel without chunks is as fast or faster (random
// 16-row-aligned groups of the MoE x operand: 257-512 groups 73-76 against
// 84-89 us, 2048 groups 182 against 211 us, 4096 groups 410 against 650 us).
constexpr int64_t kSplitMaxGroups = 64 * kSplitWaves;

ColwisePlan colwise_plan(int64_t ext, int64_t ncols, int64_t G, bool split)
{
    split = split && G <= kSplitMaxGroups;
    constexpr int CG = kJaggedStridedCG, SPS = 8 / CG;
    const int NW = split ? kSplitWaves : kJaggedStridedWaves;
    const int64_t trows = 16 * NW * (64 / CG);
    const int64_t chunk = kSplitTiles * trows;
    ColwisePlan p;
    const int64_t nstrips = (ncols + 8 * CG - 1) / (8 * CG);
    p.nsuper = (nstrips + SPS - 1) / SPS;
    const int64_t nlong = ext / (trows - 14);
    const int64_t bound = nlong + ext / trows + G / kPackMax + 1;
    p.items = std::min<int64_t>(G, bound);
    if (split)
        p.items += (ext + 15 * std::min<int64_t>(G, nlong)) / chunk;
    p.nblocks = 8 * SPS * ((p.items * p.nsuper + 7) / 8);
    // one set per (first item of a long group, strip)
    p.ws_bytes = split ? p.items * p.nsuper * SPS * kSetWords * (int64_t)sizeof(uint32_t) : 0;
    return p;
}

// The scale slots (g, c), g < G, c < ncols, are distinct words: the
// workspace-free split path keeps one column's exchange in each.
bool distinct_scale_slots(int64_t G, int64_t ncols, int64_t ss_g, int64_t ss_c)
{
    const int64_t ag = ss_g < 0 ? -ss_g : ss_g, ac = ss_c < 0 ? -ss_c : ss_c;
    if (G == 1)
        return ncols == 1 || ac != 0;
    if (ncols == 1)
        return ag != 0;
    if (ag == 0 || ac == 0)
        return false;
    return ag / ncols >= ac || ac / G >= ag;   // one stride spans the other's whole extent
}

// The split path without a workspace applies: few enough groups for the
// 4-wave workgroups' table (one group per thread), at most kSlotMaxChunks
// chunks per group (the slot's 8-bit counts), distinct scale slots.
bool colwise_in_slots(int64_t ext, int64_t ncols, int64_t G, int64_t ss_g, int64_t ss_c)
{
    const int64_t chunk = (int64_t)kSplitTiles * 16 * kSplitWaves * (64 / kJaggedStridedCG);
    return G <= kSplitMaxGroups && ext <= kSlotMaxChunks * chunk &&
           distinct_scale_slots(G, ncols, ss_g, ss_c);
}

// The colwise tile kernel: chunks of T 128-row tiles x 256 columns.
// It takes the column-major colwise calls with at most kTileMaxGroups groups,
// at most kSlotMaxChunks chunks per group (so any offsets keep every exchange
// set within a block of resident workgroups) and groups of at most
// kTileMaxAvgRows rows on average.  Longer groups make sets of many chunks,
// and the split kernel's 1536-row chunks are faster there (x (16384, 4096),
// cold, with / without a workspace: one group 57 / 69 us against 67 / 83,
// groups of 4096 and 12288 rows 59 / 64 against 57 / 72; eight MoE groups
// 51 / 61 against 58 / 63).  Chunks are two tiles (168 VGPRs, three waves
// per SIMD), or one tile (102 VGPRs, four waves) for groups of at most
// kTileShortAvgRows rows on average: 256 fine-grained MoE groups (64 rows
// on average) 55.5 against 60 us with a workspace, while the 8 MoE groups
// take 63 against 51 us and 64 groups of 256 rows 44 against 41.
constexpr int64_t kTileMaxAvgRows = 4096;
constexpr int64_t kTileShortAvgRows = 128;

// tiles per chunk for these extents, 0 when the tile kernel does not apply.
// A group's chunks cover its rows from its start rounded down to 16 rows,
// at most ext + 15 rows, so every group has at most kSlotMaxChunks chunks
// when ext + 15 <= kSlotMaxChunks * CH.
int tile_t(int64_t ext, int64_t G)
{
    if (G > kTileMaxGroups)
        return 0;
    if (ext <= kTileShortAvgRows * G && ext + 15 <= kSlotMaxChunks * 128)
        return 1;
    if (ext <= kTileMaxAvgRows * G && ext + 15 <= kSlotMaxChunks * 256)
        return 2;
    return 0;
}

bool tile_applies(int64_t ext, int64_t G) { return tile_t(ext, G) != 0; }

// Grid and workspace of the tile kernel.  A group of n > 0 rows spans
// s <= n + 15 rows from its 16-row-aligned start and has max(1, ceil(s / CH))
// <= 1 + (s - 1) / CH chunks per column tile, an empty group one, so there
// are at most G + (ext + 14 G) / CH in all; a group of more than one chunk
// spans more than CH rows, i.e. has more than CH - 15, so there are at most
// min(G, ext / (CH - 14)) of them, one workspace set per column tile each.
struct TilePlan {
    int64_t t, ch, tiles_c, nblocks, nsets, ws_bytes;
};
TilePlan tile_plan(int64_t ext, int64_t ncols, int64_t G)
{
    TilePlan p;
    p.t = tile_t(ext, G);
    p.ch = 128 * (p.t ? p.t : 1);
    p.tiles_c = (ncols + 255) / 256;
    p.nblocks = p.tiles_c * (G + (ext + 14 * G) / p.ch);
    p.nsets = std::min<int64_t>(G, ext / (p.ch - 14));
    p.ws_bytes = p.nsets * p.tiles_c * kTileSetWords * (int64_t)sizeof(uint32_t);
    return p;
}

// workspace of the workspace call (the tile kernel's, else the split kernel's)
int64_t colwise_ws_bytes(int64_t ext, int64_t ncols, int64_t G)
{
    return tile_applies(ext, G) ? tile_plan(ext, ncols, G).ws_bytes : colwise_plan(ext, ncols, G, true).ws_bytes;
}

// jagged colwise on the tile kernel (tile_applies holds): exchange through
// ws, or with no ws through the long groups' scale slots, cleared by a small
// kernel launched first (distinct_scale_slots must hold)
mxq_status run_jagged_colwise_tile(const uint16_t *x, int64_t ext, int64_t ncols, int64_t ldx,
                                   const int32_t *offs, int32_t G, uint8_t *q, int64_t ldq, float *scales,
                                   int64_t ss_g, int64_t ss_c, hipStream_t st, uint32_t *ws,
                                   int64_t ws_bytes, int spin_limit = kColwiseSpinLimit)
{
    if (ncols == 0)
        return MXQ_OK;
    if (ncols % 8 != 0 || ncols > INT32_MAX)
        return MXQ_ERR_INVALID_ARG;
    const TilePlan p = tile_plan(ext, ncols, G);
    if (p.t == 0 || p.nblocks > INT32_MAX)
        return MXQ_ERR_INVALID_ARG;
    if (ws && ws_bytes < p.ws_bytes)
        return MXQ_ERR_WORKSPACE;
    if (!ws) {
        const dim3 cgrid((unsigned)std::min<int64_t>((ncols + 255) / 256, 64), (unsigned)G);
        jagged_colwise_tile_clear_kernel<<<cgrid, dim3(256), 0, st>>>(offs, G, (int)ext, (int)ncols, scales,
                                                                      ss_g, ss_c, (int)p.ch);
    }
    // sets per column tile the workspace holds (the plan's count or more)
    const int64_t nsets =
        ws ? std::min<int64_t>(ws_bytes / (p.tiles_c * kTileSetWords * (int64_t)sizeof(uint32_t)), INT32_MAX) : 0;
    const dim3 grid((unsigned)p.nblocks), block(256);
    if (p.t == 1)
        jagged_colwise_tile_kernel<1><<<grid, block, 0, st>>>(x, ldx, (int)ext, (int)ncols, offs, G, q, ldq, scales,
                                                              ss_g, ss_c, (int)p.tiles_c, ws, (int)nsets,
                                                              spin_limit);
    else
        jagged_colwise_tile_kernel<2><<<grid, block, 0, st>>>(x, ldx, (int)ext, (int)ncols, offs, G, q, ldq, scales,
                                                              ss_g, ss_c, (int)p.tiles_c, ws, (int)nsets,
                                                              spin_limit);
    return launch_status();
}

// jagged, reduction across rows of a (ext, ncols) row-major view, column-major
// q; split mode exchanges column maxima through ws (zero between calls) or,
// with no ws and `slots`, through the long groups' scale slots (cleared by a
// small kernel launched first)
mxq_status run_jagged_strided(const uint16_t *x, int64_t ext, int64_t ncols, int64_t ldx,
                              const int32_t *offs, int32_t G, uint8_t *q, int64_t ldq,
                              float *scales, int64_t ss_g, int64_t ss_col, hipStream_t st,
                              uint32_t *ws = nullptr, int64_t ws_bytes = 0,
                              int spin_limit = kColwiseSpinLimit, bool slots = false)
{
    if (ncols == 0)
        return MXQ_OK;
    if (ncols % 8 != 0 || ncols > INT32_MAX)
        return MXQ_ERR_INVALID_ARG;
    constexpr int CG = kJaggedStridedCG, NW = kJaggedStridedWaves, T = kJaggedStridedTiles;
    constexpr int NWS = kSplitWaves, TS = kSplitTiles;
    const bool split = (ws != nullptr || slots) && G <= kSplitMaxGroups;
    if (!split)
        ws = nullptr;   // many groups: the kernel without chunks needs no workspace
    const ColwisePlan p = colwise_plan(ext, ncols, G, split);
    if (p.nblocks > INT32_MAX || p.items > INT32_MAX)
        return MXQ_ERR_INVALID_ARG;
    if (ws && ws_bytes < p.ws_bytes)
        return MXQ_ERR_WORKSPACE;
    const size_t lds = G > 64 ? (3 * (size_t)G + 2) * sizeof(int) + (size_t)G : 0;
    const dim3 grid((unsigned)p.nblocks), block(64 * (split ? NWS : NW));
    if (!ws && slots) {
        const int ch = TS * 16 * NWS * (64 / CG);
        const dim3 cgrid((unsigned)std::min<int64_t>((ncols + 255) / 256, 64), (unsigned)G);
        jagged_colwise_clear_kernel<<<cgrid, dim3(256), 0, st>>>(offs, G, (int)ext, (int)ncols, scales,
                                                                 ss_g, ss_col, ch);
    }
    if (split)
        jagged_strided_kernel<CG, TS, NWS, true><<<grid, block, lds, st>>>(
            x, ldx, (int)ext, (int)ncols, offs, G, q, ldq, scales, ss_g, ss_col, (int)p.nsuper,
            (int)p.items, ws, spin_limit);
    else
        jagged_strided_kernel<CG, T, NW, false><<<grid, block, lds, st>>>(
            x, ldx, (int)ext, (int)ncols, offs, G, q, ldq, scales, ss_g, ss_col, (int)p.nsuper,
            (int)p.items, nullptr, 0);
    return launch_status();
}

mxq_status check_jagged_common(const uint16_t *x, int64_t rows, int64_t cols, const int32_t *offs,
                               int32_t G, const uint8_t *q, const float *scales)
{
    if (rows < 0 || cols < 0 || G < 1 || G > MXQ_MAX_GROUPS)
        return MXQ_ERR_INVALID_ARG;
    if (rows > INT32_MAX || cols > INT32_MAX)
        return MXQ_ERR_INVALID_ARG;
    if (!offs || !scales)
        return MXQ_ERR_INVALID_ARG;
    if ((rows > 0 && cols > 0) && (!x || !q))
        return MXQ_ERR_INVALID_ARG;
    if (x && !aligned16(x))
        return MXQ_ERR_INVALID_ARG;
    if (q && !aligned16(q))
        return MXQ_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(scales) & 3u) != 0)
        return MXQ_ERR_INVALID_ARG;
    return MXQ_OK;
}

mxq_status check_jagged_mx(const uint16_t *x, int64_t rows, int64_t cols, const int32_t *offs,
                           int32_t G, const uint8_t *q, const uint8_t *scales, int32_t scale_mode)
{
    if (rows < 0 || cols < 0 || G < 1 || G > MXQ_MAX_GROUPS)
        return MXQ_ERR_INVALID_ARG;
    if (rows > INT32_MAX || cols > INT32_MAX)
        return MXQ_ERR_INVALID_ARG;
    if (scale_mode != MXQ_SCALE_FLOOR && scale_mode != MXQ_SCALE_RCEIL)
        return MXQ_ERR_INVALID_ARG;
    if (!offs)
        return MXQ_ERR_INVALID_ARG;
    if ((rows > 0 && cols > 0) && (!x || !q || !scales))
        return MXQ_ERR_INVALID_ARG;
    if ((x && !aligned16(x)) || (q && !aligned16(q)))
        return MXQ_ERR_INVALID_ARG;
    return MXQ_OK;
}

// blocks along the unit-stride dim of a row-major (rows, cols) tensor
mxq_status run_jagged_mx_rows(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx,
                              const int32_t *offs, int G, uint8_t *q, int64_t ldq,
                              uint8_t *scales, int64_t ss_r, int64_t ss_b, bool rceil,
                              hipStream_t st)
{
    constexpr int RW = 8;   // rows per workgroup (8 measured faster than 4, 16 or 32)
    const int64_t nbmax = (cols + 31) / 32 + G - 1;
    const int64_t nbt = (nbmax + 63) / 64;
    const int64_t nrt = (rows + RW - 1) / RW;
    if (nbt * nrt > INT32_MAX)
        return MXQ_ERR_INVALID_ARG;
    jagged_mx_rowwise_kernel<RW><<<dim3((unsigned)(nbt * nrt)), dim3(kJmxThreads), 0, st>>>(
        x, ldx, (int)rows, (int)cols, offs, G, q, ldq, scales, ss_r, ss_b, (int)nbt, rceil ? 1 : 0);
    return launch_status();
}

// blocks across the rows of a row-major (rows, cols) tensor, q column-major
mxq_status run_jagged_mx_cols(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx,
                              const int32_t *offs, int G, uint8_t *q, int64_t ldq,
                              uint8_t *scales, int64_t ss_b, int64_t ss_c, bool rceil,
                              hipStream_t st)
{
    const int64_t ntr = (rows + 127) / 128 + G - 1;
    const int64_t tiles_c = (cols + 255) / 256;
    if (ntr * tiles_c > INT32_MAX)
        return MXQ_ERR_INVALID_ARG;
    jagged_mx_colwise_kernel<<<dim3((unsigned)(ntr * tiles_c)), dim3(kJmxThreads), 0, st>>>(
        x, ldx, (int)rows, (int)cols, offs, G, q, ldq, scales, ss_b, ss_c, (int)tiles_c,
        rceil ? 1 : 0);
    return launch_status();
}

// The colwise call that allocates nothing keeps its exchange sets in this
// file-scope device array (one copy per GPU, held until the process ends).
// In host code its name is a host-side stand-in: kernels get the device
// address, looked up once per device with that device current.
constexpr int64_t kScratchBytes = MXQ_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint32_t scratch[kScratchBytes / sizeof(uint32_t)];

// device that runs `st` (the calling thread's current device for the null
// stream), or -1
int stream_device(hipStream_t st)
{
    int dev = -1;
    if (st) {
        hipDevice_t d = 0;
        if (hipStreamGetDevice(st, &d) != hipSuccess)
            return -1;
        dev = (int)d;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return -1;
    }
    return dev;
}

// device address of `scratch` on device dev (nullptr on failure)
uint32_t *scratch_on(int dev)
{
    static std::atomic<uint32_t *> addr[64];
    static std::mutex init;
    if (dev < 0 || dev >= 64)
        return nullptr;
    uint32_t *p = addr[dev].load(std::memory_order_acquire);
    if (p)
        return p;
    std::lock_guard<std::mutex> lock(init);
    p = addr[dev].load(std::memory_order_relaxed);
    if (p)
        return p;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess)
        return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess)
        return nullptr;
    void *sym = nullptr;
    const hipError_t e = hipGetSymbolAddress(&sym, HIP_SYMBOL(scratch));
    if (cur != dev)
        (void)hipSetDevice(cur);
    if (e != hipSuccess || !sym)
        return nullptr;
    p = static_cast<uint32_t *>(sym);
    addr[dev].store(p, std::memory_order_release);
    return p;
}

template <int LAYOUT, int SEG, bool XCD>
mxq_status run_relayout(const uint8_t *scales, int64_t rows, int64_t ss_r, int64_t ss_b,
                        const int32_t *offs, int G, int64_t extent, uint8_t *tiles,
                        int32_t *tile_starts, hipStream_t st)
{
    using SH = RelayoutShape<LAYOUT, SEG>;
    const int64_t rb = (rows + 15) / 16;
    const int64_t rc = (rb + SH::CR - 1) / SH::CR;
    const int64_t nchunk = std::max<int64_t>(1, (extent + (1 << SH::SHC) - 1) / (1 << SH::SHC) + G - 1);
    const int64_t nitems = rc * nchunk;
    if (nitems == 0 && tile_starts == nullptr)
        return MXQ_OK;
    // at least one workgroup (workgroup 0 writes tile_starts); a multiple of
    // 8 for the XCD-ordered item mapping
    int64_t grid = std::max<int64_t>(nitems, 1);
    if (XCD)
        grid = (grid + 7) / 8 * 8;
    if (grid > INT32_MAX)
        return MXQ_ERR_INVALID_ARG;
    relayout_mx_scales_kernel<LAYOUT, SEG, XCD>
        <<<dim3((unsigned)grid), dim3(kRelayoutThreads), relayout_lds_bytes<LAYOUT, SEG>(G), st>>>(
            scales, ss_r, ss_b, (int)rows, (int)extent, offs, G, tiles, tile_starts, (int)nchunk,
            (int)nitems);
    return launch_status();
}

}  // namespace

extern "C" {

int mxq_abi_version(void) { return MXQ_ABI_VERSION; }

const char *mxq_status_string(int status)
{
    switch (status) {
    case MXQ_OK: return "MXQ_OK";
    case MXQ_ERR_INVALID_ARG: return "MXQ_ERR_INVALID_ARG";
    case MXQ_ERR_UNSUPPORTED: return "MXQ_ERR_UNSUPPORTED";
    case MXQ_ERR_LAUNCH: return "MXQ_ERR_LAUNCH";
    case MXQ_ERR_WORKSPACE: return "MXQ_ERR_WORKSPACE";
    default: return "MXQ_ERR_UNKNOWN";
    }
}

mxq_status mxq_quantize_jagged_rowwise(const uint16_t *x, int64_t rows, int64_t cols, int64_t sx_r,
                                       int64_t sx_c, const int32_t *offs, int32_t num_groups,
                                       uint8_t *q, int64_t sq_r, int64_t sq_c, float *scales,
                                       int64_t ss_r, int64_t ss_g, void *stream)
{
    mxq_status s = check_jagged_common(x, rows, cols, offs, num_groups, q, scales);
    if (s != MXQ_OK)
        return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (rows == 0)
        return MXQ_OK;
    if (sx_c == 1 && sq_c == 1) {
        if (rows > 1 && cols >= 8 && (sx_r % 8 != 0 || sq_r % 16 != 0))
            return MXQ_ERR_INVALID_ARG;
        return run_jagged_contig(x, rows, cols, sx_r, offs, num_groups, q, sq_r, scales, ss_r, ss_g, st);
    }
    if (sx_r == 1 && sq_c == 1) {
        // x is the transpose of a row-major (cols, rows) tensor: reduce across
        // its rows, store column-major of that tensor == row-major q.  Long
        // groups are split into chunks exchanging through the scale slots
        // where they apply (the tile kernel's 256-column sets would touch
        // slots G words apart: slower here), so no row is read twice
        if (sx_c % 8 != 0 || sq_r % 16 != 0)
            return MXQ_ERR_INVALID_ARG;
        return run_jagged_strided(x, cols, rows, sx_c, offs, num_groups, q, sq_r, scales, ss_g, ss_r, st,
                                  nullptr, 0, kColwiseSpinLimit,
                                  colwise_in_slots(cols, rows, num_groups, ss_g, ss_r));
    }
    return MXQ_ERR_UNSUPPORTED;
}

mxq_status mxq_quantize_jagged_colwise(const uint16_t *x, int64_t rows, int64_t cols, int64_t sx_r,
                                       int64_t sx_c, const int32_t *offs, int32_t num_groups,
                                       uint8_t *q, int64_t sq_r, int64_t sq_c, float *scales,
                                       int64_t ss_g, int64_t ss_c, void *stream)
{
    mxq_status s = check_jagged_common(x, rows, cols, offs, num_groups, q, scales);
    if (s != MXQ_OK)
        return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (cols == 0)
        return MXQ_OK;
    if (sx_c == 1 && sq_r == 1) {
        if (sx_r % 8 != 0 || sq_c % 16 != 0)
            return MXQ_ERR_INVALID_ARG;
        if (tile_applies(rows, num_groups) && distinct_scale_slots(num_groups, cols, ss_g, ss_c))
            return run_jagged_colwise_tile(x, rows, cols, sx_r, offs, num_groups, q, sq_c, scales, ss_g,
                                           ss_c, st, nullptr, 0);
        return run_jagged_strided(x, rows, cols, sx_r, offs, num_groups, q, sq_c, scales, ss_g, ss_c, st,
                                  nullptr, 0, kColwiseSpinLimit,
                                  colwise_in_slots(rows, cols, num_groups, ss_g, ss_c));
    }
    if (sx_r == 1 && sq_r == 1) {
        // column-major in and out: the rowwise pattern on the transpose
        if (cols > 1 && rows >= 8 && (sx_c % 8 != 0 || sq_c % 16 != 0))
            return MXQ_ERR_INVALID_ARG;
        return run_jagged_contig(x, cols, rows, sx_c, offs, num_groups, q, sq_c, scales, ss_c, ss_g, st);
    }
    return MXQ_ERR_UNSUPPORTED;
}

mxq_status mxq_quantize_jagged_colwise_noalloc(const uint16_t *x, int64_t rows, int64_t cols,
                                               int64_t sx_r, int64_t sx_c, const int32_t *offs,
                                               int32_t num_groups, uint8_t *q, int64_t sq_r,
                                               int64_t sq_c, float *scales, int64_t ss_g,
                                               int64_t ss_c, void *stream)
{
    mxq_status s = check_jagged_common(x, rows, cols, offs, num_groups, q, scales);
    if (s != MXQ_OK)
        return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (cols == 0)
        return MXQ_OK;
    if (sx_c == 1 && sq_r == 1) {
        if (sx_r % 8 != 0 || sq_c % 16 != 0)
            return MXQ_ERR_INVALID_ARG;
        if (colwise_ws_bytes(rows, cols, num_groups) > kScratchBytes)
            return MXQ_ERR_WORKSPACE;
        uint32_t *ws = scratch_on(stream_device(st));
        if (!ws)
            return MXQ_ERR_LAUNCH;
        if (tile_applies(rows, num_groups))
            return run_jagged_colwise_tile(x, rows, cols, sx_r, offs, num_groups, q, sq_c, scales, ss_g,
                                           ss_c, st, ws, kScratchBytes);
        return run_jagged_strided(x, rows, cols, sx_r, offs, num_groups, q, sq_c, scales, ss_g, ss_c,
                                  st, ws, kScratchBytes);
    }
    return mxq_quantize_jagged_colwise(x, rows, cols, sx_r, sx_c, offs, num_groups, q, sq_r, sq_c,
                                       scales, ss_g, ss_c, stream);
}

int64_t mxq_jagged_colwise_workspace_bytes(int64_t rows, int64_t cols, int32_t num_groups)
{
    if (rows < 0 || cols < 0 || num_groups < 1 || num_groups > MXQ_MAX_GROUPS)
        return -1;
    return colwise_ws_bytes(rows, cols, num_groups);
}

mxq_status mxq_quantize_jagged_colwise_ws(const uint16_t *x, int64_t rows, int64_t cols,
                                          int64_t sx_r, int64_t sx_c, const int32_t *offs,
                                          int32_t num_groups, uint8_t *q, int64_t sq_r,
                                          int64_t sq_c, float *scales, int64_t ss_g, int64_t ss_c,
                                          void *workspace, int64_t workspace_bytes, void *stream)
{
    mxq_status s = check_jagged_common(x, rows, cols, offs, num_groups, q, scales);
    if (s != MXQ_OK)
        return s;
    if (workspace_bytes < 0 || (workspace && (reinterpret_cast<uintptr_t>(workspace) & 3u) != 0))
        return MXQ_ERR_INVALID_ARG;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (cols == 0)
        return MXQ_OK;
    if (sx_c == 1 && sq_r == 1) {
        if (sx_r % 8 != 0 || sq_c % 16 != 0)
            return MXQ_ERR_INVALID_ARG;
        if (num_groups > kSplitMaxGroups)   // no chunks, no workspace
            return run_jagged_strided(x, rows, cols, sx_r, offs, num_groups, q, sq_c, scales, ss_g,
                                      ss_c, st);
        if (!workspace)
            return MXQ_ERR_WORKSPACE;
        if (tile_applies(rows, num_groups))
            return run_jagged_colwise_tile(x, rows, cols, sx_r, offs, num_groups, q, sq_c, scales, ss_g,
                                           ss_c, st, reinterpret_cast<uint32_t *>(workspace),
                                           workspace_bytes);
        return run_jagged_strided(x, rows, cols, sx_r, offs, num_groups, q, sq_c, scales, ss_g, ss_c,
                                  st, reinterpret_cast<uint32_t *>(workspace), workspace_bytes);
    }
    // the other layout reads every row once without a workspace
    return mxq_quantize_jagged_colwise(x, rows, cols, sx_r, sx_c, offs, num_groups, q, sq_r, sq_c,
                                       scales, ss_g, ss_c, stream);
}

mxq_status mxq_quantize_mx_3d_colwise(const uint16_t *w, int64_t E, int64_t N, int64_t K,
                                      int64_t sw_e, int64_t sw_n, int64_t sw_k, uint8_t *q,
                                      int64_t sq_e, int64_t sq_n, int64_t sq_k, uint8_t *scales,
                                      int64_t ss_e, int64_t ss_nb, int64_t ss_k,
                                      int32_t scale_mode, void *stream)
{
    if (E < 0 || N < 0 || K < 0 || N % 32 != 0)
        return MXQ_ERR_INVALID_ARG;
    if (scale_mode != MXQ_SCALE_FLOOR && scale_mode != MXQ_SCALE_RCEIL)
        return MXQ_ERR_INVALID_ARG;
    if (E == 0 || N == 0 || K == 0)
        return MXQ_OK;
    if (!w || !q || !scales)
        return MXQ_ERR_INVALID_ARG;
    if (!(sw_k == 1 && sq_n == 1))
        return MXQ_ERR_UNSUPPORTED;
    if (!aligned16(w) || !aligned16(q) || K % 8 != 0 || sw_n % 8 != 0 || sw_e % 8 != 0 ||
        sq_k % 16 != 0 || sq_e % 16 != 0)
        return MXQ_ERR_INVALID_ARG;
    if (N > INT32_MAX || K > INT32_MAX)
        return MXQ_ERR_INVALID_ARG;
    const int64_t tiles_r = (N + 127) / 128, tiles_c = (K + 255) / 256;
    const int64_t nblocks = E * tiles_r * tiles_c;
    if (nblocks > INT32_MAX)
        return MXQ_ERR_INVALID_ARG;
    block_strided_kernel<32, 1, true><<<dim3((unsigned)nblocks), dim3(kBlockThreads), 0,
                                         reinterpret_cast<hipStream_t>(stream)>>>(
        w, sw_e, sw_n, (int)N, (int)K, q, sq_e, sq_k, scales, ss_e, ss_nb, ss_k, (int)tiles_r,
        (int)tiles_c, scale_mode == MXQ_SCALE_RCEIL, mx3d_store_mode(q, N, K, sq_k, sq_e), tile_chunk(nblocks));
    return launch_status();
}

mxq_status mxq_quantize_mx_rowwise(const uint16_t *x, int64_t rows, int64_t cols, int64_t sx_r,
                                   int64_t sx_c, uint8_t *q, int64_t sq_r, int64_t sq_c,
                                   uint8_t *scales, int64_t ss_r, int64_t ss_b,
                                   int32_t scale_mode, void *stream)
{
    if (rows < 0 || cols < 0 || cols % 32 != 0)
        return MXQ_ERR_INVALID_ARG;
    if (scale_mode != MXQ_SCALE_FLOOR && scale_mode != MXQ_SCALE_RCEIL)
        return MXQ_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0)
        return MXQ_OK;
    if (!x || !q || !scales)
        return MXQ_ERR_INVALID_ARG;
    if (!(sx_c == 1 && sq_c == 1))
        return MXQ_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(q) || sx_r % 8 != 0 || sq_r % 16 != 0)
        return MXQ_ERR_INVALID_ARG;
    constexpr int U = 4, LPB = 4;
    const int64_t nbpr = cols / 32, nblocks = rows * nbpr;
    const int64_t per_wg = (int64_t)U * (kBlockThreads / LPB);
    const int64_t grid = (nblocks + per_wg - 1) / per_wg;
    if (grid > INT32_MAX)
        return MXQ_ERR_INVALID_ARG;
    block_contig_kernel<32, LPB, true, U><<<dim3((unsigned)grid), dim3(kBlockThreads), 0,
                                            reinterpret_cast<hipStream_t>(stream)>>>(
        x, sx_r, nbpr, nblocks, q, sq_r, scales, ss_r, ss_b, scale_mode == MXQ_SCALE_RCEIL);
    return launch_status();
}

mxq_status mxq_quantize_jagged_mx_rowwise(const uint16_t *x, int64_t rows, int64_t cols,
                                          int64_t sx_r, int64_t sx_c, const int32_t *offs,
                                          int32_t num_groups, uint8_t *q, int64_t sq_r,
                                          int64_t sq_c, uint8_t *scales, int64_t ss_r,
                                          int64_t ss_b, int32_t scale_mode, void *stream)
{
    mxq_status s = check_jagged_mx(x, rows, cols, offs, num_groups, q, scales, scale_mode);
    if (s != MXQ_OK)
        return s;
    if (rows == 0 || cols == 0)
        return MXQ_OK;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const bool rc = scale_mode == MXQ_SCALE_RCEIL;
    if (sx_c == 1 && sq_c == 1) {
        if (rows > 1 && (sx_r % 8 != 0 || sq_r % 16 != 0))
            return MXQ_ERR_INVALID_ARG;
        return run_jagged_mx_rows(x, rows, cols, sx_r, offs, num_groups, q, sq_r, scales, ss_r,
                                  ss_b, rc, st);
    }
    if (sx_r == 1 && sq_c == 1) {
        // a transposed view of a row-major (cols, rows) tensor: its blocks run
        // across that tensor's rows, and its column-major q is this row-major q
        if (rows % 8 != 0 || sx_c % 8 != 0 || sq_r % 16 != 0)
            return MXQ_ERR_INVALID_ARG;
        return run_jagged_mx_cols(x, cols, rows, sx_c, offs, num_groups, q, sq_r, scales, ss_b,
                                  ss_r, rc, st);
    }
    return MXQ_ERR_UNSUPPORTED;
}

mxq_status mxq_quantize_jagged_mx_colwise(const uint16_t *x, int64_t rows, int64_t cols,
                                          int64_t sx_r, int64_t sx_c, const int32_t *offs,
                                          int32_t num_groups, uint8_t *q, int64_t sq_r,
                                          int64_t sq_c, uint8_t *scales, int64_t ss_b,
                                          int64_t ss_c, int32_t scale_mode, void *stream)
{
    mxq_status s = check_jagged_mx(x, rows, cols, offs, num_groups, q, scales, scale_mode);
    if (s != MXQ_OK)
        return s;
    if (rows == 0 || cols == 0)
        return MXQ_OK;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const bool rc = scale_mode == MXQ_SCALE_RCEIL;
    if (sx_c == 1 && sq_r == 1) {
        if (cols % 8 != 0 || sx_r % 8 != 0 || sq_c % 16 != 0)
            return MXQ_ERR_INVALID_ARG;
        return run_jagged_mx_cols(x, rows, cols, sx_r, offs, num_groups, q, sq_c, scales, ss_b,
                                  ss_c, rc, st);
    }
    if (sx_r == 1 && sq_r == 1) {
        // column-major in and out: the rowwise pattern on the transpose
        if (cols > 1 && (sx_c % 8 != 0 || sq_c % 16 != 0))
            return MXQ_ERR_INVALID_ARG;
        return run_jagged_mx_rows(x, cols, rows, sx_c, offs, num_groups, q, sq_c, scales, ss_c,
                                  ss_b, rc, st);
    }
    return MXQ_ERR_UNSUPPORTED;
}

mxq_status mxq_relayout_mx_scales_grouped(const uint8_t *scales, int64_t rows, int64_t ss_r,
                                          int64_t ss_b, const int32_t *offs, int32_t num_groups,
                                          int64_t extent, uint8_t *tiles, int32_t *tile_starts,
                                          void *stream)
{
    const int32_t G = num_groups;
    if (rows < 0 || extent < 0 || G < 1 || G > MXQ_MAX_GROUPS || !offs)
        return MXQ_ERR_INVALID_ARG;
    if (rows > INT32_MAX || extent > INT32_MAX || ss_r < 0 || ss_b < 0)
        return MXQ_ERR_INVALID_ARG;
    // tile numbers are int32 (tile_starts): bound the largest one
    const int64_t max_tiles = ((rows + 15) / 16) * ((extent + 511) / 512 + G - 1);
    if (max_tiles > INT32_MAX)
        return MXQ_ERR_INVALID_ARG;
    if (rows > 0 && extent > 0 && (!scales || !tiles))
        return MXQ_ERR_INVALID_ARG;
    if ((tiles && !aligned16(tiles)) ||
        (tile_starts && (reinterpret_cast<uintptr_t>(tile_starts) & 3u) != 0))
        return MXQ_ERR_INVALID_ARG;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (ss_b == 1)
        return run_relayout<0, 4, false>(scales, rows, ss_r, ss_b, offs, G, extent, tiles,
                                        tile_starts, st);
    if (ss_r == 1)
        return run_relayout<1, 4, true>(scales, rows, ss_r, ss_b, offs, G, extent, tiles,
                                        tile_starts, st);
    return run_relayout<2, 4, false>(scales, rows, ss_r, ss_b, offs, G, extent, tiles, tile_starts,
                                     st);
}

mxq_status mxq_quantize_blockwise(const uint16_t *x, int64_t rows, int64_t cols, int64_t sx_r,
                                  int64_t sx_c, int32_t block_r, int32_t block_c, uint8_t *q,
                                  int64_t sq_r, int64_t sq_c, float *scales, int64_t ss_rb,
                                  int64_t ss_cb, void *stream)
{
    if (rows < 0 || cols < 0 || block_r <= 0 || block_c <= 0)
        return MXQ_ERR_INVALID_ARG;
    if (rows % block_r != 0 || cols % block_c != 0)
        return MXQ_ERR_INVALID_ARG;
    const bool known = (block_r == 1 && block_c == 128) || (block_r == 128 && block_c == 128) ||
                       (block_r == 128 && block_c == 1);
    if (!known)
        return MXQ_ERR_UNSUPPORTED;
    if (rows == 0 || cols == 0)
        return MXQ_OK;
    if (!x || !q || !scales)
        return MXQ_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(scales) & 3u) != 0)
        return MXQ_ERR_INVALID_ARG;
    if (rows > INT32_MAX || cols > INT32_MAX)
        return MXQ_ERR_INVALID_ARG;
    // a column-major x (a transposed view of a row-major tensor) is the
    // row-major tensor with the block shape, the q strides and the scale
    // strides transposed
    if (sx_c != 1 && sx_r == 1) {
        std::swap(rows, cols);
        std::swap(sx_r, sx_c);
        std::swap(block_r, block_c);
        std::swap(sq_r, sq_c);
        std::swap(ss_rb, ss_cb);
    }
    if (sx_c != 1 || !(sq_c == 1 || sq_r == 1))
        return MXQ_ERR_UNSUPPORTED;
    if (!aligned16(x) || sx_r % 8 != 0 || !aligned16(q))
        return MXQ_ERR_INVALID_ARG;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const bool qrow = sq_c == 1 && (sq_r != 1 || rows == 1);
    if (block_r == 1 && qrow) {
        // 1 x 128 along the unit stride into row-major q
        if (rows > 1 && sq_r % 16 != 0)
            return MXQ_ERR_INVALID_ARG;
        constexpr int U = 4, LPB = 8;
        const int64_t nbpr = cols / 128, nblocks = rows * nbpr;
        const int64_t per_wg = (int64_t)U * (kBlockThreads / LPB);
        const int64_t grid = (nblocks + per_wg - 1) / per_wg;
        if (grid > INT32_MAX)
            return MXQ_ERR_INVALID_ARG;
        block_contig_kernel<128, LPB, false, U><<<dim3((unsigned)grid), dim3(kBlockThreads), 0, st>>>(
            x, sx_r, nbpr, nblocks, q, sq_r, scales, ss_rb, ss_cb, 0);
        return launch_status();
    }
    // the 128 x 256 tile kernel: 16-row pieces of 8 columns per lane
    if (cols % 8 != 0 || rows % 16 != 0)
        return MXQ_ERR_INVALID_ARG;
    const int64_t ldq = qrow ? sq_r : sq_c;
    if (qrow ? (rows > 1 && ldq % 8 != 0) : (cols > 1 && ldq % 16 != 0))
        return MXQ_ERR_INVALID_ARG;
    const int64_t tiles_r = (rows + 127) / 128, tiles_c = (cols + 255) / 256;
    const int64_t nblocks = tiles_r * tiles_c;
    if (nblocks > INT32_MAX)
        return MXQ_ERR_INVALID_ARG;
    const dim3 grid((unsigned)nblocks), block(kBlockThreads);
    const int nt = qrow ? 0 : line_aligned(q, ldq, 0);
#define MXQ_STRIDED(BR, BC, QR)                                                                   \
    block_strided_kernel<BR, BC, false, QR><<<grid, block, 0, st>>>(                              \
        x, 0, sx_r, (int)rows, (int)cols, q, 0, ldq, scales, 0, ss_rb, ss_cb, (int)tiles_r,        \
        (int)tiles_c, 0, nt, tile_chunk(nblocks))
    if (block_r == 1)
        MXQ_STRIDED(1, 128, false);
    else if (block_c == 128 && qrow)
        MXQ_STRIDED(128, 128, true);
    else if (block_c == 128)
        MXQ_STRIDED(128, 128, false);
    else if (qrow)
        MXQ_STRIDED(128, 1, true);
    else
        MXQ_STRIDED(128, 1, false);
#undef MXQ_STRIDED
    return launch_status();
}

}  // extern "C"

// ------------------------------------------------------------ diagnostics

namespace {
__global__ void debug_cast_kernel(const float *__restrict__ y, int64_t n, uint8_t *__restrict__ out)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t k = i; k < n; k += stride)
        out[k] = (uint8_t)mxq::cvt1(y[k]);
}

// four consecutive values per thread through the packed conversions the
// kernels use: cvt4 (clamped; e8m0 paths) or cvt4_nosat (fp32-multiplier
// paths); a short last quad is padded with zeros and stored byte by byte
__global__ void debug_cast4_kernel(const float *__restrict__ y, int64_t n, uint8_t *__restrict__ out,
                                   int unclamped)
{
    const int64_t nq = (n + 3) / 4;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t k = i; k < nq; k += stride) {
        const int64_t e = 4 * k;
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            v[j] = e + j < n ? y[e + j] : 0.0f;
        const uint32_t r = unclamped ? mxq::cvt4_nosat(v[0], v[1], v[2], v[3])
                                     : mxq::cvt4(v[0], v[1], v[2], v[3]);
        if (e + 4 <= n) {
            *reinterpret_cast<uint32_t *>(out + e) = r;
        } else {
            for (int j = 0; e + j < n; ++j)
                out[e + j] = (uint8_t)(r >> (8 * j));
        }
    }
}

unsigned debug_grid(int64_t items)
{
    int64_t blocks = (items + 255) / 256;
    return (unsigned)(blocks > 65536 ? 65536 : blocks);
}
}  // namespace

extern "C" mxq_status mxq_debug_cast_e4m3(const float *y, int64_t n, uint8_t *out, void *stream)
{
    if (n < 0)
        return MXQ_ERR_INVALID_ARG;
    if (n == 0)
        return MXQ_OK;
    if (!y || !out)
        return MXQ_ERR_INVALID_ARG;
    debug_cast_kernel<<<dim3(debug_grid(n)), dim3(256), 0, reinterpret_cast<hipStream_t>(stream)>>>(y, n, out);
    return launch_status();
}

// the split colwise path with a given wait bound (see include/mxq.h)
extern "C" mxq_status mxq_debug_jagged_colwise_ws_spin(
    const uint16_t *x, int64_t rows, int64_t cols, int64_t sx_r, int64_t sx_c, const int32_t *offs,
    int32_t num_groups, uint8_t *q, int64_t sq_r, int64_t sq_c, float *scales, int64_t ss_g,
    int64_t ss_c, void *workspace, int64_t workspace_bytes, int32_t spin_limit, void *stream)
{
    mxq_status s = check_jagged_common(x, rows, cols, offs, num_groups, q, scales);
    if (s != MXQ_OK)
        return s;
    if (!(sx_c == 1 && sq_r == 1) || workspace_bytes < 0 ||
        (reinterpret_cast<uintptr_t>(workspace) & 3u) != 0 || sx_r % 8 != 0 || sq_c % 16 != 0)
        return MXQ_ERR_INVALID_ARG;
    if (tile_applies(rows, num_groups)) {
        // no workspace: the exchange in the scale slots, where it applies
        if (!workspace && !distinct_scale_slots(num_groups, cols, ss_g, ss_c))
            return MXQ_ERR_INVALID_ARG;
        return run_jagged_colwise_tile(x, rows, cols, sx_r, offs, num_groups, q, sq_c, scales, ss_g, ss_c,
                                       reinterpret_cast<hipStream_t>(stream),
                                       reinterpret_cast<uint32_t *>(workspace), workspace_bytes, spin_limit);
    }
    if (!workspace && !colwise_in_slots(rows, cols, num_groups, ss_g, ss_c))
        return MXQ_ERR_INVALID_ARG;
    return run_jagged_strided(x, rows, cols, sx_r, offs, num_groups, q, sq_c, scales, ss_g, ss_c,
                              reinterpret_cast<hipStream_t>(stream),
                              reinterpret_cast<uint32_t *>(workspace), workspace_bytes, spin_limit,
                              workspace == nullptr);
}

extern "C" mxq_status mxq_debug_cast4_e4m3(const float *y, int64_t n, uint8_t *out, int32_t unclamped,
                                           void *stream)
{
    if (n < 0 || (unclamped != 0 && unclamped != 1))
        return MXQ_ERR_INVALID_ARG;
    if (n == 0)
        return MXQ_OK;
    if (!y || !out || (reinterpret_cast<uintptr_t>(out) & 3u) != 0)
        return MXQ_ERR_INVALID_ARG;
    debug_cast4_kernel<<<dim3(debug_grid((n + 3) / 4)), dim3(256), 0, reinterpret_cast<hipStream_t>(stream)>>>(
        y, n, out, unclamped);
    return launch_status();
}
