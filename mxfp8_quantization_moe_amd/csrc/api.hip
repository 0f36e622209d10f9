// C-ABI entry points of libmxq: argument validation, layout dispatch and
// kernel launches.  No allocation, no synchronisation, no read-back.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "mxq.h"
#include "block_kernels.hpp"
#include "jagged_kernels.hpp"
#include "jagged_mx_kernels.hpp"
#include "relayout_kernels.hpp"

namespace {

using namespace mxq;

constexpr int kJaggedStridedCG = 8;     // 64-column strips (full 128-byte row pieces)
constexpr int kJaggedStridedTiles = 3;  // register tiles per lane (233 VGPRs, 2 waves per SIMD)
constexpr int kJaggedStridedWaves = 8;  // waves per workgroup: tile = 8*16*64/CG = 1024 rows

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// column-major q whose 128-row column runs start on 128-byte lines: base and
// the column (and batch) strides on lines
int line_aligned(const void *q, int64_t ldq, int64_t sqe)
{
    return ((reinterpret_cast<uintptr_t>(q) & 127u) == 0 && ldq % 128 == 0 && sqe % 128 == 0) ? 1 : 0;
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
    const size_t lds = (size_t)3 * G * sizeof(uint32_t);
    // persistent grid: a few workgroups per compute unit, each walking rows
    const int64_t per_cu = 4;
    const int64_t nwg = std::min<int64_t>(nrows, per_cu * device_cu_count(st));
    const dim3 grid((unsigned)nwg), block(kThreads);
    const int rows = (int)nrows, cols = (int)ext;
    if (ext > 8 * kThreads * 8) {
        jagged_contig_long_kernel<8><<<dim3((unsigned)nrows), block, lds, st>>>(
            x, ldx, cols, offs, G, q, ldq, scales, ss_row, ss_g);
        return launch_status();
    }
#define MXQ_CONTIG(NR)                                                                             \
    jagged_contig_kernel<NR><<<grid, block, lds, st>>>(x, ldx, rows, cols, offs, G, q, ldq, scales, \
                                                       ss_row, ss_g)
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

// jagged, reduction across rows of a (ext, ncols) row-major view, column-major q
mxq_status run_jagged_strided(const uint16_t *x, int64_t ext, int64_t ncols, int64_t ldx,
                              const int32_t *offs, int32_t G, uint8_t *q, int64_t ldq,
                              float *scales, int64_t ss_g, int64_t ss_col, hipStream_t st)
{
    if (ncols == 0)
        return MXQ_OK;
    if (ncols % 8 != 0 || ncols > INT32_MAX)
        return MXQ_ERR_INVALID_ARG;
    constexpr int CG = kJaggedStridedCG, SPS = 8 / CG, NW = kJaggedStridedWaves;
    const int64_t nstrips = (ncols + 8 * CG - 1) / (8 * CG);
    const int64_t nsuper = (nstrips + SPS - 1) / SPS;
    // items per strip (long groups and packs of short groups; only the
    // device knows which), bounded from the extent and G alone: a long group
    // spans more than TROWS - 15 rows, so there are at most ext / (TROWS -
    // 14) of them; a run of short groups starts at group 0 or where a group
    // start enters another TROWS-row block (which includes every group
    // after a long one), so there are at most ext / TROWS + 1 runs, each
    // packed kPackMax groups at a time; and every item owns a group.
    // Workgroups past the items exit after building the table, which costs
    // about a microsecond per CU each.
    constexpr int64_t trows = 16 * NW * (64 / CG);
    const int64_t bound = ext / (trows - 14) + ext / trows + G / kPackMax + 1;
    const int64_t items = std::min<int64_t>(G, bound);
    const int64_t nblocks = 8 * SPS * ((items * nsuper + 7) / 8);
    if (nblocks > INT32_MAX)
        return MXQ_ERR_INVALID_ARG;
    const size_t lds = G > 64 ? (3 * (size_t)G + 2) * sizeof(int) + (size_t)G : 0;
    jagged_strided_kernel<CG, kJaggedStridedTiles, NW>
        <<<dim3((unsigned)nblocks), dim3(64 * NW), lds, st>>>(x, ldx, (int)ext, (int)ncols, offs, G, q,
                                                           ldq, scales, ss_g, ss_col, (int)nsuper);
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
        // its rows, store column-major of that tensor == row-major q
        if (sx_c % 8 != 0 || sq_r % 16 != 0)
            return MXQ_ERR_INVALID_ARG;
        return run_jagged_strided(x, cols, rows, sx_c, offs, num_groups, q, sq_r, scales, ss_g, ss_r, st);
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
        return run_jagged_strided(x, rows, cols, sx_r, offs, num_groups, q, sq_c, scales, ss_g, ss_c, st);
    }
    if (sx_r == 1 && sq_r == 1) {
        // column-major in and out: the rowwise pattern on the transpose
        if (cols > 1 && rows >= 8 && (sx_c % 8 != 0 || sq_c % 16 != 0))
            return MXQ_ERR_INVALID_ARG;
        return run_jagged_contig(x, cols, rows, sx_c, offs, num_groups, q, sq_c, scales, ss_c, ss_g, st);
    }
    return MXQ_ERR_UNSUPPORTED;
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
        (int)tiles_c, scale_mode == MXQ_SCALE_RCEIL, line_aligned(q, sq_k, sq_e));
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
    const bool b1x128 = block_r == 1 && block_c == 128;
    const bool b128x128 = block_r == 128 && block_c == 128;
    const bool b128x1 = block_r == 128 && block_c == 1;
    if (!b1x128 && !b128x128 && !b128x1)
        return MXQ_ERR_UNSUPPORTED;
    if (rows == 0 || cols == 0)
        return MXQ_OK;
    if (!x || !q || !scales)
        return MXQ_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(scales) & 3u) != 0)
        return MXQ_ERR_INVALID_ARG;
    if (rows > INT32_MAX || cols > INT32_MAX)
        return MXQ_ERR_INVALID_ARG;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (b1x128) {
        if (!(sx_c == 1 && sq_c == 1))
            return MXQ_ERR_UNSUPPORTED;
        if (!aligned16(x) || !aligned16(q) || sx_r % 8 != 0 || sq_r % 16 != 0)
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
    // (128, 128) and (128, 1): row-major in, column-major out
    if (!(sx_c == 1 && sq_r == 1))
        return MXQ_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(q) || cols % 8 != 0 || sx_r % 8 != 0 || sq_c % 16 != 0)
        return MXQ_ERR_INVALID_ARG;
    const int64_t tiles_r = rows / 128, tiles_c = (cols + 255) / 256;
    const int64_t nblocks = tiles_r * tiles_c;
    if (nblocks > INT32_MAX)
        return MXQ_ERR_INVALID_ARG;
    const int nt = line_aligned(q, sq_c, 0);
    if (b128x128)
        block_strided_kernel<128, 128, false><<<dim3((unsigned)nblocks), dim3(kBlockThreads), 0, st>>>(
            x, 0, sx_r, (int)rows, (int)cols, q, 0, sq_c, scales, 0, ss_rb, ss_cb, (int)tiles_r,
            (int)tiles_c, 0, nt);
    else
        block_strided_kernel<128, 1, false><<<dim3((unsigned)nblocks), dim3(kBlockThreads), 0, st>>>(
            x, 0, sx_r, (int)rows, (int)cols, q, 0, sq_c, scales, 0, ss_rb, ss_cb, (int)tiles_r,
            (int)tiles_c, 0, nt);
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
}  // namespace

extern "C" mxq_status mxq_debug_cast_e4m3(const float *y, int64_t n, uint8_t *out, void *stream)
{
    if (n < 0)
        return MXQ_ERR_INVALID_ARG;
    if (n == 0)
        return MXQ_OK;
    if (!y || !out)
        return MXQ_ERR_INVALID_ARG;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    debug_cast_kernel<<<dim3((unsigned)blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream)>>>(y, n, out);
    return launch_status();
}
