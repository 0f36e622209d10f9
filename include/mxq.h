/*
 * mxq — dynamic float8 (OCP E4M3FN) quantization of MoE grouped-GEMM operands
 * on AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every entry point takes DEVICE pointers, extents and strides counted
 * in ELEMENTS (int64), and a HIP stream passed as `void*` (NULL = the null
 * stream).  Work is enqueued on that stream and the call returns without
 * synchronising; nothing is read back to the host, in particular not the
 * group offsets.
 *
 * Numerics shared by all entry points (the pages name the formats, the
 * readings below fix the arithmetic):
 *   - input elements are bf16 bit patterns;
 *   - fp32-scale paths store the quantize multiplier
 *       s = RN32(448 / max(amax, RN32(1e-12)))
 *     and write q = E4M3FN(clamp(RN32(x * s), -448, 448)), rounding to nearest
 *     even, -0 kept (a negative value that rounds to zero gives 0x80);
 *   - e8m0 paths ("floor" mode) store code = clamp(floor(log2 amax) - 8,
 *     -127, 127) + 127 (0 for an all-zero block) and write
 *       q = E4M3FN(clamp(x * 2^(127 - code), -448, 448)).
 *   The result is unique: for finite inputs exactly one byte string and one
 *   scale string is correct.  NaN / Inf inputs are outside the contract.
 *
 * Ownership: the caller allocates and owns every buffer; outputs must not
 * alias inputs.  The library allocates nothing, keeps no state, and is
 * reentrant.
 *
 * Errors (returned before any launch unless stated):
 *   MXQ_ERR_INVALID_ARG  a scale_mode that is not an mxq_scale_mode value,
 *                        null pointer with a non-empty extent, negative
 *                        extent, num_groups outside [1, MXQ_MAX_GROUPS],
 *                        extent not divisible by the block, a pointer or a
 *                        non-unit stride that breaks 16-byte alignment, or a
 *                        unit-stride extent of a column-major store that is
 *                        not a multiple of 8.
 *   MXQ_ERR_UNSUPPORTED  a layout combination with no kernel (see each call).
 *   MXQ_ERR_LAUNCH       the launch failed (hipGetLastError after launch).
 *   MXQ_ERR_WORKSPACE    a call that takes scratch memory was given less than
 *                        it needs for these extents (nothing is launched).
 * A zero extent is not an error: the call writes whatever scales the
 * definition still assigns (an empty group's scale) and returns MXQ_OK.
 */
#ifndef MXQ_H
#define MXQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXQ_ABI_VERSION 1
#define MXQ_MAX_GROUPS 4096
/* size of the device array behind mxq_quantize_jagged_colwise_noalloc */
#define MXQ_NOALLOC_SCRATCH_BYTES (4 << 20)

typedef enum mxq_status {
    MXQ_OK = 0,
    MXQ_ERR_INVALID_ARG = 1,
    MXQ_ERR_UNSUPPORTED = 2,
    MXQ_ERR_LAUNCH = 3,
    MXQ_ERR_WORKSPACE = 4
} mxq_status;

/*
 * How an MX block's e8m0 shared exponent se (code se + 127, multiplier
 * 2^-se) is derived from the block's amax.  Both modes are named, not
 * defined, by "[mxfp8 moe training] add CUDA kernel to quantize 3d tensor
 * colwise" (the author's comment); the readings implemented:
 *   FLOOR  se = floor(log2 amax) - 8 (OCP MX v1.0 rule, emax(E4M3) = 8);
 *          magnitudes in (448, 512) * 2^se saturate to 448.
 *   RCEIL  se = the smallest integer with amax <= 448 * 2^se (amax / 448
 *          rounded up to a power of two); nothing saturates.
 * Both clamp se to [-127, 127]; a zero block gets code 0.
 */
typedef enum mxq_scale_mode { MXQ_SCALE_FLOOR = 0, MXQ_SCALE_RCEIL = 1 } mxq_scale_mode;

/* Version of this ABI (MXQ_ABI_VERSION). */
int mxq_abi_version(void);

/* Static, human-readable name of a status code. */
const char *mxq_status_string(int status);

/*
 * Jagged per-group ROWWISE quantization.
 * Source: "[scaled grouped mm] add triton kernels for float8 rowwise
 * quantization with per-group/jagged scales", Summary (first kernel): one
 * scale per row for each token group, output row-major, feeding the left
 * operand of the grad_weight grouped GEMM; Motivation: offsets stay on the
 * device, one launch covers every group.
 *
 * x       (rows, cols) bf16, strides (sx_r, sx_c).  Groups run along dim 1.
 * offs    int32[num_groups] on the device: cumulative group ends; group g is
 *         columns [offs[g-1], offs[g]) with offs[-1] = 0.  Precondition (not
 *         checkable without a sync): non-decreasing, 0 <= offs[g] <= cols.
 *         Columns at or past offs[num_groups-1] belong to no group and their
 *         q bytes are not written.
 * q       (rows, cols) e4m3 bytes, strides (sq_r, sq_c).
 * scales  (rows, num_groups) fp32, strides (ss_r, ss_g); every entry is
 *         written, an empty group gets 448 / RN32(1e-12).
 * Layouts with a kernel: sx_c == 1 && sq_c == 1 (row-major in and out), and
 * sx_r == 1 && sq_c == 1 (a transposed view of a row-major tensor, e.g.
 * grad_out^T, into a row-major q).  For the second, with num_groups <= 256,
 * cols <= 391,680 and distinct scale slots, groups longer than 1536 columns
 * are split into chunks that exchange maxima through the group's scale
 * slots: two kernels run in stream order (one zeroes those slots), and the
 * slots hold intermediate words until the second ends.
 */
mxq_status mxq_quantize_jagged_rowwise(const uint16_t *x, int64_t rows, int64_t cols, int64_t sx_r,
                                       int64_t sx_c, const int32_t *offs, int32_t num_groups,
                                       uint8_t *q, int64_t sq_r, int64_t sq_c, float *scales,
                                       int64_t ss_r, int64_t ss_g, void *stream);

/*
 * Jagged per-group COLWISE quantization.
 * Source: same page, Summary (second kernel): scales computed over the
 * logical columns of each token group, output column-major, feeding the
 * right operand of the grad_weight grouped GEMM.
 *
 * x       (rows, cols) bf16, strides (sx_r, sx_c).  Groups run along dim 0:
 *         group g is rows [offs[g-1], offs[g]); same precondition as above
 *         with `rows` as the extent.
 * q       (rows, cols) e4m3, strides (sq_r, sq_c).
 * scales  (num_groups, cols) fp32, strides (ss_g, ss_c).
 * Layouts with a kernel: sx_c == 1 && sq_r == 1 (row-major in, column-major
 * out), and sx_r == 1 && sq_r == 1 (column-major in and out).
 *
 * Row-major in, with num_groups <= 256 and distinct scale slots: token
 * groups longer than the rows one workgroup holds are cut into chunks that
 * exchange each column's maximum through the group's own scale slots, so
 * every element is read once.  Chunks are 128 rows x 256 columns when
 * rows <= 32,625 and rows <= 128 * num_groups, 256 rows x 256 columns when
 * rows <= 65,265 and rows <= 4096 * num_groups, else 1536 rows x 64 columns
 * when rows <= 391,680.  Two kernels run in stream order: one zeroes those
 * slots, the second quantizes; while it runs the slots hold intermediate
 * words (maxima and counts), and at its end the scales.  Other extents read
 * the rows of groups longer than 3072 rows twice.
 */
mxq_status mxq_quantize_jagged_colwise(const uint16_t *x, int64_t rows, int64_t cols, int64_t sx_r,
                                       int64_t sx_c, const int32_t *offs, int32_t num_groups,
                                       uint8_t *q, int64_t sq_r, int64_t sq_c, float *scales,
                                       int64_t ss_g, int64_t ss_c, void *stream);

/*
 * Jagged COLWISE quantization with a caller's workspace: the same operation,
 * arguments and results as mxq_quantize_jagged_colwise.  Source: as above;
 * the pages' kernels keep a whole token group of a column block in one
 * program, which on a GPU with 256 compute units leaves the longest group's
 * columns on a few of them.
 *
 * For a row-major x and column-major q, token groups longer than the rows one
 * workgroup holds are cut into chunks (as above: 128 or 256 x 256, or
 * 1536 x 64)
 * quantized by separate workgroups, which exchange their column maxima
 * through the workspace, so every element is read from memory once, in one
 * launch, for up to 256 groups (the call without a workspace needs a second,
 * clearing launch for the same).  More groups run the kernel without chunks.
 * The column-major-in layout needs no workspace and runs as
 * mxq_quantize_jagged_colwise.
 *
 * workspace        device memory of at least
 *                  mxq_jagged_colwise_workspace_bytes(rows, cols, num_groups)
 *                  bytes, 4-byte aligned, filled with zeros before its first
 *                  use; every call leaves it filled with zeros again, so it
 *                  can be reused by later calls (and graph replays) without
 *                  clearing.  Owned by the caller.  Two calls that overlap in
 *                  time must not share a workspace.
 * workspace_bytes  its size; too small -> MXQ_ERR_WORKSPACE, before any launch.
 */
mxq_status mxq_quantize_jagged_colwise_ws(const uint16_t *x, int64_t rows, int64_t cols,
                                          int64_t sx_r, int64_t sx_c, const int32_t *offs,
                                          int32_t num_groups, uint8_t *q, int64_t sq_r,
                                          int64_t sq_c, float *scales, int64_t ss_g, int64_t ss_c,
                                          void *workspace, int64_t workspace_bytes, void *stream);

/* Workspace bytes mxq_quantize_jagged_colwise_ws needs for these extents (a
 * bound that holds for any offsets); 0 for more than 256 groups (the call
 * then runs the kernel without chunks, which is as fast there, and needs no
 * workspace: it may be NULL); -1 for invalid arguments. */
int64_t mxq_jagged_colwise_workspace_bytes(int64_t rows, int64_t cols, int32_t num_groups);

/*
 * Jagged COLWISE quantization that allocates nothing, for callers that
 * cannot allocate device memory or call hipMalloc (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * operation, arguments and results of mxq_quantize_jagged_colwise_ws, with
 * the workspace taken from a fixed device array inside the library (one per
 * GPU, MXQ_NOALLOC_SCRATCH_BYTES = 4 MiB, held until the process ends; zero
 * at load, and every call leaves it zero).  Extents whose
 * workspace (mxq_jagged_colwise_workspace_bytes) exceeds it ->
 * MXQ_ERR_WORKSPACE before any launch (e.g. 16384 x 4096 with 8 groups needs
 * 135,168 bytes).  Calls on one GPU share the array: calls that overlap in
 * time on one GPU race and must be serialized (e.g. issued on one stream).
 * The array's device address is looked up on the first call on each device
 * (MXQ_ERR_LAUNCH if that fails).
 */
mxq_status mxq_quantize_jagged_colwise_noalloc(const uint16_t *x, int64_t rows, int64_t cols,
                                               int64_t sx_r, int64_t sx_c, const int32_t *offs,
                                               int32_t num_groups, uint8_t *q, int64_t sq_r,
                                               int64_t sq_c, float *scales, int64_t ss_g,
                                               int64_t ss_c, void *stream);

/*
 * MXFP8 quantization of 3D expert weights along N ("colwise", 32 x 1 blocks).
 * Source: "[mxfp8 moe training] add CUDA kernel to quantize 3d tensor
 * colwise", Summary: weights (E, N, K) scaled along N and written directly in
 * per-expert column-major layout, no separate transpose pass; the author's
 * comment names the floor / rceil scale modes.
 *
 * w       (E, N, K) bf16, strides (sw_e, sw_n, sw_k); N % 32 == 0.
 * q       (E, N, K) e4m3, strides (sq_e, sq_n, sq_k); default per-expert
 *         column-major is (N*K, 1, N).
 * scales  (E, N/32, K) e8m0 bytes, strides (ss_e, ss_nb, ss_k).
 * Layout with a kernel: sw_k == 1 && sq_n == 1 (K % 8 == 0).
 * scale_mode: MXQ_SCALE_FLOOR or MXQ_SCALE_RCEIL.
 */
mxq_status mxq_quantize_mx_3d_colwise(const uint16_t *w, int64_t E, int64_t N, int64_t K,
                                      int64_t sw_e, int64_t sw_n, int64_t sw_k, uint8_t *q,
                                      int64_t sq_e, int64_t sq_n, int64_t sq_k, uint8_t *scales,
                                      int64_t ss_e, int64_t ss_nb, int64_t ss_k,
                                      int32_t scale_mode, void *stream);

/*
 * MXFP8 quantization along the last dim (1 x 32 blocks), the layout `to_mx`
 * produces.  Source: same page, Summary (the `to_mx` route along the
 * contiguous dim).
 *
 * x       (rows, cols) bf16, strides (sx_r, sx_c); cols % 32 == 0.
 * q       (rows, cols) e4m3, strides (sq_r, sq_c).
 * scales  (rows, cols/32) e8m0, strides (ss_r, ss_b).
 * Layout with a kernel: sx_c == 1 && sq_c == 1.
 * scale_mode: MXQ_SCALE_FLOOR or MXQ_SCALE_RCEIL.
 */
mxq_status mxq_quantize_mx_rowwise(const uint16_t *x, int64_t rows, int64_t cols, int64_t sx_r,
                                   int64_t sx_c, uint8_t *q, int64_t sq_r, int64_t sq_c,
                                   uint8_t *scales, int64_t ss_r, int64_t ss_b,
                                   int32_t scale_mode, void *stream);

/*
 * Jagged MXFP8: e8m0 block scales with 32-element blocks inside token
 * groups, for MX grouped GEMMs whose groups run along K.  Source: "[mxfp8
 * moe training] add CUDA kernel for per-group conversion of scale factors to
 * blocked layout", stacked PR list (scales of token groups along K); the
 * blocks and scale rules are those of mxq_quantize_mx_rowwise.  Reading (the
 * pages do not pad groups): blocks restart at every group start, a group of
 * n elements has ceil(n/32) blocks and its last block may be short; block k
 * of group g has scale index B_g + k, B_g = sum over j < g of ceil(n_j/32).
 *
 * Groups as in mxq_quantize_jagged_rowwise (rowwise: along dim 1) and
 * mxq_quantize_jagged_colwise (colwise: along dim 0).  Elements at or past
 * offs[G-1] and scale entries past the last block are not written.
 *
 * rowwise: scales[r*ss_r + b*ss_b], b < ceil(cols/32) + G - 1 (the most any
 *          offsets can need; the caller's buffer must hold that many).
 *          Layouts with a kernel: sx_c == 1 && sq_c == 1 (row-major in and
 *          out; sx_r % 8 == 0, sq_r % 16 == 0), or sx_r == 1 && sq_c == 1
 *          (a transposed view; rows % 8 == 0, sx_c % 8 == 0, sq_r % 16 == 0).
 * colwise: scales[b*ss_b + c*ss_c], b < ceil(rows/32) + G - 1.
 *          Layouts with a kernel: sx_c == 1 && sq_r == 1 (row-major in,
 *          column-major out; cols % 8 == 0, sx_r % 8 == 0, sq_c % 16 == 0),
 *          or sx_r == 1 && sq_r == 1 (column-major in and out).
 * The 16-byte fast paths need group starts on multiples of 8 (rowwise) or
 * 16 (colwise); other offsets take element-wise loads or stores.
 * scale_mode: MXQ_SCALE_FLOOR or MXQ_SCALE_RCEIL.
 */
mxq_status mxq_quantize_jagged_mx_rowwise(const uint16_t *x, int64_t rows, int64_t cols,
                                          int64_t sx_r, int64_t sx_c, const int32_t *offs,
                                          int32_t num_groups, uint8_t *q, int64_t sq_r,
                                          int64_t sq_c, uint8_t *scales, int64_t ss_r,
                                          int64_t ss_b, int32_t scale_mode, void *stream);
mxq_status mxq_quantize_jagged_mx_colwise(const uint16_t *x, int64_t rows, int64_t cols,
                                          int64_t sx_r, int64_t sx_c, const int32_t *offs,
                                          int32_t num_groups, uint8_t *q, int64_t sq_r,
                                          int64_t sq_c, uint8_t *scales, int64_t ss_b,
                                          int64_t ss_c, int32_t scale_mode, void *stream);

/*
 * Per-group re-layout of jagged MX e8m0 scales into the scale-operand tiles
 * of a gfx950 scaled-MFMA grouped GEMM.  Source: "[mxfp8 moe training] add
 * CUDA kernel for per-group conversion of scale factors to blocked layout",
 * title, benchmarks and stacked PR list: after jagged MX quantization with
 * token groups along K, each group's scales are converted, on the device, to
 * the layout the grouped GEMM reads.  The page's target is another vendor's
 * MMA layout and is not printed; the layout here (reading) is the scale
 * operand order of the gfx950 scaled MFMA with 16 rows x 128 K values of
 * e4m3 (CDNA4 ISA, V_MFMA_SCALE_F32_16X16X128_F8F6F4): lane 16j + i of a
 * wave supplies the scale of row i and 32-value K block j in one 32-bit
 * register whose byte op_sel selects, so one register serves four 128-value
 * K steps.
 *
 * scales  e8m0 bytes of `rows` rows, block b of row r at
 *         scales[r*ss_r + b*ss_b], blocks numbered as the jagged MX calls
 *         number them (group g's nb_g = ceil(n_g/32) blocks from B_g).  For
 *         the rowwise operand pass its (rows, blocks) scales; for the
 *         colwise operand pass its scales with the columns as rows
 *         (ss_r = ss_c, ss_b = ss_b of mxq_quantize_jagged_mx_colwise).
 * offs, num_groups, extent
 *         the token groups and the token extent given to the jagged MX
 *         call (offsets are clamped to [0, extent] the same way).
 * tiles   output, 16-byte aligned, capacity 256 * ceil(rows/16) *
 *         (ceil(extent/512) + G - 1) bytes.  A tile is 16 rows x 16 blocks
 *         stored as 64 lane words of 4 bytes:
 *           byte 4*lane + u = scale of row lane % 16, block 4u + lane / 16
 *         (tile-local row and block).  Group g owns ceil(rows/16) x
 *         KT_g = ceil(n_g/512) tiles, tile (rb, kt) at index
 *         T_g + rb*KT_g + kt, T_g = ceil(rows/16) * sum of KT_h over h < g.
 *         Entries past the last row or past the group's last block are 0;
 *         bytes past the last tile are not written.
 * tile_starts
 *         output, G + 1 int32 (T_g, and the total at index G), or NULL.
 * Layouts with a kernel: any strides; ss_b == 1 and ss_r == 1 read whole
 * 256-byte pieces, others read bytes.
 * Errors: MXQ_ERR_INVALID_ARG also for negative strides and for a tile
 * count past INT32_MAX.
 */
mxq_status mxq_relayout_mx_scales_grouped(const uint8_t *scales, int64_t rows, int64_t ss_r,
                                          int64_t ss_b, const int32_t *offs, int32_t num_groups,
                                          int64_t extent, uint8_t *tiles, int32_t *tile_starts,
                                          void *stream);

/*
 * Blockwise ("groupwise") fp8 quantization with one fp32 multiplier per
 * block_r x block_c block.  Source: "[fp8 blockwise] load 2d chunks for
 * groupwise quant to enable coalesced gmem accesses", body: 1 x blocksize
 * blocks for activations, blocksize x blocksize for weights, loaded as 2D
 * chunks so both directions coalesce.
 *
 * x       (rows, cols) bf16, strides (sx_r, sx_c); rows % block_r == 0 and
 *         cols % block_c == 0.
 * q       (rows, cols) e4m3, strides (sq_r, sq_c).
 * scales  (rows/block_r, cols/block_c) fp32, strides (ss_rb, ss_cb).
 * Blocks: (1, 128), (128, 128) or (128, 1); others -> MXQ_ERR_UNSUPPORTED.
 * Layouts with a kernel, for every block shape:
 *   x   row-major (sx_c == 1) or a transposed view of a row-major tensor
 *       (sx_r == 1), read in place: the view is quantized as the underlying
 *       tensor with the block shape, q strides and scale strides transposed;
 *   q   row-major (sq_c == 1) or column-major (sq_r == 1).
 * x and q 16-byte aligned, x's leading stride a multiple of 8 elements,
 * scales 4-byte aligned.  In the terms of the underlying row-major tensor
 * (R, C): 1 x 128 blocks into row-major q need q's row stride % 16 == 0;
 * every other combination runs on 128 x 256 tiles and needs C % 8 == 0,
 * R % 16 == 0 and q's leading stride % 8 == 0 (row-major) or % 16 == 0
 * (column-major).  Other layouts -> MXQ_ERR_UNSUPPORTED, unmet alignments ->
 * MXQ_ERR_INVALID_ARG.
 */
mxq_status mxq_quantize_blockwise(const uint16_t *x, int64_t rows, int64_t cols, int64_t sx_r,
                                  int64_t sx_c, int32_t block_r, int32_t block_c, uint8_t *q,
                                  int64_t sq_r, int64_t sq_c, float *scales, int64_t ss_rb,
                                  int64_t ss_cb, void *stream);

/*
 * TEST-ONLY diagnostics, not part of the quantization API: the library's own
 * device conversions applied to n fp32 values, so that tests can check them
 * against the CPU definition over whole fp32 ranges.  y: n floats, out: n
 * bytes, both device pointers; errors as above.
 *
 * mxq_debug_cast_e4m3: one value at a time, clamped to +-448, then the
 * hardware round-to-nearest-even E4M3FN conversion.
 * mxq_debug_cast4_e4m3: four consecutive values at a time through the packed
 * conversion the quantization kernels use (out 4-byte aligned):
 *   unclamped == 0  the clamped form of the e8m0 (MX) paths, any finite y;
 *   unclamped == 1  the form of the fp32-multiplier paths, which omits the
 *                   clamp: defined only for |y| < 464, the range those paths
 *                   can produce (|RN32(x * 448 / max(amax, eps))| <= 448 +
 *                   2^-15 whenever |x| <= amax).
 */
/*
 * TEST-ONLY: mxq_quantize_jagged_colwise_ws for a row-major x and a
 * column-major q with the bound on how long a chunk waits for the other
 * chunks of its token group set by the caller (in polls); 0 looks once, a
 * negative value never waits, so the chunks reduce their groups' rows
 * themselves (the path taken when the others do not arrive in time).  A
 * NULL workspace selects the exchange through the scale slots of
 * mxq_quantize_jagged_colwise (extents it does not cover ->
 * MXQ_ERR_INVALID_ARG).  Other layouts -> MXQ_ERR_INVALID_ARG.
 */
mxq_status mxq_debug_jagged_colwise_ws_spin(const uint16_t *x, int64_t rows, int64_t cols,
                                            int64_t sx_r, int64_t sx_c, const int32_t *offs,
                                            int32_t num_groups, uint8_t *q, int64_t sq_r,
                                            int64_t sq_c, float *scales, int64_t ss_g,
                                            int64_t ss_c, void *workspace,
                                            int64_t workspace_bytes, int32_t spin_limit,
                                            void *stream);
mxq_status mxq_debug_cast_e4m3(const float *y, int64_t n, uint8_t *out, void *stream);
mxq_status mxq_debug_cast4_e4m3(const float *y, int64_t n, uint8_t *out, int32_t unclamped,
                                void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_H */
