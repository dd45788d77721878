/*
 * mxcast.h -- C ABI of libmxcast: bf16 -> MXFP8 casts and the 128x4 blocked
 * e8m0 scale layout on AMD Instinct MI355X (gfx950).
 *
 * The method (pytorch/ao pull-request pages):
 *  - "triton kernel to cast to mx across dim0 and dim1", Summary: cast a bf16
 *    matrix to MX along dim0 and dim1 in 32-element blocks, writing the
 *    row-major and the col-major results and both scale sets from a single
 *    read of the input.
 *  - "[mxfp8 moe training] add compile support": e8m0 scales rearranged into
 *    the blocked layout per group along M (error trace: (16640, 160) scales,
 *    int32 [G] and int64 [G+1] offsets), per group along K and per expert of
 *    3D weights (Perf analysis, item 2); output rows bounded by rows +
 *    num_groups * 128 so that no offset is read on the host (change list);
 *    3D expert weights cast along dim1 through a 2D reshape (item 4).
 *  - "[mxfp8 moe training] parallelize along col blocks in scale blocked
 *    format kernel for groups along K", Changes: the blocked layout is built
 *    at a granularity of 128x4 scales.
 *  - "FP8 linear triton with row-wise scaling", quantize_fp8_rowwise: the
 *    row-wise fp8 cast (mx_quantize_fp8_rowwise, whose rule is stated there).
 *  - "[float8nocompile]: Triton kernels for conversion to float8 dtypes for
 *    forward pass of Float8LinearNoCompile": the tensor-wise fp8 cast with a
 *    two-stage global amax (mx_quantize_fp8_tensorwise).
 *  - "[mxfp8 moe training] add compile support", Perf analysis item 1: the
 *    MXFP8 (grouped) GEMM that consumes the casts (mx_gemm_mxfp8,
 *    mx_grouped_gemm_mxfp8).
 *
 * MX rule (the pages do not spell it out; this is the reading implemented):
 *   amax  = max |x| over a block of 32 (NaN > +Inf > finite);
 *   e     = floor(log2(amax)) - 8, clamped to [-127, 127]; amax = 0 gives
 *           e = -127; the scale byte is e + 127 (e8m0); a block holding a
 *           NaN gets the e8m0 NaN byte 0xFF;
 *   q     = x / 2^e rounded to nearest-even to e4m3fn, saturated to +-448
 *           (so +-Inf -> +-448); in a NaN block every element is e4m3 NaN
 *           with its own sign (0x7F / 0xFF).
 *
 * Blocked layout of a (rows, cols) scale matrix: rows padded to a multiple
 * of 128, cols to a multiple of 4, padding bytes 0.  512-byte tiles of
 * 128 rows x 4 cols, ordered by row block, then column block; inside a tile,
 * scale (r, c) sits at byte (r % 32) * 16 + (r % 128 / 32) * 4 + c % 4.
 *
 * Conventions for every call below:
 *  - All array arguments are DEVICE pointers, contiguous, row-major.
 *  - The caller owns every buffer (scratch included) and the stream.  The
 *    library allocates nothing, never synchronises and never reads device
 *    memory from the host; all work is enqueued on `stream` (0 = the null
 *    stream) and runs asynchronously.  It keeps no state, except the
 *    per-GPU scratch array of mx_quantize_fp8_tensorwise_noalloc.
 *  - Arguments are validated on the host before any HIP call; a rejected
 *    call enqueues nothing.  A launch failure reported by the HIP runtime
 *    returns MX_ERR_HIP.
 *  - Empty inputs (a zero extent) are valid and enqueue nothing; shapes are
 *    checked first, so pointers may then be NULL.
 */
#ifndef MXCAST_H
#define MXCAST_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#if defined(__GNUC__)
#define MX_API __attribute__((visibility("default")))
#else
#define MX_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MX_OK = 0,
    MX_ERR_NULL = 1,    /* a required pointer is NULL                          */
    MX_ERR_SHAPE = 2,   /* a size is negative, not a multiple of 32 where one  */
                        /* is required, or beyond the supported maximum        */
    MX_ERR_GROUPS = 3,  /* num_groups outside [1, MX_MAX_GROUPS] or bad axis   */
    MX_ERR_HIP = 4,     /* the HIP runtime rejected a launch                   */
    MX_ERR_ALIGN = 5,   /* a pointer lacks the alignment stated for it         */
    MX_ERR_WORKSPACE = 6 /* a caller-provided workspace is too small           */
} mx_status;

#define MX_BLOCK 32          /* elements per scale block                  */
#define MX_MAX_GROUPS 1024   /* groups accepted by the grouped layout     */

/* Static text for a status code (any int: values that are not an mx_status
 * give "unknown status"). */
MX_API const char* mx_status_string(int status);

/*
 * bf16 -> MXFP8 along dim0 and dim1 from one read of the input.
 *   x      bf16 (rows, cols) row-major; 16-byte aligned.
 *   q_row  e4m3 (rows, cols): blocks of 32 along each row; 8-byte aligned.
 *   s_row  e8m0 (rows, cols / 32).
 *   q_col  e4m3 of the col-major cast: the (rows, cols) result in column-
 *          major order, i.e. a row-major (cols, rows) array whose row c holds
 *          column c of x cast in blocks of 32 consecutive rows; 16-byte
 *          aligned.
 *   s_col  e8m0 (cols, rows / 32).
 * Either output pair may be NULL to skip that direction (both members of a
 * pair NULL); both pairs NULL, a half-NULL pair or x NULL -> MX_ERR_NULL.
 * rows and cols must be >= 0 and multiples of 32, cols <= 2^25, else
 * MX_ERR_SHAPE.  Outputs must not overlap the input or each other.
 * Where rows are a multiple of 16384 and cols of 8192 (or the shape is
 * 16384 x 4096), each present scale matrix has at most 1024 columns and is
 * 16-byte aligned, the call enqueues two kernels: the cast writing the
 * scales in the 128x4 blocked layout, then their conversion to the layout
 * above in place.  Until the second has run, the scale buffers hold the
 * blocked bytes; both are on `stream`, so stream order hides this.
 */
MX_API mx_status mx_cast_dim0_dim1(const void* x, int64_t rows, int64_t cols,
                            uint8_t* q_row, uint8_t* s_row,
                            uint8_t* q_col, uint8_t* s_col,
                            hipStream_t stream);

/*
 * The same cast with both scale sets written directly in the 128x4 blocked
 * layout ("triton kernel to cast to mx across dim0 and dim1", future
 * improvement 2: write out swizzled scales), saving the separate layout
 * pass and its traffic.
 *   s_row_blocked  mx_blocked_bytes(1, rows, cols / 32) bytes: the blocked
 *                  form of the (rows, cols / 32) row scales; 16-byte aligned.
 *   s_col_blocked  mx_blocked_bytes(1, cols, rows / 32) bytes: the blocked
 *                  form of the (cols, rows / 32) column scales; 16-byte
 *                  aligned.
 * Every byte of both buffers is written (padding 0).  Codes, arguments and
 * errors as for mx_cast_dim0_dim1.
 */
MX_API mx_status mx_cast_dim0_dim1_blocked(const void* x, int64_t rows, int64_t cols,
                                           uint8_t* q_row, uint8_t* s_row_blocked,
                                           uint8_t* q_col, uint8_t* s_col_blocked,
                                           hipStream_t stream);

/*
 * The same cast for MoE activations grouped along M, with the row scales
 * written directly in the M-grouped blocked layout -- what
 * mx_scales_to_blocked_grouped(s_row, ..., group_axis 0) makes of the plain
 * row scales -- so that the grouped layout needs no pass of its own ("[mxfp8
 * moe training] add compile support": M-group layout of the (16640, 160)
 * scales with device-side offsets; "triton kernel to cast to mx across dim0
 * and dim1", future improvement 2: swizzled scales from the cast).
 *   group_end_offsets  DEVICE int32 [num_groups], cumulative END rows of the
 *                      groups (read and clamped on the device exactly as by
 *                      mx_scales_to_blocked_grouped: undefined result for
 *                      malformed offsets, but memory-safe).
 *   s_row_grouped      mx_blocked_grouped_bytes(rows, cols / 32, num_groups,
 *                      0) bytes, 16-byte aligned; every byte is written.
 *   out_group_starts   DEVICE int64 [num_groups + 1] or NULL: padded start
 *                      row of each group, then the padded total.
 *   q_row              as for mx_cast_dim0_dim1 (required).
 *   q_col, s_col       plain col-major codes and (cols, rows / 32) scales,
 *                      as for mx_cast_dim0_dim1, or both NULL (dim0 only).
 * Shapes as for mx_cast_dim0_dim1; 1 <= num_groups <= MX_MAX_GROUPS (else
 * MX_ERR_GROUPS) and rows + 128 * num_groups < 2^31.  With rows or cols 0
 * only the (all-zero) grouped buffer and the starts are written.
 */
MX_API mx_status mx_cast_dim0_dim1_mgrouped(const void* x, int64_t rows, int64_t cols,
                                            const int32_t* group_end_offsets, int32_t num_groups,
                                            uint8_t* q_row, uint8_t* s_row_grouped,
                                            int64_t* out_group_starts,
                                            uint8_t* q_col, uint8_t* s_col, hipStream_t stream);

/*
 * The MoE activation cast with BOTH scale sets written in their grouped
 * blocked layouts, for the two grouped GEMMs of MoE training: the row scales
 * M-grouped as by mx_cast_dim0_dim1_mgrouped (the forward GEMM, grouped
 * along its M), and the column scales K-grouped -- the groups of rows are
 * the groups along the K dimension of the weight-gradient GEMM, which
 * contracts over the tokens ("[mxfp8 moe training] parallelize along col
 * blocks in scale blocked format kernel for groups along K"; "triton kernel
 * to cast to mx across dim0 and dim1", future improvement 2: swizzled scales
 * from the cast).  One read of x, no layout pass of its own.
 *   group_end_offsets  DEVICE int32 [num_groups], cumulative END rows,
 *                      clamped on the device as by
 *                      mx_scales_to_blocked_grouped.
 *   q_row, s_row_grouped, row_group_starts   as for
 *                      mx_cast_dim0_dim1_mgrouped (q_row required).
 *   q_col              col-major codes (cols, rows), 16-byte aligned
 *                      (required).
 *   s_col_grouped      mx_blocked_grouped_bytes(cols, rows / 32, num_groups,
 *                      1) bytes, 16-byte aligned, every byte written: what
 *                      mx_scales_to_blocked_grouped(s_col, ends_k, group_axis
 *                      1) makes of the plain (cols, rows / 32) column scales
 *                      with ends_k[g] = end_g / 32 rounded down (a 32-row
 *                      block belongs to the group it falls in whole; group
 *                      ends at multiples of 32 keep every block whole).
 *   col_group_starts   DEVICE int64 [num_groups + 1] or NULL: padded start
 *                      column of each group, then the padded total.
 * Shapes as for mx_cast_dim0_dim1, plus cols > 0 when rows > 0 (else
 * MX_ERR_SHAPE); 1 <= num_groups <= MX_MAX_GROUPS (else MX_ERR_GROUPS), rows
 * + 128 * num_groups < 2^31.  With rows 0 only the (all-zero) grouped
 * buffers and the starts are written.
 */
MX_API mx_status mx_cast_dim0_dim1_grouped_blocked(const void* x, int64_t rows, int64_t cols,
                                                   const int32_t* group_end_offsets, int32_t num_groups,
                                                   uint8_t* q_row, uint8_t* s_row_grouped,
                                                   int64_t* row_group_starts, uint8_t* q_col,
                                                   uint8_t* s_col_grouped, int64_t* col_group_starts,
                                                   hipStream_t stream);

/*
 * dim1 cast of 3D expert weights, expert by expert.
 *   w  bf16 (experts, n, k) contiguous; 16-byte aligned.
 *   q  e4m3 (experts, k, n): expert e's (n, k) matrix cast in blocks of 32
 *      along n and stored col-major (row-major (k, n)); 16-byte aligned.
 *   s  e8m0 (experts, k, n / 32).
 * Because n is a multiple of 32, blocks never straddle experts and the
 * values equal the 2D dim1 cast of the (experts * n, k) reshape.
 * n or k not a multiple of 32, k > 2^25, or a negative size -> MX_ERR_SHAPE.
 */
MX_API mx_status mx_cast_dim1_3d(const void* w, int64_t experts, int64_t n, int64_t k,
                          uint8_t* q, uint8_t* s, hipStream_t stream);

/*
 * The 3D dim1 cast with each expert's (k, n / 32) scales written directly in
 * the 128x4 blocked layout: s_blocked holds mx_blocked_bytes(experts, k,
 * n / 32) bytes, expert e's blocked matrix at e * ceil128(k) * ceil4(n / 32);
 * every byte written (padding 0); 16-byte aligned.  n must be a multiple of
 * 128 (so that no 128-row tile of the reshape spans two experts), else
 * MX_ERR_SHAPE: use mx_cast_dim1_3d then mx_scales_to_blocked.
 */
MX_API mx_status mx_cast_dim1_3d_blocked(const void* w, int64_t experts, int64_t n, int64_t k,
                                         uint8_t* q, uint8_t* s_blocked, hipStream_t stream);

/* Bytes of the blocked form of `batch` (rows, cols) matrices:
 * batch * ceil128(rows) * ceil4(cols); -1 on a negative argument. */
MX_API int64_t mx_blocked_bytes(int64_t batch, int64_t rows, int64_t cols);

/*
 * Blocked layout of `batch` independent e8m0 (rows, cols) matrices.
 *   s    u8 (batch, rows, cols).
 *   out  mx_blocked_bytes(batch, rows, cols) bytes: matrix b's blocked form
 *        at byte b * ceil128(rows) * ceil4(cols); every byte is written
 *        (padding 0).
 * batch = 1 is the plain 2D conversion; batch = experts converts the
 * (experts, k, n / 32) scales of mx_cast_dim1_3d per expert.
 */
MX_API mx_status mx_scales_to_blocked(const uint8_t* s, int64_t batch, int64_t rows, int64_t cols,
                               uint8_t* out, hipStream_t stream);

/* Size in bytes of the grouped blocked output (host arithmetic only):
 *   axis 0: (rows + 128 * num_groups) * ceil4(cols)
 *   axis 1: ceil128(rows) * (ceil4(cols) + 4 * num_groups)
 * -1 on a negative size, num_groups outside [1, MX_MAX_GROUPS] or a bad axis. */
MX_API int64_t mx_blocked_grouped_bytes(int64_t rows, int64_t cols, int32_t num_groups,
                                 int32_t group_axis);

/*
 * Grouped blocked layout with the group offsets kept on the device.
 *   s                  u8 (rows, cols) scales.
 *   group_end_offsets  DEVICE int32 [num_groups]: cumulative END offset of
 *                      each group along the grouped axis, in rows of s
 *                      (group_axis 0, "M groups") or in scale columns of s
 *                      (group_axis 1, "K groups"); the last should equal the
 *                      extent.  Empty groups are allowed.  The offsets are
 *                      never read on the host; the kernel clamps each end to
 *                      [previous end, extent] and ignores anything past the
 *                      last end, so malformed offsets stay memory-safe.
 *   out                mx_blocked_grouped_bytes(...) bytes, every byte
 *                      written.  axis 0: group g padded to a multiple of 128
 *                      rows, starting at output row start[g] (byte
 *                      start[g] * ceil4(cols)); the whole buffer reads as one
 *                      blocked matrix of rows + 128 * G rows.  axis 1: group
 *                      g padded to a multiple of 4 columns and laid out as
 *                      its own blocked matrix of ceil128(rows) rows at byte
 *                      ceil128(rows) * start[g].  Bytes past the last group
 *                      are 0.
 *   out_group_starts   DEVICE int64 [num_groups + 1] or NULL: start[g] in
 *                      output rows (axis 0) or output columns (axis 1);
 *                      start[num_groups] is the padded total.
 * rows, cols >= 0 (rows + 128 * G and cols + 4 * G below 2^31), group_axis
 * 0 or 1, 1 <= num_groups <= MX_MAX_GROUPS; s, out and group_end_offsets
 * non-NULL (s may be NULL only when rows * cols == 0).
 */
MX_API mx_status mx_scales_to_blocked_grouped(const uint8_t* s, int64_t rows, int64_t cols,
                                       const int32_t* group_end_offsets, int32_t num_groups,
                                       int32_t group_axis, uint8_t* out,
                                       int64_t* out_group_starts, hipStream_t stream);

/*
 * Row-wise fp8 cast with one bf16 scale per row (the gist "FP8 linear triton
 * with row-wise scaling", quantize_fp8_rowwise).  For each row r of x:
 *   scale[r] = amax_r / 448, the quotient of the row's bf16 amax |x| and the
 *              largest e4m3fn value formed in binary32 and rounded to bf16
 *              (nearest-even); a row holding a NaN has scale 0x7FC0;
 *   q[r, c]  = binary32(x[r, c]) / scale[r] (correctly rounded) converted to
 *              e4m3fn, nearest-even and NOT saturated: a magnitude above 464
 *              (which would round to 480, past the largest code) and +-Inf
 *              give NaN; the sign bit of every code is the sign bit of x.
 * As in the page's code there is no guard: an all-zero row has scale 0 and
 * NaN codes, and a row whose amax / 448 underflows bf16 gets a zero or
 * subnormal scale under which its larger elements overflow to NaN.
 *   x      bf16 (rows, cols) row-major contiguous; 2-byte aligned.
 *   q      e4m3fn (rows, cols) row-major, rows * cols bytes.
 *   scale  bf16 bit patterns, rows values; 2-byte aligned.
 * rows, cols >= 0 and cols <= 2^30, else MX_ERR_SHAPE; rows or cols 0 writes
 * nothing.  Any cols is accepted; the input is read once when cols % 8 == 0,
 * cols <= 32768, x is 16-byte and q 8-byte aligned, and twice otherwise.
 */
MX_API mx_status mx_quantize_fp8_rowwise(const void* x, int64_t rows, int64_t cols, uint8_t* q,
                                         uint16_t* scale, hipStream_t stream);

/*
 * Tensor-wise fp8 cast: one bf16 scale for the whole tensor, from a global
 * amax found in two stages ("[float8nocompile]: Triton kernels for
 * conversion to float8 dtypes for forward pass of Float8LinearNoCompile",
 * review thread: block amaxes computed in parallel into a buffer, a global
 * amax from them, then the conversion).  With amax = max |x| over all n
 * elements, scale and codes follow mx_quantize_fp8_rowwise's rule:
 *   *scale = amax / 448 through binary32 to bf16 (0x7FC0 if any x is NaN);
 *   q[i]   = e4m3fn(binary32(x[i]) / *scale), not saturated, sign of x.
 *   x          bf16, n elements of any shape, contiguous; 2-byte aligned.
 *   q          n bytes.
 *   scale      one bf16 (2 bytes, 2-byte aligned), written by the call.
 *   workspace  device scratch of at least mx_tensorwise_workspace_bytes(n)
 *              bytes, 4-byte aligned, owned by the caller; it holds the
 *              block amaxes between the two launches, needs no clearing and
 *              must not be used by another call until this one has run.
 * n < 0 or n > 2^40 -> MX_ERR_SHAPE; n == 0 writes nothing; a workspace
 * smaller than required -> MX_ERR_WORKSPACE.  Three kernels are enqueued; the
 * input is read twice (the second time partly from the memory-side cache).
 * Fastest with x 16-byte and q 8-byte aligned.
 */
MX_API int64_t mx_tensorwise_workspace_bytes(int64_t n);
MX_API mx_status mx_quantize_fp8_tensorwise(const void* x, int64_t n, uint8_t* q, uint16_t* scale,
                                            void* workspace, int64_t workspace_bytes,
                                            hipStream_t stream);

/*
 * mx_quantize_fp8_tensorwise without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, rule, kernels and
 * results; the block amaxes live in a static device array of the library
 * (8 KiB, 2048 words: enough for every n <= 2^40), one per GPU, held until
 * the process ends.  The call allocates nothing; its first call on a device
 * looks the array's address up (hipGetSymbolAddress) with that device
 * current, so `stream` must belong to the current device.  Every call on a
 * GPU shares that GPU's array: calls that overlap on one GPU (two streams,
 * or two host threads) race and may return a wrong scale; serialise them.
 * The array needs no clearing (each call writes every word it reads).
 * Errors as mx_quantize_fp8_tensorwise; MX_ERR_WORKSPACE if n needed more
 * than the array holds (unreachable for n <= 2^40); MX_ERR_HIP if the
 * address lookup fails.
 */
MX_API mx_status mx_quantize_fp8_tensorwise_noalloc(const void* x, int64_t n, uint8_t* q, uint16_t* scale,
                                                    hipStream_t stream);

/*
 * MX-scaled GEMM, the consumer of the dim0 casts ("[mxfp8 moe training] add
 * compile support", Perf analysis item 1: MXFP8 grouped GEMMs of the MoE
 * activations against per-group weights), on gfx950's block-scaled MFMA:
 *   C[m][n] = sum over k of A(m, k) * B(n, k), with
 *   A(m, k) = e4m3(qa[m][k]) * 2^(S_A(m, k / 32) - 127) and B likewise.
 *   qa, sa   A codes (m, k) as mx_cast_dim0_dim1 writes q_row, and A's
 *            (m, k / 32) scales S_A in the 128 x 4 blocked layout
 *            (mx_blocked_bytes(1, m, k / 32) bytes, as
 *            mx_cast_dim0_dim1_blocked writes s_row_blocked or
 *            mx_scales_to_blocked makes); both 16-byte aligned.
 *   qb, sb   B codes (n, k), K-major the same way (the dim0 cast of a
 *            (n, k) weight), and B's (n, k / 32) scales blocked likewise;
 *            both 16-byte aligned.
 *   c        (m, n) row-major: binary32 (c_bf16 = 0, 4-byte aligned) or bf16
 *            rounded to nearest-even (c_bf16 = 1, 2-byte aligned).
 * The scale layout is the one the scaled-GEMM consumer on the MXFP8 pages
 * reads: a 32-row slab's scales for four consecutive blocks of K sit in one
 * 16-byte run.  Padding of the layout (rows past m or n, blocks past
 * k / 32) is never used for a written result.
 * The products of each 64-deep K step are summed by the MFMA with less than
 * binary32 precision (measured on MI355X: within 3.4e-4 of the step's
 * largest product); the steps accumulate in binary32.  A NaN code or scale
 * (0xFF) gives NaN where it enters.
 * m, n, k >= 0, k % 32 == 0, k <= 2^23, m, n < 2^31, else MX_ERR_SHAPE; m or
 * n 0 writes nothing; k 0 writes zeros.  Misaligned pointers give
 * MX_ERR_ALIGN.
 */
MX_API mx_status mx_gemm_mxfp8(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb,
                               int64_t m, int64_t n, int64_t k, void* c, int32_t c_bf16, hipStream_t stream);

/*
 * The same GEMM grouped along M: rows [end_{g-1}, end_g) of A (cumulative
 * END offsets on the device, clamped as by mx_scales_to_blocked_grouped)
 * are multiplied by group g's weights.  sa holds A's scales in the
 * M-grouped blocked layout (mx_blocked_grouped_bytes(m, k / 32,
 * num_groups, 0) bytes, as mx_cast_dim0_dim1_mgrouped writes
 * s_row_grouped or mx_scales_to_blocked_grouped makes with group_axis 0);
 * qb holds num_groups consecutive (n, k) code matrices and sb their
 * num_groups blocked (n, k / 32) scale layouts one after another
 * (mx_blocked_bytes(num_groups, n, k / 32) bytes).  Rows past the last end
 * are not written.  1 <= num_groups <= MX_MAX_GROUPS (else MX_ERR_GROUPS),
 * m + 256 * num_groups < 2^31; other arguments as for mx_gemm_mxfp8.
 */
MX_API mx_status mx_grouped_gemm_mxfp8(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb,
                                       const uint8_t* sb, const int32_t* group_end_offsets,
                                       int32_t num_groups, int64_t m, int64_t n, int64_t k, void* c,
                                       int32_t c_bf16, hipStream_t stream);

/*
 * The same GEMM grouped along K, the weight-gradient GEMM of MoE training:
 * for each group g, over its range of K (the tokens of expert g),
 *   C_g[m][n] = sum over k in group g of A(m, k) * B(n, k),
 * with C_g the g-th of num_groups consecutive (m, n) outputs.  The operands
 * are the col-major casts of the token-major activations and gradients --
 * qa (m, k) and qb (n, k) row-major codes as mx_cast_dim0_dim1 writes q_col --
 * and their scales in the K-grouped blocked layout of the same groups, as
 * mx_cast_dim0_dim1_grouped_blocked writes s_col_grouped
 * (mx_blocked_grouped_bytes(m, k / 32, num_groups, 1) bytes for A, likewise
 * with n for B).
 *   group_end_offsets  DEVICE int32 [num_groups], cumulative END positions
 *                      along K (tokens), clamped on the device as by
 *                      mx_scales_to_blocked_grouped; group g's K range is
 *                      its 32-blocks [lo_g / 32, hi_g / 32) (the reading of
 *                      the K-grouped scales); an empty group's C_g is zero.
 * 1 <= num_groups <= MX_MAX_GROUPS (else MX_ERR_GROUPS), k + 128 *
 * num_groups < 2^31; other arguments as for mx_gemm_mxfp8.
 */
MX_API mx_status mx_kgrouped_gemm_mxfp8(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb,
                                        const uint8_t* sb, const int32_t* group_end_offsets,
                                        int32_t num_groups, int64_t m, int64_t n, int64_t k, void* c,
                                        int32_t c_bf16, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MXCAST_H */
