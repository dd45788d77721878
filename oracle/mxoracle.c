/*
 * mxoracle.c -- CPU oracle for the bf16 -> MXFP8 cast and the 128x4 blocked
 * scale layout.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * loads this file.  Only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or helper with the
 * HIP library: it is a second, independent statement of the same method,
 * written to be read against the pages by eye, not to be fast.
 *
 * Plain C99, fp64 arithmetic, one 32-element block at a time:
 *   - the block amax is a plain fabs/max loop with an explicit NaN test;
 *   - the scale exponent is floor(log2(amax)) - 8, taken from frexp();
 *   - each element is |x| * 2^-e (exact in double), saturated at 448, and
 *     rounded to the nearest e4m3 code by a linear search of the code book,
 *     ties going to the even code.
 * An OpenMP "parallel for" over independent rows/columns is the only
 * concession to speed; it does not change any result.
 *
 * Sources (pytorch/ao pull-request pages):
 *  - "triton kernel to cast to mx across dim0 and dim1", Summary: 32-element
 *    blocks cast along dim0 and dim1 from one read, row-major and col-major
 *    outputs plus scales.
 *  - "[mxfp8 moe training] parallelize along col blocks in scale blocked format
 *    kernel for groups along K", Changes: e8m0 scales converted to the blocked
 *    layout for grouped GEMMs at a 128x4 granularity, groups along K.
 *  - "[mxfp8 moe training] add compile support", change list (padded rows
 *    bounded by rows + num_groups * 128, no host read of the offsets) and the
 *    error trace (M-group op on (16640, 160) e8m0 scales with int32 [G] and
 *    int64 [G+1] offsets); Perf analysis item 4 (3D weights cast with the 2D
 *    dim1 kernel via a reshape).
 *  - "FP8 linear triton with row-wise scaling", quantize_fp8_rowwise: the e4m3
 *    maximum is finfo(float8_e4m3fn).max = 448; and the row-wise fp8 cast
 *    itself (one bf16 scale per row), whose own readings are stated at
 *    mxo_quantize_fp8_rowwise below.
 *  - "[float8nocompile]: Triton kernels for conversion to float8 dtypes for
 *    forward pass of Float8LinearNoCompile": the tensor-wise fp8 cast (one
 *    global amax), read at mxo_quantize_fp8_tensorwise below.
 *  - "[mxfp8 moe training] add compile support", Perf analysis item 1: the
 *    MXFP8 (grouped) GEMM that consumes the casts, at mxo_mx_gemm below.
 * The pages do not write out the MX scale rule, the rounding mode, the
 * treatment of Inf/NaN or the byte order inside a 128x4 tile.  The readings
 * taken here (each stated at the function that uses it) are:
 *  - scale exponent e = floor(log2(amax)) - 8, 8 being the exponent of the
 *    largest e4m3 value (448 = 1.75 * 2^8); e clamped to the e8m0 range
 *    [-127, 127]; an all-zero block gets e = -127 (byte 0);
 *  - elements x / 2^e rounded to nearest, ties to even, saturated to +-448;
 *  - a block holding a NaN gets the e8m0 NaN byte 0xFF and every element
 *    becomes e4m3 NaN carrying its own sign (0x7F / 0xFF);
 *  - a block holding +-Inf (and no NaN) has amax = +Inf, so e clamps to 127
 *    (byte 254); +-Inf elements saturate to +-448, finite ones scale by 2^-127;
 *  - the 128x4 blocked layout is the MX scale-factor layout of block-scaled
 *    GEMMs: 512-byte tiles, row blocks outermost, column blocks next; inside
 *    a tile, byte (r % 32) * 16 + (r % 128 / 32) * 4 + (c % 4); padding 0.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define MXO_BLOCK 32          /* elements sharing one scale */
#define MXO_E4M3_MAX 448.0    /* largest finite e4m3fn value */
#define MXO_E4M3_EMAX 8       /* floor(log2(448)) */
#define MXO_E4M3_NEXT 480.0   /* 1.875 * 2^8: the step past 448, which has no finite code */
#define MXO_E8M0_NAN 0xFF

enum { MXO_OK = 0, MXO_ERR_ARG = 1 };

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

/* bf16 bit pattern -> its exact value.  bf16 is the top half of a binary32,
 * so the value is the float with those 16 bits on top; widening to double is
 * exact (denormals included). */
double mxo_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Value of an e4m3fn magnitude code 0x00..0x7E (OCP FP8 E4M3: 4 exponent
 * bits, bias 7, 3 mantissa bits, no infinities, 0x7F is NaN).
 * Exponent field 0 holds the subnormals m * 2^-9. */
double mxo_e4m3_value(int code)
{
    int exp_field = (code >> 3) & 0xF;
    int mant = code & 7;
    if (exp_field == 0)
        return ldexp((double)mant, -9);
    return ldexp(1.0 + mant / 8.0, exp_field - 7);
}

/* e8m0 byte -> the power of two it stands for (byte 255 is NaN). */
double mxo_e8m0_value(int byte)
{
    if (byte == MXO_E8M0_NAN)
        return NAN;
    return ldexp(1.0, byte - 127);
}

static double codebook[127];   /* e4m3 magnitude codes 0x00..0x7E */
static int codebook_ready = 0;

static void init_codebook(void)
{
    if (codebook_ready)
        return;
    for (int c = 0; c < 127; ++c)
        codebook[c] = mxo_e4m3_value(c);
    codebook_ready = 1;
}

/* ------------------------------------------------------------------ */
/* The MX rule, one block at a time                                    */
/* ------------------------------------------------------------------ */

/* Unbiased scale exponent of a block from its amax, before the e8m0 clamp:
 * floor(log2(amax)) - 8.  frexp writes amax = f * 2^k with f in [0.5, 1), so
 * floor(log2(amax)) = k - 1.  amax = 0 has no logarithm; it is reported as
 * below the e8m0 range (the minimum scale), amax = +Inf as above it. */
static long scale_exponent_unclamped(double amax)
{
    if (amax == 0.0)
        return -1000;
    if (isinf(amax))
        return 1000;
    int k;
    frexp(amax, &k);
    return (long)(k - 1) - MXO_E4M3_EMAX;
}

/* e8m0 scale byte of a block with the given amax (amax >= 0 or NaN).
 * Exponent clamped to [-127, 127]; byte = exponent + 127; NaN -> 0xFF. */
int mxo_scale_byte(double amax)
{
    if (isnan(amax))
        return MXO_E8M0_NAN;
    long e = scale_exponent_unclamped(amax);
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    return (int)(e + 127);
}

/* e4m3fn byte of one element x under scale byte s (0..254): the code nearest
 * to |x| / 2^(s-127), ties to the even code, saturated at 448; sign bit from
 * x (so -0.0 keeps its sign).  The scaled value is exact in double: x has 8
 * significant bits and is multiplied by a power of two within range.  The
 * distances compared below are exact whenever they can decide the result.
 * Under the e8m0 NaN scale (s = 255) every element is NaN with its own sign. */
int mxo_quantize_element(double x, int s)
{
    int sign = signbit(x) ? 0x80 : 0x00;
    if (s == MXO_E8M0_NAN || isnan(x))
        return 0x7F | sign;
    init_codebook();
    double v = ldexp(fabs(x), -(s - 127));
    if (v >= MXO_E4M3_MAX)             /* saturate (Inf included) */
        return 0x7E | sign;
    int best = 0;
    double best_d = fabs(v - codebook[0]);
    for (int c = 1; c < 127; ++c) {
        double d = fabs(v - codebook[c]);
        if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_d = d;
        }
    }
    return best | sign;
}

/* The element rule applied to n bf16 bit patterns under one scale byte. */
void mxo_quantize_elements(const uint16_t* x, int64_t n, int s, uint8_t* q)
{
    init_codebook();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        q[i] = (uint8_t)mxo_quantize_element(mxo_bf16_value(x[i]), s);
}

/* Cast one block of 32 bf16 values (given as their bit patterns, possibly
 * strided in memory) to 32 e4m3 bytes plus one e8m0 scale byte. */
static void quantize_block(const uint16_t* x, int64_t x_stride, uint8_t* q, int64_t q_stride,
                           uint8_t* scale)
{
    double v[MXO_BLOCK];
    double amax = 0.0;
    int has_nan = 0;
    for (int i = 0; i < MXO_BLOCK; ++i) {
        v[i] = mxo_bf16_value(x[i * x_stride]);
        if (isnan(v[i]))
            has_nan = 1;
        else if (fabs(v[i]) > amax)
            amax = fabs(v[i]);
    }
    int s = has_nan ? MXO_E8M0_NAN : mxo_scale_byte(amax);
    *scale = (uint8_t)s;
    for (int i = 0; i < MXO_BLOCK; ++i)
        q[i * q_stride] = (uint8_t)mxo_quantize_element(v[i], s);
}

/* Exported single-block form (contiguous input and output). */
void mxo_quantize_block(const uint16_t* x32, uint8_t* q32, uint8_t* scale)
{
    init_codebook();
    quantize_block(x32, 1, q32, 1, scale);
}

/* ------------------------------------------------------------------ */
/* dim0 / dim1 / 3D casts                                              */
/* ------------------------------------------------------------------ */

/* dim0: blocks of 32 consecutive elements along the last axis of a row-major
 * (rows, cols) bf16 matrix.  q (rows, cols) row-major, s (rows, cols/32).
 * The (16640, 5120) activations carry (16640, 160) scales in the compile
 * support page's error trace, which fixes blocks along the last axis. */
int mxo_cast_dim0(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s)
{
    if (rows < 0 || cols < 0 || cols % MXO_BLOCK != 0)
        return MXO_ERR_ARG;
    init_codebook();
    int64_t nb = cols / MXO_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < nb; ++j)
            quantize_block(x + r * cols + j * MXO_BLOCK, 1, q + r * cols + j * MXO_BLOCK, 1,
                           s + r * nb + j);
    return MXO_OK;
}

/* dim1: blocks of 32 consecutive rows within one column.  The col-major
 * output of the (rows, cols) matrix is stored as row-major (cols, rows):
 * q[c * rows + r]; scales s (cols, rows/32). */
int mxo_cast_dim1(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s)
{
    if (rows < 0 || cols < 0 || rows % MXO_BLOCK != 0)
        return MXO_ERR_ARG;
    init_codebook();
    int64_t nb = rows / MXO_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; ++c)
        for (int64_t i = 0; i < nb; ++i)
            quantize_block(x + (i * MXO_BLOCK) * cols + c, cols, q + c * rows + i * MXO_BLOCK, 1,
                           s + c * nb + i);
    return MXO_OK;
}

/* 3D expert weights W (experts, n, k) bf16: each expert's (n, k) matrix is
 * cast along dim1 (blocks of 32 along n).  q (experts, k, n), s (experts, k,
 * n/32).  The compile-support page (Perf analysis, item 4) proposes doing
 * this through the 2D dim1 kernel on a reshape; here each expert is cast on
 * its own, which is the definition. */
int mxo_cast_dim1_3d(const uint16_t* w, int64_t experts, int64_t n, int64_t k, uint8_t* q,
                     uint8_t* s)
{
    if (experts < 0 || n < 0 || k < 0 || n % MXO_BLOCK != 0)
        return MXO_ERR_ARG;
    for (int64_t e = 0; e < experts; ++e) {
        int rc = mxo_cast_dim1(w + e * n * k, n, k, q + e * k * n, s + e * k * (n / MXO_BLOCK));
        if (rc != MXO_OK)
            return rc;
    }
    return MXO_OK;
}

/* ------------------------------------------------------------------ */
/* 128x4 blocked scale layout                                           */
/* ------------------------------------------------------------------ */

static int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

/* Bytes of the blocked form of a (rows, cols) scale matrix. */
int64_t mxo_blocked_size(int64_t rows, int64_t cols)
{
    if (rows < 0 || cols < 0)
        return -1;
    return round_up(rows, 128) * round_up(cols, 4);
}

/* Position of scale (r, c) in the blocked form of a matrix with padded width
 * cols_pad (a multiple of 4).  Tiles of 128 rows x 4 columns are 512 bytes;
 * tiles are ordered row block first, column block second.  Inside a tile the
 * 128 rows are four sub-blocks of 32; byte (i, j) of the tile's 32 x 16 view
 * holds row 32 * (j / 4) + i, column j % 4. */
static int64_t blocked_index(int64_t r, int64_t c, int64_t cols_pad)
{
    int64_t col_blocks = cols_pad / 4;
    int64_t tile = (r / 128) * col_blocks + c / 4;
    int64_t within = (r % 32) * 16 + ((r % 128) / 32) * 4 + (c % 4);
    return tile * 512 + within;
}

/* Blocked form of a (rows, cols) matrix taken from a source with leading
 * dimension ld, written to out (mxo_blocked_size bytes; padding = 0). */
static void to_blocked_strided(const uint8_t* src, int64_t ld, int64_t rows, int64_t cols,
                               uint8_t* out)
{
    int64_t rows_pad = round_up(rows, 128), cols_pad = round_up(cols, 4);
    for (int64_t r = 0; r < rows_pad; ++r)
        for (int64_t c = 0; c < cols_pad; ++c)
            out[blocked_index(r, c, cols_pad)] =
                (r < rows && c < cols) ? src[r * ld + c] : (uint8_t)0;
}

int mxo_to_blocked(const uint8_t* s, int64_t rows, int64_t cols, uint8_t* out)
{
    if (rows < 0 || cols < 0)
        return MXO_ERR_ARG;
    to_blocked_strided(s, cols, rows, cols, out);
    return MXO_OK;
}

/* batch independent (rows, cols) matrices, outputs concatenated. */
int mxo_to_blocked_batched(const uint8_t* s, int64_t batch, int64_t rows, int64_t cols,
                           uint8_t* out)
{
    if (batch < 0 || rows < 0 || cols < 0)
        return MXO_ERR_ARG;
    int64_t per = mxo_blocked_size(rows, cols);
    for (int64_t b = 0; b < batch; ++b)
        to_blocked_strided(s + b * rows * cols, cols, rows, cols, out + b * per);
    return MXO_OK;
}

/* Output size of the grouped forms: the padded extent is bounded without
 * reading the offsets, by 128 extra rows (axis 0) or 4 extra columns (axis
 * 1) per group, as on the compile-support page (padded_rows = rows +
 * num_groups * 128). */
int64_t mxo_blocked_grouped_size(int64_t rows, int64_t cols, int32_t groups, int32_t axis)
{
    if (rows < 0 || cols < 0 || groups < 1 || (axis != 0 && axis != 1))
        return -1;
    if (axis == 0)
        return (rows + 128 * (int64_t)groups) * round_up(cols, 4);
    return round_up(rows, 128) * (round_up(cols, 4) + 4 * (int64_t)groups);
}

/* Grouped blocked layout.  ends[g] is the cumulative END offset of group g
 * along the grouped axis: rows of s (axis 0, "M groups") or scale columns of
 * s (axis 1, "K groups").  Offsets live in device memory on the GPU side and
 * cannot be checked there without a host read, so both sides use the same
 * memory-safe reading of malformed offsets: each end is clamped to
 * [previous end, extent], and anything past the last end is not part of any
 * group.
 *
 * axis 0: group g (rows [lo, hi)) padded to a multiple of 128 rows; its
 *   blocked form starts at output row start[g] = sum over earlier groups of
 *   round_up(size, 128), i.e. at byte start[g] * round_up(cols, 4).
 * axis 1: group g (columns [lo, hi)) padded to a multiple of 4 columns; its
 *   blocked form is its own contiguous matrix of round_up(rows, 128) rows,
 *   starting at output column start[g] = sum of earlier round_up(width, 4),
 *   i.e. at byte round_up(rows, 128) * start[g].
 * start[G] is the padded total.  Every other byte of the out_bytes-long
 * buffer is 0.  starts may be NULL. */
int mxo_to_blocked_grouped(const uint8_t* s, int64_t rows, int64_t cols, const int32_t* ends,
                           int32_t groups, int32_t axis, uint8_t* out, int64_t out_bytes,
                           int64_t* starts)
{
    int64_t need = mxo_blocked_grouped_size(rows, cols, groups, axis);
    if (need < 0 || out_bytes < need)
        return MXO_ERR_ARG;
    memset(out, 0, (size_t)out_bytes);
    int64_t extent = axis == 0 ? rows : cols;
    int64_t lo = 0, start = 0;
    int64_t cols_pad = round_up(cols, 4), rows_pad = round_up(rows, 128);
    for (int32_t g = 0; g < groups; ++g) {
        int64_t hi = ends[g];
        if (hi < lo)
            hi = lo;
        if (hi > extent)
            hi = extent;
        if (starts)
            starts[g] = start;
        int64_t size = hi - lo;
        if (axis == 0) {
            to_blocked_strided(s + lo * cols, cols, size, cols, out + start * cols_pad);
            start += round_up(size, 128);
        } else {
            to_blocked_strided(s + lo, cols, rows, size, out + rows_pad * start);
            start += round_up(size, 4);
        }
        lo = hi;
    }
    if (starts)
        starts[groups] = start;
    return MXO_OK;
}

/* ------------------------------------------------------------------ */
/* Row-wise fp8: one scale per row                                     */
/* ------------------------------------------------------------------ */
/*
 * Source: the gist "FP8 linear triton with row-wise scaling",
 * quantize_fp8_rowwise.  For a bf16 (rows, cols) matrix it takes, in order:
 *   1. amax of |x| over each row, in bf16 (exact: a max of bf16 values);
 *   2. scale = amax / 448, a bf16 tensor divided by a Python float: the
 *      quotient is formed in float32 and rounded to bf16;
 *   3. x converted to float32 and divided by the row's scale (float32);
 *   4. that quotient converted to float8_e4m3fn.
 * Readings, where the page leaves a step to the libraries it calls:
 *   - float32 division is IEEE binary32, correctly rounded; float32 -> bf16
 *     rounds to nearest, ties to even, and every NaN becomes 0x7FC0;
 *   - float32 -> e4m3fn rounds to nearest, ties to even, without saturation:
 *     a magnitude that rounds past 448 (the next step, 480, has no finite
 *     code, so anything above 464) and +-Inf become NaN;
 *   - a row holding a NaN has a NaN amax, so its scale is NaN and so is every
 *     quotient; an all-zero row has scale 0 and its quotients 0/0 are NaN; a
 *     row whose amax / 448 falls below the bf16 range gets scale 0 or a
 *     subnormal scale and its larger elements overflow to NaN -- all as the
 *     page's code computes them, with no guard added;
 *   - the sign bit of every code, NaN codes included, is the sign bit of x
 *     (the scale is never negative, so this is the quotient's sign wherever
 *     the quotient is a number).
 */

/* binary32 quotient a / b, correctly rounded.  Formed in double and then
 * rounded once to float: with 53 >= 2 * 24 + 2 bits the double rounding
 * cannot differ from rounding the exact quotient (a classical result for
 * the basic operations). */
static float f32_quotient(float a, float b)
{
    return (float)((double)a / (double)b);
}

/* float32 value -> bf16 bit pattern, rounded to nearest, ties to even.
 * Written as a comparison with the midpoint of the two bf16 neighbours (both
 * exact in double), not as bit arithmetic. */
uint16_t mxo_bf16_round(float f)
{
    if (isnan(f))
        return 0x7FC0;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000);
    if (isinf(f))
        return (uint16_t)(sign | 0x7F80);
    double v = fabs((double)f);
    uint16_t lo = (uint16_t)((u >> 16) & 0x7FFF);   /* largest bf16 magnitude <= |f| */
    double v_lo = mxo_bf16_value(lo);
    if (v_lo == v)
        return (uint16_t)(sign | lo);
    uint16_t hi = (uint16_t)(lo + 1);               /* 0x7F80 (Inf) stands for 2^128 */
    double v_hi = hi == 0x7F80 ? ldexp(1.0, 128) : mxo_bf16_value(hi);
    double mid = (v_lo + v_hi) / 2;
    uint16_t pick = v < mid ? lo : v > mid ? hi : ((lo & 1) ? hi : lo);
    return (uint16_t)(sign | pick);
}

/* float32 value -> e4m3fn byte without saturation (sign from the value). */
int mxo_e4m3fn_from_f32(float f)
{
    int sign = signbit(f) ? 0x80 : 0x00;
    if (isnan(f))
        return 0x7F | sign;
    double v = fabs((double)f);
    if (v > (MXO_E4M3_MAX + MXO_E4M3_NEXT) / 2)   /* rounds to 480 or beyond: no finite code */
        return 0x7F | sign;
    init_codebook();
    int best = 0;
    double best_d = fabs(v - codebook[0]);
    for (int c = 1; c < 127; ++c) {
        double d = fabs(v - codebook[c]);
        if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_d = d;
        }
    }
    return best | sign;
}

/* Scale of a row (bf16 bits) from its amax (a bf16 value, or NaN). */
uint16_t mxo_rowwise_scale(double amax)
{
    if (isnan(amax))
        return 0x7FC0;
    return mxo_bf16_round(f32_quotient((float)amax, (float)MXO_E4M3_MAX));
}

/* Code of one element x (a bf16 value) under a row scale given as bf16 bits. */
int mxo_rowwise_element(double x, uint16_t scale_bits)
{
    int sign = signbit(x) ? 0x80 : 0x00;
    float q = f32_quotient((float)x, (float)mxo_bf16_value(scale_bits));
    return (mxo_e4m3fn_from_f32(q) & 0x7F) | sign;
}

/* The element rule over n bf16 values under one scale given as bf16 bits. */
void mxo_rowwise_elements(const uint16_t* x, int64_t n, uint16_t scale_bits, uint8_t* q)
{
    init_codebook();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        q[i] = (uint8_t)mxo_rowwise_element(mxo_bf16_value(x[i]), scale_bits);
}

/* bf16 (rows, cols) -> q (rows, cols) e4m3fn bytes, scale (rows) bf16 bits. */
int mxo_quantize_fp8_rowwise(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q,
                             uint16_t* scale)
{
    if (rows < 0 || cols < 0)
        return MXO_ERR_ARG;
    if (cols == 0)
        return MXO_OK;
    init_codebook();
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * cols;
        double amax = 0.0;
        int has_nan = 0;
        for (int64_t i = 0; i < cols; ++i) {
            double v = mxo_bf16_value(xr[i]);
            if (isnan(v))
                has_nan = 1;
            else if (fabs(v) > amax)
                amax = fabs(v);
        }
        uint16_t s = mxo_rowwise_scale(has_nan ? NAN : amax);
        scale[r] = s;
        for (int64_t i = 0; i < cols; ++i)
            q[r * cols + i] = (uint8_t)mxo_rowwise_element(mxo_bf16_value(xr[i]), s);
    }
    return MXO_OK;
}

/* ------------------------------------------------------------------ */
/* Tensor-wise fp8: one scale for the whole tensor                     */
/* ------------------------------------------------------------------ */
/*
 * Source: "[float8nocompile]: Triton kernels for conversion to float8 dtypes
 * for forward pass of Float8LinearNoCompile" (review thread): one amax for
 * the whole tensor, found as per-block amaxes and then a global amax over
 * them, before the elements are converted.  The page states the structure,
 * not the formula.  Reading: the formula is the one the gist "FP8 linear
 * triton with row-wise scaling" states for its fp8 cast, with the amax taken
 * over every element instead of over a row -- bf16 amax; scale = amax / 448
 * through float32 to bf16; float32 x / scale to e4m3fn without saturation;
 * the same NaN and sign readings as the row-wise cast above.  The amax is a
 * max, so the order of the blocks cannot change it; the oracle takes it in
 * one plain loop.
 */
int mxo_quantize_fp8_tensorwise(const uint16_t* x, int64_t n, uint8_t* q, uint16_t* scale)
{
    if (n < 0)
        return MXO_ERR_ARG;
    if (n == 0)
        return MXO_OK;
    init_codebook();
    double amax = 0.0;
    int has_nan = 0;
    for (int64_t i = 0; i < n; ++i) {
        double v = mxo_bf16_value(x[i]);
        if (isnan(v))
            has_nan = 1;
        else if (fabs(v) > amax)
            amax = fabs(v);
    }
    uint16_t s = mxo_rowwise_scale(has_nan ? NAN : amax);
    *scale = s;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        q[i] = (uint8_t)mxo_rowwise_element(mxo_bf16_value(x[i]), s);
    return MXO_OK;
}

/* ------------------------------------------------------------------ */
/* MX-scaled GEMM: the consumer of the dim0 casts                      */
/* ------------------------------------------------------------------ */
/*
 * Source: "[mxfp8 moe training] add compile support", Perf analysis item 1:
 * MXFP8 grouped GEMMs on the (16640, 5120) activations grouped along M (4
 * groups) against per-group (8192, 5120) weights; the operands are the dim0
 * casts (32-element blocks along K, one e8m0 scale each).  The value an MX
 * operand stands for is code x 2^(scale byte - 127) (the MX rule above), so
 * the product is written out as its definition:
 *   C[m][n] = sum over k of A(m, k) * B(n, k),
 *   A(m, k) = e4m3(qa[m][k]) * 2^(sa[m][k / 32] - 127), B likewise,
 * accumulated in fp64 (every product is exact in fp64; the sum is within
 * rounding of the exact value).  absum[m][n] = sum over k of |A(m, k) B(n, k)|
 * is returned beside it: it scales the error bound of any faster summation.
 * A NaN code or a NaN scale byte (0xFF) makes the terms it touches NaN.
 */
static double mx_operand(uint8_t code, uint8_t scale)
{
    if ((code & 0x7F) == 0x7F || scale == MXO_E8M0_NAN)
        return NAN;
    double v = mxo_e4m3_value(code & 0x7F);
    return ldexp((code & 0x80) ? -v : v, (int)scale - 127);
}

int mxo_mx_gemm(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb, int64_t m,
                int64_t n, int64_t k, double* c, double* absum)
{
    if (m < 0 || n < 0 || k < 0 || k % MXO_BLOCK != 0)
        return MXO_ERR_ARG;
    int64_t kb = k / MXO_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0, mag = 0.0;
            for (int64_t t = 0; t < k; ++t) {
                double p = mx_operand(qa[i * k + t], sa[i * kb + t / MXO_BLOCK]) *
                           mx_operand(qb[j * k + t], sb[j * kb + t / MXO_BLOCK]);
                acc += p;
                mag += fabs(p);
            }
            c[i * n + j] = acc;
            if (absum)
                absum[i * n + j] = mag;
        }
    }
    return MXO_OK;
}

/* Grouped along M: rows [end_{g-1}, end_g) of A (ends clamped as for the M
 * groups of the blocked layout) are multiplied by group g's B (n, k) matrix
 * and scales; rows past the last end are left untouched. */
int mxo_mx_gemm_grouped(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb,
                        const int32_t* ends, int32_t groups, int64_t m, int64_t n, int64_t k, double* c,
                        double* absum)
{
    if (groups < 1 || m < 0 || n < 0 || k < 0 || k % MXO_BLOCK != 0)
        return MXO_ERR_ARG;
    int64_t lo = 0, kb = k / MXO_BLOCK;
    for (int32_t g = 0; g < groups; ++g) {
        int64_t hi = ends[g];
        if (hi < lo)
            hi = lo;
        if (hi > m)
            hi = m;
        int rc = mxo_mx_gemm(qa + lo * k, sa + lo * kb, qb + (int64_t)g * n * k, sb + (int64_t)g * n * kb,
                             hi - lo, n, k, c + lo * n, absum ? absum + lo * n : NULL);
        if (rc != MXO_OK)
            return rc;
        lo = hi;
    }
    return MXO_OK;
}

/* Threads the OpenMP loops above run on. */
int mxo_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following calls (timing only: results do not depend on it). */
void mxo_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
