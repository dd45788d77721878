/*
 * Driver for the AddressSanitizer + UndefinedBehaviorSanitizer build of the
 * CPU oracle (oracle/mxoracle.c), run by tests/test_sanitizers.py.  Every
 * oracle entry point is called on small seeded inputs held in buffers of
 * exactly the size the call may touch, including ragged shapes, empty and
 * malformed group offsets and special bf16 values, so that any read or write
 * past a buffer, and any undefined arithmetic, stops the run.  A few
 * results are cross-checked (dim1 = dim0 of the transpose, 3D = per-expert
 * dim1) so that the calls do real work.  Exit status 0: clean.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double mxo_bf16_value(uint16_t bits);
double mxo_e4m3_value(int code);
double mxo_e8m0_value(int byte);
int mxo_scale_byte(double amax);
int mxo_quantize_element(double x, int s);
void mxo_quantize_elements(const uint16_t* x, int64_t n, int s, uint8_t* q);
void mxo_quantize_block(const uint16_t* x32, uint8_t* q32, uint8_t* scale);
int mxo_cast_dim0(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s);
int mxo_cast_dim1(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s);
int mxo_cast_dim1_3d(const uint16_t* w, int64_t experts, int64_t n, int64_t k, uint8_t* q, uint8_t* s);
int64_t mxo_blocked_size(int64_t rows, int64_t cols);
int mxo_to_blocked(const uint8_t* s, int64_t rows, int64_t cols, uint8_t* out);
int mxo_to_blocked_batched(const uint8_t* s, int64_t batch, int64_t rows, int64_t cols, uint8_t* out);
int64_t mxo_blocked_grouped_size(int64_t rows, int64_t cols, int32_t groups, int32_t axis);
int mxo_to_blocked_grouped(const uint8_t* s, int64_t rows, int64_t cols, const int32_t* ends, int32_t groups,
                           int32_t axis, uint8_t* out, int64_t out_bytes, int64_t* starts);
uint16_t mxo_bf16_round(float f);
int mxo_e4m3fn_from_f32(float f);
uint16_t mxo_rowwise_scale(double amax);
int mxo_rowwise_element(double x, uint16_t scale_bits);
void mxo_rowwise_elements(const uint16_t* x, int64_t n, uint16_t scale_bits, uint8_t* q);
int mxo_quantize_fp8_rowwise(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, uint16_t* scale);
int mxo_quantize_fp8_tensorwise(const uint16_t* x, int64_t n, uint8_t* q, uint16_t* scale);
int mxo_mx_gemm(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb, int64_t m, int64_t n,
                int64_t k, double* c, double* absum);
int mxo_mx_gemm_grouped(const uint8_t* qa, const uint8_t* sa, const uint8_t* qb, const uint8_t* sb,
                        const int32_t* ends, int32_t groups, int64_t m, int64_t n, int64_t k, double* c,
                        double* absum);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void)
{
    /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (uint32_t)((z ^ (z >> 31)) >> 32);
}

static int failures = 0;
#define CHECK(cond)                                                          \
    do {                                                                     \
        if (!(cond)) {                                                       \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

static void* xmalloc(size_t n) { return malloc(n ? n : 1); }

/* random bf16 bits: any pattern, every 7th one a finite value near 1 */
static void fill_bf16(uint16_t* x, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        uint32_t r = next_u32();
        x[i] = (i % 7 == 0) ? (uint16_t)(0x3F00 + (r & 0xFF)) : (uint16_t)r;
    }
}

static void cast_checks(int64_t rows, int64_t cols)
{
    int64_t n = rows * cols;
    uint16_t* x = xmalloc(n * 2);
    uint16_t* t = xmalloc(n * 2);
    fill_bf16(x, n);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            t[c * rows + r] = x[r * cols + c];
    uint8_t *q0 = xmalloc(n), *s0 = xmalloc(n / 32), *q1 = xmalloc(n), *s1 = xmalloc(n / 32);
    uint8_t *qt = xmalloc(n), *st = xmalloc(n / 32);
    CHECK(mxo_cast_dim0(x, rows, cols, q0, s0) == 0);
    CHECK(mxo_cast_dim1(x, rows, cols, q1, s1) == 0);
    CHECK(mxo_cast_dim0(t, cols, rows, qt, st) == 0);
    CHECK(memcmp(q1, qt, n) == 0 && memcmp(s1, st, n / 32) == 0);
    int64_t bsz = mxo_blocked_size(rows, cols / 32);
    uint8_t* b = xmalloc(bsz);
    CHECK(mxo_to_blocked(s0, rows, cols / 32, b) == 0);
    free(b);
    free(x); free(t); free(q0); free(s0); free(q1); free(s1); free(qt); free(st);
}

static void layout_checks(void)
{
    const int64_t shapes[][2] = {{1, 1}, {130, 7}, {256, 8}, {0, 5}, {5, 0}, {300, 13}};
    for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) {
        int64_t r = shapes[i][0], c = shapes[i][1];
        uint8_t* s = xmalloc(3 * r * c);
        for (int64_t j = 0; j < 3 * r * c; ++j)
            s[j] = (uint8_t)next_u32();
        int64_t one = mxo_blocked_size(r, c);
        uint8_t* out = xmalloc(3 * one);
        CHECK(mxo_to_blocked(s, r, c, out) == 0);
        CHECK(mxo_to_blocked_batched(s, 3, r, c, out) == 0);
        free(out);
        /* grouped, both axes: ordinary, empty, decreasing and past-the-end ends */
        const int32_t ends_sets[][4] = {{1, 2, 3, 4}, {0, 0, 0, 0}, {5, 2, 1000, 3}, {-4, 7, 7, 2147483647}};
        for (int axis = 0; axis < 2; ++axis) {
            int64_t extent = axis == 0 ? r : c;
            for (size_t e = 0; e < 4; ++e) {
                int32_t ends[4];
                for (int g = 0; g < 4; ++g)
                    ends[g] = (int32_t)(ends_sets[e][g] == 2147483647 ? extent : ends_sets[e][g]);
                int64_t need = mxo_blocked_grouped_size(r, c, 4, axis);
                CHECK(need >= 0);
                uint8_t* g_out = xmalloc(need);
                int64_t starts[5];
                CHECK(mxo_to_blocked_grouped(s, r, c, ends, 4, axis, g_out, need, starts) == 0);
                CHECK(starts[4] <= (axis == 0 ? r + 4 * 128 : c + 4 * 4));
                free(g_out);
            }
        }
        free(s);
    }
}

static void rowwise_checks(void)
{
    const int64_t shapes[][2] = {{1, 1}, {5, 37}, {3, 1024}, {0, 9}, {9, 0}};
    for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) {
        int64_t r = shapes[i][0], c = shapes[i][1];
        uint16_t* x = xmalloc(r * c * 2);
        fill_bf16(x, r * c);
        uint8_t* q = xmalloc(r * c);
        uint16_t* sc = xmalloc(r * 2);
        CHECK(mxo_quantize_fp8_rowwise(x, r, c, q, sc) == 0);
        if (r * c > 0) {
            uint16_t s1;
            uint8_t* q1 = xmalloc(r * c);
            CHECK(mxo_quantize_fp8_tensorwise(x, r * c, q1, &s1) == 0);
            free(q1);
        }
        free(x); free(q); free(sc);
    }
}

static void gemm_checks(void)
{
    const int64_t m = 33, n = 17, k = 96, kb = 3;
    uint8_t *qa = xmalloc(m * k), *sa = xmalloc(m * kb), *qb = xmalloc(2 * n * k), *sb = xmalloc(2 * n * kb);
    for (int64_t i = 0; i < m * k; ++i) qa[i] = (uint8_t)next_u32();
    for (int64_t i = 0; i < 2 * n * k; ++i) qb[i] = (uint8_t)next_u32();
    for (int64_t i = 0; i < m * kb; ++i) sa[i] = (uint8_t)(120 + next_u32() % 16);
    for (int64_t i = 0; i < 2 * n * kb; ++i) sb[i] = (uint8_t)(120 + next_u32() % 16);
    double* c = xmalloc(m * n * sizeof(double));
    double* a = xmalloc(m * n * sizeof(double));
    CHECK(mxo_mx_gemm(qa, sa, qb, sb, m, n, k, c, a) == 0);
    const int32_t ends[2] = {20, 99};
    CHECK(mxo_mx_gemm_grouped(qa, sa, qb, sb, ends, 2, m, n, k, c, a) == 0);
    free(qa); free(sa); free(qb); free(sb); free(c); free(a);
}

int main(void)
{
    for (int v = 0; v < 65536; v += 7)
        (void)mxo_bf16_value((uint16_t)v);
    for (int code = 0; code < 127; ++code)
        (void)mxo_e4m3_value(code);
    for (int b = 0; b < 256; ++b)
        (void)mxo_e8m0_value(b);
    uint16_t all[256];
    uint8_t q[256];
    for (int i = 0; i < 256; ++i)
        all[i] = (uint16_t)(i * 257);
    for (int s = 0; s < 256; s += 5)
        mxo_quantize_elements(all, 256, s, q);
    uint8_t sc;
    mxo_quantize_block(all, q, &sc);
    (void)mxo_scale_byte(0.0);
    (void)mxo_scale_byte(1e300);
    (void)mxo_e4m3fn_from_f32(1e30f);
    (void)mxo_bf16_round(3.0e38f);
    (void)mxo_rowwise_scale(1e-45);
    uint8_t qr[256];
    mxo_rowwise_elements(all, 256, 0x3F80, qr);
    cast_checks(32, 32);
    cast_checks(96, 160);
    cast_checks(64, 2080);
    uint16_t* w = xmalloc(3 * 64 * 96 * 2);
    fill_bf16(w, 3 * 64 * 96);
    uint8_t *wq = xmalloc(3 * 64 * 96), *ws = xmalloc(3 * 96 * 2);
    CHECK(mxo_cast_dim1_3d(w, 3, 64, 96, wq, ws) == 0);
    free(w); free(wq); free(ws);
    layout_checks();
    rowwise_checks();
    gemm_checks();
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer run clean\n");
    return 0;
}
