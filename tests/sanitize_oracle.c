/*
 * sanitize_oracle.c -- TEST INFRASTRUCTURE: drives every entry point of the
 * CPU oracle (oracle/mxq_oracle.c) on ragged, tiny and empty shapes and on
 * inputs holding every kind of bf16 (NaN, Inf, zeros, subnormals, extremes),
 * with each output buffer allocated to exactly its documented size.  Built
 * with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_oracle_sanitize.py, so an out-of-bounds access, a use of freed
 * memory, a leak or undefined arithmetic (an out-of-range float-to-int
 * conversion, an invalid shift, signed overflow) fails the run.  It computes
 * nothing of its own; the values are pinned by the other oracle tests.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* the oracle's entry points (oracle/mxq_oracle.c has no header of its own) */
void orc_mxfp8_quantize_rowwise(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q,
                                uint8_t *scale);
int orc_mxfp8_quantize_padcrop(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q,
                               uint8_t *scale);
void orc_mxfp8_quantize_colwise(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q,
                                uint8_t *scale);
int orc_mxfp8_quantize_colwise_t(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *qt,
                                 uint8_t *st);
void orc_mxfp8_dequantize(const uint8_t *q, const uint8_t *scale, int64_t rows, int64_t cols,
                          int axis, uint16_t *out);
int orc_mxfp8_fake_quant(const uint16_t *x, int64_t rows, int64_t cols, int axis, uint16_t *out);
void orc_mxfp8_quantize_rowwise_many(int32_t n, const uint16_t *const *xs, const int64_t *rows,
                                     const int64_t *cols, uint8_t *const *qs, uint8_t *const *ss);
void orc_mxfp4_quantize(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q,
                        uint8_t *scale);
void orc_mxfp4_dequantize(const uint8_t *q, const uint8_t *scale, int64_t rows, int64_t cols,
                          uint16_t *out);
int orc_mxfp4_fake_quant(const uint16_t *x, int64_t rows, int64_t cols, uint16_t *out);
void orc_blockfp8_quantize_rect(const uint16_t *x, int64_t rows, int64_t cols, int32_t br,
                                int32_t bc, uint8_t *q, float *scale);
void orc_blockfp8_dequantize_rect(const uint8_t *q, const float *scale, int64_t rows,
                                  int64_t cols, int32_t br, int32_t bc, uint16_t *out);
void orc_blockfp8_quantize_gkn(const uint16_t *x, int64_t G, int64_t K, int64_t N, int32_t blk,
                               uint8_t *q, float *scale);
void orc_blockfp8_dequantize_gkn(const uint8_t *q, const float *scale, int64_t G, int64_t K,
                                 int64_t N, int32_t blk, uint16_t *out);
int orc_blockfp8_fake_quant_1x128(const uint16_t *x, int64_t rows, int64_t cols, uint16_t *out);
int orc_blockfp8_to_mxfp8(const uint8_t *q, const float *scale, int64_t rows, int64_t cols,
                          int32_t blk, uint8_t *q8, uint8_t *scale8);
void orc_nvfp4_quantize(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q_packed,
                        uint8_t *s_e4m3, float *global_scale);
int orc_nvfp4_quantize_grouped(int32_t n, const uint16_t *const *xs, const int64_t *rows,
                               const int64_t *cols, const int32_t *group, int32_t n_groups,
                               uint8_t *const *qs, uint8_t *const *ss, float *gs);
void orc_nvfp4_dequantize(const uint8_t *q_packed, const uint8_t *s_e4m3,
                          const float *global_scale, int64_t rows, int64_t cols, uint16_t *out);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void)
{
    /* xorshift64* */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}

/* Exactly n elements (never a zero-byte request: malloc(0) may return NULL). */
static void *alloc(size_t n, size_t elem)
{
    void *p = malloc(n ? n * elem : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}

/* bf16 input of the given kind: 0 every 16-bit pattern at random (NaN, Inf,
 * subnormals included); 1 finite, normal-range values; 2 all zero but one
 * NaN-free extreme per row. */
static uint16_t *make_input(int64_t rows, int64_t cols, int kind)
{
    size_t n = (size_t)(rows * cols);
    uint16_t *x = (uint16_t *)alloc(n, 2);
    for (size_t i = 0; i < n; ++i) {
        uint16_t v = (uint16_t)rnd();
        if (kind == 1) v = (uint16_t)((v & 0x80FFu) | (uint16_t)((0x30 + (rnd() % 0x20)) << 8));
        if (kind == 2) v = 0;
        x[i] = v;
    }
    if (kind == 2 && cols > 0)
        for (int64_t r = 0; r < rows; ++r) x[r * cols + r % cols] = r & 1 ? 0x7F7F : 0x0001;
    return x;
}

static void run_mx(int64_t rows, int64_t cols, int kind)
{
    uint16_t *x = make_input(rows, cols, kind);
    size_t e = (size_t)(rows * cols), ng = (size_t)(rows * (cols / 32));
    size_t nrg = (size_t)((rows + 31) / 32);
    uint8_t *q = (uint8_t *)alloc(e, 1), *s = (uint8_t *)alloc(ng, 1);
    uint16_t *out = (uint16_t *)alloc(e, 2);
    orc_mxfp8_quantize_rowwise(x, rows, cols, q, s);
    orc_mxfp8_dequantize(q, s, rows, cols, 1, out);
    if (orc_mxfp8_quantize_padcrop(x, rows, cols, q, s) != 0 && e) exit(3);
    uint8_t *qc = (uint8_t *)alloc(e, 1), *sc = (uint8_t *)alloc(nrg * (size_t)cols, 1);
    orc_mxfp8_quantize_colwise(x, rows, cols, qc, sc);
    orc_mxfp8_dequantize(qc, sc, rows, cols, 0, out);
    uint8_t *qt = (uint8_t *)alloc(e, 1), *st = (uint8_t *)alloc((size_t)cols * nrg, 1);
    if (orc_mxfp8_quantize_colwise_t(x, rows, cols, qt, st) != 0 && e) exit(3);
    if (orc_mxfp8_fake_quant(x, rows, cols, 0, out) != 0 && e) exit(3);
    if (orc_mxfp8_fake_quant(x, rows, cols, 1, out) != 0 && e) exit(3);
    /* MXFP4 */
    uint8_t *q4 = (uint8_t *)alloc(e / 2, 1);
    orc_mxfp4_quantize(x, rows, cols, q4, s);
    orc_mxfp4_dequantize(q4, s, rows, cols, out);
    if (orc_mxfp4_fake_quant(x, rows, cols, out) != 0 && e) exit(3);
    /* FP8 block -> MXFP8 (128 x 128 tiles, cols % 32 == 0) */
    size_t tr = (size_t)((rows + 127) / 128), tc = (size_t)((cols + 127) / 128);
    uint8_t *bq = (uint8_t *)alloc(e, 1);
    float *bS = (float *)alloc(tr * tc, sizeof(float));
    orc_blockfp8_quantize_rect(x, rows, cols, 128, 128, bq, bS);
    if (orc_blockfp8_to_mxfp8(bq, bS, rows, cols, 128, q, s) != 0 && e) exit(3);
    free(bq); free(bS); free(q4); free(qt); free(st); free(qc); free(sc);
    free(q); free(s); free(out); free(x);
}

static void run_block(int64_t rows, int64_t cols, int32_t br, int32_t bc, int kind)
{
    uint16_t *x = make_input(rows, cols, kind);
    size_t e = (size_t)(rows * cols);
    size_t tr = (size_t)((rows + br - 1) / br), tc = (size_t)((cols + bc - 1) / bc);
    uint8_t *q = (uint8_t *)alloc(e, 1);
    float *S = (float *)alloc(tr * tc, sizeof(float));
    uint16_t *out = (uint16_t *)alloc(e, 2);
    orc_blockfp8_quantize_rect(x, rows, cols, br, bc, q, S);
    orc_blockfp8_dequantize_rect(q, S, rows, cols, br, bc, out);
    if (br == 1 && bc == 128 && orc_blockfp8_fake_quant_1x128(x, rows, cols, out) != 0 && e) exit(3);
    free(q); free(S); free(out); free(x);
}

static void run_gkn(int64_t G, int64_t K, int64_t N, int kind)
{
    uint16_t *x = make_input(G * K, N, kind);
    size_t e = (size_t)(G * K * N);
    size_t ts = (size_t)(((K + 127) / 128) * ((N + 127) / 128));
    uint8_t *q = (uint8_t *)alloc(e, 1);
    float *S = (float *)alloc((size_t)G * ts, sizeof(float));
    uint16_t *out = (uint16_t *)alloc(e, 2);
    orc_blockfp8_quantize_gkn(x, G, K, N, 128, q, S);
    orc_blockfp8_dequantize_gkn(q, S, G, K, N, 128, out);
    free(q); free(S); free(out); free(x);
}

static void run_nv(int64_t rows, int64_t cols, int kind)
{
    uint16_t *x = make_input(rows, cols, kind);
    size_t e = (size_t)(rows * cols);
    uint8_t *q = (uint8_t *)alloc(e / 2, 1), *s = (uint8_t *)alloc(e / 16, 1);
    float *g = (float *)alloc(1, sizeof(float));
    uint16_t *out = (uint16_t *)alloc(e, 2);
    orc_nvfp4_quantize(x, rows, cols, q, s, g);
    orc_nvfp4_dequantize(q, s, g, rows, cols, out);
    free(q); free(s); free(g); free(out); free(x);
}

static void run_grouped(int kind)
{
    enum { N = 5 };
    const int64_t rows[N] = {33, 0, 1, 64, 7}, cols[N] = {64, 32, 96, 32, 160};
    const int32_t group[N] = {0, 1, 1, 0, 2};
    const uint16_t *xs[N];
    uint8_t *qs[N], *ss[N], *q4[N], *s16[N];
    for (int i = 0; i < N; ++i) {
        size_t e = (size_t)(rows[i] * cols[i]);
        xs[i] = make_input(rows[i], cols[i], kind);
        qs[i] = (uint8_t *)alloc(e, 1);
        ss[i] = (uint8_t *)alloc(e / 32, 1);
        q4[i] = (uint8_t *)alloc(e / 2, 1);
        s16[i] = (uint8_t *)alloc(e / 16, 1);
    }
    orc_mxfp8_quantize_rowwise_many(N, xs, rows, cols, qs, ss);
    float *gs = (float *)alloc(3, sizeof(float));
    if (orc_nvfp4_quantize_grouped(N, xs, rows, cols, group, 3, q4, s16, gs) != 0) exit(3);
    for (int i = 0; i < N; ++i) {
        free((void *)xs[i]); free(qs[i]); free(ss[i]); free(q4[i]); free(s16[i]);
    }
    free(gs);
}

int main(void)
{
    static const int64_t mx_shapes[][2] = {{1, 32}, {31, 64}, {33, 96}, {129, 160}, {64, 256},
                                           {0, 32}, {2, 0}};
    static const int64_t blk_shapes[][2] = {{1, 1}, {5, 130}, {129, 257}, {200, 128}, {0, 7}};
    static const int64_t nv_shapes[][2] = {{1, 16}, {17, 48}, {64, 256}, {0, 16}};
    for (int kind = 0; kind < 3; ++kind) {
        for (size_t i = 0; i < sizeof(mx_shapes) / sizeof(mx_shapes[0]); ++i)
            run_mx(mx_shapes[i][0], mx_shapes[i][1], kind);
        for (size_t i = 0; i < sizeof(blk_shapes) / sizeof(blk_shapes[0]); ++i) {
            run_block(blk_shapes[i][0], blk_shapes[i][1], 128, 128, kind);
            run_block(blk_shapes[i][0], blk_shapes[i][1], 1, 128, kind);
        }
        run_gkn(3, 130, 257, kind);
        run_gkn(1, 1, 1, kind);
        for (size_t i = 0; i < sizeof(nv_shapes) / sizeof(nv_shapes[0]); ++i)
            run_nv(nv_shapes[i][0], nv_shapes[i][1], kind);
        run_grouped(kind);
    }
    printf("sanitized oracle run: ok\n");
    return 0;
}
