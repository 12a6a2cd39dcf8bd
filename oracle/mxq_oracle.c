/*
 * mxq_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * The plain, slow, single-threaded CPU definition of every byte the HIP
 * library produces.  Only the tests, the smoke check and the benchmark's CPU
 * baseline may load this file's library; the product path never does, and it
 * shares no code, header, table or constant generator with the HIP sources.
 *
 * Arithmetic conventions
 *   - Exact steps are done in IEEE double: a bf16, E4M3 or E2M1 value times a
 *     power of two is always exact there, so the only rounding is the one the
 *     format conversion defines.
 *   - Steps the method defines in fp32 (the block-FP8 and NVFP4 scale and
 *     element divisions, the fp32 products of their dequantization) are done
 *     in C `float` with one IEEE operation per statement.  The build uses
 *     -ffp-contract=off -fno-fast-math on x86-64 SSE (FLT_EVAL_METHOD == 0),
 *     with no flush-to-zero, so each such statement rounds exactly once.
 *   - Rounding to a narrower format is round-to-nearest, ties-to-even, via
 *     nearbyint() of a quotient by a power of two (exact) under the default
 *     rounding mode.
 *
 * Sources (the pages name the formats and the method; the bit layouts are the
 * public format definitions those names refer to):
 *   [MX-adapter]  "PR #1935 完整报告 / Use TransformerEngine for MXFP8
 *                 quantization", section 实现拆解 item 1 (group of 32,
 *                 32-row zero pad then crop, compact non-swizzled qweight +
 *                 scale) and 关键源码片段 (the scale is stored as
 *                 `<name>.weight_scale_inv`).
 *   [V4-mxfp4]    "V4 mxfp4" (miles PR #1372), PR description: Blackwell MXFP8
 *                 uses power-of-two scales; E8M0 (`float8_e8m0fnu`) scale
 *                 dtype; fp4 output packed two per byte (`float4_e2m1fn_x2`,
 *                 N/2 bytes per row) in the review of `fp4_act_quant`;
 *                 fake-quant (simulate-QAT) with blocks of 32 and 128.
 *   [xorl]        "Add FP8, NVFP4, and QARL training and export" (xorl PR #30),
 *                 deep review, "What looked solid": block-FP8 absmax scaling;
 *                 NVFP4 two-level global + FP8-block scaling with
 *                 effective = block_scale * global_scale, clamped, zero block
 *                 guarded.
 *   [OFP8]        OCP 8-bit floating point: E4M3 "fn" (bias 7, no infinity,
 *                 S.1111.111 is NaN, max finite 448).
 *   [OCP-MX]      OCP Microscaling formats v1.0: E8M0 scale 2^(b-127), 0xFF NaN;
 *                 E2M1 element {0, .5, 1, 1.5, 2, 3, 4, 6}; conversion to MX
 *                 takes the shared scale as the largest power of two <= amax
 *                 divided by the largest power of two of the element format
 *                 (2^8 for E4M3, 2^2 for E2M1), and clamps elements to the
 *                 max normal.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes): RNE everywhere; saturation to the max finite value; the sign
 * bit is kept on zero results; a group (tile, tensor) holding NaN or Inf is
 * quantized to all-NaN; an all-zero MX group gets scale byte 0; columns are
 * never padded (cols % 32 != 0 is an error at the boundary).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Formats                                                                   */
/* ------------------------------------------------------------------------ */

/* bf16 (1-8-7, bias 127, IEEE subnormals/Inf/NaN) decoded exactly. */
double orc_bf16_to_double(uint16_t b)
{
    int sign = b >> 15;
    int e = (b >> 7) & 0xFF;
    int m = b & 0x7F;
    double v;
    if (e == 0xFF)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -133);            /* 0.m * 2^-126 */
    else
        v = ldexp((double)(128 + m), e - 134); /* 1.m * 2^(e-127) */
    return sign ? -v : v;
}

/* floor(log2(a)) for finite a > 0, exact via frexp. */
static int floor_log2(double a)
{
    int e;
    frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
    return e - 1;
}

/* bf16 round-to-nearest-even of a double.  NaN maps to the quiet NaN with the
 * input's sign (0x7FC0 / 0xFFC0); overflow after rounding gives +-Inf. */
uint16_t orc_double_to_bf16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (isnan(v)) return sign | 0x7FC0;
    double a = fabs(v);
    if (isinf(a)) return sign | 0x7F80;
    if (a == 0.0) return sign;
    int E = floor_log2(a);
    if (E < -126) E = -126;                 /* subnormal binade: quantum 2^-133 */
    double quantum = ldexp(1.0, E - 7);     /* 7 fraction bits */
    double n = nearbyint(a / quantum);      /* exact division, RNE */
    double r = n * quantum;
    if (r >= ldexp(1.0, 128)) return sign | 0x7F80;
    if (r < ldexp(1.0, -126)) return sign | (uint16_t)n; /* subnormal: bits = n */
    int Er = floor_log2(r);
    int frac = (int)(ldexp(r, -Er) * 128.0) - 128;       /* 7-bit fraction */
    return sign | (uint16_t)(((Er + 127) << 7) | frac);
}

/* E4M3 ("fn"): bias 7, no Inf, NaN = S.1111.111, subnormal m * 2^-9. */
double orc_e4m3_to_double(uint8_t c)
{
    int sign = c >> 7;
    int e = (c >> 3) & 0xF;
    int m = c & 7;
    double v;
    if (e == 0xF && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 10);
    return sign ? -v : v;
}

/* E4M3 encode: nearest finite code, ties to the even code, saturating at
 * +-448.  NaN -> 0x7F | sign, +-Inf -> +-448, the sign bit always kept. */
uint8_t orc_double_to_e4m3(double v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0;
    if (isnan(v)) return sign | 0x7F;
    double a = fabs(v);
    if (isinf(a)) return sign | 0x7E;
    if (a == 0.0) return sign;
    int E = floor_log2(a);
    if (E < -6) E = -6;                     /* subnormals share the 2^-6 binade's quantum */
    double quantum = ldexp(1.0, E - 3);     /* 3 fraction bits */
    double n = nearbyint(a / quantum);
    double r = n * quantum;
    if (r > 448.0) return sign | 0x7E;      /* saturate */
    if (r < ldexp(1.0, -6)) return sign | (uint8_t)n; /* subnormal code = n */
    int Er = floor_log2(r);
    int frac = (int)(ldexp(r, -Er) * 8.0) - 8;
    return sign | (uint8_t)(((Er + 7) << 3) | frac);
}

/* E8M0 scale byte: 2^(b-127) for b in 0..254, 0xFF = NaN. */
double orc_e8m0_to_double(uint8_t b)
{
    if (b == 0xFF) return NAN;
    return ldexp(1.0, (int)b - 127);
}

/* E2M1: sign bit 0x8, bias 1; magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}. */
double orc_e2m1_to_double(uint8_t nib)
{
    int sign = (nib >> 3) & 1;
    int e = (nib >> 1) & 3;
    int m = nib & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -v : v;
}

/* E2M1 encode: nearest, ties to even code, saturating at +-6; the format has
 * no NaN, so NaN maps to 0x7 | sign (only reached under the all-NaN rule). */
uint8_t orc_double_to_e2m1(double v)
{
    uint8_t sign = signbit(v) ? 0x8 : 0;
    if (isnan(v)) return sign | 0x7;
    double a = fabs(v);
    if (isinf(a)) return sign | 0x7;
    if (a == 0.0) return sign;
    int E = floor_log2(a);
    if (E < 0) E = 0;                       /* subnormal 0.5 shares the [1,2) quantum */
    double quantum = ldexp(1.0, E - 1);     /* 1 fraction bit */
    double n = nearbyint(a / quantum);
    double r = n * quantum;
    if (r > 6.0) return sign | 0x7;
    if (r < 1.0) return sign | (uint8_t)n;  /* 0 -> 0, 0.5 -> 1 */
    int Er = floor_log2(r);
    int frac = (int)(ldexp(r, -Er) * 2.0) - 2;
    return sign | (uint8_t)(((Er + 1) << 1) | frac);
}

/* The element encoders over runs of fp32 bit patterns, for the exhaustive
 * sweeps of the library's fp32 -> E4M3 / E2M1 / bf16 converters: out[i] is
 * the encoding of the fp32 value whose bit pattern is first + i * stride
 * (as a double, which holds every fp32 value exactly).  Plain loops over the
 * scalar encoders above. */
void orc_f32_bits_to_e4m3(uint32_t first, int64_t n, uint32_t stride, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u = first + (uint32_t)i * stride;
        float f;
        memcpy(&f, &u, sizeof f);
        out[i] = orc_double_to_e4m3((double)f);
    }
}

void orc_f32_bits_to_e2m1(uint32_t first, int64_t n, uint32_t stride, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u = first + (uint32_t)i * stride;
        float f;
        memcpy(&f, &u, sizeof f);
        out[i] = orc_double_to_e2m1((double)f);
    }
}

void orc_f32_bits_to_bf16(uint32_t first, int64_t n, uint32_t stride, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u = first + (uint32_t)i * stride;
        float f;
        memcpy(&f, &u, sizeof f);
        out[i] = orc_double_to_bf16((double)f);
    }
}

/* ------------------------------------------------------------------------ */
/* MXFP8: groups of 32, one E8M0 scale, E4M3 elements                        */
/* ------------------------------------------------------------------------ */

#define MX_GROUP 32

/* Shared scale byte of one group [OCP-MX, V4-mxfp4]: the power of two
 * 2^(floor(log2 amax) - 8) as an E8M0 byte, clamped at 0 (2^-127); an
 * all-zero group gets 0; a group holding NaN or Inf gets 0xFF. */
static uint8_t mx_scale_byte(const double *vals, int n)
{
    double amax = 0.0;
    for (int i = 0; i < n; ++i) {
        double a = fabs(vals[i]);
        if (!isfinite(a)) return 0xFF;
        if (a > amax) amax = a;
    }
    if (amax == 0.0) return 0;
    int E = floor_log2(amax) - 8;           /* 8 = exponent of 256, E4M3's largest power of two */
    if (E < -127) E = -127;
    if (E > 127) E = 127;
    return (uint8_t)(E + 127);
}

/* One element of a group with scale byte s: x / 2^(s-127), exact, then E4M3;
 * a NaN group encodes every element as NaN with the element's sign. */
static uint8_t mx_encode(double x, uint8_t s)
{
    if (s == 0xFF) return (signbit(x) ? 0x80 : 0) | 0x7F;
    return orc_double_to_e4m3(ldexp(x, 127 - (int)s));
}

/* Row-wise MXFP8 [MX-adapter item 1]: x [rows, cols] bf16 row-major,
 * groups of 32 along each row.  q [rows, cols] E4M3 bytes and scale
 * [rows, cols/32] E8M0 bytes, both compact and row-major.  cols % 32 == 0. */
void orc_mxfp8_quantize_rowwise(const uint16_t *x, int64_t rows, int64_t cols,
                                uint8_t *q, uint8_t *scale)
{
    double g[MX_GROUP];
    int64_t ng = cols / MX_GROUP;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t k = 0; k < ng; ++k) {
            const uint16_t *src = x + r * cols + k * MX_GROUP;
            for (int i = 0; i < MX_GROUP; ++i) g[i] = orc_bf16_to_double(src[i]);
            uint8_t s = mx_scale_byte(g, MX_GROUP);
            scale[r * ng + k] = s;
            for (int i = 0; i < MX_GROUP; ++i)
                q[r * cols + k * MX_GROUP + i] = mx_encode(g[i], s);
        }
    }
}

/* The adapter's literal route [MX-adapter item 1]: zero-pad rows up to a
 * multiple of 32, quantize row-wise, crop back to the real rows. */
int orc_mxfp8_quantize_padcrop(const uint16_t *x, int64_t rows, int64_t cols,
                               uint8_t *q, uint8_t *scale)
{
    int64_t prows = (rows + 31) / 32 * 32;
    int64_t ng = cols / MX_GROUP;
    uint16_t *xp = (uint16_t *)calloc((size_t)(prows * cols), sizeof(uint16_t));
    uint8_t *qp = (uint8_t *)malloc((size_t)(prows * cols));
    uint8_t *sp = (uint8_t *)malloc((size_t)(prows * ng));
    if (!xp || !qp || !sp) { free(xp); free(qp); free(sp); return -1; }
    memcpy(xp, x, (size_t)(rows * cols) * sizeof(uint16_t));
    orc_mxfp8_quantize_rowwise(xp, prows, cols, qp, sp);
    memcpy(q, qp, (size_t)(rows * cols));
    memcpy(scale, sp, (size_t)(rows * ng));
    free(xp); free(qp); free(sp);
    return 0;
}

/* Column-wise MXFP8: groups of 32 consecutive rows within each column.
 * q keeps x's [rows, cols] layout; scale is [ceil(rows/32), cols] row-major.
 * A last group of fewer than 32 rows is quantized over the rows it has, which
 * equals zero-padding it (zeros never raise the amax). */
void orc_mxfp8_quantize_colwise(const uint16_t *x, int64_t rows, int64_t cols,
                                uint8_t *q, uint8_t *scale)
{
    double g[MX_GROUP];
    int64_t nrg = (rows + MX_GROUP - 1) / MX_GROUP;
    for (int64_t j = 0; j < nrg; ++j) {
        int64_t r0 = j * MX_GROUP;
        int n = (int)((rows - r0) < MX_GROUP ? (rows - r0) : MX_GROUP);
        for (int64_t c = 0; c < cols; ++c) {
            for (int i = 0; i < n; ++i) g[i] = orc_bf16_to_double(x[(r0 + i) * cols + c]);
            uint8_t s = mx_scale_byte(g, n);
            scale[j * cols + c] = s;
            for (int i = 0; i < n; ++i) q[(r0 + i) * cols + c] = mx_encode(g[i], s);
        }
    }
}

/* Column-wise MXFP8 in the transposed layout a backward-pass GEMM reads: the
 * groups and codes of orc_mxfp8_quantize_colwise, stored as qt [cols, rows]
 * (qt[c * rows + r] is the code of x[r, c]) and st [cols, ceil(rows/32)]
 * (st[c * ceil(rows/32) + j] is the scale of rows 32j.. of column c). */
int orc_mxfp8_quantize_colwise_t(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *qt,
                                 uint8_t *st)
{
    int64_t nrg = (rows + MX_GROUP - 1) / MX_GROUP;
    uint8_t *q = (uint8_t *)malloc((size_t)(rows * cols));
    uint8_t *s = (uint8_t *)malloc((size_t)(nrg * cols));
    if (!q || !s) { free(q); free(s); return -1; }
    orc_mxfp8_quantize_colwise(x, rows, cols, q, s);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) qt[c * rows + r] = q[r * cols + c];
    for (int64_t j = 0; j < nrg; ++j)
        for (int64_t c = 0; c < cols; ++c) st[c * nrg + j] = s[j * cols + c];
    free(q); free(s);
    return 0;
}

/* MXFP8 dequantization: bf16_RNE(E4M3(q) * 2^(s-127)).  The product is exact
 * in double; NaN (code or scale 0xFF) gives the quiet NaN with the code's
 * sign.  axis 1: scale [rows, cols/32]; axis 0: scale [ceil(rows/32), cols]. */
void orc_mxfp8_dequantize(const uint8_t *q, const uint8_t *scale, int64_t rows,
                          int64_t cols, int axis, uint16_t *out)
{
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c) {
            uint8_t code = q[r * cols + c];
            uint8_t s = axis == 1 ? scale[r * (cols / MX_GROUP) + c / MX_GROUP]
                                  : scale[(r / MX_GROUP) * cols + c];
            double v = orc_e4m3_to_double(code);
            uint16_t o;
            if (isnan(v) || s == 0xFF)
                o = (uint16_t)((code & 0x80) ? 0xFFC0 : 0x7FC0);
            else
                o = orc_double_to_bf16(v * orc_e8m0_to_double(s));
            out[r * cols + c] = o;
        }
    }
}

/* Fake quantization (simulate-QAT) [V4-mxfp4]: quantize, then dequantize
 * back to bf16, along `axis` (1 = row-wise groups, 0 = column-wise). */
int orc_mxfp8_fake_quant(const uint16_t *x, int64_t rows, int64_t cols, int axis,
                         uint16_t *out)
{
    int64_t ns = axis == 1 ? rows * (cols / MX_GROUP)
                           : ((rows + MX_GROUP - 1) / MX_GROUP) * cols;
    uint8_t *q = (uint8_t *)malloc((size_t)(rows * cols));
    uint8_t *s = (uint8_t *)malloc((size_t)ns);
    if (!q || !s) { free(q); free(s); return -1; }
    if (axis == 1) orc_mxfp8_quantize_rowwise(x, rows, cols, q, s);
    else orc_mxfp8_quantize_colwise(x, rows, cols, q, s);
    orc_mxfp8_dequantize(q, s, rows, cols, axis, out);
    free(q); free(s);
    return 0;
}

/* Grouped row-wise quantization: each tensor independently, in order. */
void orc_mxfp8_quantize_rowwise_many(int32_t n, const uint16_t *const *xs,
                                     const int64_t *rows, const int64_t *cols,
                                     uint8_t *const *qs, uint8_t *const *ss)
{
    for (int32_t t = 0; t < n; ++t)
        orc_mxfp8_quantize_rowwise(xs[t], rows[t], cols[t], qs[t], ss[t]);
}

/* ------------------------------------------------------------------------ */
/* MXFP4: groups of 32, one E8M0 scale, E2M1 elements [V4-mxfp4]             */
/* ------------------------------------------------------------------------ */

/* Shared scale byte [OCP-MX]: 2^(floor(log2 amax) - 2) -- 4 = 2^2 is E2M1's
 * largest power of two -- as an E8M0 byte clamped at 0 (2^-127); an all-zero
 * group gets 0; a group holding NaN or Inf gets 0xFF. */
static uint8_t mx4_scale_byte(const double *vals, int n)
{
    double amax = 0.0;
    for (int i = 0; i < n; ++i) {
        double a = fabs(vals[i]);
        if (!isfinite(a)) return 0xFF;
        if (a > amax) amax = a;
    }
    if (amax == 0.0) return 0;
    int E = floor_log2(amax) - 2;           /* 2 = exponent of 4, E2M1's largest power of two */
    if (E < -127) E = -127;
    if (E > 127) E = 127;
    return (uint8_t)(E + 127);
}

/* Row-wise MXFP4 (the simulate-QAT groups of 32 along the last dimension
 * [V4-mxfp4]): x [rows, cols] bf16, cols % 32 == 0.  Element nibble =
 * E2M1(x / 2^(s-127)) (exact quotient, RNE, saturating at +-6, sign kept);
 * a NaN group (scale 0xFF) has nibbles 0x7 | sign, E2M1 having no NaN.
 * q [rows, cols/2]: element 2j in the low nibble of byte j, element 2j+1 in
 * the high nibble (`float4_e2m1fn_x2`); scale [rows, cols/32] E8M0. */
void orc_mxfp4_quantize(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q,
                        uint8_t *scale)
{
    double g[MX_GROUP];
    uint8_t nib[MX_GROUP];
    int64_t ng = cols / MX_GROUP;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t k = 0; k < ng; ++k) {
            const uint16_t *src = x + r * cols + k * MX_GROUP;
            for (int i = 0; i < MX_GROUP; ++i) g[i] = orc_bf16_to_double(src[i]);
            uint8_t s = mx4_scale_byte(g, MX_GROUP);
            scale[r * ng + k] = s;
            for (int i = 0; i < MX_GROUP; ++i)
                nib[i] = s == 0xFF ? (uint8_t)((signbit(g[i]) ? 0x8 : 0) | 0x7)
                                   : orc_double_to_e2m1(ldexp(g[i], 127 - (int)s));
            for (int i = 0; i < MX_GROUP; i += 2)
                q[r * (cols / 2) + (k * MX_GROUP + i) / 2] = (uint8_t)(nib[i] | (nib[i + 1] << 4));
        }
    }
}

/* MXFP4 dequantization: bf16_RNE(E2M1(nibble) * 2^(s-127)), the product exact
 * in double; scale 0xFF gives the quiet NaN with the nibble's sign. */
void orc_mxfp4_dequantize(const uint8_t *q, const uint8_t *scale, int64_t rows, int64_t cols,
                          uint16_t *out)
{
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c) {
            uint8_t byte = q[r * (cols / 2) + c / 2];
            uint8_t nib = (c % 2 == 0) ? (byte & 0xF) : (byte >> 4);
            uint8_t s = scale[r * (cols / MX_GROUP) + c / MX_GROUP];
            uint16_t o;
            if (s == 0xFF)
                o = (uint16_t)((nib & 0x8) ? 0xFFC0 : 0x7FC0);
            else
                o = orc_double_to_bf16(orc_e2m1_to_double(nib) * orc_e8m0_to_double(s));
            out[r * cols + c] = o;
        }
    }
}

/* MXFP4 fake quantization (`mxfp4_simulate_qat(x, 32)` [V4-mxfp4, compressor
 * review]): quantize row-wise, then dequantize back to bf16. */
int orc_mxfp4_fake_quant(const uint16_t *x, int64_t rows, int64_t cols, uint16_t *out)
{
    uint8_t *q = (uint8_t *)malloc((size_t)(rows * cols / 2));
    uint8_t *s = (uint8_t *)malloc((size_t)(rows * (cols / MX_GROUP)));
    if (!q || !s) { free(q); free(s); return -1; }
    orc_mxfp4_quantize(x, rows, cols, q, s);
    orc_mxfp4_dequantize(q, s, rows, cols, out);
    free(q); free(s);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Block-FP8: blk x blk tiles, fp32 absmax scale [xorl, "What looked solid"] */
/* ------------------------------------------------------------------------ */

/* S = fl32(amax / 448); q = E4M3(fl32(x / S)).  Edge tiles use their valid
 * region.  A zero tile stores S = 0 and divides by 1 (all codes +-0).  A tile
 * holding NaN or Inf stores S = NaN and every code is NaN with x's sign.
 * scale is [ceil(rows/blk), ceil(cols/blk)] fp32 row-major. */
void orc_blockfp8_quantize_rect(const uint16_t *x, int64_t rows, int64_t cols, int32_t br,
                                int32_t bc, uint8_t *q, float *scale)
{
    int64_t tr = (rows + br - 1) / br, tc = (cols + bc - 1) / bc;
    for (int64_t bi = 0; bi < tr; ++bi) {
        for (int64_t bj = 0; bj < tc; ++bj) {
            int64_t r0 = bi * br, c0 = bj * bc;
            int64_t r1 = r0 + br < rows ? r0 + br : rows;
            int64_t c1 = c0 + bc < cols ? c0 + bc : cols;
            double amax = 0.0;
            int nonfinite = 0;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c) {
                    double a = fabs(orc_bf16_to_double(x[r * cols + c]));
                    if (!isfinite(a)) nonfinite = 1;
                    else if (a > amax) amax = a;
                }
            float S, divisor;
            if (nonfinite) {
                S = NAN;
                divisor = NAN;
            } else {
                S = (float)amax / 448.0f;       /* one IEEE fp32 division */
                divisor = (amax == 0.0) ? 1.0f : S;
            }
            scale[bi * tc + bj] = S;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c) {
                    uint16_t xb = x[r * cols + c];
                    uint8_t code;
                    if (nonfinite) {
                        code = (uint8_t)(((xb >> 8) & 0x80) | 0x7F);
                    } else {
                        float xf = (float)orc_bf16_to_double(xb);
                        float t = xf / divisor;  /* one IEEE fp32 division */
                        code = orc_double_to_e4m3((double)t);
                    }
                    q[r * cols + c] = code;
                }
        }
    }
}

/* Square blk x blk tiles (the weight recipe). */
void orc_blockfp8_quantize(const uint16_t *x, int64_t rows, int64_t cols, int32_t blk,
                           uint8_t *q, float *scale)
{
    orc_blockfp8_quantize_rect(x, rows, cols, blk, blk, q, scale);
}

/* Block-FP8 dequantization: bf16_RNE(fl32(E4M3(q) * S)).  A NaN product
 * (NaN code, NaN scale, 0 * Inf) gives the quiet NaN with the code's sign. */
void orc_blockfp8_dequantize_rect(const uint8_t *q, const float *scale, int64_t rows,
                                  int64_t cols, int32_t br, int32_t bc, uint16_t *out)
{
    int64_t tc = (cols + bc - 1) / bc;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            uint8_t code = q[r * cols + c];
            float S = scale[(r / br) * tc + c / bc];
            float v = (float)orc_e4m3_to_double(code);
            float p = v * S;                    /* one IEEE fp32 multiplication */
            out[r * cols + c] = isnan(p) ? (uint16_t)((code & 0x80) ? 0xFFC0 : 0x7FC0)
                                         : orc_double_to_bf16((double)p);
        }
}

void orc_blockfp8_dequantize(const uint8_t *q, const float *scale, int64_t rows, int64_t cols,
                             int32_t blk, uint16_t *out)
{
    orc_blockfp8_dequantize_rect(q, scale, rows, cols, blk, blk, out);
}

/* Block-FP8 of a stack of G matrices [G, K, N] (grouped GEMM weights, the
 * `_gkn` variant [xorl, "What looked solid"]): every slice [K, N] is
 * quantized on its own with blk x blk tiles, so no tile crosses slices;
 * scale is [G, ceil(K/blk), ceil(N/blk)]. */
void orc_blockfp8_quantize_gkn(const uint16_t *x, int64_t G, int64_t K, int64_t N, int32_t blk,
                               uint8_t *q, float *scale)
{
    int64_t ts = ((K + blk - 1) / blk) * ((N + blk - 1) / blk);
    for (int64_t g = 0; g < G; ++g)
        orc_blockfp8_quantize(x + g * K * N, K, N, blk, q + g * K * N, scale + g * ts);
}

void orc_blockfp8_dequantize_gkn(const uint8_t *q, const float *scale, int64_t G, int64_t K,
                                 int64_t N, int32_t blk, uint16_t *out)
{
    int64_t ts = ((K + blk - 1) / blk) * ((N + blk - 1) / blk);
    for (int64_t g = 0; g < G; ++g)
        orc_blockfp8_dequantize(q + g * K * N, scale + g * ts, K, N, blk, out + g * K * N);
}

/* 1 x 128 blocks along each row: the activation recipe, and with
 * dequantization right after it the fake quantization fp8_simulate_qat(x,
 * 128) ["V4 mxfp4" (miles PR #1372), compressor review; fp32 scale storage per
 * the PR description].  scale is [rows, ceil(cols/128)]. */
int orc_blockfp8_fake_quant_1x128(const uint16_t *x, int64_t rows, int64_t cols, uint16_t *out)
{
    int64_t tc = (cols + 127) / 128;
    uint8_t *q = (uint8_t *)malloc((size_t)(rows * cols));
    float *S = (float *)malloc((size_t)(rows * tc) * sizeof(float));
    if (!q || !S) { free(q); free(S); return -1; }
    orc_blockfp8_quantize_rect(x, rows, cols, 1, 128, q, S);
    orc_blockfp8_dequantize_rect(q, S, rows, cols, 1, 128, out);
    free(q); free(S);
    return 0;
}

/* FP8 block -> BF16 -> MXFP8 re-quantization [MX-adapter, 实现拆解 item 5:
 * the FP8->BF16->MXFP8 checkpoint conversion]: dequantize a block-FP8 tensor
 * (codes q [rows, cols], fp32 scales [ceil(rows/blk), ceil(cols/blk)]) to
 * bf16 as orc_blockfp8_dequantize does, then quantize that bf16 tensor
 * row-wise to MXFP8.  cols % 32 == 0. */
int orc_blockfp8_to_mxfp8(const uint8_t *q, const float *scale, int64_t rows, int64_t cols,
                          int32_t blk, uint8_t *q8, uint8_t *scale8)
{
    uint16_t *bf = (uint16_t *)malloc((size_t)(rows * cols) * sizeof(uint16_t));
    if (!bf) return -1;
    orc_blockfp8_dequantize(q, scale, rows, cols, blk, bf);
    orc_mxfp8_quantize_rowwise(bf, rows, cols, q8, scale8);
    free(bf);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* NVFP4: global fp32 scale, per-16 E4M3 block scale, E2M1 elements          */
/* [xorl, "What looked solid"; V4-mxfp4, review of fp4_act_quant]            */
/* ------------------------------------------------------------------------ */

#define NV_BLOCK 16

/* Steps, in order:
 *   A   = max |x| over the tensor (exact)
 *   g   = fl32(A / 2688)                      2688 = 448 * 6
 *   per block of 16 along a row, amax b:
 *   d   = fl32(6 * g)
 *   s   = E4M3(fl32(b / d))                   saturates at 448 (the clamp)
 *   eff = fl32(E4M3(s) * g)                   effective scale
 *   q   = E2M1(fl32(x / eff)), or sign-only zero when eff == 0 (the guard)
 * Element 2j goes to the low nibble of byte j, 2j+1 to the high nibble.
 * q_packed [rows, cols/2], s [rows, cols/16], global_scale[0] = g.
 * A tensor holding NaN or Inf: g = NaN, every scale byte 0x7F, every nibble
 * 0x7 | sign. */
/* max |x| over n bf16 values, and whether any of them is NaN or Inf. */
static void nv_amax(const uint16_t *x, int64_t n, double *A, int *nonfinite)
{
    for (int64_t i = 0; i < n; ++i) {
        double a = fabs(orc_bf16_to_double(x[i]));
        if (!isfinite(a)) *nonfinite = 1;
        else if (a > *A) *A = a;
    }
}

/* The global scale g of an amax A (NaN when the values held NaN or Inf). */
static float nv_global(double A, int nonfinite)
{
    if (nonfinite) return NAN;
    float g = (float)A / 2688.0f;
    return g;
}

/* The per-block steps of one tensor under a given global scale g. */
static void nv_quantize_given(const uint16_t *x, int64_t rows, int64_t cols, float g,
                              int nonfinite, uint8_t *q_packed, uint8_t *s_e4m3)
{
    int64_t nb = cols / NV_BLOCK;
    if (nonfinite) {
        for (int64_t i = 0; i < rows * nb; ++i) s_e4m3[i] = 0x7F;
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t c = 0; c < cols; c += 2) {
                uint8_t lo = (uint8_t)(((x[r * cols + c] >> 12) & 0x8) | 0x7);
                uint8_t hi = (uint8_t)(((x[r * cols + c + 1] >> 12) & 0x8) | 0x7);
                q_packed[r * (cols / 2) + c / 2] = (uint8_t)(lo | (hi << 4));
            }
        return;
    }
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t k = 0; k < nb; ++k) {
            const uint16_t *src = x + r * cols + k * NV_BLOCK;
            double b = 0.0;
            for (int i = 0; i < NV_BLOCK; ++i) {
                double a = fabs(orc_bf16_to_double(src[i]));
                if (a > b) b = a;
            }
            uint8_t s;
            if (g == 0.0f) {
                s = 0;
            } else {
                float d = 6.0f * g;
                float ratio = (float)b / d;
                s = orc_double_to_e4m3((double)ratio);
            }
            s_e4m3[r * nb + k] = s;
            float eff = (float)orc_e4m3_to_double(s) * g;
            uint8_t nib[NV_BLOCK];
            for (int i = 0; i < NV_BLOCK; ++i) {
                uint16_t xb = src[i];
                if (eff == 0.0f) {
                    nib[i] = (uint8_t)((xb >> 12) & 0x8);
                } else {
                    float t = (float)orc_bf16_to_double(xb) / eff;
                    nib[i] = orc_double_to_e2m1((double)t);
                }
            }
            for (int i = 0; i < NV_BLOCK; i += 2)
                q_packed[r * (cols / 2) + (k * NV_BLOCK + i) / 2] =
                    (uint8_t)(nib[i] | (nib[i + 1] << 4));
        }
    }
}

void orc_nvfp4_quantize(const uint16_t *x, int64_t rows, int64_t cols,
                        uint8_t *q_packed, uint8_t *s_e4m3, float *global_scale)
{
    double A = 0.0;
    int nonfinite = 0;
    nv_amax(x, rows * cols, &A, &nonfinite);
    float g = nv_global(A, nonfinite);
    global_scale[0] = g;
    nv_quantize_given(x, rows, cols, g, nonfinite, q_packed, s_e4m3);
}

/* NVFP4 of several tensors whose global scale is shared within caller-given
 * scale groups: tensor i belongs to group[i] in [0, n_groups); A of a group is
 * the max |x| over all its tensors (NaN/Inf in any of them makes the whole
 * group non-finite), g = fl32(A / 2688) is written to gs[group], and every
 * member is quantized with that g.  A group with no member gets g = 0.  This
 * covers the two gate/up conventions of a fused gated-MoE weight [xorl PR #30,
 * deep review item 3]: a global scale per half (gate and up in separate
 * groups, the QAT form) and one shared weight_scale_2 (gate and up in one
 * group, the export form). */
int orc_nvfp4_quantize_grouped(int32_t n, const uint16_t *const *xs, const int64_t *rows,
                               const int64_t *cols, const int32_t *group, int32_t n_groups,
                               uint8_t *const *qs, uint8_t *const *ss, float *gs)
{
    double *A = (double *)calloc((size_t)n_groups, sizeof(double));
    int *nf = (int *)calloc((size_t)n_groups, sizeof(int));
    if (!A || !nf) { free(A); free(nf); return -1; }
    for (int32_t i = 0; i < n; ++i) nv_amax(xs[i], rows[i] * cols[i], &A[group[i]], &nf[group[i]]);
    for (int32_t j = 0; j < n_groups; ++j) gs[j] = nv_global(A[j], nf[j]);
    for (int32_t i = 0; i < n; ++i)
        nv_quantize_given(xs[i], rows[i], cols[i], gs[group[i]], nf[group[i]], qs[i], ss[i]);
    free(A); free(nf);
    return 0;
}

/* NVFP4 dequantization: bf16_RNE(fl32(E2M1(q) * eff)), eff = fl32(E4M3(s) * g).
 * A NaN product gives the quiet NaN with the nibble's sign. */
void orc_nvfp4_dequantize(const uint8_t *q_packed, const uint8_t *s_e4m3,
                          const float *global_scale, int64_t rows, int64_t cols,
                          uint16_t *out)
{
    float g = global_scale[0];
    int64_t nb = cols / NV_BLOCK;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            uint8_t byte = q_packed[r * (cols / 2) + c / 2];
            uint8_t nib = (c & 1) ? (byte >> 4) : (byte & 0xF);
            float eff = (float)orc_e4m3_to_double(s_e4m3[r * nb + c / NV_BLOCK]) * g;
            float v = (float)orc_e2m1_to_double(nib);
            float p = v * eff;
            out[r * cols + c] = isnan(p) ? (uint16_t)((nib & 0x8) ? 0xFFC0 : 0x7FC0)
                                         : orc_double_to_bf16((double)p);
        }
}
