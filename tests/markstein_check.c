/*
 * markstein_check.c -- host check of the division the block-FP8 and NVFP4
 * kernels use in place of an IEEE fp32 division (test infrastructure).
 *
 * The kernels compute x / d as
 *     y  = RN(1 / d)          (one IEEE division, per tile or per table entry)
 *     q0 = RN(x * y)
 *     r  = fma(-q0, d, x)     (exact remainder)
 *     q  = fma(r, y, q0), with the sign of x
 * (Markstein's correction step), and take it only when the divisor lies in
 * [2^-60, 2^60] and |x / d| <= 512 (their callers: bf16 x, block-FP8
 * x / S with S = amax / 448, NVFP4 b / (6g) and x / eff).  The claim their
 * comments make: in that domain the result is bit for bit the IEEE quotient
 * RN(x / d), except for quotients below 2^-30, where both are below 2^-30
 * with the same sign -- far under the first rounding threshold of E4M3
 * (2^-10) and of E2M1 (2^-2), so the encoded codes agree.
 *
 * This program replays exactly those fp32 operations on the host (SSE
 * arithmetic, FLT_EVAL_METHOD 0, fmaf correctly rounded, no flush to zero)
 * and checks the claim on:
 *   A  every bf16 significand of x, both signs x fp32 significands of d (in
 *      full mode all 2^23 in the divisor binade [1, 2) and every 61st in the
 *      others) x quotient binades around the E4M3/E2M1 rounding ranges x
 *      divisor binades across the domain, both edges included;
 *   B  every bf16 bit pattern x (both signs, zeros, subnormals) with
 *      |x| <= 512 d, against divisors 2^-60, 2^-30, 1, 2^30 and 2^59 times
 *      every 61st significand (full mode), and 2^60.
 * Quick mode takes every 409th (A) and 8191st (B) significand instead.
 * Usage: markstein_check quick|full.  Prints "markstein check: ok ..." and
 * exits 0 when the claim holds; prints the first counterexamples otherwise.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* The kernels' quotient, operation by operation (each line one fp32 rounding). */
static float markstein(float x, float d, float y)
{
    const float q0 = x * y;
    const float r = fmaf(-q0, d, x);
    return copysignf(fmaf(r, y, q0), x);
}

typedef struct { long long cases, tiny, bad; } counts;

static void check(float x, float d, float y, counts *c)
{
    const float want = x / d;               /* IEEE fp32 division, RNE */
    if (fabsf(want) > 512.0f) return;       /* outside the domain the kernels use */
    const float got = markstein(x, d, y);
    ++c->cases;
    if (u_of(got) == u_of(want)) return;
    /* allowed: both below 2^-30 in magnitude with the same sign */
    if (fabsf(want) < 0x1p-30f && fabsf(got) < 0x1p-30f && signbit(got) == signbit(want)) {
        ++c->tiny;
        return;
    }
    if (c->bad++ < 4) {
#pragma omp critical
        printf("MISMATCH x=%a d=%a: markstein %a (0x%08x) ieee %a (0x%08x)\n", x, d, got,
               u_of(got), want, u_of(want));
    }
}

int main(int argc, char **argv)
{
    const int full = argc > 1 && strcmp(argv[1], "full") == 0;
    /* full: every significand of d in the central divisor binade and every
     * 61st elsewhere (A), every 61st (B); quick: every 409th / 8191st */
    const uint32_t STRIDE_A = full ? 61u : 409u, STRIDE_A0 = full ? 1u : 409u;
    const uint32_t STRIDE_B = full ? 61u : 8191u;
    long long n_cases = 0, n_tiny = 0, n_bad = 0;

    /* A: x = (1 + mx/128) 2^(ed + k), d = (1 + md 2^-23) 2^ed, so x / d lies in
     * (2^(k-1), 2^(k+1)).  Quotient binades k cover E2M1 (k = -2..3) and E4M3
     * (k = -10..9) rounding ranges; divisor binades span the domain edges. */
    static const int ks[] = {-10, -6, -2, 0, 1, 2, 3, 5, 8, 9};
    static const int eds[] = {-60, -59, -40, -1, 0, 1, 40, 59};
    const int nk = sizeof ks / sizeof ks[0], ned = full ? sizeof eds / sizeof eds[0] : 4;
    static const int eds_quick[] = {-60, 0, 1, 59};
    for (int ie = 0; ie < ned; ++ie) {
        const int ed = full ? eds[ie] : eds_quick[ie];
        const int64_t stride = ed == 0 ? STRIDE_A0 : STRIDE_A;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : n_cases, n_tiny, n_bad)
        for (int64_t md = 0; md < (1 << 23); md += stride) {
            counts c = {0, 0, 0};
            const float d = ldexpf(1.0f + (float)md * 0x1p-23f, ed);
            const float y = 1.0f / d;
            for (int ik = 0; ik < nk; ++ik) {
                const int k = ks[ik];
                if (ed + k > 127 || ed + k < -126) continue;
                for (uint32_t mx = 0; mx < 128; ++mx) {
                    const float x = ldexpf(1.0f + (float)mx / 128.0f, ed + k);
                    check(x, d, y, &c);
                    check(-x, d, y, &c);
                }
            }
            n_cases += c.cases;
            n_tiny += c.tiny;
            n_bad += c.bad;
        }
    }
    /* B: every bf16 pattern with |x| <= 512 d */
    static const int ebs[] = {-60, -30, 0, 30, 59, 60};
    for (int ie = 0; ie < 6; ++ie) {
        /* 2^60 is the largest divisor taken: only its first significand */
        const int64_t end = ebs[ie] == 60 ? 1 : (1 << 23);
#pragma omp parallel for schedule(dynamic, 16) reduction(+ : n_cases, n_tiny, n_bad)
        for (int64_t md = 0; md < end; md += STRIDE_B) {
            counts c = {0, 0, 0};
            const float d = ldexpf(1.0f + (float)md * 0x1p-23f, ebs[ie]);
            const float y = 1.0f / d;
            const float lim = 512.0f * d;
            for (uint32_t b = 0; b < 0x10000u; ++b) {
                const float x = f_of(b << 16);
                if (!(fabsf(x) <= lim)) continue;   /* also drops NaN and Inf */
                check(x, d, y, &c);
            }
            n_cases += c.cases;
            n_tiny += c.tiny;
            n_bad += c.bad;
        }
    }
    if (n_bad) {
        printf("markstein check: FAILED %lld of %lld cases\n", n_bad, n_cases);
        return 1;
    }
    printf("markstein check: ok (%s), %lld cases, %lld equal-sign quotients below 2^-30\n",
           full ? "full" : "quick", n_cases, n_tiny);
    return 0;
}
