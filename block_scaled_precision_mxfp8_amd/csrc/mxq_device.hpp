// mxq_device.hpp -- device-side building blocks shared by the gfx950 kernels.
//
// Number formats (bit layouts as the OCP 8-bit floating point and OCP
// microscaling definitions give them; the pages name the formats):
//   bf16  1-8-7, bias 127            E4M3 ("fn") 1-4-3, bias 7, max 448 = 0x7E,
//   E8M0  2^(b-127), 0xFF = NaN       S.1111.111 = NaN, subnormals m * 2^-9
//   E2M1  1-2-1, bias 1, magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}
//
// Everything here is integer or exactly-rounded fp32 arithmetic: no fast-math
// and no flush of denormals (the library is built with
// -fno-gpu-flush-denormals-to-zero; the rebias tricks below rely on fp32
// subnormals being kept).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mxq {

// Compile-time loop: f(std::integral_constant<int, I>) for I = B, B+S, ... < E.
// Keeps register-array indices static where a #pragma unroll could give up on
// a large body (and fall back to scratch memory for the array).
template <int B, int E, int S, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + S, E, S>(f);
    }
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// amax of bf16 data: magnitude bit patterns (bits & 0x7FFF) order exactly like
// the magnitudes they encode, with Inf (0x7F80) and NaN (> 0x7F80) on top, so
// the group max is an unsigned integer max -- two elements per v_pk_max_u16.
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

__device__ __forceinline__ uint32_t mag2(uint32_t w) { return w & 0x7FFF7FFFu; }

// Max magnitude bits of the 8 bf16 in one 16-byte vector.
__device__ __forceinline__ uint32_t amax8(const uint4 v)
{
    uint32_t m = pk_max_u16(pk_max_u16(mag2(v.x), mag2(v.y)), pk_max_u16(mag2(v.z), mag2(v.w)));
    return max(m & 0xFFFFu, m >> 16);
}

// DPP quad permutations: [1,0,3,2] swaps neighbours, [2,3,0,1] swaps pairs.
__device__ __forceinline__ uint32_t dpp_swap1(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_swap2(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
}

// Row-block-per-XCD tile order for kernels whose per-row scale bytes are a
// short piece (16 or 32 bytes) of a 128-byte line per 512-column segment.
// Workgroup i runs on XCD i % 8.  Row block rb goes to XCD rb % 8, and its
// segments run there one after another, so each scale line is fetched (or
// written back) by one L2 instead of by several (HBM reads of MXFP4
// dequantization were +36% over the algorithmic bytes, NVFP4's +34%; the
// order gains 7-12% there on MI355X).  The
// grid has xcd_row_grid(nseg, nrb) workgroups; the padding ones (rb >= nrb)
// get false.
__host__ __device__ inline int64_t xcd_row_grid(int64_t nseg, int64_t nrb)
{
    return nseg * 8 * ((nrb + 7) / 8);
}
__device__ __forceinline__ bool xcd_row_tile(int64_t nseg, int64_t nrb, int64_t &seg, int64_t &rb)
{
    const int64_t k = blockIdx.x / 8;
    rb = (k / nseg) * 8 + blockIdx.x % 8;
    seg = k % nseg;
    return rb < nrb;
}

// A pointer read from memory (an entry of a grouped launch table) carries no
// address space, so the compiler would reach it with flat instructions, whose
// completion waits also cover LDS and scalar loads.  Table pointers always
// point to global memory; saying so gives global loads and stores.
template <class T>
__device__ __forceinline__ T *global_ptr(T *p)
{
    using G = __attribute__((address_space(1))) T *;
    return (T *)(G)__builtin_bit_cast(uintptr_t, p);
}

// Index of the last entry whose first tile is <= t, for strictly increasing
// starts[0..n) with starts[0] == 0 (grouped launches).  64-way search: each
// round, lane k samples starts[lo + k*step]; the sampled values increase with
// k, so the lanes that pass form a prefix and the highest one narrows the
// range to one step.  384 entries take two dependent reads instead of nine.
// The result is wave-uniform.
__device__ __forceinline__ int find_entry(const int32_t *__restrict__ starts, int n, int32_t t)
{
    const int lane = threadIdx.x & (kWave - 1);
    int lo = 0, m = n;  // invariant: starts[lo] <= t, and the answer is in [lo, lo + m)
    while (m > 1) {
        const int step = (m + kWave - 1) / kWave;
        const int off = lane * step;
        const bool le = off < m && starts[lo + off] <= t;
        const int last = 63 - __builtin_clzll(__ballot(le));  // lane 0 always passes
        lo += last * step;
        m = min(step, m - last * step);
    }
    return __builtin_amdgcn_readfirstlane(lo);
}

// Max over the 4 lanes of a quad (one 32-element row group = 4 lanes x 8).
__device__ __forceinline__ uint32_t quad_max(uint32_t v)
{
    v = max(v, dpp_swap1(v));
    return max(v, dpp_swap2(v));
}

// Max over all 64 lanes (result valid in every lane).
__device__ __forceinline__ uint32_t wave_max(uint32_t v)
{
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1)
        v = max(v, (uint32_t)__shfl_xor((int)v, off, kWave));
    return v;
}

// ---------------------------------------------------------------------------
// MX scale unit: the shared scale is 2^(floor(log2 amax) - 8) (the OCP
// microscaling rule with E4M3's largest power of two, 2^8).  For a bf16 amax
// floor(log2 amax) + 127 is its exponent field (0 for zero and subnormals,
// which the clamp at byte 0 = 2^-127 covers), so the E8M0 byte is
// max(expfield - 8, 0); a group with Inf/NaN (expfield 0xFF) gets 0xFF.
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t amag)
{
    uint32_t e = amag >> 7;
    return e >= 0xFFu ? 0xFFu : (e > 8u ? e - 8u : 0u);
}

// ---------------------------------------------------------------------------
// E4M3 encoding of bf16 inputs under an MX scale.
//
// w = |x| * 2^(127 - s) * 2^-120 = |x| * 2^(7 - s).  The extra 2^-120 moves
// E4M3's exponent bias (7) onto fp32's (127): an E4M3 normal value becomes an
// fp32 normal whose top bits (>> 20) are exactly the E4M3 code, and an E4M3
// subnormal m * 2^-9 becomes the fp32 subnormal m * 2^-129, whose bits >> 20
// are again m.  Round-to-nearest-even at bit 20 of the bit pattern is then the
// E4M3 rounding, carries into the exponent included; saturation is a clamp
// of the bit pattern at 448 * 2^-120 (0x07E00000).  w is exact because bf16
// has 8 significant bits: every w that can round to a nonzero code is at
// least 2^-130 with its lowest bit at or above 2^-137; anything smaller is
// below 2^-141 after ldexp's own rounding and encodes to 0 either way.
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t e4m3_mag_rebiased(uint32_t bits)
{
    bits = min(bits, 0x07E00000u);
    return (bits + 0x7FFFFu + ((bits >> 20) & 1u)) >> 20;
}

// Magnitude code of one bf16 held in the HIGH half of `hi` (low half zero).
__device__ __forceinline__ uint32_t e4m3_mag_bf16hi(uint32_t hi, int e)
{
    float w = __builtin_amdgcn_ldexpf(__builtin_fabsf(__uint_as_float(hi)), e);
    return e4m3_mag_rebiased(__float_as_uint(w));
}

// Sign bits of the 4 bf16 in (w0, w1), moved to bit 7 of bytes 0..3.
__device__ __forceinline__ uint32_t signs4(uint32_t w0, uint32_t w1)
{
    return __builtin_amdgcn_perm(w1, w0, 0x07050301u) & 0x80808080u;
}

// 4 E4M3 codes (bytes 0..3 <- elements 0..3 of (w0, w1)) in software, with a
// separate ldexp exponent e = 7 - s and NaN flag per element (column groups).
__device__ __forceinline__ uint32_t e4m3x4_col(uint32_t w0, uint32_t w1, int e0, int e1, int e2,
                                               int e3, bool n0, bool n1, bool n2, bool n3)
{
    uint32_t c0 = n0 ? 0x7Fu : e4m3_mag_bf16hi(w0 << 16, e0);
    uint32_t c1 = n1 ? 0x7Fu : e4m3_mag_bf16hi(w0 & 0xFFFF0000u, e1);
    uint32_t c2 = n2 ? 0x7Fu : e4m3_mag_bf16hi(w1 << 16, e2);
    uint32_t c3 = n3 ? 0x7Fu : e4m3_mag_bf16hi(w1 & 0xFFFF0000u, e3);
    return (c0 | (c1 << 8) | (c2 << 16) | (c3 << 24)) | signs4(w0, w1);
}

// ---------------------------------------------------------------------------
// Decoding and bf16 rounding
// ---------------------------------------------------------------------------

// fp32 -> bf16 round-to-nearest-even on the bit pattern (finite or Inf input;
// overflow carries into the exponent and gives Inf; the sign rides along).
__device__ __forceinline__ uint32_t bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 (finite or Inf) -> packed bf16 (a in the low half), RNE.  One
// v_cvt_pk_bf16_f32.  tests/test_gpu_converters.py runs it (and bf16_rne
// above) on every non-NaN fp32 pattern of both signs against the CPU
// reference's bf16 rounding: identical, subnormals kept, overflow to Inf.
// NaN inputs give a NaN of the same sign, but callers route NaN elsewhere.
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b)
{
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// E4M3 magnitude code (0..0x7E) as fp32: the rebias trick in reverse.
__device__ __forceinline__ float e4m3_mag_value(uint32_t mag)
{
    return __builtin_amdgcn_ldexpf(__uint_as_float(mag << 20), 120);
}

// MXFP8 element back to bf16: bf16_RNE(E4M3(code) * 2^(s - 127)).  The fp32
// product (code << 20 as a rebiased fp32, times 2^(s - 7)) is exact: E4M3 has
// 4 significant bits and the smallest product, 2^-136, is far above fp32's
// subnormal step.  NaN code or NaN scale -> 0x7FC0 with the code's sign.
__device__ __forceinline__ uint32_t mx_dequant1(uint32_t code, int e_dq, bool nan_scale)
{
    uint32_t mag = code & 0x7Fu;
    uint32_t b = bf16_rne(__builtin_amdgcn_ldexpf(__uint_as_float(mag << 20), e_dq));
    b = (nan_scale || mag == 0x7Fu) ? 0x7FC0u : b;
    return b | ((code & 0x80u) << 8);
}

// 4 codes (bytes of c) -> 4 bf16 in two dwords.
__device__ __forceinline__ uint2 mx_dequant4(uint32_t c, int e_dq, bool nan_scale)
{
    uint32_t b0 = mx_dequant1(c & 0xFFu, e_dq, nan_scale);
    uint32_t b1 = mx_dequant1((c >> 8) & 0xFFu, e_dq, nan_scale);
    uint32_t b2 = mx_dequant1((c >> 16) & 0xFFu, e_dq, nan_scale);
    uint32_t b3 = mx_dequant1(c >> 24, e_dq, nan_scale);
    return make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
}

// ---------------------------------------------------------------------------
// fp32 -> E4M3 / E2M1 (block-FP8 and NVFP4, whose quotients are full fp32)
// ---------------------------------------------------------------------------

// |t| (nonneg fp32, not NaN) -> E4M3 magnitude code, RNE, saturating at 0x7E.
// Normal range (t >= 2^-6): round the fp32 pattern at bit 20 and rebias the
// exponent by 120.  Subnormal range: adding 2^14 rounds t to a multiple of
// 2^-9 (fp32's step at 2^14), and the low bits of the sum count those steps.
// Swept with cvt_fp8x2_f32 in tests/test_gpu_converters.py.
__device__ __forceinline__ uint32_t e4m3_mag_from_f32(float t)
{
    uint32_t a = __float_as_uint(t);
    uint32_t nrm = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
    uint32_t sub = __float_as_uint(t + 16384.0f) - 0x46800000u;
    uint32_t c = a >= 0x3C800000u ? nrm : sub;
    return min(c, 0x7Eu);
}

// |t| (nonneg fp32, not NaN) -> E2M1 magnitude code 0..7, RNE, saturating.
// Normal range (t >= 1): round at fp32 bit 22 and rebias by 126.  Below 1:
// adding 2^22 rounds to a multiple of 0.5.  Swept with cvt_fp4x2_f32 in
// tests/test_gpu_converters.py.
__device__ __forceinline__ uint32_t e2m1_mag_from_f32(float t)
{
    uint32_t a = __float_as_uint(t);
    uint32_t nrm = ((a + 0x1FFFFFu + ((a >> 22) & 1u)) >> 22) - (126u << 1);
    uint32_t sub = __float_as_uint(t + 4194304.0f) - 0x4A800000u;
    uint32_t c = a >= 0x3F800000u ? nrm : sub;
    return min(c, 7u);
}

// E2M1 magnitude code (0..7) as fp32 (rebias by 2^126: code << 22 is the
// fp32 pattern of value * 2^-126, subnormal for 0.5).
__device__ __forceinline__ float e2m1_mag_value(uint32_t mag)
{
    return __builtin_amdgcn_ldexpf(__uint_as_float(mag << 22), 126);
}

// ---------------------------------------------------------------------------
// Hardware-assisted MX encode / decode (gfx950 scaled converts).
//
// v_cvt_scalef32_pk_fp8_bf16 converts two bf16 to E4M3 as RNE(x / scale),
// exactly for every |x / scale| <= 464 (E4M3 subnormals, signed zeros and
// bf16 subnormal inputs included); above that it returns the NaN code
// instead of saturating.  Clamping each magnitude to 448 * scale first
// (exact: a bf16 value) therefore makes it the saturating RNE encoder of the
// method.  tests/test_gpu_parity.py runs every (bf16 value, reachable scale
// byte) pair through the row kernels (test_rowwise_every_value_every_scale)
// and the column kernels (test_colwise_edge_values) against the CPU reference.
// ---------------------------------------------------------------------------

typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

// bf16 bits of 448 * 2^(s - 127) (exponent field s + 8, fraction 0.75).
__device__ __forceinline__ uint32_t mx_limit_bf16(uint32_t s) { return ((s + 8u) << 7) | 0x60u; }

// 2^(s - 127) as fp32 (s <= 254; s = 0 is the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s)
{
    return __uint_as_float(s ? (s << 23) : 0x00400000u);
}

// Clamp both bf16 magnitudes of w to the packed limit lim2, keeping signs.
__device__ __forceinline__ uint32_t clamp_mag2(uint32_t w, uint32_t lim2)
{
    return (w & 0x80008000u) | pk_min_u16(w & 0x7FFF7FFFu, lim2);
}

// Two E4M3 codes of the (already clamped) bf16 pair w into half `kHi` of old.
template <bool kHi>
__device__ __forceinline__ uint32_t cvt_fp8x2(uint32_t old, uint32_t w, float scale)
{
    const i16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(
        __builtin_bit_cast(i16x2, old), __builtin_bit_cast(bf16x2, w), scale, kHi);
    return __builtin_bit_cast(uint32_t, r);
}

// 4 codes of one row group (finite scale byte s): bytes 0..3 <- (w0.lo, w0.hi, w1.lo, w1.hi).
__device__ __forceinline__ uint32_t e4m3x4_row_hw(uint32_t w0, uint32_t w1, uint32_t lim2,
                                                  float scale)
{
    return cvt_fp8x2<true>(cvt_fp8x2<false>(0u, clamp_mag2(w0, lim2), scale),
                           clamp_mag2(w1, lim2), scale);
}

// Row-wise MXFP8 of one lane's 8 bf16 when its lane quad holds one group of
// 32: the group's scale byte (the same in all 4 lanes), its fp32 value, and
// the lane's 8 E4M3 codes (elements 0..3 in c0).  A NaN/Inf group gives
// 0x7F with each element's sign.
struct MxRow8 {
    uint32_t s;
    float sf;
    uint32_t c0, c1;
};

__device__ __forceinline__ MxRow8 mx_row_encode8(uint4 v)
{
    MxRow8 m;
    m.s = mx_scale_byte(quad_max(amax8(v)));
    const uint32_t lim = mx_limit_bf16(m.s);
    const uint32_t lim2 = lim | (lim << 16);
    m.sf = e8m0_to_f32(m.s);
    m.c0 = e4m3x4_row_hw(v.x, v.y, lim2, m.sf);
    m.c1 = e4m3x4_row_hw(v.z, v.w, lim2, m.sf);
    if (m.s == 0xFFu) {
        m.c0 = 0x7F7F7F7Fu | signs4(v.x, v.y);
        m.c1 = 0x7F7F7F7Fu | signs4(v.z, v.w);
    }
    return m;
}

// Column groups: the pair fed to one convert must share a scale, so it is
// made of the same column in two consecutive rows.  For dword k (columns 2k,
// 2k+1) of rows i and i+1 (already clamped): returns bytes
// [(i,2k), (i+1,2k), (i,2k+1), (i+1,2k+1)].
__device__ __forceinline__ uint32_t e4m3_colpair_hw(uint32_t a, uint32_t b, float s_lo, float s_hi)
{
    const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x05040100u);  // (a.lo, b.lo)
    const uint32_t hi = __builtin_amdgcn_perm(b, a, 0x07060302u);  // (a.hi, b.hi)
    return cvt_fp8x2<true>(cvt_fp8x2<false>(0u, lo, s_lo), hi, s_hi);
}

// MX dequantization with v_cvt_scalef32_pk_bf16_fp8 (E4M3 * scale -> bf16):
// exact for every code and every E8M0 scale 2^-127..2^127 -- bf16 subnormal
// results and overflow to Inf included -- except the NaN codes, which it
// turns into 0xFFC0 whatever their sign; callers route groups that can hold
// NaN to mx_dequant4.  tests/test_gpu_parity.py
// (test_dequant_hw_path_all_finite_pairs) runs every finite code with every
// scale byte through this path against the CPU reference.
__device__ __forceinline__ uint2 mx_dequant4_hw(uint32_t c, float scale)
{
    const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, scale, false);
    const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, scale, true);
    return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// ---------------------------------------------------------------------------
// fp32 quotients and fp32 -> E4M3 / E2M1 with the hardware converts
// ---------------------------------------------------------------------------

// x / d for d > 0 from y = RN(1/d) with two FMAs (Markstein's correction
// step), the sign taken from x (the correction alone turns -0 into +0).
// tests/markstein_check.c replays these fp32 operations on the host against
// IEEE division over the domain the callers use -- d in [2^-60, 2^60],
// quotients of magnitude <= 512 -- on every bf16 significand of x against
// every fp32 significand of d in one divisor binade and every 61st in seven
// others, at ten quotient binades, and on every bf16 pattern of x (zeros,
// subnormals, both signs) against divisors at 2^-60, 2^-30, 1, 2^30, 2^59
// times every 61st significand and 2^60 (4.7e10 cases with --runslow, a
// sample by default): identical except quotients below 2^-30, where both stay
// below 2^-30 with the same sign -- far under every rounding threshold of
// E4M3 and E2M1.  Outside that domain callers divide.
__device__ __forceinline__ float div_markstein(float x, float d, float y)
{
    const float q0 = x * y;
    const float r = __builtin_fmaf(-q0, d, x);
    return __builtin_copysignf(__builtin_fmaf(r, y, q0), x);
}

__device__ __forceinline__ bool markstein_ok(float d)
{
    return d >= 0x1p-60f && d <= 0x1p60f;
}

// Two fp32 -> E4M3 codes (RNE, saturating) into half kHi of old.
// v_cvt_pk_fp8_f32 gives the NaN code above 448, hence the clamp; with it,
// tests/test_gpu_converters.py finds both halves equal to the CPU
// reference's E4M3 encoding for every fp32 in [-512, 512] and every 4099th
// pattern up to +-Inf (the quotients x / S stay within 448 (1 + 2^-23)).
template <bool kHi>
__device__ __forceinline__ uint32_t cvt_fp8x2_f32(uint32_t old, float a, float b)
{
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, kHi);
}

// Two fp32 -> E2M1 nibbles (RNE, saturating at +-6; lo nibble <- a) into byte
// kByte of old.  tests/test_gpu_converters.py finds v_cvt_scalef32_pk_fp4_f32
// (scale 1) equal to the CPU reference's E2M1 encoding in all four byte
// slots for every fp32 in [-16, 16] and every 4099th pattern up to +-Inf,
// saturation included (the quotients x / eff stay below 9).
template <int kByte>
__device__ __forceinline__ uint32_t cvt_fp4x2_f32(uint32_t old, float a, float b)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, kByte);
}

// ---------------------------------------------------------------------------
// Global memory access with an optional non-temporal (streaming) hint: every
// byte here is touched once, so keeping it out of the caches' working set
// can only help.  kNT selects the hinted form.
// ---------------------------------------------------------------------------
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

template <bool kNT>
__device__ __forceinline__ uint4 ld16(const void *p)
{
    if (kNT) {
        const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    }
    return *reinterpret_cast<const uint4 *>(p);
}

template <bool kNT>
__device__ __forceinline__ uint2 ld8(const void *p)
{
    if (kNT) {
        const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
        return make_uint2(v.x, v.y);
    }
    return *reinterpret_cast<const uint2 *>(p);
}

template <bool kNT>
__device__ __forceinline__ uint32_t ld4(const void *p)
{
    if (kNT) return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
    return *reinterpret_cast<const uint32_t *>(p);
}

template <bool kNT>
__device__ __forceinline__ void st16(void *p, uint4 v)
{
    if (kNT) {
        const u32x4_t w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t *>(p));
    } else {
        *reinterpret_cast<uint4 *>(p) = v;
    }
}

template <bool kNT>
__device__ __forceinline__ void st8(void *p, uint2 v)
{
    if (kNT) {
        const u32x2_t w = {v.x, v.y};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t *>(p));
    } else {
        *reinterpret_cast<uint2 *>(p) = v;
    }
}

template <bool kNT>
__device__ __forceinline__ void st4(void *p, uint32_t v)
{
    if (kNT) __builtin_nontemporal_store(v, reinterpret_cast<uint32_t *>(p));
    else *reinterpret_cast<uint32_t *>(p) = v;
}

// Wave-uniform OR of a lane predicate.
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// bf16 bits in the low half of u -> fp32 value.
// ---------------------------------------------------------------------------
// MXFP4: groups of 32 share an E8M0 scale 2^(floor(log2 amax) - 2) (E2M1's
// largest power of two is 4 = 2^2); elements are E2M1 nibbles, element 2j in
// the low nibble of byte j.
// ---------------------------------------------------------------------------

// Scale byte from the group's max magnitude bits: max(expfield - 2, 0), 0xFF
// for Inf/NaN.
__device__ __forceinline__ uint32_t mx4_scale_byte(uint32_t amag)
{
    uint32_t e = amag >> 7;
    return e >= 0xFFu ? 0xFFu : (e > 2u ? e - 2u : 0u);
}

// 8 bf16 (v.x holds elements 0, 1; v.w elements 6, 7) -> 8 E2M1 nibbles of
// x / sf.  v_cvt_scalef32_pk_fp4_bf16 computes exactly the round-to-nearest-
// even, +-6-saturating, sign-keeping nibble of x / sf for every bf16 x and
// power-of-two sf from 2^-127 to 2^127; tests/test_gpu_mxfp4.py runs every
// (bf16 value, reachable scale byte) pair through the MXFP4 kernel against
// the CPU reference.
__device__ __forceinline__ uint32_t e2m1x8_hw(uint4 v, float sf)
{
    uint32_t o = 0u;
    o = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(o, __builtin_bit_cast(bf16x2, v.x), sf, 0);
    o = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(o, __builtin_bit_cast(bf16x2, v.y), sf, 1);
    o = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(o, __builtin_bit_cast(bf16x2, v.z), sf, 2);
    o = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(o, __builtin_bit_cast(bf16x2, v.w), sf, 3);
    return o;
}

// Nibbles of a NaN group: 0x7 with each element's sign (E2M1 has no NaN).
__device__ __forceinline__ uint32_t e2m1x8_nan(uint4 v)
{
    // bf16 sign bits 15 / 31 of each word -> nibble sign bits 3 / 7 of its byte
    const uint32_t b0 = ((v.x >> 12) & 0x8u) | ((v.x >> 24) & 0x80u);
    const uint32_t b1 = ((v.y >> 12) & 0x8u) | ((v.y >> 24) & 0x80u);
    const uint32_t b2 = ((v.z >> 12) & 0x8u) | ((v.z >> 24) & 0x80u);
    const uint32_t b3 = ((v.w >> 12) & 0x8u) | ((v.w >> 24) & 0x80u);
    return 0x77777777u | b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

// Upper halves of two fp32 (a -> low half): their bf16 when the values are
// exactly representable in bf16.
__device__ __forceinline__ uint32_t bf16x2_exact(float a, float b)
{
    return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// 8 E2M1 nibbles -> 8 bf16 of nibble * sf for a finite power-of-two sf.  The
// nibble decodes exactly (v_cvt_scalef32_pk_f32_fp4, scale 1); its value
// (two significant bits) times sf >= 2^-127 is exact in fp32 and in bf16, or
// overflows to Inf in both, so the bf16 is the fp32's upper half.
__device__ __forceinline__ uint4 e2m1x8_dequant_hw(uint32_t packed, float sf)
{
    const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 0);
    const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 1);
    const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 2);
    const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 3);
    return make_uint4(bf16x2_exact(p0.x * sf, p0.y * sf), bf16x2_exact(p1.x * sf, p1.y * sf),
                      bf16x2_exact(p2.x * sf, p2.y * sf), bf16x2_exact(p3.x * sf, p3.y * sf));
}

// Dequantized NaN group: the quiet NaN 0x7FC0 with each nibble's sign.
__device__ __forceinline__ uint4 e2m1x8_dequant_nan(uint32_t packed)
{
    // nibble sign bits 8j+3 / 8j+7 -> bf16 sign bits 15 / 31 of word j
    const uint32_t w0 = ((packed << 12) & 0x8000u) | ((packed << 24) & 0x80000000u);
    const uint32_t w1 = ((packed << 4) & 0x8000u) | ((packed << 16) & 0x80000000u);
    const uint32_t w2 = ((packed >> 4) & 0x8000u) | ((packed << 8) & 0x80000000u);
    const uint32_t w3 = ((packed >> 12) & 0x8000u) | (packed & 0x80000000u);
    return make_uint4(0x7FC07FC0u | w0, 0x7FC07FC0u | w1, 0x7FC07FC0u | w2, 0x7FC07FC0u | w3);
}

__device__ __forceinline__ float bf16lo_to_f32(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

}  // namespace mxq
