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

namespace mxq {

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

// 4 E4M3 codes (bytes 0..3 <- elements 0..3 of (w0, w1)), with one ldexp
// exponent e = 7 - s for all four (a row group).  NaN group -> 0x7F | sign.
__device__ __forceinline__ uint32_t e4m3x4_row(uint32_t w0, uint32_t w1, int e, bool nan_group)
{
    uint32_t c0 = e4m3_mag_bf16hi(w0 << 16, e);
    uint32_t c1 = e4m3_mag_bf16hi(w0 & 0xFFFF0000u, e);
    uint32_t c2 = e4m3_mag_bf16hi(w1 << 16, e);
    uint32_t c3 = e4m3_mag_bf16hi(w1 & 0xFFFF0000u, e);
    uint32_t mags = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    mags = nan_group ? 0x7F7F7F7Fu : mags;
    return mags | signs4(w0, w1);
}

// Same with a separate exponent / NaN flag per element (column groups).
__device__ __forceinline__ uint32_t e4m3x4_col(uint32_t w0, uint32_t w1, const int e[4],
                                               const bool nan[4])
{
    uint32_t c0 = nan[0] ? 0x7Fu : e4m3_mag_bf16hi(w0 << 16, e[0]);
    uint32_t c1 = nan[1] ? 0x7Fu : e4m3_mag_bf16hi(w0 & 0xFFFF0000u, e[1]);
    uint32_t c2 = nan[2] ? 0x7Fu : e4m3_mag_bf16hi(w1 << 16, e[2]);
    uint32_t c3 = nan[3] ? 0x7Fu : e4m3_mag_bf16hi(w1 & 0xFFFF0000u, e[3]);
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
// adding 2^22 rounds to a multiple of 0.5.
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

// bf16 bits in the low half of u -> fp32 value.
__device__ __forceinline__ float bf16lo_to_f32(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

}  // namespace mxq
