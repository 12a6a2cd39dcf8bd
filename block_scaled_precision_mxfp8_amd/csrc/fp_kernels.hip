// fp_kernels.hip -- block-FP8 and NVFP4 for gfx950: block-FP8 over 128 x 128
// tiles (also per slice of a [G, K, N] stack) and over 1 x 128 activation
// blocks with their fake quantization, the FP8 block -> BF16 -> MXFP8
// re-quantization in one pass, NVFP4 (global fp32 scale x per-16 E4M3 scale,
// E2M1 elements) single-tensor and grouped with shared global scales, and the
// dequantizers.
//
// Method (xorl PR #30 "Add FP8, NVFP4, and QARL training and export", deep
// review, "What looked solid"): block-FP8 absmax scaling; NVFP4 two-level
// global + FP8-block scaling with effective = block_scale * global_scale,
// clamped (the E4M3 block scale saturates at 448) and zero blocks guarded;
// FP4 output packed two per byte, [..., N/2] (miles PR #1372 "V4 mxfp4",
// review of fp4_act_quant).  The steps the method defines in fp32 -- the
// scale divisions, the element quotients and the dequantization products --
// give the correctly rounded fp32 result: an IEEE division, or a reciprocal
// with one FMA correction where that is proven to give the same quotient
// (div_markstein); no fast-math, denormals kept.
#include <math.h>

#include <mutex>

#include "launch.hpp"
#include "mxq_device.hpp"

namespace mxq {

constexpr int kBlk = 128;   // block-FP8 tile edge
constexpr int kSegNv = 512; // NVFP4 columns per wave segment (64 lanes x 8)
constexpr int kRowsNv = 32; // rows per workgroup tile of the grouped NVFP4 passes
// Rows per tile of the single-tensor NVFP4 encoding pass: 16 measured 9%
// faster than 32 there with cold inputs, while the grouped passes ran 3%
// slower with 16.
constexpr int kRowsNvQ = 16;
// Rows per workgroup tile of the NVFP4 dequantizer and the FP8 -> MXFP8 pass
// (4 waves x 4 rows).  With cold inputs, 16-row tiles measured 6-7% faster
// than 32-row ones, 8-row ones no faster.
constexpr int kRowsDq = 16;
// Rows per tile of the block-FP8 dequantizer and the 1 x 128 quantizer (4
// waves x 2 rows): 8 rows measured 5% (dequantize) and 4% (1 x 128
// simulate-QAT) faster than 16, which were 4-7% faster than 32.
constexpr int kRowsBq = 8;
static_assert(kBlk % kRowsDq == 0 && kBlk % kRowsBq == 0,
              "a tile's rows share one 128-row block row");
// Streaming (non-temporal) hints, chosen by measurement on MI355X with
// inputs read cold from HBM.  Outputs are written once.  Hinted 16-byte loads
// of x help block-FP8 (+3%); the dequantizers' 4- and 8-byte code loads do
// better unhinted (NVFP4: 4.3 -> 5.0 TB/s), while the FP8 -> MXFP8 pass's
// 8-byte code loads measured 2% faster hinted.  The single-tensor NVFP4 amax
// pass loads unhinted so that x can stay in the Infinity Cache for the
// encoding pass; the grouped amax pass streams (its tensors together far
// exceed that cache: 2.87 -> 2.72 ms on 256 MoE gate/up tensors).
constexpr bool kNTStore = true;
// Resident-workgroup cap for the single-tensor NVFP4 launches (amax pass,
// encoding pass, dequantize): 23 KiB of dynamic LDS that no kernel touches
// leaves room for 6 of their 4-wave workgroups in a CU's 160 KiB instead of
// the 8 their VGPRs allow.  MI355X, [8192, 8192] cold in HBM, variants
// interleaved in one process, medians of 6 rounds: quantize (three launches)
// 49.99 -> 49.16 us, dequantize 30.12 -> 29.25 us; 5 resident measured the
// same for quantize and 1% slower for dequantize.  The grouped NVFP4 passes
// ran 10% slower under such a cap and the block-FP8 quantizers and
// dequantizer slower or no faster; they keep 0.
constexpr size_t kLdsCap6 = 23 * 1024;
constexpr bool kNTLoad = true;
constexpr bool kNTLoadDq = false;
constexpr bool kNTLoadRequant = true;
constexpr bool kNTLoadNvAmax = false;
constexpr bool kNTLoadNvGAmax = true;
constexpr bool kNTLoadNvQuant = true;

// 8 bf16 -> 8 E4M3 codes of fl32(x / div): by reciprocal + FMA correction
// when `fast` (the divisor is in the exact domain), else by IEEE division;
// all NaN with each element's sign for a NaN/Inf block.
__device__ __forceinline__ uint2 bfp8_encode8(uint4 v, float div, float y, bool fast,
                                              bool nonfinite)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t c[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t w0 = w[2 * h], w1 = w[2 * h + 1];
        const float f0 = bf16lo_to_f32(w0), f1 = bf16hi_to_f32(w0);
        const float f2 = bf16lo_to_f32(w1), f3 = bf16hi_to_f32(w1);
        if (nonfinite) {
            c[h] = 0x7F7F7F7Fu | signs4(w0, w1);
        } else if (fast) {
            c[h] = cvt_fp8x2_f32<true>(cvt_fp8x2_f32<false>(0u, div_markstein(f0, div, y),
                                                            div_markstein(f1, div, y)),
                                       div_markstein(f2, div, y), div_markstein(f3, div, y));
        } else {
            c[h] = cvt_fp8x2_f32<true>(cvt_fp8x2_f32<false>(0u, f0 / div, f1 / div), f2 / div,
                                       f3 / div);   // IEEE fp32 divisions
        }
    }
    return make_uint2(c[0], c[1]);
}

// ---------------------------------------------------------------------------
// Block-FP8: one workgroup of 8 waves per 128 x 128 tile.  Thread t loads 4
// rows (t/16 + 32k) x 8 columns ((t%16)*8): each wave load covers 4 rows x
// 256 B.  8 waves of 16 rows measured 5% faster on MI355X than 4 waves of 32
// ([8192, 8192], cold): after the tile's barrier each wave encodes half as
// much; 16 waves of 8 rows were 7% slower.
// A stack of slices [G, rows, cols] (ts tiles each) is quantized slice by
// slice: no tile crosses a slice boundary.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) void bfp8_quant_kernel(const uint16_t *__restrict__ x,
                                                         int64_t rows, int64_t cols,
                                                         uint8_t *__restrict__ q,
                                                         float *__restrict__ scale, int64_t tc,
                                                         int64_t ts)
{
    __shared__ uint32_t red[8];
    const int64_t slice = blockIdx.x / ts, t = blockIdx.x % ts;
    x += slice * rows * cols;
    q += slice * rows * cols;
    scale += slice * ts;
    const int64_t bi = t / tc, bj = t % tc;
    const int tid = threadIdx.x;
    const int64_t col = bj * kBlk + (tid & 15) * 8;
    const int64_t rbase = bi * kBlk + (tid >> 4);
    const bool cin = col < cols;  // cols % 8 == 0: a chunk is all in or all out

    uint4 v[4];
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t r = rbase + 32 * k;
        v[k] = make_uint4(0, 0, 0, 0);
        if (cin && r < rows) v[k] = ld16<kNTLoad>(x + r * cols + col);
        m = max(m, amax8(v[k]));
    }
    m = wave_max(m);
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = m;
    __syncthreads();
    m = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) m = max(m, red[w]);

    const bool nonfinite = m >= 0x7F80u;
    const float A = __uint_as_float(m << 16);      // exact: amax is a bf16 value
    const float S = nonfinite ? __builtin_nanf("") : A / 448.0f;
    const float div = (m == 0u) ? 1.0f : S;        // zero tile: codes are +-0
    if (tid == 0) scale[bi * tc + bj] = S;

    // Tile-uniform choice: reciprocal + FMA correction (exact for divisors in
    // [2^-60, 2^60] and |x / S| <= 448 * (1 + 2^-23)), IEEE division
    // otherwise, all-NaN for a NaN/Inf tile.
    const bool fast = !nonfinite && markstein_ok(div);
    const float y = fast ? 1.0f / div : 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t r = rbase + 32 * k;
        const uint2 c = bfp8_encode8(v[k], div, y, fast, nonfinite);
        if (cin && r < rows) st8<kNTStore>(q + r * cols + col, c);
    }
}

// E4M3 code (with sign) to fp32, NaN for S.1111.111.
__device__ __forceinline__ float e4m3_to_f32(uint32_t code)
{
    const uint32_t mag = code & 0x7Fu;
    float v = e4m3_mag_value(mag);
    v = mag == 0x7Fu ? __builtin_nanf("") : v;
    return (code & 0x80u) ? -v : v;
}

// bf16 of an fp32 product; NaN -> quiet NaN with the element code's sign.
__device__ __forceinline__ uint32_t bf16_of_product(float p, uint32_t code_sign)
{
    return p != p ? (0x7FC0u | (code_sign ? 0x8000u : 0u)) : bf16_rne(p);
}

// One 8-element chunk of block-FP8 codes -> 8 bf16 (two words of 4 codes).
__device__ __forceinline__ uint4 bfp8_dequant8(uint2 c, float S, bool slow)
{
    uint32_t o[4];
    if (!slow) {
        // E4M3 -> fp32 exactly (v_cvt_pk_f32_fp8), one fp32 product, RNE to bf16
        const uint32_t cw[2] = {c.x, c.y};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[h], false);
            const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[h], true);
            o[2 * h] = bf16x2_rne(a.x * S, a.y * S);
            o[2 * h + 1] = bf16x2_rne(b.x * S, b.y * S);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            const uint32_t cw = j < 4 ? c.x : c.y;
            const int sh = 8 * (j & 3);
            const uint32_t c0 = (cw >> sh) & 0xFFu, c1 = (cw >> (sh + 8)) & 0xFFu;
            const float p0 = e4m3_to_f32(c0) * S;   // one IEEE fp32 multiplication
            const float p1 = e4m3_to_f32(c1) * S;
            o[j / 2] = bf16_of_product(p0, c0 & 0x80u) | (bf16_of_product(p1, c1 & 0x80u) << 16);
        }
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// Tiles: 512-column segment x kRowsBq rows (4 waves x 2 rows).  128 x 128
// blocks (kRowScales false): a tile's rows lie inside one 128-row block row,
// so each lane needs one scale; 1 x 128 blocks (kRowScales true): one scale
// per row.
template <bool kRowScales>
__global__ __launch_bounds__(256) void bfp8_dequant_kernel(const uint8_t *__restrict__ q,
                                                           const float *__restrict__ scale,
                                                           int64_t rows, int64_t cols,
                                                           uint16_t *__restrict__ out, int64_t tc,
                                                           int64_t nseg, int64_t slice_tiles,
                                                           int64_t slice_scales)
{
    // slices [G, rows, cols] of 128 x 128 tiles: slice_tiles launch tiles and
    // slice_scales scales each (one slice when slice_tiles is the grid size)
    const int64_t slice = blockIdx.x / slice_tiles;
    q += slice * rows * cols;
    out += slice * rows * cols;
    scale += slice * slice_scales;
    const int64_t tile = blockIdx.x % slice_tiles;
    const int64_t seg = tile % nseg;
    const int64_t rb = tile / nseg;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    const int64_t col = seg * kSegNv + lane * 8;
    if (col >= cols) return;  // cols % 8 == 0; no barriers below
    const int64_t r0 = rb * kRowsBq + wave;
    constexpr int kR = kRowsBq / 4;
    float S[kR];
    uint2 c[kR];
    bool bad = false;
#pragma unroll
    for (int i = 0; i < kR; ++i) {
        const int64_t r = r0 + 4 * i;
        c[i] = make_uint2(0, 0);
        S[i] = 0.0f;
        if (kRowScales) {
            if (r < rows) S[i] = scale[r * tc + col / kBlk];
        } else {
            S[i] = i == 0 ? scale[((rb * kRowsBq) / kBlk) * tc + col / kBlk] : S[0];
        }
        if (r < rows) c[i] = ld8<kNTLoadDq>(q + r * cols + col);
        const uint32_t tx = c[i].x & 0x7F7F7F7Fu, ty = c[i].y & 0x7F7F7F7Fu;
        // NaN products (NaN code, NaN or infinite scale) take the exact sign rule
        bad |= (((tx + 0x01010101u) | (ty + 0x01010101u)) & 0x80808080u) != 0u;
        bad |= !__builtin_isfinite(S[i]);
    }
    const bool slow = wave_any(bad);
#pragma unroll
    for (int i = 0; i < kR; ++i) {
        const int64_t r = r0 + 4 * i;
        const uint4 o = slow ? bfp8_dequant8(c[i], S[i], true) : bfp8_dequant8(c[i], S[i], false);
        if (r < rows) st16<kNTStore>(out + r * cols + col, o);
    }
}

// ---------------------------------------------------------------------------
// Block-FP8 with 1 x 128 blocks (the activation recipe; with kFQ the fake
// quantization fp8_simulate_qat(x, 128)).  Tiles as the dequantizer; 16
// lanes (8 columns each) hold one block of a row, reduced with 4 DPP steps.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t row16_max(uint32_t v)
{
    v = quad_max(v);
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // half mirror
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // mirror
}

template <bool kQ, bool kFQ>
__global__ __launch_bounds__(256) void bfp8_1x128_kernel(const uint16_t *__restrict__ x,
                                                         int64_t rows, int64_t cols,
                                                         uint8_t *__restrict__ q,
                                                         float *__restrict__ scale,
                                                         uint16_t *__restrict__ fq, int64_t tc,
                                                         int64_t nseg)
{
    // with scales to write, a row block's segments run on one XCD, so each
    // row's scale line fills inside one L2 (no barriers below)
    int64_t seg, rb;
    if (kQ) {
        if (!xcd_row_tile(nseg, (rows + kRowsBq - 1) / kRowsBq, seg, rb)) return;
    } else {
        seg = blockIdx.x % nseg;
        rb = blockIdx.x / nseg;
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    const int64_t col = seg * kSegNv + lane * 8;
    const bool cin = col < cols;  // cols % 8 == 0; lanes past the edge still join the DPP
    const int64_t r0 = rb * kRowsBq + wave;
    constexpr int kR = kRowsBq / 4;
    uint4 v[kR];
#pragma unroll
    for (int i = 0; i < kR; ++i) {
        const int64_t r = r0 + 4 * i;
        v[i] = make_uint4(0, 0, 0, 0);
        if (cin && r < rows) v[i] = ld16<kNTLoad>(x + r * cols + col);
    }
#pragma unroll
    for (int i = 0; i < kR; ++i) {
        const int64_t r = r0 + 4 * i;
        const bool ok = cin && r < rows;
        const uint32_t m = row16_max(amax8(v[i]));
        const bool nonfinite = m >= 0x7F80u;
        const float A = __uint_as_float(m << 16);      // exact: amax is a bf16 value
        const float S = nonfinite ? __builtin_nanf("") : A / 448.0f;
        const float div = (m == 0u) ? 1.0f : S;        // zero block: codes are +-0
        const bool fast = !nonfinite && markstein_ok(div);
        const bool wave_fast = !wave_any(!fast);
        const float y = fast ? 1.0f / div : 0.0f;
        const uint2 c = wave_fast ? bfp8_encode8(v[i], div, y, true, false)
                                  : bfp8_encode8(v[i], div, y, fast, nonfinite);
        if (kQ && ok) {
            st8<kNTStore>(q + r * cols + col, c);
            scale[r * tc + col / kBlk] = S;  // the same value from the block's 16 lanes
        }
        if (kFQ) {
            const bool slow = wave_any(nonfinite);
            const uint4 d = slow ? bfp8_dequant8(c, S, true) : bfp8_dequant8(c, S, false);
            if (ok) st16<kNTStore>(fq + r * cols + col, d);
        }
    }
}

// ---------------------------------------------------------------------------
// FP8 block -> BF16 -> MXFP8 in one pass (the checkpoint conversion): each
// lane dequantizes 8 codes of a row exactly as bfp8_dequant_kernel does and
// quantizes the 8 bf16 row-wise as the MXFP8 row-wise kernel does (a lane
// quad is one group of 32), so the bf16 tensor never reaches memory: 1 byte
// read and 1 + 1/32 written per element instead of 6.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bfp8_to_mx_kernel(const uint8_t *__restrict__ q,
                                                         const float *__restrict__ scale,
                                                         int64_t rows, int64_t cols,
                                                         uint8_t *__restrict__ q8,
                                                         uint8_t *__restrict__ s8, int64_t tc,
                                                         int64_t nseg)
{
    // a row block's segments run on one XCD, so each row's scale line fills
    // inside one L2 (no barriers below)
    int64_t seg, rb;
    if (!xcd_row_tile(nseg, (rows + kRowsDq - 1) / kRowsDq, seg, rb)) return;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    const int64_t col = seg * kSegNv + lane * 8;
    if (col >= cols) return;  // cols % 32 == 0: whole quads leave; no barriers below
    const int64_t r0 = rb * kRowsDq + wave;
    const float S = scale[((rb * kRowsDq) / kBlk) * tc + col / kBlk];
    constexpr int kR = kRowsDq / 4;
    uint2 c[kR];
    bool nan_code = false;
#pragma unroll
    for (int i = 0; i < kR; ++i) {
        const int64_t r = r0 + 4 * i;
        c[i] = make_uint2(0, 0);
        if (r < rows) c[i] = ld8<kNTLoadRequant>(q + r * cols + col);
        const uint32_t tx = c[i].x & 0x7F7F7F7Fu, ty = c[i].y & 0x7F7F7F7Fu;
        nan_code |= (((tx + 0x01010101u) | (ty + 0x01010101u)) & 0x80808080u) != 0u;
    }
    const bool slow = wave_any(nan_code || !__builtin_isfinite(S));
#pragma unroll
    for (int i = 0; i < kR; ++i) {
        const int64_t r = r0 + 4 * i;
        const uint4 bf = slow ? bfp8_dequant8(c[i], S, true) : bfp8_dequant8(c[i], S, false);
        const MxRow8 m = mx_row_encode8(bf);
        if (r < rows) {
            st8<kNTStore>(q8 + r * cols + col, make_uint2(m.c0, m.c1));
            s8[r * (cols >> 5) + (col >> 5)] = (uint8_t)m.s;  // same byte from a quad's 4 lanes
        }
    }
}

// ---------------------------------------------------------------------------
// NVFP4.  Pass 1: each workgroup writes the max magnitude (bf16 bits) of its
// share of x to a partials array; one workgroup reduces the partials (an
// unsigned max: order-independent, deterministic) to g, written to the
// caller's global-scale word; pass 2 reads g and quantizes.  Measured on
// MI355X ([8192, 8192], cold): reducing the partials in the encoding pass
// instead -- in one wave behind a barrier, or in every wave, 256 or 512 of
// them, or once per workgroup of a persistent encoding grid -- made that pass
// 2 to 13 us slower, more than the reducing launch costs (about 5 us).  In
// pass 2 a lane pair owns one 16-element block: 16 bytes of x, 4 bytes of
// packed codes and (both lanes) its scale byte each.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void nvfp4_amax_kernel(const uint16_t *__restrict__ x,
                                                         int64_t nvec, uint32_t *__restrict__ partial)
{
    __shared__ uint32_t red[4];
    constexpr int kU = 8;  // 16-byte loads in flight per thread
    // each workgroup reads kU * 4 KiB of contiguous x per step, then strides
    // by the grid (contiguous chunks keep DRAM pages open)
    const uint4 *xv = reinterpret_cast<const uint4 *>(x);
    constexpr int64_t kChunk = 256 * kU;
    uint32_t m = 0;
    for (int64_t base = (int64_t)blockIdx.x * kChunk; base < nvec; base += (int64_t)gridDim.x * kChunk) {
        uint4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t i = base + u * 256 + threadIdx.x;
            v[u] = i < nvec ? ld16<kNTLoadNvAmax>(xv + i) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) m = max(m, amax8(v[u]));
    }
    m = wave_max(m);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = m;
    __syncthreads();
    if (threadIdx.x == 0) partial[blockIdx.x] = max(max(red[0], red[1]), max(red[2], red[3]));
}

// 8 E2M1 codes (half a block, four words of x pairs) under effective scale
// eff, packed into one word (element 2j -> low nibble of byte j).
__device__ __forceinline__ uint32_t nvfp4_codes8(const uint4 a, float eff, float y, bool fast,
                                                 bool nonfinite)
{
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
    uint32_t out = 0u;
    if (fast) {
        // reciprocal + FMA correction (exact here), E2M1 by the hardware
        out = cvt_fp4x2_f32<0>(out, div_markstein(bf16lo_to_f32(w[0]), eff, y),
                               div_markstein(bf16hi_to_f32(w[0]), eff, y));
        out = cvt_fp4x2_f32<1>(out, div_markstein(bf16lo_to_f32(w[1]), eff, y),
                               div_markstein(bf16hi_to_f32(w[1]), eff, y));
        out = cvt_fp4x2_f32<2>(out, div_markstein(bf16lo_to_f32(w[2]), eff, y),
                               div_markstein(bf16hi_to_f32(w[2]), eff, y));
        out = cvt_fp4x2_f32<3>(out, div_markstein(bf16lo_to_f32(w[3]), eff, y),
                               div_markstein(bf16hi_to_f32(w[3]), eff, y));
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float f0 = bf16lo_to_f32(w[j]), f1 = bf16hi_to_f32(w[j]);
            uint32_t n0, n1;
            if (nonfinite) {
                n0 = n1 = 7u;
            } else if (eff == 0.0f) {
                n0 = n1 = 0u;
            } else {
                n0 = e2m1_mag_from_f32(__builtin_fabsf(f0) / eff);   // one IEEE fp32 division
                n1 = e2m1_mag_from_f32(__builtin_fabsf(f1) / eff);
            }
            n0 |= (w[j] >> 12) & 0x8u;          // sign of the low bf16
            n1 |= (w[j] >> 28) & 0x8u;          // sign of the high bf16
            out |= (n0 | (n1 << 4)) << (8 * j);
        }
    }
    return out;
}

// Tiles: 512-column segment x kRowsNvQ rows (single tensor) or kRowsNv rows
// (grouped); wave w of a tile holds rows w, w + 4, ...  Lane pair (2k, 2k+1)
// holds one 16-element block, 8 elements each, so every load and store
// instruction of a wave is contiguous; the block amax is one DPP swap.
//
// With g fixed for the workgroup, a block's effective scale can take only 127
// values, one per E4M3 magnitude code: the workgroup tabulates
// eff = fl32(val(m) * g) and RN(1 / eff) once (one IEEE division per entry)
// in LDS, so a block looks its pair up instead of dividing.  Every thread of
// the workgroup must call this (it holds a barrier).
__device__ __forceinline__ void nvfp4_scale_table(float2 *tab, float g)
{
    if (threadIdx.x < 128) {
        const float eff = e4m3_mag_value(threadIdx.x) * g;  // one IEEE fp32 multiplication
        tab[threadIdx.x] = make_float2(eff, markstein_ok(eff) ? 1.0f / eff : 0.0f);
    }
    __syncthreads();
}

// The per-block steps for one wave's kR rows of a tile (rows r0 + 4i), given
// the global scale g (NaN when the tensor or scale group holds NaN/Inf) and
// the workgroup's table for g.  The block-scale quotient b / (6g) is IEEE
// division's result either way: by the reciprocal-FMA step when 6g lies in
// its proven domain (b <= A keeps the quotient under 449), else by division.
template <int kR>
__device__ __forceinline__ void nvfp4_encode_rows(const uint4 (&v)[kR], int64_t r0,
                                                  int64_t rows, int64_t cols, int64_t col,
                                                  uint8_t *__restrict__ q,
                                                  uint8_t *__restrict__ s_out, float g,
                                                  bool nonfinite, const float2 *tab)
{
    const bool cin = col < cols;  // cols % 16 == 0: a block (lane pair) is all in or all out
    const float d = 6.0f * g;
    const bool dfast = markstein_ok(d);           // uniform: g is the workgroup's
    const float yd = dfast ? 1.0f / d : 0.0f;     // RN(1 / d), one IEEE division per thread
#pragma unroll
    for (int i = 0; i < kR; ++i) {
        const int64_t r = r0 + 4 * i;
        const bool ok = cin && r < rows;
        const uint32_t h = amax8(v[i]);
        const uint32_t b = max(h, dpp_swap1(h));  // the block's amax (lane pair)
        uint32_t s;
        if (nonfinite) {
            s = 0x7Fu;
        } else if (g == 0.0f) {
            s = 0u;
        } else {
            const float bf = __uint_as_float(b << 16);
            const float ratio = dfast ? div_markstein(bf, d, yd) : bf / d;
            s = e4m3_mag_from_f32(ratio);
        }
        const float2 t = tab[s & 0x7Fu];
        const float eff = t.x;
        const bool fast = !wave_any(nonfinite || !markstein_ok(eff));
        const float y = t.y;
        const uint32_t codes = fast ? nvfp4_codes8(v[i], eff, y, true, false)
                                    : nvfp4_codes8(v[i], eff, 0.0f, false, nonfinite);
        if (ok) {
            st4<kNTStore>(q + r * (cols >> 1) + (col >> 1), codes);
            // both lanes of the pair hold the same byte: storing it from each
            // avoids an exec-mask change per row
            s_out[r * (cols >> 4) + (col >> 4)] = (uint8_t)s;
        }
    }
}

// This wave's kR rows of a tile (16 bytes of x per lane and row).
template <bool kNT, int kR>
__device__ __forceinline__ void nvfp4_load_rows(const uint16_t *__restrict__ x, int64_t r0,
                                                int64_t rows, int64_t cols, int64_t col,
                                                uint4 (&v)[kR])
{
#pragma unroll
    for (int i = 0; i < kR; ++i) {
        const int64_t r = r0 + 4 * i;
        v[i] = make_uint4(0, 0, 0, 0);
        if (col < cols && r < rows) v[i] = ld16<kNT>(x + r * cols + col);
    }
}

// One workgroup: the global amax from the partials (one per thread, so every
// load is in flight at once), g = fl32(A / 2688) (NaN when x holds NaN/Inf),
// written once for the encoding pass to read.
__global__ __launch_bounds__(kNvAmaxBlocks) void nvfp4_finalize_kernel(
    const uint32_t *__restrict__ partial, int npartial, float *__restrict__ g_out)
{
    __shared__ uint32_t red[kNvAmaxBlocks / kWave];
    uint32_t am = (int)threadIdx.x < npartial ? partial[threadIdx.x] : 0u;
    am = wave_max(am);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = am;
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int w = 1; w < kNvAmaxBlocks / kWave; ++w) am = max(am, red[w]);
        const bool nonfinite = am >= 0x7F80u;
        *g_out = nonfinite ? __builtin_nanf("") : __uint_as_float(am << 16) / 2688.0f;  // 448 * 6
    }
}

__global__ __launch_bounds__(256) void nvfp4_quant_kernel(const uint16_t *__restrict__ x,
                                                          int64_t rows, int64_t cols,
                                                          uint8_t *__restrict__ q,
                                                          uint8_t *__restrict__ s_out,
                                                          const float *__restrict__ g_in,
                                                          int64_t nseg)
{
    // a row block's segments run on one XCD (2% faster end to end on
    // [8192, 8192] than the plain order); padding workgroups leave before the
    // barrier in nvfp4_scale_table, whole
    int64_t seg, rb;
    if (!xcd_row_tile(nseg, (rows + kRowsNvQ - 1) / kRowsNvQ, seg, rb)) return;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    const int64_t col = seg * kSegNv + lane * 8;
    const int64_t r0 = rb * kRowsNvQ + wave;
    __shared__ float2 tab[128];
    uint4 v[kRowsNvQ / 4];
    nvfp4_load_rows<kNTLoadNvQuant>(x, r0, rows, cols, col, v);
    const float g = *g_in;
    nvfp4_scale_table(tab, g);
    nvfp4_encode_rows(v, r0, rows, cols, col, q, s_out, g, g != g, tab);
}

// ---------------------------------------------------------------------------
// Grouped NVFP4: many tensors, the global scale shared within caller-given
// scale groups (a fused gated-MoE gate_up weight uses one group per half for
// QAT, or one group for both halves to export a shared weight_scale_2).  Three
// launches over the flattened (tensor, tile) space of 512-column x 32-row
// tiles: per-tile amax partials; one workgroup per scale group reducing its
// members' partials to g; per-tile encoding with the tensor's group scale.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void nvfp4_g_amax_kernel(const NvEntry *__restrict__ table,
                                                           const int32_t *__restrict__ starts,
                                                           int32_t n, uint32_t *__restrict__ partial)
{
    __shared__ uint32_t red[4];
    const int32_t t = (int32_t)blockIdx.x;
    const NvEntry E = table[find_entry(starts, n, t)];
    const int32_t local = t - E.tile_begin;
    const int64_t seg = local % E.nseg, rb = local / E.nseg;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    uint4 v[kRowsNv / 4];
    nvfp4_load_rows<kNTLoadNvGAmax>(global_ptr(E.x), rb * kRowsNv + wave, E.rows, E.cols,
                                    seg * kSegNv + lane * 8, v);
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < kRowsNv / 4; ++i) m = max(m, amax8(v[i]));
    m = wave_max(m);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) partial[t] = max(max(red[0], red[1]), max(red[2], red[3]));
}

__global__ __launch_bounds__(256) void nvfp4_g_reduce_kernel(const int32_t *__restrict__ starts,
                                                             const int32_t *__restrict__ groups,
                                                             int32_t n, int32_t total_tiles,
                                                             const uint32_t *__restrict__ partial,
                                                             float *__restrict__ gs)
{
    __shared__ uint32_t red[4];
    const int32_t j = (int32_t)blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t m = 0;
    // 64 entries per step: a ballot finds this group's members (the same mask
    // in every wave), whose partial ranges the whole workgroup then reduces
    for (int32_t base = 0; base < n; base += kWave) {
        const int32_t i = base + lane;
        uint64_t mask = __ballot(i < n && groups[i] == j);
        while (mask) {
            const int32_t k = base + __builtin_ctzll(mask);
            mask &= mask - 1;
            const int32_t t1 = k + 1 < n ? starts[k + 1] : total_tiles;
            for (int32_t t = starts[k] + (int32_t)threadIdx.x; t < t1; t += 256)
                m = max(m, partial[t]);
        }
    }
    m = wave_max(m);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        m = max(max(red[0], red[1]), max(red[2], red[3]));
        const bool nonfinite = m >= 0x7F80u;
        gs[j] = nonfinite ? __builtin_nanf("") : __uint_as_float(m << 16) / 2688.0f;
    }
}

__global__ __launch_bounds__(256) void nvfp4_g_quant_kernel(const NvEntry *__restrict__ table,
                                                            const int32_t *__restrict__ starts,
                                                            int32_t n, const float *__restrict__ gs)
{
    const int32_t t = (int32_t)blockIdx.x;
    const NvEntry E = table[find_entry(starts, n, t)];
    const int32_t local = t - E.tile_begin;
    const int64_t seg = local % E.nseg, rb = local / E.nseg;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t col = seg * kSegNv + lane * 8, r0 = rb * kRowsNv + wave;
    __shared__ float2 tab[128];
    uint4 v[kRowsNv / 4];
    nvfp4_load_rows<kNTLoadNvQuant>(global_ptr(E.x), r0, E.rows, E.cols, col, v);
    const float g = gs[E.group];
    nvfp4_scale_table(tab, g);
    nvfp4_encode_rows(v, r0, E.rows, E.cols, col, global_ptr(E.q), global_ptr(E.s), g, g != g,
                      tab);
}

// 8 packed E2M1 nibbles (one word) -> 8 bf16, effective scale eff.
__device__ __forceinline__ uint4 nvfp4_dequant8(uint32_t packed, float eff, bool slow)
{
    uint32_t o[4];
    if (!slow) {
        // E2M1 -> fp32 exactly (v_cvt_scalef32_pk_f32_fp4, scale 1), one product, RNE
        const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 0);
        const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 1);
        const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 2);
        const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 3);
        o[0] = bf16x2_rne(p0.x * eff, p0.y * eff);
        o[1] = bf16x2_rne(p1.x * eff, p1.y * eff);
        o[2] = bf16x2_rne(p2.x * eff, p2.y * eff);
        o[3] = bf16x2_rne(p3.x * eff, p3.y * eff);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t byte = (packed >> (8 * j)) & 0xFFu;
            const uint32_t n0 = byte & 0xFu, n1 = byte >> 4;
            float v0 = e2m1_mag_value(n0 & 7u), v1 = e2m1_mag_value(n1 & 7u);
            v0 = (n0 & 8u) ? -v0 : v0;
            v1 = (n1 & 8u) ? -v1 : v1;
            const float q0 = v0 * eff, q1 = v1 * eff;       // one IEEE fp32 multiplication each
            o[j] = bf16_of_product(q0, n0 & 8u) | (bf16_of_product(q1, n1 & 8u) << 16);
        }
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// Each lane owns 8 consecutive outputs (half a block), so every 16-byte store
// instruction of a wave covers 1 KiB of contiguous memory: partial-line
// streaming stores cost whole-line bandwidth.
__global__ __launch_bounds__(256) void nvfp4_dequant_kernel(const uint8_t *__restrict__ q,
                                                            const uint8_t *__restrict__ s_in,
                                                            const float *__restrict__ g_in,
                                                            int64_t rows, int64_t cols,
                                                            uint16_t *__restrict__ out,
                                                            int64_t nseg)
{
    int64_t seg, rb;
    if (!xcd_row_tile(nseg, (rows + kRowsDq - 1) / kRowsDq, seg, rb)) return;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    const int64_t col = seg * kSegNv + lane * 8;
    if (col >= cols) return;  // cols % 16 == 0; no barriers below
    const int64_t r0 = rb * kRowsDq + wave;
    constexpr int kR = kRowsDq / 4;
    uint32_t pk[kR], sb[kR];
    // all of the wave's loads are issued before any is used (decoding a
    // scale in this loop made the compiler wait for each row's loads in turn)
#pragma unroll
    for (int i = 0; i < kR; ++i) {
        const int64_t r = r0 + 4 * i;
        pk[i] = 0u;
        sb[i] = 0u;
        if (r < rows) {
            pk[i] = ld4<kNTLoadDq>(q + r * (cols >> 1) + (col >> 1));
            sb[i] = s_in[r * (cols >> 4) + (col >> 4)];
        }
    }
    const float g = *g_in;
    float eff[kR];
    bool bad = false;
#pragma unroll
    for (int i = 0; i < kR; ++i) {
        // one IEEE fp32 multiplication; rows past the end stay 0
        eff[i] = r0 + 4 * i < rows ? e4m3_to_f32(sb[i]) * g : 0.0f;
        bad |= !__builtin_isfinite(eff[i]);  // NaN products (x * NaN, 0 * Inf) take the sign rule
    }
    const bool slow = wave_any(bad);
#pragma unroll
    for (int i = 0; i < kR; ++i) {
        const int64_t r = r0 + 4 * i;
        const uint4 o = slow ? nvfp4_dequant8(pk[i], eff[i], true) : nvfp4_dequant8(pk[i], eff[i], false);
        if (r < rows) st16<kNTStore>(out + r * cols + col, o);
    }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------

hipError_t launch_bfp8_quant(const uint16_t *x, int64_t slices, int64_t rows, int64_t cols,
                             uint8_t *q, float *scale, hipStream_t stream)
{
    const int64_t tr = (rows + kBlk - 1) / kBlk, tc = (cols + kBlk - 1) / kBlk;
    const int64_t ts = tr * tc;
    if (ts <= 0 || slices <= 0) return hipSuccess;
    if (ts > 0x7FFFFFFF / slices) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bfp8_quant_kernel, dim3((unsigned)(ts * slices)), dim3(512), 0, stream, x,
                       rows, cols, q, scale, tc, ts);
    return hipGetLastError();
}

hipError_t launch_bfp8_dequant(const uint8_t *q, const float *scale, int64_t slices,
                               int64_t rows, int64_t cols, bool row_scales, uint16_t *out,
                               hipStream_t stream)
{
    const int64_t nseg = (cols + kSegNv - 1) / kSegNv;
    const int64_t per = nseg * ((rows + kRowsBq - 1) / kRowsBq);
    if (per <= 0 || slices <= 0) return hipSuccess;
    if (per > 0x7FFFFFFF / slices) return hipErrorInvalidConfiguration;
    const int64_t tiles = per * slices;
    const int64_t tc = (cols + kBlk - 1) / kBlk;
    const int64_t scales = (row_scales ? rows : (rows + kBlk - 1) / kBlk) * tc;
    if (row_scales)
        hipLaunchKernelGGL((bfp8_dequant_kernel<true>), dim3((unsigned)tiles), dim3(256), 0,
                           stream, q, scale, rows, cols, out, tc, nseg, per, scales);
    else
        hipLaunchKernelGGL((bfp8_dequant_kernel<false>), dim3((unsigned)tiles), dim3(256), 0,
                           stream, q, scale, rows, cols, out, tc, nseg, per, scales);
    return hipGetLastError();
}

hipError_t launch_bfp8_1x128(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q,
                             float *scale, uint16_t *fq, hipStream_t stream)
{
    const int64_t tc = (cols + kBlk - 1) / kBlk;
    const int64_t nseg = (cols + kSegNv - 1) / kSegNv;
    const int64_t nrb = (rows + kRowsBq - 1) / kRowsBq;
    if (nseg <= 0 || nrb <= 0) return hipSuccess;
    const int64_t tiles = q ? xcd_row_grid(nseg, nrb) : nseg * nrb;  // the kernel's order
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)tiles), block(256);
    if (q && fq)
        hipLaunchKernelGGL((bfp8_1x128_kernel<true, true>), grid, block, 0, stream, x, rows, cols,
                           q, scale, fq, tc, nseg);
    else if (q)
        hipLaunchKernelGGL((bfp8_1x128_kernel<true, false>), grid, block, 0, stream, x, rows, cols,
                           q, scale, fq, tc, nseg);
    else
        hipLaunchKernelGGL((bfp8_1x128_kernel<false, true>), grid, block, 0, stream, x, rows, cols,
                           q, scale, fq, tc, nseg);
    return hipGetLastError();
}

hipError_t launch_bfp8_to_mx(const uint8_t *q, const float *scale, int64_t rows, int64_t cols,
                             uint8_t *q8, uint8_t *s8, hipStream_t stream)
{
    const int64_t tc = (cols + kBlk - 1) / kBlk;
    const int64_t nseg = (cols + kSegNv - 1) / kSegNv;
    const int64_t nrb = (rows + kRowsDq - 1) / kRowsDq;
    if (nseg <= 0 || nrb <= 0) return hipSuccess;
    const int64_t tiles = xcd_row_grid(nseg, nrb);
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bfp8_to_mx_kernel, dim3((unsigned)tiles), dim3(256), 0, stream, q, scale,
                       rows, cols, q8, s8, tc, nseg);
    return hipGetLastError();
}

hipError_t launch_nvfp4_quant(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q,
                              uint8_t *s, float *g, uint32_t *ws, int64_t ws_words,
                              hipStream_t stream)
{
    const int64_t nvec = rows * cols / 8;
    if (nvec <= 0) return hipSuccess;
    const int64_t want = (nvec + 255) / 256;
    const int ablocks = (int)(want < kNvAmaxBlocks ? want : kNvAmaxBlocks);
    if (ablocks > ws_words) return hipErrorInvalidValue;  // one partial per amax workgroup
    const int64_t nseg = (cols + kSegNv - 1) / kSegNv;
    const int64_t tiles = xcd_row_grid(nseg, (rows + kRowsNvQ - 1) / kRowsNvQ);
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(nvfp4_amax_kernel, dim3((unsigned)ablocks), dim3(256), kLdsCap6, stream, x,
                       nvec, ws);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(nvfp4_finalize_kernel, dim3(1), dim3(kNvAmaxBlocks), 0, stream, ws, ablocks,
                       g);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(nvfp4_quant_kernel, dim3((unsigned)tiles), dim3(256), kLdsCap6, stream, x,
                       rows, cols, q, s, g, nseg);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// NVFP4 for callers that cannot allocate: the amax partials go to `scratch`,
// a fixed array of this library (kNvAmaxBlocks words, 2 KiB) that each GPU
// holds until the process ends, instead of a caller workspace.  In host code
// `scratch` names a host-side stand-in, not device memory: its address on a
// device comes from hipGetSymbolAddress, resolved once per device with that
// device current and kept below.  Every call on a GPU shares that GPU's
// array, so calls that overlap on one GPU race.  Each call writes every
// partial it later reads, so nothing needs clearing between calls.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint32_t scratch[kNvAmaxBlocks];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
uint32_t *scratch_on[kMaxDevices];  // device address of `scratch` per device, once resolved

// The device address of `scratch` on the device that runs `stream`.
hipError_t scratch_for(hipStream_t stream, uint32_t **out)
{
    int dev = -1;
    hipError_t err = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_on[dev]) {
        int cur = -1;
        err = hipGetDevice(&cur);
        if (err != hipSuccess) return err;
        if (cur != dev && (err = hipSetDevice(dev)) != hipSuccess) return err;
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t back = hipSetDevice(cur);
            if (err == hipSuccess) err = back;
        }
        if (err != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        scratch_on[dev] = static_cast<uint32_t *>(p);
    }
    *out = scratch_on[dev];
    return hipSuccess;
}

}  // namespace

hipError_t launch_nvfp4_quant_noalloc(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q,
                                      uint8_t *s, float *g, hipStream_t stream)
{
    uint32_t *ws = nullptr;
    const hipError_t err = scratch_for(stream, &ws);
    if (err != hipSuccess) return err;
    return launch_nvfp4_quant(x, rows, cols, q, s, g, ws, kNvAmaxBlocks, stream);
}

int64_t nvfp4_tiles(int64_t rows, int64_t cols, int64_t *nseg)
{
    const int64_t ns = (cols + kSegNv - 1) / kSegNv;
    if (nseg) *nseg = ns;
    return ns * ((rows + kRowsNv - 1) / kRowsNv);
}

hipError_t launch_nvfp4_grouped(const NvEntry *table, const int32_t *starts, const int32_t *groups,
                                int32_t n, uint32_t *partial, int64_t total_tiles, float *gs,
                                int32_t n_groups, hipStream_t stream)
{
    if (n <= 0 && n_groups <= 0) return hipSuccess;
    if (total_tiles > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    if (total_tiles > 0) {
        hipLaunchKernelGGL(nvfp4_g_amax_kernel, dim3((unsigned)total_tiles), dim3(256), 0, stream,
                           table, starts, n, partial);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(nvfp4_g_reduce_kernel, dim3((unsigned)n_groups), dim3(256), 0, stream,
                       starts, groups, n, (int32_t)total_tiles, partial, gs);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || total_tiles == 0) return err;
    hipLaunchKernelGGL(nvfp4_g_quant_kernel, dim3((unsigned)total_tiles), dim3(256), 0, stream,
                       table, starts, n, gs);
    return hipGetLastError();
}

hipError_t launch_nvfp4_dequant(const uint8_t *q, const uint8_t *s, const float *g, int64_t rows,
                                int64_t cols, uint16_t *out, hipStream_t stream)
{
    const int64_t nseg = (cols + kSegNv - 1) / kSegNv;
    const int64_t nrb = (rows + kRowsDq - 1) / kRowsDq;
    if (nseg <= 0 || nrb <= 0) return hipSuccess;
    const int64_t tiles = xcd_row_grid(nseg, nrb);
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(nvfp4_dequant_kernel, dim3((unsigned)tiles), dim3(256), kLdsCap6, stream, q,
                       s, g, rows, cols, out, nseg);
    return hipGetLastError();
}

}  // namespace mxq
