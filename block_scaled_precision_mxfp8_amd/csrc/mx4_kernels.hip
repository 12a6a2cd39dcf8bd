// mx4_kernels.hip -- MXFP4 quantization, fake quantization and dequantization
// for gfx950.
//
// MXFP4: every group of 32 consecutive values of a row shares one power-of-two
// scale 2^(floor(log2 amax) - 2), stored as an E8M0 byte (0 for an all-zero
// group, 0xFF for a group holding NaN or Inf); elements are E2M1 nibbles of
// x / scale (round to nearest even, saturating at +-6, sign kept), packed two
// per byte with element 2j in the low nibble (miles PR #1372 "V4 mxfp4": the
// simulate-QAT groups of 32 in the compressor review, the [..., N/2] packed
// output in the review of fp4_act_quant; the exponent rule is the OCP
// microscaling conversion, E2M1's largest power of two being 2^2).
//
// Layout: x [rows, cols] bf16, q [rows, cols/2], scale [rows, cols/32], fake
// quant [rows, cols] bf16, all contiguous.  Tiles as the MXFP8 row-wise
// kernel: a wave covers 512 columns (8 per lane, a lane quad per group) and 8
// rows; a workgroup 32 rows.

#include "launch.hpp"
#include "mxq_device.hpp"

namespace mxq {

namespace {

constexpr int kSeg4 = 512;       // columns per wave segment
constexpr int kRows4 = 16;       // rows per workgroup tile (4 waves x 4 rows): quantize and
                                 // simulate-QAT 4% faster than 32 with cold inputs on MI355X
constexpr int kRowsDq4 = 16;     // rows per dequantize tile: 5% faster than 32
constexpr int kU4 = 4;           // rows each wave keeps in flight: all 4 of its tile rows
constexpr bool kNTLoad4 = true;  // streaming hints: every byte is touched once
constexpr bool kNTStore4 = true;

template <bool kQ, bool kFQ, bool kFull>
__device__ __forceinline__ void mx4_tile(const uint16_t *__restrict__ x, int64_t rows, int64_t cols,
                                         uint8_t *__restrict__ q, uint8_t *__restrict__ scale,
                                         uint16_t *__restrict__ fq, int64_t seg, int64_t rb)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    const int64_t col = seg * kSeg4 + lane * 8;
    const bool cin = kFull || col < cols;  // cols % 32 == 0: a quad is all in or all out
    const int64_t r0 = rb * kRows4 + wave;
#pragma unroll
    for (int it = 0; it < kRows4 / (4 * kU4); ++it) {
        uint4 v[kU4];
#pragma unroll
        for (int u = 0; u < kU4; ++u) {
            const int64_t r = r0 + 4 * (it * kU4 + u);
            v[u] = make_uint4(0, 0, 0, 0);
            if (kFull || (cin && r < rows)) v[u] = ld16<kNTLoad4>(x + r * cols + col);
        }
#pragma unroll
        for (int u = 0; u < kU4; ++u) {
            const int64_t r = r0 + 4 * (it * kU4 + u);
            const bool ok = kFull || (cin && r < rows);
            const uint32_t s = mx4_scale_byte(quad_max(amax8(v[u])));
            const bool nan_group = s == 0xFFu;
            const float sf = e8m0_to_f32(s);
            const uint32_t codes = nan_group ? e2m1x8_nan(v[u]) : e2m1x8_hw(v[u], sf);
            if (kQ && ok) {
                st4<kNTStore4>(q + r * (cols >> 1) + (col >> 1), codes);
                // all 4 lanes of the quad hold the same byte: storing it from
                // each avoids an exec-mask change per row
                scale[r * (cols >> 5) + (col >> 5)] = (uint8_t)s;
            }
            if (kFQ) {
                uint4 d = e2m1x8_dequant_hw(codes, sf);
                if (wave_any(nan_group))  // rare: a NaN/Inf group in this row of the wave
                    d = nan_group ? e2m1x8_dequant_nan(codes) : d;
                if (ok) st16<kNTStore4>(fq + r * cols + col, d);
            }
        }
    }
}

template <bool kQ, bool kFQ>
__global__ __launch_bounds__(256) void mx4_quant_kernel(const uint16_t *__restrict__ x,
                                                        int64_t rows, int64_t cols,
                                                        uint8_t *__restrict__ q,
                                                        uint8_t *__restrict__ scale,
                                                        uint16_t *__restrict__ fq, int64_t nseg)
{
    // quantize-only: row blocks per XCD, so the 16-byte pieces of each scale
    // line are written back from one L2 (+2% on MI355X; with the bf16
    // fake-quant output the plain order measured 1% faster)
    int64_t seg, rb;
    if (kQ && !kFQ) {
        if (!xcd_row_tile(nseg, (rows + kRows4 - 1) / kRows4, seg, rb)) return;
    } else {
        seg = blockIdx.x % nseg;
        rb = blockIdx.x / nseg;
    }
    if ((seg + 1) * kSeg4 <= cols && (rb + 1) * kRows4 <= rows)
        mx4_tile<kQ, kFQ, true>(x, rows, cols, q, scale, fq, seg, rb);
    else
        mx4_tile<kQ, kFQ, false>(x, rows, cols, q, scale, fq, seg, rb);
}

// out = bf16(E2M1(q) * 2^(s - 127)); scale 0xFF gives the quiet NaN with the
// nibble's sign.  Each lane decodes 8 elements (4 code bytes, one scale byte)
// per row and writes 16 contiguous bytes.
__global__ __launch_bounds__(256) void mx4_dequant_kernel(const uint8_t *__restrict__ q,
                                                          const uint8_t *__restrict__ scale,
                                                          int64_t rows, int64_t cols,
                                                          uint16_t *__restrict__ out, int64_t nseg)
{
    int64_t seg, rb;
    if (!xcd_row_tile(nseg, (rows + kRowsDq4 - 1) / kRowsDq4, seg, rb)) return;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    const int64_t col = seg * kSeg4 + lane * 8;
    if (col >= cols) return;  // no barriers below
    const int64_t r0 = rb * kRowsDq4 + wave;
    constexpr int kR = kRowsDq4 / 4;
    uint32_t pk[kR], sb[kR];
    bool bad = false;
#pragma unroll
    for (int i = 0; i < kR; ++i) {
        const int64_t r = r0 + 4 * i;
        pk[i] = 0u;
        sb[i] = 0u;
        if (r < rows) {
            pk[i] = ld4<false>(q + r * (cols >> 1) + (col >> 1));
            sb[i] = scale[r * (cols >> 5) + (col >> 5)];
        }
        bad |= sb[i] == 0xFFu;
    }
    const bool slow = wave_any(bad);
#pragma unroll
    for (int i = 0; i < kR; ++i) {
        const int64_t r = r0 + 4 * i;
        uint4 d = e2m1x8_dequant_hw(pk[i], e8m0_to_f32(sb[i]));
        if (slow && sb[i] == 0xFFu) d = e2m1x8_dequant_nan(pk[i]);
        if (r < rows) st16<kNTStore4>(out + r * cols + col, d);
    }
}

}  // namespace

hipError_t launch_mx4_quant(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q,
                            uint8_t *scale, uint16_t *fq, hipStream_t stream)
{
    const int64_t nseg = (cols + kSeg4 - 1) / kSeg4;
    const int64_t nrb = (rows + kRows4 - 1) / kRows4;
    if (nseg <= 0 || nrb <= 0) return hipSuccess;
    const int64_t tiles = (q && !fq) ? xcd_row_grid(nseg, nrb) : nseg * nrb;
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)tiles), block(256);
    if (q && fq)
        hipLaunchKernelGGL((mx4_quant_kernel<true, true>), grid, block, 0, stream, x, rows, cols, q,
                           scale, fq, nseg);
    else if (q)
        hipLaunchKernelGGL((mx4_quant_kernel<true, false>), grid, block, 0, stream, x, rows, cols,
                           q, scale, fq, nseg);
    else
        hipLaunchKernelGGL((mx4_quant_kernel<false, true>), grid, block, 0, stream, x, rows, cols,
                           q, scale, fq, nseg);
    return hipGetLastError();
}

hipError_t launch_mx4_dequant(const uint8_t *q, const uint8_t *scale, int64_t rows, int64_t cols,
                              uint16_t *out, hipStream_t stream)
{
    const int64_t nseg = (cols + kSeg4 - 1) / kSeg4;
    const int64_t nrb = (rows + kRowsDq4 - 1) / kRowsDq4;
    if (nseg <= 0 || nrb <= 0) return hipSuccess;
    const int64_t tiles = xcd_row_grid(nseg, nrb);
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(mx4_dequant_kernel, dim3((unsigned)tiles), dim3(256), 0, stream, q, scale,
                       rows, cols, out, nseg);
    return hipGetLastError();
}

}  // namespace mxq
