// mx_kernels.hip -- MXFP8 kernels for gfx950: row-wise quantize (+ fused
// fake-quant), one-pass column-wise + row-wise + fake-quant (columns in x's
// layout or transposed), dequantize, the E8M0 -> fp32 scale view, and the
// grouped row-wise launch over many tensors.
//
// Method ("PR #1935 完整报告 / Use TransformerEngine for MXFP8 quantization",
// section 实现拆解 item 1): groups of 32 consecutive values share one
// power-of-two E8M0 scale; elements are E4M3 codes; outputs are compact and
// non-swizzled.  Rows need no padding: row groups never span rows, so the
// zero-pad-to-32-rows-then-crop route gives the same bytes as predicating the
// missing rows off, which is what the kernels do.
//
// Work layout.  A wave owns a 512-column segment (64 lanes x 8 bf16 = one
// 16-byte load per lane, 1 KiB contiguous per load instruction) of a run of
// rows.  A row group of 32 is 4 adjacent lanes, so its amax is two DPP
// steps; a column group of 32 is 32 rows of the same lane, so its amax stays
// in the lane.  All of this is HBM streaming: there is no reuse across
// workgroups, so the blockIdx -> tile order only keeps each workgroup's
// accesses contiguous, except where workgroups share a scale line (the
// transposed column-only launch groups those on one XCD).
#include "launch.hpp"
#include "mxq_device.hpp"

namespace mxq {

constexpr int kSeg = 512;          // columns per wave segment
// Rows per row-wise workgroup tile; each of the 4 waves keeps all its rows in
// flight.  With cold inputs on [16384, 7168], against 32-row tiles, 16 rows
// made fake-quant 4% and the grouped MoE launch 6% faster, and 8 rows gained
// another 1.6% for single-tensor fake-quant but lost 4.5% on the grouped
// launch.  For single-tensor quantize-only launches, 16 rows measured 1.5-1.8%
// faster than 8 on [16384, 7168] and 2-3.5% on [4097, 7168] (interleaved A/B
// timing, two boxes); launches that write the fake-quant keep 8.
constexpr int kRowsRowQ = 16;     // single tensor, codes and scales only (4 waves x 4 rows)
constexpr int kRowsRowFQ = 8;     // single tensor with fake-quant output (4 waves x 2 rows)
constexpr int kRowsGrouped = 16;  // grouped launch (4 waves x 4 rows)

// Tile rows of a single-tensor row-wise launch.
constexpr int rows_row_tile(bool q, bool fq) { return (q && !fq) ? kRowsRowQ : kRowsRowFQ; }
// Rows per dequantize tile (4 waves x 2 rows).  Against 32-row tiles, 16 rows
// were 3% (row groups) and 7% (column groups) faster, and 8 rows another 1%
// and 1.5%.
constexpr int kRowsDq = 8;
// Resident-workgroup cap for the single-output row-wise launches (codes and
// scales only, or fake-quant only) and the grouped launch.  Their 4-wave
// workgroups need few VGPRs (27-52), so 8 fit on a CU; each launch reserves
// 27 KiB of dynamic LDS that no kernel touches, which leaves room for 5 in a
// CU's 160 KiB.  MI355X, inputs cold in HBM, variants interleaved in one
// process, medians of 5 rounds: row-wise quantize of [16384, 7168]
// 55.5 -> 54.3 us, fake-quant only 72.5 -> 70.9 us, the grouped launch over
// the 384 MoE tensors 2747 -> 2717 us; 6 resident measured close behind, 4
// and 3 slower.  The column-wise launches hold 4 (by VGPRs) and ran slower
// with fewer; the same cap slowed the 1 x 128 block-FP8 quantizer (12%) and
// the column-group dequantizer (5%), which keep 0.
constexpr size_t kLdsCap5 = 27 * 1024;
constexpr int kColTileRows = 128;  // rows per transposed column-wise workgroup tile (4 waves x 32)
// Streaming (non-temporal) hints on every load and store: each byte is
// touched once.  Measured on MI355X with the [16384, 7168] activation read
// cold from HBM (launches cycling over 4 resident batches): row-wise
// 5.19 -> 5.91 TB/s, column-wise 5.27 -> 5.83, fake-quant 5.51 -> 5.89,
// the one-pass kernel 4.84 -> 5.16, against unhinted loads and stores.
constexpr bool kNTLoad = true;
constexpr bool kNTStore = true;

// ---------------------------------------------------------------------------
// Row-wise tile: rows [rb*kRowsT, (rb+1)*kRowsT) x columns of segment `seg`.
// kFull: the whole tile is inside the tensor (wave-uniform), so no load or
// store needs a predicate.
// ---------------------------------------------------------------------------
template <bool kQ, bool kFQ, bool kFull, int kRowsT>
__device__ __forceinline__ void mx_row_tile_impl(const uint16_t *__restrict__ x, int64_t rows,
                                                 int64_t cols, int64_t ldx, uint8_t *__restrict__ q,
                                                 int64_t ldq, uint8_t *__restrict__ scale,
                                                 int64_t lds, uint16_t *__restrict__ fq, int64_t ldf,
                                                 int64_t seg, int64_t rb)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    const int64_t col = seg * kSeg + lane * 8;
    const bool cin = kFull || col < cols;  // cols % 32 == 0: a quad is all in or all out
    const int64_t r0 = rb * kRowsT + wave;
    constexpr int kU = kRowsT / 4;  // the wave's rows, all in flight at once

#pragma unroll
    for (int it = 0; it < kRowsT / (4 * kU); ++it) {
        uint4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t r = r0 + 4 * (it * kU + u);
            v[u] = make_uint4(0, 0, 0, 0);
            if (kFull || (cin && r < rows)) v[u] = ld16<kNTLoad>(x + r * ldx + col);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t r = r0 + 4 * (it * kU + u);
            const bool ok = kFull || (cin && r < rows);
            const MxRow8 m = mx_row_encode8(v[u]);
            const uint32_t s = m.s, c0 = m.c0, c1 = m.c1;
            const float sf = m.sf;
            const bool nan_group = s == 0xFFu;
            if (kQ && ok) {
                st8<kNTStore>(q + r * ldq + col, make_uint2(c0, c1));
                // all 4 lanes of the quad hold the same byte: storing it from
                // each avoids an exec-mask change per row
                scale[r * lds + (col >> 5)] = (uint8_t)s;
            }
            if (kFQ) {
                uint2 lo, hi;
                if (wave_any(nan_group)) {   // rare: a NaN/Inf group in this row of the wave
                    lo = mx_dequant4(c0, (int)s - 7, nan_group);
                    hi = mx_dequant4(c1, (int)s - 7, nan_group);
                } else {
                    lo = mx_dequant4_hw(c0, sf);
                    hi = mx_dequant4_hw(c1, sf);
                }
                if (ok) st16<kNTStore>(fq + r * ldf + col, make_uint4(lo.x, lo.y, hi.x, hi.y));
            }
        }
    }
}

template <bool kQ, bool kFQ, int kRowsT>
__device__ __forceinline__ void mx_row_tile(const uint16_t *__restrict__ x, int64_t rows,
                                            int64_t cols, int64_t ldx, uint8_t *__restrict__ q,
                                            int64_t ldq, uint8_t *__restrict__ scale, int64_t lds,
                                            uint16_t *__restrict__ fq, int64_t ldf, int64_t seg,
                                            int64_t rb)
{
    if ((seg + 1) * kSeg <= cols && (rb + 1) * kRowsT <= rows)
        mx_row_tile_impl<kQ, kFQ, true, kRowsT>(x, rows, cols, ldx, q, ldq, scale, lds, fq, ldf,
                                                seg, rb);
    else
        mx_row_tile_impl<kQ, kFQ, false, kRowsT>(x, rows, cols, ldx, q, ldq, scale, lds, fq, ldf,
                                                 seg, rb);
}

template <bool kQ, bool kFQ>
__global__ __launch_bounds__(256) void mx_rowwise_kernel(const uint16_t *__restrict__ x,
                                                         int64_t rows, int64_t cols, int64_t ldx,
                                                         uint8_t *__restrict__ q, int64_t ldq,
                                                         uint8_t *__restrict__ scale, int64_t lds,
                                                         uint16_t *__restrict__ fq, int64_t ldf,
                                                         int64_t nseg)
{
    // quantize-only: a row block's segments run on one XCD, so each row's
    // scale line fills inside one L2 (as the MXFP4 quantizer does)
    constexpr int kRowsT = rows_row_tile(kQ, kFQ);
    int64_t seg, rb;
    if (kQ && !kFQ) {
        if (!xcd_row_tile(nseg, (rows + kRowsT - 1) / kRowsT, seg, rb)) return;
    } else {
        seg = blockIdx.x % nseg;
        rb = blockIdx.x / nseg;
    }
    mx_row_tile<kQ, kFQ, kRowsT>(x, rows, cols, ldx, q, ldq, scale, lds, fq, ldf, seg, rb);
}

// ---------------------------------------------------------------------------
// Body of the transposed column-wise kernel (+ row-wise + fake-quant), one
// read of x.  Two waves hold one 32-row group x 256 columns in registers,
// 16 rows each (16 x 8 bytes per lane, 4 columns each): the column amax is an
// in-lane max over a wave's 16 loads, combined with the other half's through
// LDS behind one barrier; the row amax is a max over the 8 lanes of a
// 32-element group.  Column codes go through the hardware convert two rows
// at a time (the pair it converts must share one scale, i.e. one column).
// ---------------------------------------------------------------------------
// Column codes go to the transposed layout: staged in LDS as
// lds_t[column slot][row] (column slot j*64 + lane for the lane's column j,
// kTPitch dwords per slot) for the workgroup to write out as whole rows of
// qt; the column scales are staged after them, one dword (the workgroup's 4
// groups) per column, for st [cols, nrg].
constexpr int kTPitch = 33;  // dwords per LDS column slot: 128 rows of codes + 1 (no bank conflicts)
constexpr int kSegT = 256;   // columns per transposed workgroup tile (64 lanes x 4)

// Max over the 8 lanes of one 32-element row group (4 columns per lane).
__device__ __forceinline__ uint32_t oct_max(uint32_t v)
{
    v = max(v, dpp_swap1(v));
    v = max(v, dpp_swap2(v));
    return max(v, (uint32_t)__shfl_xor((int)v, 4, kWave));
}

template <bool kRow, bool kFQRow, bool kFull>
__device__ __forceinline__ void mx_colwise_t_body(const uint16_t *__restrict__ x, int64_t rows,
                                                   int64_t cols, uint8_t *__restrict__ qr,
                                                   uint8_t *__restrict__ sr,
                                                   uint16_t *__restrict__ fq_row, int64_t g,
                                                   int half, int64_t col,
                                                   uint32_t *__restrict__ lds_t,
                                                   uint2 *__restrict__ xm, bool active)
{
    constexpr bool kRowAny = kRow || kFQRow;
    const bool cin = kFull || col < cols;
    const int64_t r0 = g * 32 + half * 16;
    const int64_t ngr = cols >> 5;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    uint2 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        v[i] = make_uint2(0, 0);
        if (active && (kFull || (cin && r0 + i < rows))) v[i] = ld8<kNTLoad>(x + (r0 + i) * cols + col);
    }
    // column scales: in-lane amax over this half's 16 rows, then the other
    // half's (the partner wave, wave ^ 1) through LDS
    uint32_t m0 = 0, m1 = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        m0 = pk_max_u16(m0, mag2(v[i].x));
        m1 = pk_max_u16(m1, mag2(v[i].y));
    }
    xm[wave * kWave + lane] = make_uint2(m0, m1);
    __syncthreads();
    const uint2 o = xm[(wave ^ 1) * kWave + lane];
    m0 = pk_max_u16(m0, o.x);
    m1 = pk_max_u16(m1, o.y);
    if (!active) return;  // wave-uniform: a group past the last row (after the barrier)
    uint32_t s[4];
    bool nan[4];
    uint32_t lim2[2];
    float sf[4];
    int e[4];
    bool col_slow;
    {
        const uint32_t am[4] = {m0 & 0xFFFFu, m0 >> 16, m1 & 0xFFFFu, m1 >> 16};
        bool any_nan = false;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            s[j] = mx_scale_byte(am[j]);
            nan[j] = s[j] == 0xFFu;
            any_nan |= nan[j];
            sf[j] = e8m0_to_f32(s[j]);
            e[j] = 7 - (int)s[j];
        }
#pragma unroll
        for (int k = 0; k < 2; ++k)
            lim2[k] = mx_limit_bf16(s[2 * k]) | (mx_limit_bf16(s[2 * k + 1]) << 16);
        if (cin && half == 0) {
            // byte `group` of the column's dword: the workgroup's 4 groups of it
            uint8_t *lds_s = reinterpret_cast<uint8_t *>(lds_t + kSegT * kTPitch);
            const int gl = wave >> 1;
#pragma unroll
            for (int j = 0; j < 4; ++j) lds_s[(lane * 4 + j) * 4 + gl] = (uint8_t)s[j];
        }
        col_slow = wave_any(any_nan);  // a NaN/Inf column in the wave: exact software path
    }
    // codes of rows i-2, i-1 wait here until rows i, i+1 complete a 4-row
    // dword per column
    uint32_t tq0 = 0u, tq1 = 0u;
    const int dw0 = (wave >> 1) * 8 + half * 4;  // first dword of this half's rows in a slot
    static_for<0, 16, 2>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        uint32_t a0, b0;  // rows i and i+1, the lane's 4 columns
        if (!col_slow) {
            // the pair fed to one convert shares a scale: same column, rows i and i+1
            const uint32_t rp0 = e4m3_colpair_hw(clamp_mag2(v[i].x, lim2[0]),
                                                 clamp_mag2(v[i + 1].x, lim2[0]), sf[0], sf[1]);
            const uint32_t rp1 = e4m3_colpair_hw(clamp_mag2(v[i].y, lim2[1]),
                                                 clamp_mag2(v[i + 1].y, lim2[1]), sf[2], sf[3]);
            a0 = __builtin_amdgcn_perm(rp1, rp0, 0x06040200u);
            b0 = __builtin_amdgcn_perm(rp1, rp0, 0x07050301u);
        } else {
            a0 = e4m3x4_col(v[i].x, v[i].y, e[0], e[1], e[2], e[3], nan[0], nan[1], nan[2], nan[3]);
            b0 = e4m3x4_col(v[i + 1].x, v[i + 1].y, e[0], e[1], e[2], e[3], nan[0], nan[1], nan[2],
                            nan[3]);
        }
        if (i % 4 == 0) {
            tq0 = a0;
            tq1 = b0;
        } else {
            // 4x4 byte transpose: rows i-2..i+1 x the lane's 4 columns -> one
            // dword (4 consecutive rows) per column
            const uint32_t lo01 = __builtin_amdgcn_perm(tq1, tq0, 0x05010400u);
            const uint32_t hi01 = __builtin_amdgcn_perm(tq1, tq0, 0x07030602u);
            const uint32_t lo23 = __builtin_amdgcn_perm(b0, a0, 0x05010400u);
            const uint32_t hi23 = __builtin_amdgcn_perm(b0, a0, 0x07030602u);
            const uint32_t cw[4] = {__builtin_amdgcn_perm(lo23, lo01, 0x05040100u),
                                    __builtin_amdgcn_perm(lo23, lo01, 0x07060302u),
                                    __builtin_amdgcn_perm(hi23, hi01, 0x05040100u),
                                    __builtin_amdgcn_perm(hi23, hi01, 0x07060302u)};
#pragma unroll
            for (int j = 0; j < 4; ++j)
                lds_t[(j * kWave + lane) * kTPitch + dw0 + i / 4] = cw[j];
        }
    });
    // then the row-wise work, row by row: a group of 32 is 8 lanes, each with
    // one dword of 4 codes
    if (kRowAny) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t r = r0 + i;
            const bool ok = kFull || (cin && r < rows);
            const uint32_t am = pk_max_u16(mag2(v[i].x), mag2(v[i].y));
            const uint32_t sb = mx_scale_byte(oct_max(max(am & 0xFFFFu, am >> 16)));
            const uint32_t lim = mx_limit_bf16(sb);
            const float rsf = e8m0_to_f32(sb);
            uint32_t c = e4m3x4_row_hw(v[i].x, v[i].y, lim | (lim << 16), rsf);
            const bool nan_group = sb == 0xFFu;
            if (nan_group) c = 0x7F7F7F7Fu | signs4(v[i].x, v[i].y);
            if (kRow && ok) {
                st4<kNTStore>(qr + r * cols + col, c);
                sr[r * ngr + (col >> 5)] = (uint8_t)sb;  // same byte from the group's 8 lanes
            }
            if (kFQRow) {  // a NaN/Inf group in this row of the wave: exact software path
                const uint2 d = wave_any(nan_group) ? mx_dequant4(c, (int)sb - 7, nan_group)
                                                    : mx_dequant4_hw(c, rsf);
                if (ok) st8<kNTStore>(fq_row + r * cols + col, d);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Column-wise (+ row-wise + fake-quant) in one read of x, one 32-row group x
// 512 columns per workgroup: kW waves hold 32 / kW rows each (rows
// g*32 + wave + kW*i), so a wave keeps few rows in registers and more waves
// fit on a SIMD.  The column amax is each wave's in-lane max over its rows,
// combined through 4 (kW = 4) or 8 KiB of LDS after one barrier.  Each wave
// stores its rows' row-wise codes and scales before that barrier; after it,
// the wave encodes its rows column-wise, then writes their fake-quant rows.
// Against the earlier form, one wave per 32-row
// group (128 VGPRs of x, 2 waves per SIMD), on MI355X with cold inputs: the
// one pass 11% faster with 8 waves, column-only 10% faster with 4; 16 waves
// of 2 rows were slower, and so was a cap of 64 VGPRs for 8 waves.
// ---------------------------------------------------------------------------
template <bool kCol, bool kRow, bool kFQRow, bool kFQCol, bool kFull, int kW>
__device__ __forceinline__ void mx_colsplit_body(
    const uint16_t *__restrict__ x, int64_t rows, int64_t cols, uint8_t *__restrict__ qc,
    uint8_t *__restrict__ sc, uint8_t *__restrict__ qr, uint8_t *__restrict__ sr,
    uint16_t *__restrict__ fq_row, uint16_t *__restrict__ fq_col, int64_t g, int64_t col,
    uint4 *__restrict__ part)
{
    constexpr int kRW = 32 / kW;  // rows per wave
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const bool cin = kFull || col < cols;
    const int64_t r0 = g * 32 + wave;
    const int64_t ngr = cols >> 5;

    uint4 v[kRW];
#pragma unroll
    for (int i = 0; i < kRW; ++i) {
        const int64_t r = r0 + kW * i;
        v[i] = make_uint4(0, 0, 0, 0);
        if (kFull || (cin && r < rows)) v[i] = ld16<kNTLoad>(x + r * cols + col);
    }
    uint32_t m0 = 0, m1 = 0, m2 = 0, m3 = 0;
#pragma unroll
    for (int i = 0; i < kRW; ++i) {
        m0 = pk_max_u16(m0, mag2(v[i].x));
        m1 = pk_max_u16(m1, mag2(v[i].y));
        m2 = pk_max_u16(m2, mag2(v[i].z));
        m3 = pk_max_u16(m3, mag2(v[i].w));
    }
    auto row_codes = [&](int i) __attribute__((always_inline)) {
        const int64_t r = r0 + kW * i;
        const bool ok = kFull || (cin && r < rows);
        const MxRow8 m = mx_row_encode8(v[i]);
        if (ok) {
            st8<kNTStore>(qr + r * cols + col, make_uint2(m.c0, m.c1));
            sr[r * ngr + (col >> 5)] = (uint8_t)m.s;  // same byte from the 4 lanes of a quad
        }
    };
    // the row-wise codes and scales need no other wave's data: storing them
    // before the barrier keeps this wave's stores in flight while it waits.
    // On the one pass this measured 1.9% faster than storing them after the
    // column codes (117.9 against 120.1 us, faster in 15 of 15 paired rounds;
    // 2% for the launch without fake-quant)
    if (kRow) {
        static_for<0, kRW, 1>([&](auto ic) __attribute__((always_inline)) {
            row_codes(decltype(ic)::value);
        });
    }
    part[wave * kWave + lane] = make_uint4(m0, m1, m2, m3);
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kW; ++w) {
        const uint4 p = part[w * kWave + lane];
        m0 = pk_max_u16(m0, p.x);
        m1 = pk_max_u16(m1, p.y);
        m2 = pk_max_u16(m2, p.z);
        m3 = pk_max_u16(m3, p.w);
    }
    const uint32_t am[8] = {m0 & 0xFFFFu, m0 >> 16, m1 & 0xFFFFu, m1 >> 16,
                            m2 & 0xFFFFu, m2 >> 16, m3 & 0xFFFFu, m3 >> 16};
    uint32_t s[8];
    bool nan[8];
    float sf[8];
    int e[8];
    bool any_nan = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        s[j] = mx_scale_byte(am[j]);
        nan[j] = s[j] == 0xFFu;
        any_nan |= nan[j];
        sf[j] = e8m0_to_f32(s[j]);
        e[j] = 7 - (int)s[j];
    }
    uint32_t lim2[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        lim2[k] = mx_limit_bf16(s[2 * k]) | (mx_limit_bf16(s[2 * k + 1]) << 16);
    if (kCol && cin && wave == 0) {
        const uint32_t lo = s[0] | (s[1] << 8) | (s[2] << 16) | (s[3] << 24);
        const uint32_t hi = s[4] | (s[5] << 8) | (s[6] << 16) | (s[7] << 24);
        st8<kNTStore>(sc + g * cols + col, make_uint2(lo, hi));
    }
    const bool col_slow = wave_any(any_nan);

    auto put_col_row = [&](int i, uint32_t c0, uint32_t c1) __attribute__((always_inline)) {
        const int64_t r = r0 + kW * i;
        const bool ok = kFull || (cin && r < rows);
        if (kCol && ok) st8<kNTStore>(qc + r * cols + col, make_uint2(c0, c1));
        if (kFQCol) {
            uint32_t bb[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bb[j] = mx_dequant1((c0 >> (8 * j)) & 0xFFu, (int)s[j] - 7, nan[j]);
                bb[4 + j] = mx_dequant1((c1 >> (8 * j)) & 0xFFu, (int)s[4 + j] - 7, nan[4 + j]);
            }
            if (ok)
                st16<kNTStore>(fq_col + r * cols + col,
                               make_uint4(bb[0] | (bb[1] << 16), bb[2] | (bb[3] << 16),
                                          bb[4] | (bb[5] << 16), bb[6] | (bb[7] << 16)));
        }
    };
    auto row_fake_quant = [&](int i) __attribute__((always_inline)) {
        const int64_t r = r0 + kW * i;
        const bool ok = kFull || (cin && r < rows);
        const MxRow8 m = mx_row_encode8(v[i]);
        const bool nan_group = m.s == 0xFFu;
        uint2 lo, hi;
        if (wave_any(nan_group)) {
            lo = mx_dequant4(m.c0, (int)m.s - 7, nan_group);
            hi = mx_dequant4(m.c1, (int)m.s - 7, nan_group);
        } else {
            lo = mx_dequant4_hw(m.c0, m.sf);
            hi = mx_dequant4_hw(m.c1, m.sf);
        }
        if (ok) st16<kNTStore>(fq_row + r * cols + col, make_uint4(lo.x, lo.y, hi.x, hi.y));
    };
    static_for<0, kRW, 2>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        uint32_t a0, a1, b0, b1;  // rows i and i+1 of the wave: columns 0-3 and 4-7 of the lane
        if (!col_slow) {
            const uint32_t a[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
            const uint32_t b[4] = {v[i + 1].x, v[i + 1].y, v[i + 1].z, v[i + 1].w};
            uint32_t rp[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                rp[k] = e4m3_colpair_hw(clamp_mag2(a[k], lim2[k]), clamp_mag2(b[k], lim2[k]),
                                        sf[2 * k], sf[2 * k + 1]);
            a0 = __builtin_amdgcn_perm(rp[1], rp[0], 0x06040200u);
            a1 = __builtin_amdgcn_perm(rp[3], rp[2], 0x06040200u);
            b0 = __builtin_amdgcn_perm(rp[1], rp[0], 0x07050301u);
            b1 = __builtin_amdgcn_perm(rp[3], rp[2], 0x07050301u);
        } else {
            a0 = e4m3x4_col(v[i].x, v[i].y, e[0], e[1], e[2], e[3], nan[0], nan[1], nan[2], nan[3]);
            a1 = e4m3x4_col(v[i].z, v[i].w, e[4], e[5], e[6], e[7], nan[4], nan[5], nan[6], nan[7]);
            b0 = e4m3x4_col(v[i + 1].x, v[i + 1].y, e[0], e[1], e[2], e[3], nan[0], nan[1], nan[2],
                            nan[3]);
            b1 = e4m3x4_col(v[i + 1].z, v[i + 1].w, e[4], e[5], e[6], e[7], nan[4], nan[5], nan[6],
                            nan[7]);
        }
        put_col_row(i, a0, a1);
        put_col_row(i + 1, b0, b1);
    });
    // then the fake-quant rows, each row encoded again from x (still in
    // registers).  Writing each row's codes and fake-quant together measured
    // 0.8% slower on the one pass than codes first (119.6 against 118.7 us),
    // and keeping the codes in registers for this loop instead of re-encoding
    // was slower again
    if (kFQRow) {
        static_for<0, kRW, 1>([&](auto ic) __attribute__((always_inline)) {
            row_fake_quant(decltype(ic)::value);
        });
    }
}

template <bool kCol, bool kRow, bool kFQRow, bool kFQCol, int kW>
__global__ __launch_bounds__(64 * kW) void mx_colwise_kernel(
    const uint16_t *__restrict__ x, int64_t rows, int64_t cols, uint8_t *__restrict__ qc,
    uint8_t *__restrict__ sc, uint8_t *__restrict__ qr, uint8_t *__restrict__ sr,
    uint16_t *__restrict__ fq_row, uint16_t *__restrict__ fq_col, int64_t nseg)
{
    __shared__ uint4 part[kW * kWave];
    // With row-wise outputs, all segments of a group run on one XCD (1.2% faster
    // there on MI355X; column-only measured 1.5% slower that way, so it keeps
    // the segment-fastest order).  Workgroup-uniform exit, before the barrier.
    int64_t seg, g;  // g: 32-row group
    if (kRow || kFQRow) {
        if (!xcd_row_tile(nseg, (rows + 31) / 32, seg, g)) return;
    } else {
        seg = blockIdx.x % nseg;
        g = blockIdx.x / nseg;
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t col = seg * kSeg + lane * 8;
    if ((seg + 1) * kSeg <= cols && g * 32 + 32 <= rows)
        mx_colsplit_body<kCol, kRow, kFQRow, kFQCol, true, kW>(x, rows, cols, qc, sc, qr, sr,
                                                               fq_row, fq_col, g, col, part);
    else
        mx_colsplit_body<kCol, kRow, kFQRow, kFQCol, false, kW>(x, rows, cols, qc, sc, qr, sr,
                                                                fq_row, fq_col, g, col, part);
}

// ---------------------------------------------------------------------------
// Column-wise in the transposed layout (+ optional row-wise and fake-quant),
// one read of x.  The eight waves of a workgroup quantize 128 rows x 256
// columns (mx_colwise_t_body, two waves per 32-row group), staging the
// column codes and scales in LDS; after a barrier the workgroup writes them out:
// column c's 128 codes are 128 contiguous bytes of qt (8 lanes, 16-byte
// stores) and its 4 scales one dword of st.  Measured on MI355X against
// alternatives (cold [16384, 7168] input): 4 columns per lane (256-column
// tiles, a wave per group, 156 VGPRs, 3 waves per SIMD) ran 4% faster than 8
// per lane (512-column tiles, 2 waves per SIMD) both column-only and in one
// pass -- after its loads a wave converts half as much; splitting each group
// over two waves of 16 rows (93 VGPRs, two 8-wave workgroups per CU) gained
// another 1.5% in one pass (135.4 against 137.4 us), within 1% column-only.
// For column codes only, earlier forms: codes stored straight from registers,
// 16-byte pieces of 64 lines per instruction, 3.1 TB/s (1.4 with streaming stores);
// scale bytes stored straight from registers 4.67 TB/s; a persistent
// workgroup loading its next tile while writing one out was 3-5% slower.
// ---------------------------------------------------------------------------
// Workgroup order.  A line of st (128 groups of one column) collects 4 bytes
// from each of 32 workgroups: the 32 row bands of one segment.  Column-only
// launches run those 32 back to back on one XCD, so the pieces merge in that
// XCD's L2 before write-back: on MI355X this removed the +9.7% of extra HBM
// writes and took [16384, 7168] from 73.6 to 68.1 us.  With the row-wise
// outputs as well, the plain segment-fastest order measured 1-3% faster than
// a row block's segments on one XCD, with 512- and with 256-column tiles, and
// 2-11% faster than units of 8, 32 or 128 row bands per XCD.
template <bool kRow, bool kFQRow>
constexpr bool kColTUnits = !kRow && !kFQRow;

template <bool kRow, bool kFQRow>
__global__ __launch_bounds__(512) void mx_colwise_t_kernel(
    const uint16_t *__restrict__ x, int64_t rows, int64_t cols, uint8_t *__restrict__ qt,
    int64_t ldt, uint8_t *__restrict__ st, uint8_t *__restrict__ qr, uint8_t *__restrict__ sr,
    uint16_t *__restrict__ fq_row, int64_t nseg)
{
    __shared__ uint32_t lds_t[kSegT * kTPitch + kSegT];
    __shared__ uint2 xm[8 * kWave];  // the two halves' column maxima of each group
    int64_t seg, rb;
    if (kColTUnits<kRow, kFQRow>) {
        // workgroups in units of 32 consecutive row bands of one segment,
        // unit u on XCD u % 8 (workgroup i runs on XCD i % 8)
        const int64_t nrb = (rows + kColTileRows - 1) / kColTileRows, nrbb = (nrb + 31) / 32;
        const int64_t kk = blockIdx.x / 8;
        const int64_t unit = (kk / 32) * 8 + blockIdx.x % 8;
        if (unit >= nseg * nrbb) return;  // workgroup-uniform, before any barrier
        seg = unit / nrbb;
        rb = (unit % nrbb) * 32 + kk % 32;
        if (rb >= nrb) return;            // workgroup-uniform
    } else {
        seg = blockIdx.x % nseg;
        rb = blockIdx.x / nseg;
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    const int64_t col = seg * kSegT + lane * 4;
    const int64_t g = rb * (kColTileRows / 32) + (wave >> 1);  // 32-row group index
    const int half = wave & 1;                                  // its rows 16*half..16*half+15
    const int64_t nrg = (rows + 31) / 32;
    {
        const bool active = g * 32 < rows;  // wave-uniform; every wave reaches both barriers
        if ((seg + 1) * kSegT <= cols && g * 32 + 32 <= rows)
            mx_colwise_t_body<kRow, kFQRow, true>(x, rows, cols, qr, sr, fq_row, g, half, col,
                                                  lds_t, xm, active);
        else
            mx_colwise_t_body<kRow, kFQRow, false>(x, rows, cols, qr, sr, fq_row, g, half, col,
                                                   lds_t, xm, active);
    }
    __syncthreads();
    {
        // scales: the tile's 4 groups of each column, one dword when st rows
        // are dword-aligned (nrg % 4 == 0; st itself is 4-byte aligned)
        const uint32_t *lds_s = lds_t + kSegT * kTPitch;
        const int64_t g0 = rb * 4;
        for (int cl = threadIdx.x; cl < kSegT; cl += 512) {
            const int64_t c = seg * kSegT + cl;
            if (c >= cols) continue;
            const uint32_t w4 = lds_s[cl];
            if (g0 + 4 <= nrg && (nrg & 3) == 0) {
                *reinterpret_cast<uint32_t *>(st + c * nrg + g0) = w4;
            } else {
                for (int b = 0; b < 4 && g0 + b < nrg; ++b)
                    st[c * nrg + g0 + b] = (uint8_t)(w4 >> (8 * b));
            }
        }
    }
    // write-out: LDS slot ridx holds column (ridx % 64) * 4 + ridx / 64 of the
    // tile; 8 threads per slot, 16 rows (one dword quad) each.  Rows and
    // columns past the tensor's edge hold codes of nothing and are skipped.
    const int k = threadIdx.x & 7;
    const int64_t r = rb * kColTileRows + k * 16;
#pragma unroll 4
    for (int it = 0; it < kSegT / 64; ++it) {
        const int ridx = it * 64 + (threadIdx.x >> 3);
        const int64_t c = seg * kSegT + (ridx & (kWave - 1)) * 4 + (ridx >> 6);
        const uint32_t *src = lds_t + ridx * kTPitch + k * 4;
        const uint4 w = make_uint4(src[0], src[1], src[2], src[3]);
        if (c >= cols || r >= rows) continue;
        uint8_t *dst = qt + c * ldt + r;
        if (r + 16 <= rows) {
            st16<kNTStore>(dst, w);
        } else {
            for (int b = 0; b < (int)(rows - r); ++b) {
                const uint32_t word = b < 4 ? w.x : b < 8 ? w.y : b < 12 ? w.z : w.w;
                dst[b] = (uint8_t)(word >> (8 * (b & 3)));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Dequantize: out = bf16_RNE(E4M3(q) * 2^(s - 127)), row (axis 1) or column
// (axis 0) groups.  Tiles: 512-column segment x kRowsDq rows.
// ---------------------------------------------------------------------------
template <int kAxis>
__global__ __launch_bounds__(256) void mx_dequant_kernel(const uint8_t *__restrict__ q,
                                                         const uint8_t *__restrict__ scale,
                                                         int64_t rows, int64_t cols,
                                                         uint16_t *__restrict__ out, int64_t nseg)
{
    int64_t seg, rb;
    if (kAxis == 0) {
        // the 32 / kRowsDq tiles of one column group run back to back on one
        // XCD, so its scale row is fetched into one L2 once
        constexpr int kSub = 32 / kRowsDq;
        int64_t sp, gi;
        if (!xcd_row_tile(nseg * kSub, (rows + 31) / 32, sp, gi)) return;
        seg = sp / kSub;
        rb = gi * kSub + sp % kSub;
    } else {
        // a row block's segments run back to back on one XCD, so each row's
        // scale line is fetched into one L2 once (+18.6% HBM reads with the
        // plain order, time within noise either way)
        if (!xcd_row_tile(nseg, (rows + kRowsDq - 1) / kRowsDq, seg, rb)) return;
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    const int64_t col = seg * kSeg + lane * 8;
    if (col >= cols) return;  // no barriers below
    const int64_t r0 = rb * kRowsDq + wave;
    // all of the wave's codes and scales in flight before any is decoded
    constexpr int kR = kRowsDq / 4;
    uint2 cc[kR];
    uint32_t ss[kR];
    // column groups: the tile's rows lie in one group row, so one scale load
    static_assert(32 % kRowsDq == 0, "a dequantize tile lies in one column-group row");
    const int64_t grow = (rb * kRowsDq) >> 5;  // the tile's column-group row
    const uint2 sv = kAxis == 0 && r0 < rows
                         ? *reinterpret_cast<const uint2 *>(scale + grow * cols + col)
                         : make_uint2(0, 0);
#pragma unroll
    for (int i = 0; i < kR; ++i) {
        const int64_t r = r0 + 4 * i;
        cc[i] = make_uint2(0, 0);
        ss[i] = 0u;
        if (r < rows) {
            cc[i] = *reinterpret_cast<const uint2 *>(q + r * cols + col);
            if (kAxis == 1) ss[i] = scale[r * (cols >> 5) + (col >> 5)];
        }
    }
    // a 0xFF (NaN) scale byte among the column scales?
    const bool nan_scale = ((((~sv.x) - 0x01010101u) & sv.x) | (((~sv.y) - 0x01010101u) & sv.y)) &
                           0x80808080u;
#pragma unroll
    for (int i = 0; i < kR; ++i) {
        const int64_t r = r0 + 4 * i;
        if (r >= rows) break;  // wave-uniform
        const uint2 c = cc[i];
        uint32_t b[8];
        if (kAxis == 1) {
            const uint32_t s = ss[i];
            const bool nan = s == 0xFFu;
            // a byte of the form S.1111.111 (NaN code) in either word?
            const uint32_t tx = c.x & 0x7F7F7F7Fu, ty = c.y & 0x7F7F7F7Fu;
            const bool nan_code = (((tx + 0x01010101u) | (ty + 0x01010101u)) & 0x80808080u) != 0u;
            uint2 lo, hi;
            if (wave_any(nan || nan_code)) {
                lo = mx_dequant4(c.x, (int)s - 7, nan);
                hi = mx_dequant4(c.y, (int)s - 7, nan);
            } else {
                const float sf = e8m0_to_f32(s);
                lo = mx_dequant4_hw(c.x, sf);
                hi = mx_dequant4_hw(c.y, sf);
            }
            b[0] = lo.x; b[1] = lo.y; b[2] = hi.x; b[3] = hi.y;
        } else {
            const uint32_t tx = c.x & 0x7F7F7F7Fu, ty = c.y & 0x7F7F7F7Fu;
            const bool nan_code = (((tx + 0x01010101u) | (ty + 0x01010101u)) & 0x80808080u) != 0u;
            uint32_t w[4];
            if (wave_any(nan_code || nan_scale)) {
#pragma unroll
                for (int j = 0; j < 8; j += 2) {
                    const uint32_t cw = j < 4 ? c.x : c.y;
                    const uint32_t sw = j < 4 ? sv.x : sv.y;
                    const int sh = 8 * (j & 3);
                    const uint32_t s0 = (sw >> sh) & 0xFFu, s1 = (sw >> (sh + 8)) & 0xFFu;
                    const uint32_t d0 = mx_dequant1((cw >> sh) & 0xFFu, (int)s0 - 7, s0 == 0xFFu);
                    const uint32_t d1 = mx_dequant1((cw >> (sh + 8)) & 0xFFu, (int)s1 - 7,
                                                    s1 == 0xFFu);
                    w[j / 2] = d0 | (d1 << 16);
                }
            } else {
                // one scale per column: E4M3 -> fp32 exactly (v_cvt_pk_f32_fp8), times
                // the column's power of two (exact, subnormals kept), bf16 RNE
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t cw = h ? c.y : c.x, sw = h ? sv.y : sv.x;
                    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw, false);
                    const f32x2 bb = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw, true);
                    w[2 * h] = bf16x2_rne(a.x * e8m0_to_f32(sw & 0xFFu),
                                          a.y * e8m0_to_f32((sw >> 8) & 0xFFu));
                    w[2 * h + 1] = bf16x2_rne(bb.x * e8m0_to_f32((sw >> 16) & 0xFFu),
                                              bb.y * e8m0_to_f32(sw >> 24));
                }
            }
            b[0] = w[0]; b[1] = w[1]; b[2] = w[2]; b[3] = w[3];
        }
        st16<kNTStore>(out + r * cols + col, make_uint4(b[0], b[1], b[2], b[3]));
    }
}

// ---------------------------------------------------------------------------
// Grouped row-wise: one workgroup per tile of the flattened (tensor, tile)
// space.  The tensor is found by a 64-way search over a compact int32 array
// of first-tile indices (1.5 KiB for 384 tensors), so a workgroup reaches its
// first load after a few short dependent reads.
// (Measured against a persistent grid walking runs of tiles: the one-shot form
// was 7% faster on the 384 MoE expert tensors, letting the hardware overlap
// the tail of one tile with the next.)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mx_grouped_kernel(const GroupEntry *__restrict__ table,
                                                         const int32_t *__restrict__ starts,
                                                         int32_t n)
{
    const int32_t t = (int32_t)blockIdx.x;
    const int lo = find_entry(starts, n, t);
    const GroupEntry E = table[lo];
    const int32_t local = t - starts[lo];
    const int32_t nseg = (int32_t)E.nseg;
    mx_row_tile<true, false, kRowsGrouped>(global_ptr(E.x), E.rows, E.cols, E.ldx, global_ptr(E.q),
                                        E.ldq, global_ptr(E.scale), E.lds, nullptr, 0, local % nseg,
                                        local / nseg);
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------

int64_t mx_grouped_tiles(int64_t rows, int64_t cols, int64_t *nseg)
{
    const int64_t ns = (cols + kSeg - 1) / kSeg;
    if (nseg) *nseg = ns;
    return ns * ((rows + kRowsGrouped - 1) / kRowsGrouped);
}

hipError_t launch_mx_rowwise(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t *q, int64_t ldq, uint8_t *scale, int64_t lds, uint16_t *fq,
                             int64_t ldf, hipStream_t stream)
{
    const int64_t nseg = (cols + kSeg - 1) / kSeg;
    const int kRowsT = rows_row_tile(q != nullptr, fq != nullptr);
    const int64_t nrb = (rows + kRowsT - 1) / kRowsT;
    if (nseg <= 0 || nrb <= 0) return hipSuccess;
    const int64_t tiles = (q && !fq) ? xcd_row_grid(nseg, nrb) : nseg * nrb;  // the kernel's order
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)tiles), block(256);
    if (q && fq)
        hipLaunchKernelGGL((mx_rowwise_kernel<true, true>), grid, block, 0, stream, x, rows, cols,
                           ldx, q, ldq, scale, lds, fq, ldf, nseg);
    else if (q)
        hipLaunchKernelGGL((mx_rowwise_kernel<true, false>), grid, block, kLdsCap5, stream, x,
                           rows, cols, ldx, q, ldq, scale, lds, fq, ldf, nseg);
    else
        hipLaunchKernelGGL((mx_rowwise_kernel<false, true>), grid, block, kLdsCap5, stream, x,
                           rows, cols, ldx, q, ldq, scale, lds, fq, ldf, nseg);
    return hipGetLastError();
}

hipError_t launch_mx_colwise(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *qc,
                             uint8_t *sc, uint8_t *qr, uint8_t *sr, uint16_t *fq_row,
                             uint16_t *fq_col, hipStream_t stream)
{
    const int64_t nseg = (cols + kSeg - 1) / kSeg;
    const int64_t ngroups = (rows + 31) / 32;  // one workgroup per (segment, 32-row group)
    if (nseg <= 0 || ngroups <= 0) return hipSuccess;
    const bool col = qc != nullptr, row = qr != nullptr;
    // the kernel's order: XCD-grouped when it writes row-wise outputs
    const int64_t tiles = (row || fq_row) ? xcd_row_grid(nseg, ngroups) : nseg * ngroups;
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    // 8 waves of 4 rows when row-wise outputs come too, 4 waves of 8 rows otherwise
#define MXQ_COLWISE(C, R, FR, FC, W)                                                               \
    hipLaunchKernelGGL((mx_colwise_kernel<C, R, FR, FC, W>), dim3((unsigned)tiles), dim3(64 * W), \
                       0, stream, x, rows, cols, qc, sc, qr, sr, fq_row, fq_col, nseg)
    if (col && row && fq_row) MXQ_COLWISE(true, true, true, false, 8);
    else if (col && row) MXQ_COLWISE(true, true, false, false, 8);
    else if (col && fq_row) MXQ_COLWISE(true, false, true, false, 8);
    else if (col) MXQ_COLWISE(true, false, false, false, 4);
    else if (fq_col) MXQ_COLWISE(false, false, false, true, 4);
    else return hipErrorInvalidValue;
#undef MXQ_COLWISE
    return hipGetLastError();
}

hipError_t launch_mx_colwise_t(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *qt,
                               int64_t ldt, uint8_t *st, uint8_t *qr, uint8_t *sr,
                               uint16_t *fq_row, hipStream_t stream)
{
    const int64_t nseg = (cols + kSegT - 1) / kSegT;
    const int64_t nrb = (rows + kColTileRows - 1) / kColTileRows;
    if (nseg <= 0 || nrb <= 0) return hipSuccess;
    // column-only: 32-band units spread over the 8 XCDs (kColTUnits)
    const int64_t tiles = (qr || fq_row) ? nseg * nrb : 8 * 32 * ((nseg * ((nrb + 31) / 32) + 7) / 8);
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)tiles), block(512);
#define MXQ_COLWISE_T(R, FR)                                                                       \
    hipLaunchKernelGGL((mx_colwise_t_kernel<R, FR>), grid, block, 0, stream, x, rows, cols, qt,    \
                       ldt, st, qr, sr, fq_row, nseg)
    if (qr && fq_row) MXQ_COLWISE_T(true, true);
    else if (qr) MXQ_COLWISE_T(true, false);
    else if (fq_row) MXQ_COLWISE_T(false, true);
    else MXQ_COLWISE_T(false, false);
#undef MXQ_COLWISE_T
    return hipGetLastError();
}

// E8M0 bytes -> fp32 values (2^(b - 127), 0xFF -> quiet NaN), grid-stride.
__global__ __launch_bounds__(256) void e8m0_to_f32_kernel(const uint8_t *__restrict__ s,
                                                          int64_t n, float *__restrict__ out)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * 256) {
        const uint32_t b = s[i];
        out[i] = b == 0xFFu ? __uint_as_float(0x7FC00000u) : e8m0_to_f32(b);
    }
}

hipError_t launch_e8m0_to_f32(const uint8_t *scale, int64_t n, float *out, hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    const int64_t want = (n + 255) / 256;
    const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
    hipLaunchKernelGGL(e8m0_to_f32_kernel, dim3(blocks), dim3(256), 0, stream, scale, n, out);
    return hipGetLastError();
}

hipError_t launch_mx_dequant(const uint8_t *q, const uint8_t *scale, int64_t rows, int64_t cols,
                             int axis, uint16_t *out, hipStream_t stream)
{
    const int64_t nseg = (cols + kSeg - 1) / kSeg;
    if (nseg <= 0 || rows <= 0) return hipSuccess;
    // the kernel's order: column groups (axis 0) or row blocks (axis 1) per XCD
    const int64_t tiles = axis == 0 ? xcd_row_grid(nseg * (32 / kRowsDq), (rows + 31) / 32)
                                    : xcd_row_grid(nseg, (rows + kRowsDq - 1) / kRowsDq);
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)tiles), block(256);
    if (axis == 1)
        hipLaunchKernelGGL((mx_dequant_kernel<1>), grid, block, 0, stream, q, scale, rows, cols,
                           out, nseg);
    else
        hipLaunchKernelGGL((mx_dequant_kernel<0>), grid, block, 0, stream, q, scale, rows, cols,
                           out, nseg);
    return hipGetLastError();
}

hipError_t launch_mx_grouped(const GroupEntry *table_dev, const int32_t *starts_dev, int32_t n,
                             int64_t total_tiles, hipStream_t stream)
{
    if (n <= 0 || total_tiles <= 0) return hipSuccess;
    if (total_tiles > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(mx_grouped_kernel, dim3((unsigned)total_tiles), dim3(256), kLdsCap5,
                       stream, table_dev, starts_dev, n);
    return hipGetLastError();
}

}  // namespace mxq
