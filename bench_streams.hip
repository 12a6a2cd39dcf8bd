// bench_streams.hip -- streaming-ceiling kernels for bench.py (measurement
// only; not part of the quantizer library).
//
// Each kernel moves the bytes of one quantizer's read:write mix with trivial
// arithmetic, so its rate is what the memory system gives that mix and that
// access pattern.  bench.py takes, per mix, the best of several patterns as
// the ceiling it reports beside the quantizer kernels:
//   tiled  one workgroup per 512-column x (4 waves x R rows) tile of a
//          [rows, cols] tensor (the quantizers' own tile shape), in the
//          plain segment-fastest order or the quantizers' XCD order, per lane and
//          row the mix's bytes: 16 bytes of bf16 or 8 (4) bytes of codes read,
//          8 / 16 / 4 bytes written per plane, and one byte per lane quad and
//          row (a scale byte per 32 elements) where the mix has scales; and
//          the same with half-width lanes: 256-column tiles, 4 elements per
//          lane (8 bytes of bf16), a scale byte per lane octet;
//   flat   a grid-stride walk over the tensor as one array, U vectors in
//          flight per lane, the same bytes per element without scales.
// Read-only kernels fold what they load into a word that is stored only if it
// equals a value no input here produces (so the loads stay); write-only
// kernels store a pattern without loading.
//
// Mixes, bytes per element read : written (kind numbers in parentheses):
//   read 2:0 (0)   write 0:2 (1)   copy 2:2 (2, fake-quant)
//   row 2:1+1/32 (3, MXFP8 quantize)   onepass 2:4+1/32 (4, codes of both axes,
//   row scales, fake-quant)   dequant 1+1/32:2 (5, MXFP8 / FP8 dequantize)
//   fp4 2:1/2+1/32 (6, MXFP4 / NVFP4 encode)   fp4dq 1/2+1/32:2 (7, FP4 dequantize)
//   requant 1:1+1/32 (8, FP8 block -> MXFP8: codes in, codes and scales out)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq_device.hpp"

namespace {

using mxq::ld16;
using mxq::ld4;
using mxq::ld8;
using mxq::st16;
using mxq::st4;
using mxq::st8;

constexpr uint32_t kNever = 0x9E3779B9u;  // the fold of loaded words is compared against this
constexpr int kKinds = 9;

// What each mix reads and writes per lane and row (tiled) or per element group (flat).
template <int K>
struct Mix {
    static constexpr int rd = (K == 1) ? 0 : (K == 5 || K == 8) ? 8 : (K == 7) ? 4 : 16;  // read
    static constexpr int w8 = (K == 3) ? 1 : (K == 4) ? 2 : 0;                  // 8-byte planes
    static constexpr int w16 = (K == 1 || K == 2 || K == 4 || K == 5 || K == 7) ? 1 : 0;
    static constexpr int w4 = (K == 6) ? 1 : 0;                                 // 4-byte planes
    static constexpr int w8b = (K == 8) ? 1 : 0;  // 8-byte plane in o8b (codes read from o8a)
    static constexpr bool sc_wr = K == 3 || K == 4 || K == 6 || K == 8;         // scale byte written
    static constexpr bool sc_rd = K == 5 || K == 7;                             // scale byte read
    static constexpr bool writes = w8 + w16 + w4 + w8b > 0 || sc_wr;
};

// x: the bf16 input for 16-byte reads; codes (o8a) for 8- and 4-byte reads.
template <int R, int K, bool X>
__global__ __launch_bounds__(256) void tiled_kernel(const uint16_t *__restrict__ x, int64_t rows,
                                                    int64_t cols, int64_t nseg,
                                                    uint8_t *__restrict__ o8a,
                                                    uint8_t *__restrict__ o8b,
                                                    uint16_t *__restrict__ o16,
                                                    uint8_t *__restrict__ sc,
                                                    uint32_t *__restrict__ sink)
{
    using M = Mix<K>;
    // X: the quantizers' order, a row block's segments on one XCD (so a
    // row's scale line fills inside one L2); else segment-fastest
    int64_t seg, rb;
    if (X) {
        if (!mxq::xcd_row_tile(nseg, (rows + 4 * R - 1) / (4 * R), seg, rb)) return;
    } else {
        seg = blockIdx.x % nseg;
        rb = blockIdx.x / nseg;
    }
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t col = seg * 512 + lane * 8;
    const int64_t r0 = rb * (4 * R) + wave;
    uint4 v[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int64_t r = r0 + 4 * i;
        v[i] = make_uint4((uint32_t)r, (uint32_t)col, 1u, 2u);
        if (r >= rows) continue;
        if (M::rd == 16) {
            v[i] = ld16<true>(x + r * cols + col);
        } else if (M::rd == 8) {
            const uint2 c = ld8<false>(o8a + r * cols + col);
            v[i] = make_uint4(c.x, c.y, c.x ^ 1u, c.y ^ 2u);
        } else if (M::rd == 4) {
            const uint32_t c = ld4<false>(o8a + r * (cols >> 1) + (col >> 1));
            v[i] = make_uint4(c, c ^ 1u, c ^ 2u, c ^ 3u);
        }
        if (M::sc_rd) v[i].w ^= sc[r * (cols >> 5) + (col >> 5)];
    }
    uint32_t fold = 0;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int64_t r = r0 + 4 * i;
        if (r >= rows) continue;
        const uint2 c = make_uint2(__builtin_amdgcn_perm(v[i].y, v[i].x, 0x06040200u),
                                   __builtin_amdgcn_perm(v[i].w, v[i].z, 0x06040200u));
        if (M::w8 > 0) st8<true>(o8a + r * cols + col, c);
        if (M::w8 > 1) st8<true>(o8b + r * cols + col, make_uint2(c.y, c.x));
        if (M::w16 > 0) st16<true>(o16 + r * cols + col, v[i]);
        if (M::w4 > 0) st4<true>(o8b + r * (cols >> 1) + (col >> 1), c.x ^ c.y);
        if (M::w8b > 0) st8<true>(o8b + r * cols + col, c);
        if (M::sc_wr) sc[r * (cols >> 5) + (col >> 5)] = (uint8_t)c.x;
        fold ^= v[i].x ^ v[i].w;
    }
    if (!M::writes && fold == kNever) sink[0] = fold;
}

// The tiled pattern with half-width lanes: 256-column tiles, 4 elements per
// lane and row (8 bytes of bf16, 4 of 8-bit codes, 2 of 4-bit codes read;
// 4 / 8 / 2 bytes written per plane).
template <int R, int K, bool X>
__global__ __launch_bounds__(256) void half_kernel(const uint16_t *__restrict__ x, int64_t rows,
                                                  int64_t cols, int64_t nseg,
                                                  uint8_t *__restrict__ o8a,
                                                  uint8_t *__restrict__ o8b,
                                                  uint16_t *__restrict__ o16,
                                                  uint8_t *__restrict__ sc,
                                                  uint32_t *__restrict__ sink)
{
    using M = Mix<K>;
    int64_t seg, rb;
    if (X) {
        if (!mxq::xcd_row_tile(nseg, (rows + 4 * R - 1) / (4 * R), seg, rb)) return;
    } else {
        seg = blockIdx.x % nseg;
        rb = blockIdx.x / nseg;
    }
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t col = seg * 256 + lane * 4;
    const int64_t r0 = rb * (4 * R) + wave;
    uint2 v[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int64_t r = r0 + 4 * i;
        v[i] = make_uint2((uint32_t)r, (uint32_t)col);
        if (r >= rows) continue;
        if (M::rd == 16) {
            v[i] = ld8<true>(x + r * cols + col);
        } else if (M::rd == 8) {
            const uint32_t c = ld4<false>(o8a + r * cols + col);
            v[i] = make_uint2(c, c ^ 1u);
        } else if (M::rd == 4) {
            const uint32_t c = *reinterpret_cast<const uint16_t *>(o8a + r * (cols >> 1) + (col >> 1));
            v[i] = make_uint2(c, c ^ 2u);
        }
        if (M::sc_rd) v[i].y ^= sc[r * (cols >> 5) + (col >> 5)];
    }
    uint32_t fold = 0;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int64_t r = r0 + 4 * i;
        if (r >= rows) continue;
        const uint32_t c = __builtin_amdgcn_perm(v[i].y, v[i].x, 0x06040200u);
        if (M::w8 > 0) st4<true>(o8a + r * cols + col, c);
        if (M::w8 > 1) st4<true>(o8b + r * cols + col, c ^ 0x01010101u);
        if (M::w16 > 0) st8<true>(o16 + r * cols + col, v[i]);
        if (M::w4 > 0)
            *reinterpret_cast<uint16_t *>(o8b + r * (cols >> 1) + (col >> 1)) = (uint16_t)(c ^ (c >> 16));
        if (M::w8b > 0) st4<true>(o8b + r * cols + col, c);
        if (M::sc_wr) sc[r * (cols >> 5) + (col >> 5)] = (uint8_t)c;
        fold ^= v[i].x ^ v[i].y;
    }
    if (!M::writes && fold == kNever) sink[0] = fold;
}

// One element group per 16 bytes of bf16 (8 elements): x as nvec 16-byte
// vectors; codes o8a as nvec 8-byte vectors (4-byte for the FP4 mixes); o8b
// nvec 8-byte vectors; o16 nvec 16-byte vectors.
template <int U, int K>
__global__ __launch_bounds__(256) void flat_kernel(const uint4 *__restrict__ x, int64_t nvec,
                                                   uint2 *__restrict__ o8a,
                                                   uint2 *__restrict__ o8b,
                                                   uint4 *__restrict__ o16,
                                                   uint32_t *__restrict__ sink)
{
    using M = Mix<K>;
    uint32_t fold = 0;
    const int64_t chunk = 256 * U;
    for (int64_t base = (int64_t)blockIdx.x * chunk; base < nvec;
         base += (int64_t)gridDim.x * chunk) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + u * 256 + threadIdx.x;
            v[u] = make_uint4((uint32_t)i, 3u, 5u, 7u);
            if (i >= nvec) continue;
            if (M::rd == 16) {
                v[u] = ld16<true>(x + i);
            } else if (M::rd == 8) {
                const uint2 c = ld8<false>(o8a + i);
                v[u] = make_uint4(c.x, c.y, c.x ^ 1u, c.y ^ 2u);
            } else if (M::rd == 4) {
                const uint32_t c = ld4<false>(reinterpret_cast<const uint32_t *>(o8a) + i);
                v[u] = make_uint4(c, c ^ 1u, c ^ 2u, c ^ 3u);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + u * 256 + threadIdx.x;
            if (i >= nvec) continue;
            if (M::w16 > 0) st16<true>(o16 + i, v[u]);
            if (M::w8 > 0) st8<true>(o8a + i, make_uint2(v[u].x, v[u].z));
            if (M::w8 > 1) st8<true>(o8b + i, make_uint2(v[u].y, v[u].w));
            if (M::w4 > 0) st4<true>(reinterpret_cast<uint32_t *>(o8b) + i, v[u].x ^ v[u].y);
            if (M::w8b > 0) st8<true>(o8b + i, make_uint2(v[u].x, v[u].z));
            fold ^= v[u].x;
        }
    }
    if (!M::writes && fold == kNever) sink[0] = fold;
}

}  // namespace

#ifndef STREAMS_BUILD_ID
#define STREAMS_BUILD_ID "unidentified"
#endif

extern "C" {

const char *bench_streams_build_id(void) { return STREAMS_BUILD_ID; }

int bench_streams_kinds(void) { return kKinds; }

// Tiled variants: variant = R index (0: R=1, 1: R=2, 2: R=4, 3: R=8) + 4 * kind
// + 4 * kinds * order (0: segment-fastest, 1: a row block's segments on one XCD)
// + 8 * kinds * width (0: 512-column tiles, 16 bytes of bf16 per lane; 1:
// 256-column tiles, 8 bytes) + 16 * kinds * cap (1: 27 KiB of unused dynamic
// LDS per workgroup, so at most 5 workgroups reside on a CU, as the row-wise
// quantizers launch).  x [rows, cols] bf16 with cols a multiple of the
// tile width; o8a, o8b [rows, cols] bytes (the codes the 8- and 4-byte reading
// kinds read are o8a); o16 [rows, cols] bf16; sc [rows, cols/32] bytes; sink
// one word.  Returns 0, 1 for a bad argument (nothing launched), 2 for a
// launch error.
int bench_stream_tiled(int variant, const void *x, int64_t rows, int64_t cols, void *o8a,
                       void *o8b, void *o16, void *sc, void *sink, void *stream)
{
    if (variant < 0 || variant >= 32 * kKinds || rows <= 0 || cols <= 0) return 1;
    const bool half = (variant / (8 * kKinds)) % 2 == 1;
    const size_t dyn = variant >= 16 * kKinds ? 27 * 1024 : 0;
    const int64_t tw = half ? 256 : 512;
    if (cols % tw != 0) return 1;
    if (!x || !o8a || !o8b || !o16 || !sc || !sink) return 1;
    const int64_t nseg = cols / tw;
    const int ri = variant % 4, kind = (variant / 4) % kKinds, xcd = (variant / (4 * kKinds)) & 1;
    const int R = 1 << ri;
    const int64_t nrb = (rows + 4 * R - 1) / (4 * R);
    const int64_t tiles = xcd ? mxq::xcd_row_grid(nseg, nrb) : nseg * nrb;
    if (tiles > 0x7FFFFFFF) return 1;
    const hipStream_t s = (hipStream_t)stream;
    const uint16_t *xp = (const uint16_t *)x;
    uint8_t *a = (uint8_t *)o8a, *b = (uint8_t *)o8b, *c = (uint8_t *)sc;
    uint16_t *f = (uint16_t *)o16;
    uint32_t *k = (uint32_t *)sink;
#define TL(RR, KK)                                                                                 \
    do {                                                                                           \
        if (half && xcd)                                                                           \
            hipLaunchKernelGGL((half_kernel<RR, KK, true>), dim3((unsigned)tiles), dim3(256), dyn, \
                               s, xp, rows, cols, nseg, a, b, f, c, k);                            \
        else if (half)                                                                             \
            hipLaunchKernelGGL((half_kernel<RR, KK, false>), dim3((unsigned)tiles), dim3(256), dyn, \
                               s, xp, rows, cols, nseg, a, b, f, c, k);                            \
        else if (xcd)                                                                              \
            hipLaunchKernelGGL((tiled_kernel<RR, KK, true>), dim3((unsigned)tiles), dim3(256), dyn, \
                               s, xp, rows, cols, nseg, a, b, f, c, k);                            \
        else                                                                                       \
            hipLaunchKernelGGL((tiled_kernel<RR, KK, false>), dim3((unsigned)tiles), dim3(256), dyn,\
                               s, xp, rows, cols, nseg, a, b, f, c, k);                            \
    } while (0)
#define TL_KIND(RR)                                                                                \
    switch (kind) {                                                                                \
    case 0: TL(RR, 0); break;                                                                      \
    case 1: TL(RR, 1); break;                                                                      \
    case 2: TL(RR, 2); break;                                                                      \
    case 3: TL(RR, 3); break;                                                                      \
    case 4: TL(RR, 4); break;                                                                      \
    case 5: TL(RR, 5); break;                                                                      \
    case 6: TL(RR, 6); break;                                                                      \
    case 7: TL(RR, 7); break;                                                                      \
    default: TL(RR, 8); break;                                                                     \
    }
    switch (R) {
    case 1: TL_KIND(1); break;
    case 2: TL_KIND(2); break;
    case 4: TL_KIND(4); break;
    default: TL_KIND(8); break;
    }
#undef TL_KIND
#undef TL
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Flat variants: variant = U index (0: U=2, 1: U=4, 2: U=8) + 3 * kind.
// x: nvec 16-byte vectors; o8a, o8b: nvec 8-byte vectors; o16: nvec 16-byte
// vectors; grid workgroups (1..65536).
int bench_stream_flat(int variant, const void *x, int64_t nvec, void *o8a, void *o8b, void *o16,
                      void *sink, int grid, void *stream)
{
    if (variant < 0 || variant >= 3 * kKinds || nvec <= 0 || grid < 1 || grid > 65536) return 1;
    if (!x || !o8a || !o8b || !o16 || !sink) return 1;
    const int ui = variant % 3, kind = variant / 3;
    const hipStream_t s = (hipStream_t)stream;
    const uint4 *xp = (const uint4 *)x;
    uint2 *a = (uint2 *)o8a, *b = (uint2 *)o8b;
    uint4 *f = (uint4 *)o16;
    uint32_t *k = (uint32_t *)sink;
#define FL(UU, KK)                                                                                 \
    hipLaunchKernelGGL((flat_kernel<UU, KK>), dim3((unsigned)grid), dim3(256), 0, s, xp, nvec, a, \
                       b, f, k)
#define FL_KIND(UU)                                                                                \
    switch (kind) {                                                                                \
    case 0: FL(UU, 0); break;                                                                      \
    case 1: FL(UU, 1); break;                                                                      \
    case 2: FL(UU, 2); break;                                                                      \
    case 3: FL(UU, 3); break;                                                                      \
    case 4: FL(UU, 4); break;                                                                      \
    case 5: FL(UU, 5); break;                                                                      \
    case 6: FL(UU, 6); break;                                                                      \
    case 7: FL(UU, 7); break;                                                                      \
    default: FL(UU, 8); break;                                                                     \
    }
    switch (ui) {
    case 0: FL_KIND(2); break;
    case 1: FL_KIND(4); break;
    default: FL_KIND(8); break;
    }
#undef FL_KIND
#undef FL
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
