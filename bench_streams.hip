// bench_streams.hip -- streaming-ceiling kernels for bench.py (measurement
// only; not part of the quantizer library).
//
// Each kernel moves the bytes of one quantizer's read:write mix with trivial
// arithmetic, so its rate is what the memory system gives that mix and that
// access pattern.  bench.py takes, per mix, the best of several patterns as
// the ceiling it reports beside the quantizer kernels:
//   tiled  one workgroup per 512-column x (4 waves x R rows) tile of a
//          [rows, cols] bf16 tensor, 16-byte streaming loads per lane and row
//          (the quantizers' own tile shape), writing N8 planes of 8 bytes and
//          N16 planes of 16 bytes per lane and row, plus one byte per lane
//          quad and row (a scale byte per 32 elements) when SC;
//   flat   a grid-stride walk over the tensor as one array of 16-byte
//          vectors, U loads in flight per lane, writing the same planes.
// Read-only variants fold what they load into a word that is stored only if
// it equals a value no input here produces (so the loads stay); write-only
// variants store a pattern without loading.
//
// Mixes (bytes per bf16 element read : written):
//   read 2:0  write 0:2  copy 2:2 (fake-quant)  row 2:1+1/32 (MXFP8 quantize)
//   onepass 2:4+1/32 (codes of both axes, row scales, fake-quant)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq_device.hpp"

namespace {

using mxq::ld16;
using mxq::st16;
using mxq::st8;

constexpr uint32_t kNever = 0x9E3779B9u;  // the fold of loaded words is compared against this

template <int R, bool kRead, int N8, int N16, bool SC>
__global__ __launch_bounds__(256) void tiled_kernel(const uint16_t *__restrict__ x, int64_t rows,
                                                    int64_t cols, int64_t nseg,
                                                    uint8_t *__restrict__ o8a,
                                                    uint8_t *__restrict__ o8b,
                                                    uint16_t *__restrict__ o16,
                                                    uint8_t *__restrict__ sc,
                                                    uint32_t *__restrict__ sink)
{
    const int64_t seg = blockIdx.x % nseg, rb = blockIdx.x / nseg;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t col = seg * 512 + lane * 8;
    const int64_t r0 = rb * (4 * R) + wave;
    uint4 v[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int64_t r = r0 + 4 * i;
        v[i] = make_uint4((uint32_t)r, (uint32_t)col, 1u, 2u);
        if (kRead && r < rows) v[i] = ld16<true>(x + r * cols + col);
    }
    uint32_t fold = 0;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int64_t r = r0 + 4 * i;
        if (r >= rows) continue;
        const uint2 c = make_uint2(__builtin_amdgcn_perm(v[i].y, v[i].x, 0x06040200u),
                                   __builtin_amdgcn_perm(v[i].w, v[i].z, 0x06040200u));
        if (N8 > 0) st8<true>(o8a + r * cols + col, c);
        if (N8 > 1) st8<true>(o8b + r * cols + col, make_uint2(c.y, c.x));
        if (N16 > 0) st16<true>(o16 + r * cols + col, v[i]);
        if (SC) sc[r * (cols >> 5) + (col >> 5)] = (uint8_t)c.x;
        fold ^= v[i].x ^ v[i].w;
    }
    if (N8 == 0 && N16 == 0 && fold == kNever) sink[0] = fold;
}

// MODE: 0 read only, 1 copy (16 B out per 16 in), 2 row mix (8 B out), 3 one-pass
// mix (8 + 8 + 16 B out), 4 write only (16 B out).
template <int U, int MODE>
__global__ __launch_bounds__(256) void flat_kernel(const uint4 *__restrict__ x, int64_t nvec,
                                                   uint2 *__restrict__ o8a,
                                                   uint2 *__restrict__ o8b,
                                                   uint4 *__restrict__ o16,
                                                   uint32_t *__restrict__ sink)
{
    uint32_t fold = 0;
    const int64_t chunk = 256 * U;
    for (int64_t base = (int64_t)blockIdx.x * chunk; base < nvec;
         base += (int64_t)gridDim.x * chunk) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + u * 256 + threadIdx.x;
            v[u] = make_uint4((uint32_t)i, 3u, 5u, 7u);
            if (MODE != 4 && i < nvec) v[u] = ld16<true>(x + i);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + u * 256 + threadIdx.x;
            if (i >= nvec) continue;
            if (MODE == 1 || MODE == 3 || MODE == 4) st16<true>(o16 + i, v[u]);
            if (MODE == 2 || MODE == 3) st8<true>(o8a + i, make_uint2(v[u].x, v[u].z));
            if (MODE == 3) st8<true>(o8b + i, make_uint2(v[u].y, v[u].w));
            fold ^= v[u].x;
        }
    }
    if (MODE == 0 && fold == kNever) sink[0] = fold;
}

}  // namespace

#ifndef STREAMS_BUILD_ID
#define STREAMS_BUILD_ID "unidentified"
#endif

extern "C" {

const char *bench_streams_build_id(void) { return STREAMS_BUILD_ID; }

// Tiled variants: variant = R index (0: R=1, 1: R=2, 2: R=4, 3: R=8) + 4 * mix
// (0 read, 1 write, 2 copy, 3 row, 4 one-pass).  x [rows, cols] bf16 with
// cols % 512 == 0; o8a, o8b [rows, cols] bytes; o16 [rows, cols] bf16; sc
// [rows, cols/32] bytes; sink one word.  Returns 0, 1 for a bad argument
// (nothing launched), 2 for a launch error.
int bench_stream_tiled(int variant, const void *x, int64_t rows, int64_t cols, void *o8a,
                       void *o8b, void *o16, void *sc, void *sink, void *stream)
{
    if (variant < 0 || variant >= 20 || rows <= 0 || cols <= 0 || cols % 512 != 0) return 1;
    if (!x || !o8a || !o8b || !o16 || !sc || !sink) return 1;
    const int64_t nseg = cols / 512;
    const int ri = variant % 4, mix = variant / 4;
    const int R = 1 << ri;
    const int64_t tiles = nseg * ((rows + 4 * R - 1) / (4 * R));
    if (tiles > 0x7FFFFFFF) return 1;
    const hipStream_t s = (hipStream_t)stream;
    const uint16_t *xp = (const uint16_t *)x;
    uint8_t *a = (uint8_t *)o8a, *b = (uint8_t *)o8b, *c = (uint8_t *)sc;
    uint16_t *f = (uint16_t *)o16;
    uint32_t *k = (uint32_t *)sink;
#define TL(RR, RD, N8, N16, SC)                                                                    \
    hipLaunchKernelGGL((tiled_kernel<RR, RD, N8, N16, SC>), dim3((unsigned)tiles), dim3(256), 0,  \
                       s, xp, rows, cols, nseg, a, b, f, c, k)
#define TL_MIX(RR)                                                                                 \
    switch (mix) {                                                                                 \
    case 0: TL(RR, true, 0, 0, false); break;                                                      \
    case 1: TL(RR, false, 0, 1, false); break;                                                     \
    case 2: TL(RR, true, 0, 1, false); break;                                                      \
    case 3: TL(RR, true, 1, 0, true); break;                                                       \
    default: TL(RR, true, 2, 1, true); break;                                                      \
    }
    switch (R) {
    case 1: TL_MIX(1); break;
    case 2: TL_MIX(2); break;
    case 4: TL_MIX(4); break;
    default: TL_MIX(8); break;
    }
#undef TL_MIX
#undef TL
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Flat variants: variant = U index (0: U=2, 1: U=4, 2: U=8) + 3 * mode (0 read,
// 1 copy, 2 row, 3 one-pass, 4 write).  x: nvec 16-byte vectors; o8a, o8b:
// nvec 8-byte vectors; o16: nvec 16-byte vectors; grid workgroups (1..65536).
int bench_stream_flat(int variant, const void *x, int64_t nvec, void *o8a, void *o8b, void *o16,
                      void *sink, int grid, void *stream)
{
    if (variant < 0 || variant >= 15 || nvec <= 0 || grid < 1 || grid > 65536) return 1;
    if (!x || !o8a || !o8b || !o16 || !sink) return 1;
    const int ui = variant % 3, mode = variant / 3;
    const hipStream_t s = (hipStream_t)stream;
    const uint4 *xp = (const uint4 *)x;
    uint2 *a = (uint2 *)o8a, *b = (uint2 *)o8b;
    uint4 *f = (uint4 *)o16;
    uint32_t *k = (uint32_t *)sink;
#define FL(UU, MM)                                                                                 \
    hipLaunchKernelGGL((flat_kernel<UU, MM>), dim3((unsigned)grid), dim3(256), 0, s, xp, nvec, a, \
                       b, f, k)
#define FL_MODE(UU)                                                                                \
    switch (mode) {                                                                                \
    case 0: FL(UU, 0); break;                                                                      \
    case 1: FL(UU, 1); break;                                                                      \
    case 2: FL(UU, 2); break;                                                                      \
    case 3: FL(UU, 3); break;                                                                      \
    default: FL(UU, 4); break;                                                                     \
    }
    switch (ui) {
    case 0: FL_MODE(2); break;
    case 1: FL_MODE(4); break;
    default: FL_MODE(8); break;
    }
#undef FL_MODE
#undef FL
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
