// launch.hpp -- host-side launchers of the gfx950 kernels (internal).
// Arguments arrive already validated by the C ABI layer (mxq_abi.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

// Launch table entry for the grouped row-wise kernel (staged in the caller's
// device workspace, followed by an int32 array of each entry's first tile).
// Tiles are (512-column segment, 16-row block) pairs, numbered tensor by
// tensor; one workgroup runs one tile.
struct GroupEntry {
    const uint16_t *x;
    uint8_t *q;
    uint8_t *scale;
    int64_t rows, cols, ldx, ldq, lds;
    int64_t tile_begin;
    int64_t nseg;  // 512-column segments per row block
};

hipError_t launch_mx_rowwise(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t *q, int64_t ldq, uint8_t *scale, int64_t lds,
                             uint16_t *fq, int64_t ldf, hipStream_t stream);

hipError_t launch_mx_colwise(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *qc,
                             uint8_t *sc, uint8_t *qr, uint8_t *sr, uint16_t *fq_row,
                             uint16_t *fq_col, hipStream_t stream);

hipError_t launch_mx_colwise_t(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *qt,
                               int64_t ldt, uint8_t *st, uint8_t *qr, uint8_t *sr,
                               uint16_t *fq_row, hipStream_t stream);

hipError_t launch_e8m0_to_f32(const uint8_t *scale, int64_t n, float *out, hipStream_t stream);

hipError_t launch_mx_dequant(const uint8_t *q, const uint8_t *scale, int64_t rows, int64_t cols,
                             int axis, uint16_t *out, hipStream_t stream);

hipError_t launch_mx_grouped(const GroupEntry *table_dev, const int32_t *starts_dev, int32_t n,
                             int64_t total_tiles, hipStream_t stream);

// Tiles of one tensor in a grouped row-wise launch (and its 512-column segments).
int64_t mx_grouped_tiles(int64_t rows, int64_t cols, int64_t *nseg);

hipError_t launch_mx4_quant(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q,
                            uint8_t *scale, uint16_t *fq, hipStream_t stream);
hipError_t launch_mx4_dequant(const uint8_t *q, const uint8_t *scale, int64_t rows, int64_t cols,
                              uint16_t *out, hipStream_t stream);

// slices: a stack [slices, rows, cols] quantized slice by slice (1 for 2-D).
hipError_t launch_bfp8_quant(const uint16_t *x, int64_t slices, int64_t rows, int64_t cols,
                             uint8_t *q, float *scale, hipStream_t stream);
// row_scales: 1 x 128 blocks (scale [rows, ceil(cols/128)]); else 128 x 128.
hipError_t launch_bfp8_dequant(const uint8_t *q, const float *scale, int64_t slices,
                               int64_t rows, int64_t cols, bool row_scales, uint16_t *out,
                               hipStream_t stream);
hipError_t launch_bfp8_1x128(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q,
                             float *scale, uint16_t *fq, hipStream_t stream);

hipError_t launch_bfp8_to_mx(const uint8_t *q, const float *scale, int64_t rows, int64_t cols,
                             uint8_t *q8, uint8_t *s8, hipStream_t stream);

// NVFP4 amax partials: at most this many workgroups write one word each, and
// one workgroup of as many threads reduces them, one load per thread.  512
// measured 1.5-2% faster than 1024 on [8192, 8192] (384 alike, 256 slower).
constexpr int kNvAmaxBlocks = 512;
static_assert(kNvAmaxBlocks % 64 == 0 && kNvAmaxBlocks <= 1024, "one thread per partial");

// ws: ws_words words of amax partials (hipErrorInvalidValue when the amax
// pass would need more; it needs at most kNvAmaxBlocks).
hipError_t launch_nvfp4_quant(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q,
                              uint8_t *s, float *g, uint32_t *ws, int64_t ws_words,
                              hipStream_t stream);
// The same with the partials in the library's own per-device array.
hipError_t launch_nvfp4_quant_noalloc(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q,
                                      uint8_t *s, float *g, hipStream_t stream);
// Launch table entry of grouped NVFP4 (staged in the caller's workspace,
// followed by int32 arrays of first tiles and scale groups, then one uint32
// amax partial per tile).  Tiles: 512 columns x 32 rows.
struct NvEntry {
    const uint16_t *x;
    uint8_t *q;
    uint8_t *s;
    int64_t rows, cols;
    int64_t nseg;
    int32_t tile_begin;
    int32_t group;
};

hipError_t launch_nvfp4_grouped(const NvEntry *table, const int32_t *starts, const int32_t *groups,
                                int32_t n, uint32_t *partial, int64_t total_tiles, float *gs,
                                int32_t n_groups, hipStream_t stream);
int64_t nvfp4_tiles(int64_t rows, int64_t cols, int64_t *nseg);

hipError_t launch_nvfp4_dequant(const uint8_t *q, const uint8_t *s, const float *g,
                                int64_t rows, int64_t cols, uint16_t *out, hipStream_t stream);

}  // namespace mxq
