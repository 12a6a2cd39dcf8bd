/*
 * mxq.h -- C ABI of the MI355X (gfx950) block-scaled quantization library.
 *
 * What the library computes (sources are the pages' titles and sections):
 *   - MXFP8: every group of 32 consecutive values shares one power-of-two
 *     scale stored as an E8M0 byte; the values are cast to FP8 E4M3.  The
 *     output is a compact, non-swizzled qweight plus a scale tensor, the one
 *     a checkpoint stores as `<name>.weight_scale_inv`, and rows that are not a
 *     multiple of 32 behave exactly as the zero-pad-then-crop route ("PR #1935
 *     完整报告 / Use TransformerEngine for MXFP8 quantization", section 实现拆解
 *     item 1 and 关键源码片段).  Power-of-two scales and the E8M0 scale dtype:
 *     miles PR #1372 "V4 mxfp4", PR description.  The scale exponent is
 *     floor(log2 amax) - 8 (the OCP microscaling conversion for E4M3, whose
 *     largest power of two is 2^8); elements round to nearest even and
 *     saturate at +-448.
 *   - Fake quantization (quantize, then dequantize back to bf16) for
 *     simulated QAT: miles PR #1372 "V4 mxfp4", the compressor review.
 *   - MXFP4 (the same groups of 32 and E8M0 scales, E2M1 elements packed two
 *     per byte) and its simulate-QAT fake quantization: the same page.
 *   - Block-FP8 (128 x 128 absmax, fp32 scale) and NVFP4 (global fp32 scale x
 *     per-16 E4M3 scale, E2M1 elements packed two per byte): xorl PR #30 "Add
 *     FP8, NVFP4, and QARL training and export", deep review, "What looked
 *     solid"; the packed FP4 output shape [..., N/2] from the review of
 *     fp4_act_quant in miles PR #1372.
 *
 * Conventions for every entry point
 *   - Data pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronizes; every call is asynchronous on
 *     `stream` (a hipStream_t passed as void*, NULL = the default stream).
 *     The two one-call grouped forms are the exception: they copy a launch
 *     table from host memory, which may block the host until the copy has
 *     read it, and they refuse to run while `stream` is being captured
 *     (their prepared-plan forms do neither).
 *   - bf16 tensors are passed as uint16_t bit patterns; E4M3, E8M0 and packed
 *     E2M1 codes as uint8_t; fp32 scales as float.  All are row-major.
 *   - Arguments are checked on the host before anything is launched; a
 *     rejected call launches nothing and writes nothing.  A launch the HIP
 *     runtime refuses returns MXQ_EHIP.  Faults that happen on the device
 *     surface at the caller's next synchronization.
 *   - Outputs are fully overwritten; no byte outside them is written.
 *   - rows == 0 is accepted and launches nothing (all pointers may then be
 *     NULL).  Sizes must satisfy the per-call shape rules and fit int64.
 *   - The library keeps no state, except the one device array per GPU that
 *     nvfp4_quantize_noalloc uses in place of a workspace: calls from several
 *     host threads are safe, apart from overlapping nvfp4_quantize_noalloc
 *     calls on one GPU.
 *   - Non-finite inputs: an MX group, block-FP8 tile or NVFP4 tensor that
 *     holds NaN or Inf is quantized as all-NaN (E8M0 byte 0xFF / fp32 NaN
 *     scale / E4M3 0x7F with each element's sign; NVFP4, whose E2M1 has no
 *     NaN: global scale NaN, block scales 0x7F, nibbles 0x7 with the sign).
 */
#ifndef MXQ_H
#define MXQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXQ_ABI_VERSION 2

typedef enum mxq_status {
    MXQ_OK = 0,
    MXQ_EINVAL = 1, /* NULL pointer where one is needed, negative size, bad axis */
    MXQ_ESHAPE = 2, /* shape the operation does not accept (e.g. cols % 32 != 0) */
    MXQ_EALIGN = 3, /* pointer or leading dimension misaligned for vector access */
    MXQ_EHIP = 4,   /* the HIP runtime rejected a launch or copy */
    MXQ_ESIZE = 5,  /* workspace too small, or a size overflows the index type */
    MXQ_ECAPTURE = 6 /* a call that copies from host memory, made while `stream`
                        is being captured into a graph (use the plan form) */
} mxq_status;

/* Static English text for a status code (never NULL). */
const char *mxq_status_string(int status);

/* MXQ_ABI_VERSION of the built library. */
int mxq_abi_version(void);

/* Identifier of the sources the library was built from: the first 16 hex
 * digits of a sha256 over the compiler flags and every source and header
 * file.  A loader compares it with the same hash of the tree it ships with
 * and refuses a library built from other sources. */
const char *mxq_build_id(void);

/*
 * Row-wise MXFP8 quantization ("PR #1935 完整报告", 实现拆解 item 1).
 *   x      [rows, cols] bf16, row stride ldx elements
 *   q      [rows, cols] E4M3 codes, row stride ldq bytes
 *   scale  [rows, cols/32] E8M0 bytes, row stride lds bytes (weight_scale_inv)
 *   fq     optional [rows, cols] bf16 fake-quant output (dequantize(q, scale)),
 *          row stride ldf elements; NULL to skip
 * Shape: cols % 32 == 0 (MXQ_ESHAPE otherwise); any rows >= 0.  Rows need no
 * padding: the result equals zero-padding to a multiple of 32 rows and
 * cropping back.  ldx >= cols, ldq >= cols, lds >= cols/32, ldf >= cols.
 * Alignment (MXQ_EALIGN): x and fq 16-byte aligned with ldx, ldf multiples of
 * 8; q 8-byte aligned with ldq a multiple of 8.
 */
mxq_status mxq_quantize_rowwise(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx,
                                uint8_t *q, int64_t ldq, uint8_t *scale, int64_t lds,
                                uint16_t *fq, int64_t ldf, void *stream);

/*
 * Column-wise MXFP8 quantization: groups of 32 consecutive rows within each
 * column (the token axis of an activation [tokens, hidden]).  One pass over x
 * can also produce the row-wise result and the row-wise fake-quant.
 *   x      [rows, cols] bf16, contiguous
 *   qc     [rows, cols] E4M3 codes in x's layout, contiguous
 *   sc     [ceil(rows/32), cols] E8M0 bytes, contiguous; a last group of
 *          fewer than 32 rows equals zero-padding it
 *   qr, sr optional row-wise outputs as mxq_quantize_rowwise (contiguous,
 *          sr [rows, cols/32]); both NULL or both set
 *   fq     optional [rows, cols] bf16 = row-wise dequantize(qr, sr) (the
 *          row-wise codes need not be stored to get it)
 * Shape: cols % 32 == 0.  Alignment: x, fq 16 bytes; qc, sc, qr 8 bytes.
 */
mxq_status mxq_quantize_colwise(const uint16_t *x, int64_t rows, int64_t cols,
                                uint8_t *qc, uint8_t *sc,
                                uint8_t *qr, uint8_t *sr, uint16_t *fq, void *stream);

/*
 * Column-wise MXFP8 in the transposed layout a backward-pass (weight-gradient)
 * GEMM reads, with optional row-wise outputs, in one read of x.  The groups,
 * scales and codes are those of mxq_quantize_colwise (32 consecutive rows of
 * one column; a short last group equals zero padding); only the storage
 * differs, which makes qt / st the row-wise MXFP8 of x transposed:
 *   qt  [cols, rows] E4M3 codes, row stride ldt bytes: qt[c * ldt + r] is the
 *       code of x[r, c]; ldt >= rows, ldt % 16 == 0, qt 16-byte aligned
 *   st  [cols, ceil(rows/32)] E8M0 bytes, compact, 4-byte aligned:
 *       st[c * ceil(rows/32) + j] is the scale of rows 32j..32j+31 of column c
 *   qr, sr, fq  optional row-wise codes [rows, cols], scales [rows, cols/32]
 *       and row-wise fake-quant [rows, cols] bf16, as mxq_quantize_colwise
 *       (qr and sr together or neither; fq alone is allowed)
 * x [rows, cols] bf16 contiguous, 16-byte aligned.  Shape: cols % 32 == 0;
 * any rows >= 0.  Bytes of qt between rows and ldt are not written.
 * Performance: with the row-wise outputs requested and ldt a multiple of
 * 4096, every row of qt starts on the same 4 KiB boundary; on MI355X a stride
 * of ldt + 256 measured about 4% faster for that call (the compact stride is
 * the faster one for the column-only call).
 */
mxq_status mxq_quantize_colwise_t(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *qt,
                                  int64_t ldt, uint8_t *st, uint8_t *qr, uint8_t *sr,
                                  uint16_t *fq, void *stream);

/*
 * MXFP8 dequantization: out = bf16_RNE(E4M3(q) * 2^(scale - 127)).  NaN code
 * or scale byte 0xFF gives the quiet NaN 0x7FC0 with the code's sign bit.
 *   q      [rows, cols] E4M3, contiguous
 *   scale  axis = 1: [rows, cols/32]; axis = 0: [ceil(rows/32), cols]; contiguous
 *   out    [rows, cols] bf16, contiguous
 * Shape: cols % 32 == 0.  Alignment: q 8 bytes, out 16 bytes.
 */
mxq_status mxq_dequantize(const uint8_t *q, const uint8_t *scale, int64_t rows, int64_t cols,
                          int axis, uint16_t *out, void *stream);

/*
 * E8M0 scale bytes as fp32 values, for consumers that take fp32 scales only
 * (miles PR #1372 "V4 mxfp4", PR description: scale storage forced to fp32
 * for fp8_simulate; E8M0 per the OCP microscaling definition):
 * out[i] = 2^(scale[i] - 127), exact (byte 0 gives the fp32 subnormal
 * 2^-127); byte 0xFF (NaN) gives the quiet NaN 0x7FC00000.
 *   scale  n bytes, any alignment     out  n floats, 4-byte aligned
 * Works for MXFP8 and MXFP4 scales of either axis (any layout: elementwise).
 */
mxq_status mxq_e8m0_to_fp32(const uint8_t *scale, int64_t n, float *out, void *stream);

/*
 * MXFP8 fake quantization (simulated QAT, miles PR #1372 "V4 mxfp4"):
 * out = dequantize(quantize(x)) along `axis` (1 = row-wise groups, 0 =
 * column-wise), written as bf16 without materializing the codes.
 * Shape: cols % 32 == 0.  Contiguous; x and out 16-byte aligned.
 */
mxq_status mxq_fake_quant(const uint16_t *x, int64_t rows, int64_t cols, int axis,
                          uint16_t *out, void *stream);

/*
 * Grouped row-wise MXFP8: many independent tensors (e.g. every expert of an
 * MoE layer) in one launch.  Each descriptor is validated as in
 * mxq_quantize_rowwise (fq is not offered here).
 */
typedef struct mxq_group_desc {
    const uint16_t *x; /* [rows, cols] bf16, row stride ldx */
    uint8_t *q;        /* [rows, cols] E4M3, row stride ldq */
    uint8_t *scale;    /* [rows, cols/32] E8M0, row stride lds */
    int64_t rows, cols, ldx, ldq, lds;
} mxq_group_desc;

/* Bytes of device workspace mxq_quantize_rowwise_grouped needs for n tensors. */
size_t mxq_grouped_workspace_size(int32_t n);

/*
 *   descs      HOST array of n descriptors (read during the call only)
 *   workspace  DEVICE buffer of >= mxq_grouped_workspace_size(n) bytes,
 *              16-byte aligned; the library stages a launch table there with
 *              a host-to-device copy on `stream` from a host buffer that
 *              lives only during the call (so the call may block the host
 *              until the copy has read it), and the buffer must not be
 *              reused until the launch has finished
 * Returns MXQ_EINVAL for n < 0 or NULL pointers, MXQ_ESIZE for a small
 * workspace, else the first failing descriptor's status; MXQ_ECAPTURE, with
 * nothing enqueued, while `stream` is being captured (a captured copy would
 * read the freed host buffer on replay: capture the plan form instead).
 * n == 0 launches nothing.
 */
mxq_status mxq_quantize_rowwise_grouped(const mxq_group_desc *descs, int32_t n,
                                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * Block-FP8 quantization (xorl PR #30, "What looked solid": block-FP8
 * absmax): per blk x blk tile, S = fl32(amax / 448), q = E4M3_RNE_sat(fl32(x / S))
 * with one IEEE fp32 division; an all-zero tile stores S = 0 and codes +-0.
 * Edge tiles use their valid region.
 *   x      [rows, cols] bf16, contiguous, 16-byte aligned
 *   q      [rows, cols] E4M3, contiguous, 8-byte aligned
 *   scale  [ceil(rows/blk), ceil(cols/blk)] fp32, contiguous
 * Shape: blk == 128; cols % 8 == 0.
 */
mxq_status blockfp8_quantize(const uint16_t *x, int64_t rows, int64_t cols, int32_t blk,
                             uint8_t *q, float *scale, void *stream);

/* Block-FP8 dequantization: out = bf16_RNE(fl32(E4M3(q) * S)); a NaN product
 * gives the quiet NaN with the code's sign.  Same shapes and rules as above. */
mxq_status blockfp8_dequantize(const uint8_t *q, const float *scale, int64_t rows, int64_t cols,
                               int32_t blk, uint16_t *out, void *stream);

/*
 * Block-FP8 of a stack of G matrices (grouped-GEMM weights [G, K, N], the
 * `_gkn` variant named in xorl PR #30 "What looked solid"): each slice
 * [K, N] is quantized as blockfp8_quantize would quantize it alone, so no
 * 128 x 128 tile crosses a slice boundary.
 *   x      [G, K, N] bf16, contiguous, 16-byte aligned
 *   q      [G, K, N] E4M3 codes, 8-byte aligned
 *   scale  [G, ceil(K/128), ceil(N/128)] fp32, 4-byte aligned
 * Shape: blk == 128; N % 8 == 0.
 */
mxq_status blockfp8_quantize_gkn(const uint16_t *x, int64_t G, int64_t K, int64_t N, int32_t blk,
                                 uint8_t *q, float *scale, void *stream);

/* Dequantization of blockfp8_quantize_gkn's output, slice by slice; out
 * [G, K, N] bf16, 16-byte aligned. */
mxq_status blockfp8_dequantize_gkn(const uint8_t *q, const float *scale, int64_t G, int64_t K,
                                   int64_t N, int32_t blk, uint16_t *out, void *stream);

/*
 * Block-FP8 with 1 x 128 blocks along each row (the activation recipe):
 * per block of 128 consecutive values of a row (the last one shorter when
 * cols % 128 != 0), S = fl32(amax / 448) and q = E4M3_RNE_sat(fl32(x / S)),
 * with the same zero-block and non-finite rules as blockfp8_quantize.
 *   x      [rows, cols] bf16, contiguous, 16-byte aligned
 *   q      [rows, cols] E4M3 codes, contiguous, 8-byte aligned
 *   scale  [rows, ceil(cols/128)] fp32, 4-byte aligned
 *   fq     optional [rows, cols] bf16 = blockfp8_dequantize_1x128(q, scale),
 *          16-byte aligned; NULL to skip
 * Shape: cols % 8 == 0.
 */
mxq_status blockfp8_quantize_1x128(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q,
                                   float *scale, uint16_t *fq, void *stream);

/* 1 x 128 block-FP8 dequantization: out = bf16_RNE(fl32(E4M3(q) * S)); a NaN
 * product gives the quiet NaN with the code's sign.  Shapes as above. */
mxq_status blockfp8_dequantize_1x128(const uint8_t *q, const float *scale, int64_t rows,
                                     int64_t cols, uint16_t *out, void *stream);

/* Fake quantization fp8_simulate_qat(x, 128) (miles PR #1372 "V4 mxfp4", the
 * compressor review; fp32 scales per its PR description): out =
 * blockfp8_dequantize_1x128(blockfp8_quantize_1x128(x)) in one pass. */
mxq_status blockfp8_fake_quant_1x128(const uint16_t *x, int64_t rows, int64_t cols,
                                     uint16_t *out, void *stream);

/*
 * FP8 block -> BF16 -> MXFP8 re-quantization in one pass: the conversion of
 * a block-FP8 checkpoint to MXFP8 ("PR #1935 完整报告", 实现拆解 item 5,
 * the FP8->BF16->MXFP8 conversion).  The result equals
 * mxq_quantize_rowwise(blockfp8_dequantize(q, scale)) byte for byte; the
 * bf16 intermediate is never written.
 *   q       [rows, cols] E4M3 codes, contiguous, 8-byte aligned
 *   scale   [ceil(rows/128), ceil(cols/128)] fp32 tile scales, 4-byte aligned
 *   q8      [rows, cols] E4M3 codes out, contiguous, 8-byte aligned
 *   scale8  [rows, cols/32] E8M0 bytes out, contiguous
 * Shape: blk == 128; cols % 32 == 0; any rows >= 0.
 */
mxq_status blockfp8_to_mxfp8(const uint8_t *q, const float *scale, int64_t rows, int64_t cols,
                             int32_t blk, uint8_t *q8, uint8_t *scale8, void *stream);

/*
 * MXFP4 quantization (miles PR #1372 "V4 mxfp4": mxfp4_simulate_qat with
 * groups of 32 in the compressor review; the packed [..., N/2] FP4 output in
 * the review of fp4_act_quant).  Every 32 consecutive values of a row share
 * one E8M0 scale byte floor(log2 amax) - 2 + 127, clamped at 0 (the OCP
 * microscaling conversion for E2M1, whose largest power of two is 2^2); 0
 * for an all-zero group, 0xFF for a group holding NaN or Inf.  Elements are
 * E2M1 nibbles of x / 2^(byte - 127), round to nearest even, saturating at
 * +-6, sign kept (a NaN group: 0x7 with each element's sign).
 *   x          [rows, cols] bf16, contiguous, 16-byte aligned
 *   q_packed   [rows, cols/2] bytes, contiguous, 4-byte aligned; element 2j
 *              in the low nibble of byte j, 2j+1 in the high nibble
 *   scale      [rows, cols/32] E8M0 bytes, contiguous
 *   fq         optional [rows, cols] bf16 = mxfp4_dequantize(q_packed,
 *              scale), contiguous, 16-byte aligned; NULL to skip
 * Shape: cols % 32 == 0 (MXQ_ESHAPE otherwise); any rows >= 0.
 */
mxq_status mxfp4_quantize(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q_packed,
                          uint8_t *scale, uint16_t *fq, void *stream);

/* MXFP4 dequantization: out = bf16(E2M1(nibble) * 2^(byte - 127)), exact (the
 * value has two significant bits and the scale is at least 2^-127) or +-Inf
 * when it overflows bf16; scale byte 0xFF gives the quiet NaN with the
 * nibble's sign.  Shapes as mxfp4_quantize; out 16-byte aligned. */
mxq_status mxfp4_dequantize(const uint8_t *q_packed, const uint8_t *scale, int64_t rows,
                            int64_t cols, uint16_t *out, void *stream);

/* MXFP4 fake quantization, mxfp4_simulate_qat(x, 32): out =
 * mxfp4_dequantize(mxfp4_quantize(x)) in one pass, without writing codes or
 * scales.  x and out [rows, cols] bf16, contiguous, 16-byte aligned. */
mxq_status mxfp4_fake_quant(const uint16_t *x, int64_t rows, int64_t cols, uint16_t *out,
                            void *stream);

/*
 * NVFP4 two-level quantization (xorl PR #30, "What looked solid":
 * effective = block_scale * global_scale, clamped, zero block guarded):
 *   A = max|x| over the tensor; g = fl32(A / 2688)  (2688 = 448 * 6)
 *   per 16 consecutive values of a row with amax b:
 *     s = E4M3_RNE_sat(fl32(b / fl32(6 * g))), eff = fl32(E4M3(s) * g)
 *     q = E2M1_RNE_sat(fl32(x / eff)), or +-0 when eff == 0
 *   element 2j -> low nibble of byte j, 2j+1 -> high nibble
 *   x          [rows, cols] bf16, contiguous, 16-byte aligned
 *   q_packed   [rows, cols/2] bytes, contiguous, 4-byte aligned
 *   s_e4m3     [rows, cols/16] E4M3 bytes, contiguous
 *   global_scale  one float (device), written with g
 *   workspace  >= nvfp4_workspace_size() bytes of device memory, 4-byte
 *              aligned, caller-owned: per-workgroup partial maxima passed
 *              between the two launches (no initial contents needed; calls
 *              that overlap on one workspace race)
 * Shape: cols % 16 == 0.
 */
size_t nvfp4_workspace_size(void);

mxq_status nvfp4_quantize(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q_packed,
                          uint8_t *s_e4m3, float *global_scale, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * nvfp4_quantize for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, results and errors minus the workspace.  The amax
 * partials go to a fixed array of the library instead: 512 words (2 KiB)
 * per GPU, held until the process ends, its device address resolved once per
 * device on the first call there.  Every size nvfp4_quantize accepts fits
 * (the amax pass writes at most 512 partials whatever the size; a launch
 * that would need more returns MXQ_ESIZE).  The call allocates nothing and
 * copies nothing.  All calls on one GPU share the array: calls that overlap
 * on one GPU (several streams or host threads at once) race, so serialize
 * them.  Nothing in the array needs clearing between calls.
 */
mxq_status nvfp4_quantize_noalloc(const uint16_t *x, int64_t rows, int64_t cols,
                                  uint8_t *q_packed, uint8_t *s_e4m3, float *global_scale,
                                  void *stream);

/*
 * Grouped NVFP4 with global scales shared within scale groups (xorl PR #30,
 * deep review item 3: a fused gated-MoE gate_up weight is quantized with one
 * global scale per half for QAT, and with one weight_scale_2 shared by gate
 * and up for the fused serving kernel).  Tensor i belongs to scale group
 * descs[i].scale_group in [0, n_groups); a group's A is the max |x| over all
 * its tensors (NaN/Inf in any makes the group all-NaN as in nvfp4_quantize),
 * global_scales[group] = fl32(A / 2688), and every member is quantized with
 * that scale exactly as nvfp4_quantize does.  A group without members gets
 * 0.  One call; tensors with rows == 0 or cols == 0 are skipped.
 *   descs          host array of n descriptors: x [rows, cols] bf16
 *                  contiguous 16-byte aligned, q [rows, cols/2] 4-byte
 *                  aligned, s [rows, cols/16]; cols % 16 == 0
 *   global_scales  device float[n_groups], 4-byte aligned
 *   workspace      >= nvfp4_grouped_workspace_size(descs, n) bytes of device
 *                  memory, 16-byte aligned, caller-owned: the launch table and
 *                  one amax partial per 512 x 32 tile (no initial contents
 *                  needed; calls that overlap on one workspace race).  It is
 *                  filled by a host-to-device copy on `stream` from a host
 *                  buffer that lives only during the call, so the call may
 *                  block the host until the copy has read it, and it returns
 *                  MXQ_ECAPTURE, with nothing enqueued, while `stream` is
 *                  being captured (capture the plan form instead).
 */
typedef struct nvfp4_group_desc {
    const uint16_t *x;
    uint8_t *q;
    uint8_t *s;
    int64_t rows, cols;
    int32_t scale_group;
    int32_t reserved; /* set to 0 */
} nvfp4_group_desc;

size_t nvfp4_grouped_workspace_size(const nvfp4_group_desc *descs, int32_t n);

mxq_status nvfp4_quantize_grouped(const nvfp4_group_desc *descs, int32_t n, float *global_scales,
                                  int32_t n_groups, void *workspace, size_t workspace_bytes,
                                  void *stream);

/*
 * Grouped launches prepared once.  Both grouped calls above rebuild their
 * launch table on the host and copy it to the device on every call.  A caller
 * that quantizes the same set of buffers every step (the experts of an MoE
 * layer; work replayed from a captured HIP graph) can instead build the table
 * once and then launch from it: the launch makes no copy and allocates
 * nothing, so a graph capture records kernels only.  The results equal the
 * one-call forms' bit for bit.
 *   1. mxq_grouped_plan_build / nvfp4_grouped_plan_build with table_host ==
 *      NULL check the descriptors exactly as the one-call form does and fill
 *      *plan, sizes included.
 *   2. Called again with plan->table_bytes of host memory at table_host, they
 *      write the table image there.  The image holds the descriptors' device
 *      pointers and shapes, so it is valid while those buffers are.
 *   3. The caller copies the image into the first plan->table_bytes bytes of
 *      a 16-byte aligned device buffer of >= plan->workspace_bytes bytes.
 *   4. The *_grouped_plan call launches, as often as wanted.  It checks the
 *      plan and the buffer's size; the device bytes it trusts to be the image.
 * A plan of one kind is refused by the other kind's launch (MXQ_EINVAL).
 * MXFP8 launches only read their buffer; an NVFP4 buffer also holds amax
 * partials after the image, so NVFP4 launches that overlap on one buffer race.
 */
typedef struct mxq_grouped_plan {
    int32_t kind;             /* written by the build call, checked by the launch */
    int32_t n_entries;        /* descriptors with rows > 0 and cols > 0 */
    int32_t n_groups;         /* NVFP4 scale groups (global_scales length); 0 for MXFP8 */
    int32_t reserved;         /* 0 */
    int64_t total_tiles;      /* workgroups of the quantize kernel */
    uint64_t table_bytes;     /* size of the table image */
    uint64_t workspace_bytes; /* device buffer size the launch needs, image first */
} mxq_grouped_plan;

/* Errors as mxq_quantize_rowwise_grouped, plus MXQ_EINVAL for plan == NULL
 * and MXQ_ESIZE for table_host_bytes < plan->table_bytes.  n == 0 gives an
 * empty plan whose launch does nothing. */
mxq_status mxq_grouped_plan_build(const mxq_group_desc *descs, int32_t n, mxq_grouped_plan *plan,
                                  void *table_host, size_t table_host_bytes);

/* table_dev: the device copy of the image.  MXQ_EINVAL for a NULL or foreign
 * plan, MXQ_EALIGN / MXQ_ESIZE for the buffer. */
mxq_status mxq_quantize_rowwise_grouped_plan(const mxq_grouped_plan *plan, const void *table_dev,
                                             size_t table_dev_bytes, void *stream);

/* Errors as nvfp4_quantize_grouped (the workspace checks move to the launch),
 * plus those of mxq_grouped_plan_build. */
mxq_status nvfp4_grouped_plan_build(const nvfp4_group_desc *descs, int32_t n, int32_t n_groups,
                                    mxq_grouped_plan *plan, void *table_host,
                                    size_t table_host_bytes);

/* workspace: the image, then room for the amax partials
 * (plan->workspace_bytes in all; may be NULL when that is 0);
 * global_scales: plan->n_groups floats, 4-byte aligned, written as by
 * nvfp4_quantize_grouped. */
mxq_status nvfp4_quantize_grouped_plan(const mxq_grouped_plan *plan, float *global_scales,
                                       void *workspace, size_t workspace_bytes, void *stream);

/* NVFP4 dequantization: out = bf16_RNE(fl32(E2M1(q) * eff)),
 * eff = fl32(E4M3(s) * g); a NaN product gives the quiet NaN with the
 * nibble's sign.  Shapes as nvfp4_quantize; out 16-byte aligned. */
mxq_status nvfp4_dequantize(const uint8_t *q_packed, const uint8_t *s_e4m3,
                            const float *global_scale, int64_t rows, int64_t cols,
                            uint16_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_H */
