// mxq_abi.hip -- the extern "C" entry points declared in include/mxq.h.
//
// Every argument is checked on the host before anything is launched, so a
// rejected call has no side effect and every error path can be exercised
// without a GPU.  A failure is always reported, never downgraded to another
// code path (the fail-visible rule the pages argue for: fusion-mlx issue #425
// keeps its explicit raise instead of a silent downgrade, and the xorl PR #30
// review objects to a swallowed RuntimeError that hides a broken fast path).
#include <string.h>

#include <vector>

#include "launch.hpp"
#include "mxq.h"

using mxq::GroupEntry;

namespace {

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// rows * ld + cols fits int64 (all kernels index with int64).
inline bool fits(int64_t rows, int64_t ld)
{
    int64_t t;
    return !__builtin_mul_overflow(rows, ld, &t);
}

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

inline mxq_status from_hip(hipError_t e) { return e == hipSuccess ? MXQ_OK : MXQ_EHIP; }

// MXQ_ECAPTURE while `stream` is being captured into a graph.  The one-call
// grouped forms copy their launch table from a host buffer that is freed when
// the call returns; a captured copy node would read that freed memory on every
// replay.  (A query the runtime refuses, e.g. of the legacy stream during
// another stream's global-mode capture, also refuses the call.)
inline mxq_status refuse_capture(hipStream_t stream)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return MXQ_EHIP;
    return cs == hipStreamCaptureStatusNone ? MXQ_OK : MXQ_ECAPTURE;
}

mxq_status check_rowwise(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx,
                         const uint8_t *q, int64_t ldq, const uint8_t *scale, int64_t lds,
                         const uint16_t *fq, int64_t ldf, bool need_q)
{
    if (rows < 0 || cols < 0) return MXQ_EINVAL;
    if (cols % 32 != 0) return MXQ_ESHAPE;
    if (rows == 0 || cols == 0) return MXQ_OK;
    if (!x || (need_q && (!q || !scale)) || (!need_q && !fq)) return MXQ_EINVAL;
    if (ldx < cols) return MXQ_ESHAPE;
    if (!aligned(x, 16) || ldx % 8 != 0) return MXQ_EALIGN;
    if (q) {
        if (!scale) return MXQ_EINVAL;
        if (ldq < cols || lds < cols / 32) return MXQ_ESHAPE;
        if (!aligned(q, 8) || ldq % 8 != 0) return MXQ_EALIGN;
        if (!fits(rows, ldq) || !fits(rows, lds)) return MXQ_ESIZE;
    }
    if (fq) {
        if (ldf < cols) return MXQ_ESHAPE;
        if (!aligned(fq, 16) || ldf % 8 != 0) return MXQ_EALIGN;
        if (!fits(rows, ldf)) return MXQ_ESIZE;
    }
    if (!fits(rows, ldx)) return MXQ_ESIZE;
    return MXQ_OK;
}

size_t round16(size_t v) { return (v + 15) / 16 * 16; }

// Launch tables of the grouped calls, as one host image copied to the front
// of the device buffer:
//   MXFP8  [GroupEntry x m][int32 first tile x m]
//   NVFP4  [NvEntry x m][int32 first tile x m][int32 scale group x m],
//          followed in the buffer by one uint32 amax partial per tile
// each padded to 16 bytes, m = the non-empty descriptors.
constexpr int32_t kPlanMx = 0x3158584D;  // "MXX1"
constexpr int32_t kPlanNv = 0x3134564E;  // "NV41"

size_t mx_table_bytes(size_t m) { return round16(m * (sizeof(GroupEntry) + sizeof(int32_t))); }

size_t nv_table_bytes(size_t m)
{
    return round16(m * (sizeof(mxq::NvEntry) + 2 * sizeof(int32_t)));
}

template <class T>
void put(std::vector<unsigned char> &img, size_t off, const std::vector<T> &v)
{
    if (!v.empty()) memcpy(img.data() + off, v.data(), v.size() * sizeof(T));
}

// Checks descs as mxq_quantize_rowwise does and builds the MXFP8 table image.
mxq_status mx_build(const mxq_group_desc *descs, int32_t n, std::vector<unsigned char> &img,
                    mxq_grouped_plan &plan)
{
    if (n < 0 || (n > 0 && !descs)) return MXQ_EINVAL;
    std::vector<GroupEntry> table;
    std::vector<int32_t> starts;
    int64_t tiles = 0;
    for (int32_t i = 0; i < n; ++i) {
        const mxq_group_desc &d = descs[i];
        mxq_status st = check_rowwise(d.x, d.rows, d.cols, d.ldx, d.q, d.ldq, d.scale, d.lds,
                                      nullptr, 0, true);
        if (st != MXQ_OK) return st;
        if (d.rows == 0 || d.cols == 0) continue;
        GroupEntry e;
        e.x = d.x;
        e.q = d.q;
        e.scale = d.scale;
        e.rows = d.rows;
        e.cols = d.cols;
        e.ldx = d.ldx;
        e.ldq = d.ldq;
        e.lds = d.lds;
        e.tile_begin = tiles;
        const int64_t t = mxq::mx_grouped_tiles(d.rows, d.cols, &e.nseg);
        if (__builtin_add_overflow(tiles, t, &tiles) || tiles > 0x7FFFFFFF) return MXQ_ESIZE;
        table.push_back(e);
        starts.push_back((int32_t)e.tile_begin);
    }
    const size_t m = table.size();
    img.assign(mx_table_bytes(m), 0);
    put(img, 0, table);
    put(img, m * sizeof(GroupEntry), starts);
    plan = mxq_grouped_plan{};
    plan.kind = kPlanMx;
    plan.n_entries = (int32_t)m;
    plan.total_tiles = tiles;
    plan.table_bytes = img.size();
    plan.workspace_bytes = img.size();
    return MXQ_OK;
}

// Checks descs as nvfp4_quantize_grouped does and builds the NVFP4 table image.
mxq_status nv_build(const nvfp4_group_desc *descs, int32_t n, int32_t n_groups,
                    std::vector<unsigned char> &img, mxq_grouped_plan &plan)
{
    if (n < 0 || n_groups < 0) return MXQ_EINVAL;
    if (n > 0 && (!descs || n_groups == 0)) return MXQ_EINVAL;
    std::vector<mxq::NvEntry> table;
    std::vector<int32_t> starts, groups;
    int64_t tiles = 0;
    for (int32_t i = 0; i < n; ++i) {
        const nvfp4_group_desc &d = descs[i];
        if (d.rows < 0 || d.cols < 0 || d.scale_group < 0 || d.scale_group >= n_groups)
            return MXQ_EINVAL;
        if (d.cols % 16 != 0) return MXQ_ESHAPE;
        if (d.rows == 0 || d.cols == 0) continue;
        if (!d.x || !d.q || !d.s) return MXQ_EINVAL;
        if (!aligned(d.x, 16) || !aligned(d.q, 4)) return MXQ_EALIGN;
        if (!fits(d.rows, d.cols)) return MXQ_ESIZE;
        mxq::NvEntry e;
        e.x = d.x;
        e.q = d.q;
        e.s = d.s;
        e.rows = d.rows;
        e.cols = d.cols;
        const int64_t t = mxq::nvfp4_tiles(d.rows, d.cols, &e.nseg);
        e.tile_begin = (int32_t)tiles;
        e.group = d.scale_group;
        if (__builtin_add_overflow(tiles, t, &tiles) || tiles > 0x7FFFFFFF) return MXQ_ESIZE;
        table.push_back(e);
        starts.push_back(e.tile_begin);
        groups.push_back(e.group);
    }
    const size_t m = table.size();
    img.assign(nv_table_bytes(m), 0);
    put(img, 0, table);
    put(img, m * sizeof(mxq::NvEntry), starts);
    put(img, m * (sizeof(mxq::NvEntry) + sizeof(int32_t)), groups);
    plan = mxq_grouped_plan{};
    plan.kind = kPlanNv;
    plan.n_entries = (int32_t)m;
    plan.n_groups = n_groups;
    plan.total_tiles = tiles;
    plan.table_bytes = img.size();
    plan.workspace_bytes = img.size() + round16((size_t)tiles * sizeof(uint32_t));
    return MXQ_OK;
}

// A plan as the build call of its kind leaves it.
bool plan_ok(const mxq_grouped_plan *p, int32_t kind)
{
    if (!p || p->kind != kind || p->n_entries < 0 || p->reserved != 0) return false;
    if (p->total_tiles < 0 || p->total_tiles > 0x7FFFFFFF) return false;
    if ((p->n_entries == 0) != (p->total_tiles == 0)) return false;
    if (kind == kPlanMx)
        return p->n_groups == 0 && p->table_bytes == mx_table_bytes((size_t)p->n_entries) &&
               p->workspace_bytes == p->table_bytes;
    return p->n_groups >= 0 && (p->n_entries == 0 || p->n_groups > 0) &&
           p->table_bytes == nv_table_bytes((size_t)p->n_entries) &&
           p->workspace_bytes ==
               p->table_bytes + round16((size_t)p->total_tiles * sizeof(uint32_t));
}

mxq_status launch_mx_plan(const mxq_grouped_plan &p, const void *table, hipStream_t stream)
{
    const unsigned char *t = static_cast<const unsigned char *>(table);
    return from_hip(mxq::launch_mx_grouped(
        reinterpret_cast<const GroupEntry *>(t),
        reinterpret_cast<const int32_t *>(t + (size_t)p.n_entries * sizeof(GroupEntry)),
        p.n_entries, p.total_tiles, stream));
}

mxq_status launch_nv_plan(const mxq_grouped_plan &p, float *gs, void *workspace,
                          hipStream_t stream)
{
    unsigned char *w = static_cast<unsigned char *>(workspace);
    const size_t m = (size_t)p.n_entries;
    return from_hip(mxq::launch_nvfp4_grouped(
        reinterpret_cast<const mxq::NvEntry *>(w),
        reinterpret_cast<const int32_t *>(w + m * sizeof(mxq::NvEntry)),
        reinterpret_cast<const int32_t *>(w + m * (sizeof(mxq::NvEntry) + sizeof(int32_t))),
        p.n_entries, reinterpret_cast<uint32_t *>(w + p.table_bytes), p.total_tiles, gs,
        p.n_groups, stream));
}

// Writes the image for a build call: NULL table_host only reports the plan.
mxq_status hand_over(const std::vector<unsigned char> &img, void *table_host, size_t bytes)
{
    if (!table_host) return MXQ_OK;
    if (bytes < img.size()) return MXQ_ESIZE;
    if (!img.empty()) memcpy(table_host, img.data(), img.size());
    return MXQ_OK;
}

}  // namespace

extern "C" {

const char *mxq_status_string(int status)
{
    switch (status) {
    case MXQ_OK: return "ok";
    case MXQ_EINVAL: return "invalid argument (null pointer, negative size or bad axis)";
    case MXQ_ESHAPE: return "unsupported shape (group/block divisibility or leading dimension)";
    case MXQ_EALIGN: return "misaligned pointer or leading dimension";
    case MXQ_EHIP: return "HIP runtime error at launch";
    case MXQ_ESIZE: return "workspace too small or size overflow";
    case MXQ_ECAPTURE:
        return "stream is being captured: this call copies from host memory (capture the plan form)";
    default: return "unknown status";
    }
}

int mxq_abi_version(void) { return MXQ_ABI_VERSION; }

#ifndef MXQ_BUILD_ID
#define MXQ_BUILD_ID "unidentified"  // built without the package's build script
#endif
const char *mxq_build_id(void) { return MXQ_BUILD_ID; }

mxq_status mxq_quantize_rowwise(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx,
                                uint8_t *q, int64_t ldq, uint8_t *scale, int64_t lds,
                                uint16_t *fq, int64_t ldf, void *stream)
{
    mxq_status st = check_rowwise(x, rows, cols, ldx, q, ldq, scale, lds, fq, ldf, true);
    if (st != MXQ_OK || rows == 0 || cols == 0) return st;
    return from_hip(mxq::launch_mx_rowwise(x, rows, cols, ldx, q, ldq, scale, lds, fq, ldf,
                                           as_stream(stream)));
}

mxq_status mxq_quantize_colwise(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *qc,
                                uint8_t *sc, uint8_t *qr, uint8_t *sr, uint16_t *fq, void *stream)
{
    if (rows < 0 || cols < 0) return MXQ_EINVAL;
    if (cols % 32 != 0) return MXQ_ESHAPE;
    if (rows == 0 || cols == 0) return MXQ_OK;
    if (!x || !qc || !sc) return MXQ_EINVAL;
    if ((qr == nullptr) != (sr == nullptr)) return MXQ_EINVAL;
    if (!aligned(x, 16) || !aligned(qc, 8) || !aligned(sc, 8)) return MXQ_EALIGN;
    if (qr && !aligned(qr, 8)) return MXQ_EALIGN;
    if (fq && !aligned(fq, 16)) return MXQ_EALIGN;
    if (!fits(rows, cols)) return MXQ_ESIZE;
    return from_hip(mxq::launch_mx_colwise(x, rows, cols, qc, sc, qr, sr, fq, nullptr,
                                           as_stream(stream)));
}

mxq_status mxq_dequantize(const uint8_t *q, const uint8_t *scale, int64_t rows, int64_t cols,
                          int axis, uint16_t *out, void *stream)
{
    if (rows < 0 || cols < 0 || (axis != 0 && axis != 1)) return MXQ_EINVAL;
    if (cols % 32 != 0) return MXQ_ESHAPE;
    if (rows == 0 || cols == 0) return MXQ_OK;
    if (!q || !scale || !out) return MXQ_EINVAL;
    if (!aligned(q, 8) || !aligned(out, 16)) return MXQ_EALIGN;
    if (axis == 0 && !aligned(scale, 8)) return MXQ_EALIGN;
    if (!fits(rows, cols)) return MXQ_ESIZE;
    return from_hip(mxq::launch_mx_dequant(q, scale, rows, cols, axis, out, as_stream(stream)));
}

mxq_status mxq_e8m0_to_fp32(const uint8_t *scale, int64_t n, float *out, void *stream)
{
    if (n < 0) return MXQ_EINVAL;
    if (n == 0) return MXQ_OK;
    if (!scale || !out) return MXQ_EINVAL;
    if (!aligned(out, 4)) return MXQ_EALIGN;
    return from_hip(mxq::launch_e8m0_to_f32(scale, n, out, as_stream(stream)));
}

mxq_status mxq_fake_quant(const uint16_t *x, int64_t rows, int64_t cols, int axis, uint16_t *out,
                          void *stream)
{
    if (rows < 0 || cols < 0 || (axis != 0 && axis != 1)) return MXQ_EINVAL;
    if (cols % 32 != 0) return MXQ_ESHAPE;
    if (rows == 0 || cols == 0) return MXQ_OK;
    if (!x || !out) return MXQ_EINVAL;
    if (!aligned(x, 16) || !aligned(out, 16)) return MXQ_EALIGN;
    if (!fits(rows, cols)) return MXQ_ESIZE;
    hipError_t e;
    if (axis == 1)
        e = mxq::launch_mx_rowwise(x, rows, cols, cols, nullptr, 0, nullptr, 0, out, cols,
                                   as_stream(stream));
    else
        e = mxq::launch_mx_colwise(x, rows, cols, nullptr, nullptr, nullptr, nullptr, nullptr, out,
                                   as_stream(stream));
    return from_hip(e);
}

mxq_status mxq_quantize_colwise_t(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *qt,
                                  int64_t ldt, uint8_t *st, uint8_t *qr, uint8_t *sr,
                                  uint16_t *fq, void *stream)
{
    if (rows < 0 || cols < 0) return MXQ_EINVAL;
    if (cols % 32 != 0) return MXQ_ESHAPE;
    if (rows == 0 || cols == 0) return MXQ_OK;
    if (!x || !qt || !st || (qr && !sr) || (sr && !qr)) return MXQ_EINVAL;
    if (ldt < rows) return MXQ_ESHAPE;
    if (!aligned(x, 16) || !aligned(qt, 16) || ldt % 16 != 0 || !aligned(st, 4)) return MXQ_EALIGN;
    if (qr && !aligned(qr, 8)) return MXQ_EALIGN;
    if (fq && !aligned(fq, 16)) return MXQ_EALIGN;
    if (!fits(rows, cols) || !fits(cols, ldt)) return MXQ_ESIZE;
    return from_hip(mxq::launch_mx_colwise_t(x, rows, cols, qt, ldt, st, qr, sr, fq,
                                             as_stream(stream)));
}

mxq_status mxfp4_quantize(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q_packed,
                          uint8_t *scale, uint16_t *fq, void *stream)
{
    if (rows < 0 || cols < 0) return MXQ_EINVAL;
    if (cols % 32 != 0) return MXQ_ESHAPE;
    if (rows == 0 || cols == 0) return MXQ_OK;
    if (!x || !q_packed || !scale) return MXQ_EINVAL;
    if (!aligned(x, 16) || !aligned(q_packed, 4) || (fq && !aligned(fq, 16))) return MXQ_EALIGN;
    if (!fits(rows, cols)) return MXQ_ESIZE;
    return from_hip(mxq::launch_mx4_quant(x, rows, cols, q_packed, scale, fq, as_stream(stream)));
}

mxq_status mxfp4_dequantize(const uint8_t *q_packed, const uint8_t *scale, int64_t rows,
                            int64_t cols, uint16_t *out, void *stream)
{
    if (rows < 0 || cols < 0) return MXQ_EINVAL;
    if (cols % 32 != 0) return MXQ_ESHAPE;
    if (rows == 0 || cols == 0) return MXQ_OK;
    if (!q_packed || !scale || !out) return MXQ_EINVAL;
    if (!aligned(q_packed, 4) || !aligned(out, 16)) return MXQ_EALIGN;
    if (!fits(rows, cols)) return MXQ_ESIZE;
    return from_hip(mxq::launch_mx4_dequant(q_packed, scale, rows, cols, out, as_stream(stream)));
}

mxq_status mxfp4_fake_quant(const uint16_t *x, int64_t rows, int64_t cols, uint16_t *out,
                            void *stream)
{
    if (rows < 0 || cols < 0) return MXQ_EINVAL;
    if (cols % 32 != 0) return MXQ_ESHAPE;
    if (rows == 0 || cols == 0) return MXQ_OK;
    if (!x || !out) return MXQ_EINVAL;
    if (!aligned(x, 16) || !aligned(out, 16)) return MXQ_EALIGN;
    if (!fits(rows, cols)) return MXQ_ESIZE;
    return from_hip(mxq::launch_mx4_quant(x, rows, cols, nullptr, nullptr, out, as_stream(stream)));
}

size_t mxq_grouped_workspace_size(int32_t n)
{
    // [GroupEntry x n][int32 first tile x n], rounded up to 16 bytes
    return n <= 0 ? 0 : ((size_t)n * (sizeof(GroupEntry) + sizeof(int32_t)) + 15) / 16 * 16;
}

size_t nvfp4_workspace_size(void) { return (size_t)mxq::kNvAmaxBlocks * sizeof(uint32_t); }

mxq_status mxq_quantize_rowwise_grouped(const mxq_group_desc *descs, int32_t n, void *workspace,
                                        size_t workspace_bytes, void *stream)
{
    if (n < 0) return MXQ_EINVAL;
    if (n == 0) return MXQ_OK;
    if (!descs || !workspace) return MXQ_EINVAL;
    if (!aligned(workspace, 16)) return MXQ_EALIGN;
    if (workspace_bytes < mxq_grouped_workspace_size(n)) return MXQ_ESIZE;
    std::vector<unsigned char> img;
    mxq_grouped_plan plan;
    mxq_status st = mx_build(descs, n, img, plan);
    if (st != MXQ_OK || plan.n_entries == 0) return st;
    st = refuse_capture(as_stream(stream));
    if (st != MXQ_OK) return st;
    // pageable source: the copy has read it by the time hipMemcpyAsync returns
    if (hipMemcpyAsync(workspace, img.data(), img.size(), hipMemcpyHostToDevice,
                       as_stream(stream)) != hipSuccess)
        return MXQ_EHIP;
    return launch_mx_plan(plan, workspace, as_stream(stream));
}

mxq_status mxq_grouped_plan_build(const mxq_group_desc *descs, int32_t n, mxq_grouped_plan *plan,
                                  void *table_host, size_t table_host_bytes)
{
    if (!plan) return MXQ_EINVAL;
    std::vector<unsigned char> img;
    mxq_grouped_plan p;
    mxq_status st = mx_build(descs, n, img, p);
    if (st != MXQ_OK) return st;
    st = hand_over(img, table_host, table_host_bytes);
    if (st == MXQ_OK) *plan = p;
    return st;
}

mxq_status mxq_quantize_rowwise_grouped_plan(const mxq_grouped_plan *plan, const void *table_dev,
                                             size_t table_dev_bytes, void *stream)
{
    if (!plan_ok(plan, kPlanMx)) return MXQ_EINVAL;
    if (plan->n_entries == 0) return MXQ_OK;
    if (!table_dev) return MXQ_EINVAL;
    if (!aligned(table_dev, 16)) return MXQ_EALIGN;
    if (table_dev_bytes < plan->workspace_bytes) return MXQ_ESIZE;
    return launch_mx_plan(*plan, table_dev, as_stream(stream));
}

mxq_status blockfp8_quantize(const uint16_t *x, int64_t rows, int64_t cols, int32_t blk,
                             uint8_t *q, float *scale, void *stream)
{
    if (rows < 0 || cols < 0) return MXQ_EINVAL;
    if (blk != 128 || cols % 8 != 0) return MXQ_ESHAPE;
    if (rows == 0 || cols == 0) return MXQ_OK;
    if (!x || !q || !scale) return MXQ_EINVAL;
    if (!aligned(x, 16) || !aligned(q, 8) || !aligned(scale, 4)) return MXQ_EALIGN;
    if (!fits(rows, cols)) return MXQ_ESIZE;
    return from_hip(mxq::launch_bfp8_quant(x, 1, rows, cols, q, scale, as_stream(stream)));
}

mxq_status blockfp8_dequantize(const uint8_t *q, const float *scale, int64_t rows, int64_t cols,
                               int32_t blk, uint16_t *out, void *stream)
{
    if (rows < 0 || cols < 0) return MXQ_EINVAL;
    if (blk != 128 || cols % 8 != 0) return MXQ_ESHAPE;
    if (rows == 0 || cols == 0) return MXQ_OK;
    if (!q || !scale || !out) return MXQ_EINVAL;
    if (!aligned(q, 8) || !aligned(out, 16) || !aligned(scale, 4)) return MXQ_EALIGN;
    if (!fits(rows, cols)) return MXQ_ESIZE;
    return from_hip(mxq::launch_bfp8_dequant(q, scale, 1, rows, cols, false, out,
                                             as_stream(stream)));
}

mxq_status blockfp8_quantize_gkn(const uint16_t *x, int64_t G, int64_t K, int64_t N, int32_t blk,
                                 uint8_t *q, float *scale, void *stream)
{
    if (G < 0 || K < 0 || N < 0) return MXQ_EINVAL;
    if (blk != 128 || N % 8 != 0) return MXQ_ESHAPE;
    if (G == 0 || K == 0 || N == 0) return MXQ_OK;
    if (!x || !q || !scale) return MXQ_EINVAL;
    if (!aligned(x, 16) || !aligned(q, 8) || !aligned(scale, 4)) return MXQ_EALIGN;
    int64_t kn;
    if (__builtin_mul_overflow(K, N, &kn) || !fits(G, kn)) return MXQ_ESIZE;
    return from_hip(mxq::launch_bfp8_quant(x, G, K, N, q, scale, as_stream(stream)));
}

mxq_status blockfp8_dequantize_gkn(const uint8_t *q, const float *scale, int64_t G, int64_t K,
                                   int64_t N, int32_t blk, uint16_t *out, void *stream)
{
    if (G < 0 || K < 0 || N < 0) return MXQ_EINVAL;
    if (blk != 128 || N % 8 != 0) return MXQ_ESHAPE;
    if (G == 0 || K == 0 || N == 0) return MXQ_OK;
    if (!q || !scale || !out) return MXQ_EINVAL;
    if (!aligned(q, 8) || !aligned(out, 16) || !aligned(scale, 4)) return MXQ_EALIGN;
    int64_t kn;
    if (__builtin_mul_overflow(K, N, &kn) || !fits(G, kn)) return MXQ_ESIZE;
    return from_hip(mxq::launch_bfp8_dequant(q, scale, G, K, N, false, out, as_stream(stream)));
}

mxq_status blockfp8_quantize_1x128(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q,
                                   float *scale, uint16_t *fq, void *stream)
{
    if (rows < 0 || cols < 0) return MXQ_EINVAL;
    if (cols % 8 != 0) return MXQ_ESHAPE;
    if (rows == 0 || cols == 0) return MXQ_OK;
    if (!x || !q || !scale) return MXQ_EINVAL;
    if (!aligned(x, 16) || !aligned(q, 8) || !aligned(scale, 4) || (fq && !aligned(fq, 16)))
        return MXQ_EALIGN;
    if (!fits(rows, cols)) return MXQ_ESIZE;
    return from_hip(mxq::launch_bfp8_1x128(x, rows, cols, q, scale, fq, as_stream(stream)));
}

mxq_status blockfp8_dequantize_1x128(const uint8_t *q, const float *scale, int64_t rows,
                                     int64_t cols, uint16_t *out, void *stream)
{
    if (rows < 0 || cols < 0) return MXQ_EINVAL;
    if (cols % 8 != 0) return MXQ_ESHAPE;
    if (rows == 0 || cols == 0) return MXQ_OK;
    if (!q || !scale || !out) return MXQ_EINVAL;
    if (!aligned(q, 8) || !aligned(out, 16) || !aligned(scale, 4)) return MXQ_EALIGN;
    if (!fits(rows, cols)) return MXQ_ESIZE;
    return from_hip(mxq::launch_bfp8_dequant(q, scale, 1, rows, cols, true, out,
                                             as_stream(stream)));
}

mxq_status blockfp8_fake_quant_1x128(const uint16_t *x, int64_t rows, int64_t cols,
                                     uint16_t *out, void *stream)
{
    if (rows < 0 || cols < 0) return MXQ_EINVAL;
    if (cols % 8 != 0) return MXQ_ESHAPE;
    if (rows == 0 || cols == 0) return MXQ_OK;
    if (!x || !out) return MXQ_EINVAL;
    if (!aligned(x, 16) || !aligned(out, 16)) return MXQ_EALIGN;
    if (!fits(rows, cols)) return MXQ_ESIZE;
    return from_hip(mxq::launch_bfp8_1x128(x, rows, cols, nullptr, nullptr, out,
                                           as_stream(stream)));
}

mxq_status blockfp8_to_mxfp8(const uint8_t *q, const float *scale, int64_t rows, int64_t cols,
                             int32_t blk, uint8_t *q8, uint8_t *scale8, void *stream)
{
    if (rows < 0 || cols < 0) return MXQ_EINVAL;
    if (blk != 128 || cols % 32 != 0) return MXQ_ESHAPE;
    if (rows == 0 || cols == 0) return MXQ_OK;
    if (!q || !scale || !q8 || !scale8) return MXQ_EINVAL;
    if (!aligned(q, 8) || !aligned(scale, 4) || !aligned(q8, 8)) return MXQ_EALIGN;
    if (!fits(rows, cols)) return MXQ_ESIZE;
    return from_hip(mxq::launch_bfp8_to_mx(q, scale, rows, cols, q8, scale8, as_stream(stream)));
}

// Checks shared by the two single-tensor NVFP4 entry points.
static mxq_status check_nvfp4(const uint16_t *x, int64_t rows, int64_t cols,
                              const uint8_t *q_packed, const uint8_t *s_e4m3,
                              const float *global_scale)
{
    if (rows < 0 || cols < 0) return MXQ_EINVAL;
    if (cols % 16 != 0) return MXQ_ESHAPE;
    if (rows == 0 || cols == 0) return MXQ_OK;
    if (!x || !q_packed || !s_e4m3 || !global_scale) return MXQ_EINVAL;
    if (!aligned(x, 16) || !aligned(q_packed, 4) || !aligned(global_scale, 4)) return MXQ_EALIGN;
    if (!fits(rows, cols)) return MXQ_ESIZE;
    return MXQ_OK;
}

mxq_status nvfp4_quantize(const uint16_t *x, int64_t rows, int64_t cols, uint8_t *q_packed,
                          uint8_t *s_e4m3, float *global_scale, void *workspace,
                          size_t workspace_bytes, void *stream)
{
    mxq_status st = check_nvfp4(x, rows, cols, q_packed, s_e4m3, global_scale);
    if (st != MXQ_OK || rows == 0 || cols == 0) return st;
    if (!workspace) return MXQ_EINVAL;
    if (workspace_bytes < nvfp4_workspace_size()) return MXQ_ESIZE;
    if (!aligned(workspace, 4)) return MXQ_EALIGN;
    return from_hip(mxq::launch_nvfp4_quant(x, rows, cols, q_packed, s_e4m3, global_scale,
                                            static_cast<uint32_t *>(workspace),
                                            (int64_t)(workspace_bytes / sizeof(uint32_t)),
                                            as_stream(stream)));
}

mxq_status nvfp4_quantize_noalloc(const uint16_t *x, int64_t rows, int64_t cols,
                                  uint8_t *q_packed, uint8_t *s_e4m3, float *global_scale,
                                  void *stream)
{
    mxq_status st = check_nvfp4(x, rows, cols, q_packed, s_e4m3, global_scale);
    if (st != MXQ_OK || rows == 0 || cols == 0) return st;
    const hipError_t err = mxq::launch_nvfp4_quant_noalloc(x, rows, cols, q_packed, s_e4m3,
                                                           global_scale, as_stream(stream));
    return err == hipErrorInvalidValue ? MXQ_ESIZE : from_hip(err);
}

size_t nvfp4_grouped_workspace_size(const nvfp4_group_desc *descs, int32_t n)
{
    if (n <= 0 || !descs) return 0;
    size_t tiles = 0;
    for (int32_t i = 0; i < n; ++i)
        if (descs[i].rows > 0 && descs[i].cols > 0)
            tiles += (size_t)mxq::nvfp4_tiles(descs[i].rows, descs[i].cols, nullptr);
    return nv_table_bytes((size_t)n) + round16(tiles * sizeof(uint32_t));
}

mxq_status nvfp4_quantize_grouped(const nvfp4_group_desc *descs, int32_t n, float *global_scales,
                                  int32_t n_groups, void *workspace, size_t workspace_bytes,
                                  void *stream)
{
    if (n < 0 || n_groups < 0) return MXQ_EINVAL;
    if (n > 0 && (!descs || n_groups == 0)) return MXQ_EINVAL;
    if (n_groups == 0) return MXQ_OK;
    if (!global_scales) return MXQ_EINVAL;
    if (!aligned(global_scales, 4)) return MXQ_EALIGN;
    std::vector<unsigned char> img;
    mxq_grouped_plan plan;
    mxq_status st = nv_build(descs, n, n_groups, img, plan);
    if (st != MXQ_OK) return st;
    if (!workspace) return MXQ_EINVAL;
    if (!aligned(workspace, 16)) return MXQ_EALIGN;
    if (workspace_bytes < nvfp4_grouped_workspace_size(descs, n)) return MXQ_ESIZE;
    st = refuse_capture(as_stream(stream));
    if (st != MXQ_OK) return st;
    // pageable source: the copy has read it by the time it returns
    if (!img.empty() && hipMemcpyAsync(workspace, img.data(), img.size(), hipMemcpyHostToDevice,
                                       as_stream(stream)) != hipSuccess)
        return MXQ_EHIP;
    return launch_nv_plan(plan, global_scales, workspace, as_stream(stream));
}

mxq_status nvfp4_grouped_plan_build(const nvfp4_group_desc *descs, int32_t n, int32_t n_groups,
                                    mxq_grouped_plan *plan, void *table_host,
                                    size_t table_host_bytes)
{
    if (!plan) return MXQ_EINVAL;
    std::vector<unsigned char> img;
    mxq_grouped_plan p;
    mxq_status st = nv_build(descs, n, n_groups, img, p);
    if (st != MXQ_OK) return st;
    st = hand_over(img, table_host, table_host_bytes);
    if (st == MXQ_OK) *plan = p;
    return st;
}

mxq_status nvfp4_quantize_grouped_plan(const mxq_grouped_plan *plan, float *global_scales,
                                       void *workspace, size_t workspace_bytes, void *stream)
{
    if (!plan_ok(plan, kPlanNv)) return MXQ_EINVAL;
    if (plan->n_groups == 0) return MXQ_OK;
    if (!global_scales) return MXQ_EINVAL;
    if (!aligned(global_scales, 4)) return MXQ_EALIGN;
    if (plan->workspace_bytes > 0) {  // else no member has elements: only the scales are written
        if (!workspace) return MXQ_EINVAL;
        if (!aligned(workspace, 16)) return MXQ_EALIGN;
        if (workspace_bytes < plan->workspace_bytes) return MXQ_ESIZE;
    }
    return launch_nv_plan(*plan, global_scales, workspace, as_stream(stream));
}

mxq_status nvfp4_dequantize(const uint8_t *q_packed, const uint8_t *s_e4m3,
                            const float *global_scale, int64_t rows, int64_t cols, uint16_t *out,
                            void *stream)
{
    if (rows < 0 || cols < 0) return MXQ_EINVAL;
    if (cols % 16 != 0) return MXQ_ESHAPE;
    if (rows == 0 || cols == 0) return MXQ_OK;
    if (!q_packed || !s_e4m3 || !global_scale || !out) return MXQ_EINVAL;
    if (!aligned(q_packed, 4) || !aligned(out, 16) || !aligned(global_scale, 4)) return MXQ_EALIGN;
    if (!fits(rows, cols)) return MXQ_ESIZE;
    return from_hip(mxq::launch_nvfp4_dequant(q_packed, s_e4m3, global_scale, rows, cols, out,
                                              as_stream(stream)));
}

}  // extern "C"
