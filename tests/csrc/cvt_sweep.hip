// cvt_sweep.hip -- TEST ONLY: runs the library's fp32 -> E4M3 / E2M1 / bf16
// converters (mxq_device.hpp) over runs of fp32 bit patterns, so a test can
// compare every pattern with the CPU oracle's encoders.  Pattern i of a call
// is first + i * stride; the host checks that none wraps past 0xFFFFFFFF.
//
// For each pattern t (an fp32 value) and its negation:
//   e4m3  hw[i] = bytes (code(t), code(-t), code(-t), code(t)) from the two
//                 halves of cvt_fp8x2_f32 (v_cvt_pk_fp8_f32 after the clamp)
//         sw[i] = e4m3_mag_from_f32(t)           (t >= 0 only)
//   e2m1  hw[i] = bytes (c(t) | c(-t) << 4, c(-t) | c(t) << 4, c(t) | c(t) << 4,
//                 c(-t) | c(-t) << 4) from the four byte slots of cvt_fp4x2_f32
//         sw[i] = e2m1_mag_from_f32(t)
//   bf16  hw[i] = bf16x2_rne(t, -t) (v_cvt_pk_bf16_f32: bf16(t) low, bf16(-t) high)
//         sw[i] = bf16_rne(t)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq_device.hpp"

#ifndef SWEEP_BUILD_ID
#define SWEEP_BUILD_ID "unidentified"
#endif

namespace {

__device__ __forceinline__ float pattern(uint32_t first, int64_t i, uint32_t stride)
{
    return __uint_as_float(first + (uint32_t)i * stride);
}

__global__ __launch_bounds__(256) void sweep_e4m3(uint32_t first, int64_t n, uint32_t stride,
                                                  uint32_t *__restrict__ hw,
                                                  uint8_t *__restrict__ sw)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float t = pattern(first, i, stride);
    hw[i] = mxq::cvt_fp8x2_f32<true>(mxq::cvt_fp8x2_f32<false>(0u, t, -t), -t, t);
    sw[i] = (uint8_t)mxq::e4m3_mag_from_f32(__builtin_fabsf(t));
}

__global__ __launch_bounds__(256) void sweep_e2m1(uint32_t first, int64_t n, uint32_t stride,
                                                  uint32_t *__restrict__ hw,
                                                  uint8_t *__restrict__ sw)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float t = pattern(first, i, stride);
    uint32_t w = mxq::cvt_fp4x2_f32<0>(0u, t, -t);
    w = mxq::cvt_fp4x2_f32<1>(w, -t, t);
    w = mxq::cvt_fp4x2_f32<2>(w, t, t);
    hw[i] = mxq::cvt_fp4x2_f32<3>(w, -t, -t);
    sw[i] = (uint8_t)mxq::e2m1_mag_from_f32(__builtin_fabsf(t));
}

__global__ __launch_bounds__(256) void sweep_bf16(uint32_t first, int64_t n, uint32_t stride,
                                                  uint32_t *__restrict__ hw,
                                                  uint16_t *__restrict__ sw)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float t = pattern(first, i, stride);
    hw[i] = mxq::bf16x2_rne(t, -t);
    sw[i] = (uint16_t)mxq::bf16_rne(t);
}

// 0 on success, 1 for bad arguments (nothing launched), 2 for a launch error.
template <class K, class S>
int launch(K kernel, uint32_t first, int64_t n, uint32_t stride, uint32_t *hw, S *sw,
           void *stream)
{
    if (n <= 0 || n > (int64_t(1) << 30) || !hw || !sw || stride == 0) return 1;
    if ((uint64_t)first + (uint64_t)(n - 1) * stride > 0xFFFFFFFFull) return 1;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, first, n, stride,
                       hw, sw);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // namespace

extern "C" {

const char *cvt_sweep_build_id(void) { return SWEEP_BUILD_ID; }

int cvt_sweep_e4m3(uint32_t first, int64_t n, uint32_t stride, uint32_t *hw, uint8_t *sw,
                   void *stream)
{
    return launch(sweep_e4m3, first, n, stride, hw, sw, stream);
}

int cvt_sweep_e2m1(uint32_t first, int64_t n, uint32_t stride, uint32_t *hw, uint8_t *sw,
                   void *stream)
{
    return launch(sweep_e2m1, first, n, stride, hw, sw, stream);
}

int cvt_sweep_bf16(uint32_t first, int64_t n, uint32_t stride, uint32_t *hw, uint16_t *sw,
                   void *stream)
{
    return launch(sweep_bf16, first, n, stride, hw, sw, stream);
}

}  // extern "C"
