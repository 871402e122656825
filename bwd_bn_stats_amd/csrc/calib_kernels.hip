// Calibration streams: a plain copy and a two-read/one-write add with the
// same access pattern as the elementwise passes.  They give the measured
// bandwidth floor that Aether-ML PR #18 ("Backward finalize" section) uses to
// call its elementwise backward "at the DRAM floor": a plain add with the
// same reads and writes takes as long.
#include "nh_internal.hpp"

namespace nh {

constexpr int kCalibThreads = 256;
constexpr int kCalibUnroll = 4;

__global__ void __launch_bounds__(kCalibThreads)
calib_copy16_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst, int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * kCalibThreads;
    for (int64_t base = (int64_t)blockIdx.x * kCalibThreads + threadIdx.x; base < n16;
         base += stride * kCalibUnroll) {
        uint4 v[kCalibUnroll];
#pragma unroll
        for (int k = 0; k < kCalibUnroll; ++k) {
            const int64_t i = base + k * stride;
            if (i < n16) v[k] = src[i];
        }
#pragma unroll
        for (int k = 0; k < kCalibUnroll; ++k) {
            const int64_t i = base + k * stride;
            if (i < n16) dst[i] = v[k];
        }
    }
}

__global__ void __launch_bounds__(kCalibThreads)
calib_copy1_kernel(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * kCalibThreads;
    for (int64_t i = (int64_t)blockIdx.x * kCalibThreads + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

__global__ void __launch_bounds__(kCalibThreads)
calib_add4_kernel(const float4 *__restrict__ a, const float4 *__restrict__ b,
                  float4 *__restrict__ o, int64_t n4)
{
    const int64_t stride = (int64_t)gridDim.x * kCalibThreads;
    for (int64_t base = (int64_t)blockIdx.x * kCalibThreads + threadIdx.x; base < n4;
         base += stride * kCalibUnroll) {
        float4 va[kCalibUnroll], vb[kCalibUnroll];
#pragma unroll
        for (int k = 0; k < kCalibUnroll; ++k) {
            const int64_t i = base + k * stride;
            if (i < n4) { va[k] = a[i]; vb[k] = b[i]; }
        }
#pragma unroll
        for (int k = 0; k < kCalibUnroll; ++k) {
            const int64_t i = base + k * stride;
            if (i < n4)
                o[i] = make_float4(va[k].x + vb[k].x, va[k].y + vb[k].y, va[k].z + vb[k].z,
                                   va[k].w + vb[k].w);
        }
    }
}

__global__ void __launch_bounds__(kCalibThreads)
calib_add1_kernel(const float *__restrict__ a, const float *__restrict__ b, float *__restrict__ o,
                  int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * kCalibThreads;
    for (int64_t i = (int64_t)blockIdx.x * kCalibThreads + threadIdx.x; i < n; i += stride)
        o[i] = a[i] + b[i];
}

static unsigned calib_grid(int64_t items, int slots)
{
    int64_t g = ceil_div(items, (int64_t)kCalibThreads * kCalibUnroll);
    if (g > slots) g = slots;
    if (g < 1) g = 1;
    return (unsigned)g;
}

hipError_t calib_copy_launch(const void *src, void *dst, size_t bytes, int slots, hipStream_t s)
{
    const bool vec = bytes % 16 == 0 && ((uintptr_t)src % 16) == 0 && ((uintptr_t)dst % 16) == 0;
    if (vec) {
        const int64_t n16 = (int64_t)(bytes / 16);
        return launch(NH_K_CALIB, calib_copy16_kernel, dim3(calib_grid(n16, slots)),
                      dim3(kCalibThreads), 0u, s, (const uint4 *)src, (uint4 *)dst, n16);
    }
    return launch(NH_K_CALIB, calib_copy1_kernel, dim3(calib_grid((int64_t)bytes, slots)),
                  dim3(kCalibThreads), 0u, s, (const uint8_t *)src, (uint8_t *)dst, (int64_t)bytes);
}

hipError_t calib_add_launch(const float *a, const float *b, float *o, int64_t n, int slots, hipStream_t s)
{
    const bool vec = n % 4 == 0 && ((uintptr_t)a % 16) == 0 && ((uintptr_t)b % 16) == 0 &&
                     ((uintptr_t)o % 16) == 0;
    if (vec)
        return launch(NH_K_CALIB, calib_add4_kernel, dim3(calib_grid(n / 4, slots)),
                      dim3(kCalibThreads), 0u, s, (const float4 *)a, (const float4 *)b, (float4 *)o,
                      n / 4);
    return launch(NH_K_CALIB, calib_add1_kernel, dim3(calib_grid(n, slots)), dim3(kCalibThreads),
                  0u, s, a, b, o, n);
}

} // namespace nh
