// Calibration streams: a plain copy and a two-read/one-write add with the
// same access pattern as the elementwise passes.  They give the measured
// bandwidth floor that Aether-ML PR #18 ("Backward finalize" section) uses to
// call its elementwise backward "at the DRAM floor": a plain add with the
// same reads and writes takes as long.
#include "nh_internal.hpp"

namespace nh {

constexpr int kCalibThreads = 256;
constexpr int kCalibUnroll = 4;

// Each block streams one contiguous chunk, kCalibUnroll 16-byte accesses in
// flight per thread, every access nontemporal: the fastest plain stream
// shape measured on MI355X.
__global__ void __launch_bounds__(kCalibThreads)
calib_copy16_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst, int64_t n16, int64_t chunk)
{
    const int64_t b0 = (int64_t)blockIdx.x * chunk;
    const int64_t b1 = b0 + chunk < n16 ? b0 + chunk : n16;
    const u32x4_t *s4 = reinterpret_cast<const u32x4_t *>(src);
    u32x4_t *d4 = reinterpret_cast<u32x4_t *>(dst);
    for (int64_t base = b0 + threadIdx.x; base < b1; base += kCalibThreads * kCalibUnroll) {
        u32x4_t v[kCalibUnroll];
#pragma unroll
        for (int k = 0; k < kCalibUnroll; ++k) {
            const int64_t i = base + k * kCalibThreads;
            if (i < b1) v[k] = nt_load(s4 + i);
        }
#pragma unroll
        for (int k = 0; k < kCalibUnroll; ++k) {
            const int64_t i = base + k * kCalibThreads;
            if (i < b1) __builtin_nontemporal_store(v[k], d4 + i);
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
                  float4 *__restrict__ o, int64_t n4, int64_t chunk)
{
    const int64_t b0 = (int64_t)blockIdx.x * chunk;
    const int64_t b1 = b0 + chunk < n4 ? b0 + chunk : n4;
    const f32x4_t *a4 = reinterpret_cast<const f32x4_t *>(a);
    const f32x4_t *c4 = reinterpret_cast<const f32x4_t *>(b);
    f32x4_t *o4 = reinterpret_cast<f32x4_t *>(o);
    for (int64_t base = b0 + threadIdx.x; base < b1; base += kCalibThreads * kCalibUnroll) {
        f32x4_t va[kCalibUnroll], vb[kCalibUnroll];
#pragma unroll
        for (int k = 0; k < kCalibUnroll; ++k) {
            const int64_t i = base + k * kCalibThreads;
            if (i < b1) { va[k] = nt_load(a4 + i); vb[k] = nt_load(c4 + i); }
        }
#pragma unroll
        for (int k = 0; k < kCalibUnroll; ++k) {
            const int64_t i = base + k * kCalibThreads;
            if (i < b1) __builtin_nontemporal_store(va[k] + vb[k], o4 + i);
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

// A read-only reduction stream shaped like the BatchNorm stats pass: one
// contiguous chunk per block, kCalibUnroll cacheable 16-byte loads in flight
// per thread, a block sum at the end, one float written per block.
__global__ void __launch_bounds__(kCalibThreads)
calib_read4_kernel(const float4 *__restrict__ a, int64_t n4, int64_t chunk, float *__restrict__ sums)
{
    __shared__ float red[kCalibThreads / kWave];
    const int64_t b0 = (int64_t)blockIdx.x * chunk;
    const int64_t b1 = b0 + chunk < n4 ? b0 + chunk : n4;
    float acc = 0.f;
    for (int64_t base = b0 + threadIdx.x; base < b1; base += kCalibThreads * kCalibUnroll) {
        float4 v[kCalibUnroll];
#pragma unroll
        for (int k = 0; k < kCalibUnroll; ++k) {
            const int64_t i = base + k * kCalibThreads;
            if (i < b1) v[k] = a[i];
        }
#pragma unroll
        for (int k = 0; k < kCalibUnroll; ++k) {
            const int64_t i = base + k * kCalibThreads;
            if (i < b1) acc += (v[k].x + v[k].y) + (v[k].z + v[k].w);
        }
    }
    acc = wave_sum(acc);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = red[0];
#pragma unroll
        for (int w = 1; w < kCalibThreads / kWave; ++w) t += red[w];
        sums[blockIdx.x] = t;
    }
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
        const unsigned grid = calib_grid(n16, slots);
        return launch(NH_K_CALIB, calib_copy16_kernel, dim3(grid), dim3(kCalibThreads), 0u, s,
                      (const uint4 *)src, (uint4 *)dst, n16, ceil_div(n16, grid));
    }
    return launch(NH_K_CALIB, calib_copy1_kernel, dim3(calib_grid((int64_t)bytes, slots)),
                  dim3(kCalibThreads), 0u, s, (const uint8_t *)src, (uint8_t *)dst, (int64_t)bytes);
}

hipError_t calib_add_launch(const float *a, const float *b, float *o, int64_t n, int slots, hipStream_t s)
{
    const bool vec = n % 4 == 0 && ((uintptr_t)a % 16) == 0 && ((uintptr_t)b % 16) == 0 &&
                     ((uintptr_t)o % 16) == 0;
    if (vec) {
        const unsigned grid = calib_grid(n / 4, slots);
        return launch(NH_K_CALIB, calib_add4_kernel, dim3(grid), dim3(kCalibThreads), 0u, s,
                      (const float4 *)a, (const float4 *)b, (float4 *)o, n / 4,
                      ceil_div(n / 4, grid));
    }
    return launch(NH_K_CALIB, calib_add1_kernel, dim3(calib_grid(n, slots)), dim3(kCalibThreads),
                  0u, s, a, b, o, n);
}

hipError_t calib_read_launch(const float *a, int64_t n, float *sums, int64_t max_blocks, int slots,
                             hipStream_t s)
{
    int64_t cap = max_blocks < slots ? max_blocks : slots;
    const unsigned grid = calib_grid(n / 4, (int)cap);
    return launch(NH_K_CALIB, calib_read4_kernel, dim3(grid), dim3(kCalibThreads), 0u, s,
                  (const float4 *)a, n / 4, ceil_div(n / 4, grid), sums);
}

} // namespace nh
