// Shared host-side plumbing of the kernel sources: timed launches, ceil_div,
// the calibration kernels.  Per-family interfaces: nh_bn.hpp, nh_rows.hpp.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nh_device.hpp"
#include "normhip.h"

namespace nh {

// ---- per-kernel timing (api.cpp) -------------------------------------------
bool timing_on();
// Hands out a start/stop event pair recorded under kernel id `kid`.
void timing_events(int kid, hipEvent_t *start, hipEvent_t *stop);

// Launch through hipExtLaunchKernel so that, with timing on, the dispatch
// packet itself carries the start/stop timestamps.
template <typename... KArgs, typename... Args>
inline hipError_t launch(int kid, void (*kernel)(KArgs...), dim3 grid, dim3 block,
                         uint32_t shmem, hipStream_t stream, Args... args)
{
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (timing_on()) timing_events(kid, &e0, &e1);
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, e0, e1, 0u,
                          static_cast<KArgs>(args)...);
    return hipGetLastError();
}

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---- calibration --------------------------------------------------------------
hipError_t calib_copy_launch(const void *src, void *dst, size_t bytes, int slots, hipStream_t s);
hipError_t calib_add_launch(const float *a, const float *b, float *o, int64_t n, int slots, hipStream_t s);
hipError_t calib_read_launch(const float *a, int64_t n, float *sums, int64_t max_blocks, int slots,
                             hipStream_t s);

} // namespace nh
