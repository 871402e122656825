// Host-side interface between the C ABI (api.cpp) and the kernel sources.
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

// ---- BatchNorm -------------------------------------------------------------
constexpr int kBnThreads = 256;
constexpr int kBnUnroll = 4;     // vector units in flight per thread

// Blocks per channel for a channel of `units` vector units: enough blocks
// that all C*grid_y blocks fill the device's resident slots once, but no
// block gets less than one full unrolled sweep of its threads.
inline int64_t bn_auto_grid_y(int64_t units, int64_t C, int64_t slots)
{
    int64_t per_channel = slots / (C > 0 ? C : 1);
    if (per_channel < 1) per_channel = 1;
    int64_t want = ceil_div(units, (int64_t)kBnThreads * kBnUnroll);
    if (want < 1) want = 1;
    return want < per_channel ? want : per_channel;
}

// Geometry of a BatchNorm launch: channel c's M elements in units of V
// consecutive elements inside one plane, block (c, yb) owning units
// [yb*upb, min((yb+1)*upb, units)).
struct BnGeom {
    int C;
    int HW;
    int HWv;        // units per plane
    FastDiv div_hwv;
    int units;      // units per channel (N * HWv)
    int upb;        // units per block
    int grid_y;
};

// Element offset of unit u of channel c.  Unsigned arithmetic: callers may
// form the offset of a unit past the end (never dereferenced), which must
// not be signed overflow.
template <int V>
__host__ __device__ __forceinline__ int bn_unit_offset(const BnGeom &g, int c, uint32_t u)
{
    const uint32_t n = g.div_hwv.div(u);
    const uint32_t j = u - n * (uint32_t)g.HWv;
    return (int)((n * (uint32_t)g.C + (uint32_t)c) * (uint32_t)g.HW + j * (uint32_t)V);
}

inline BnGeom make_bn_geom(int N, int C, int HW, int vec, int grid_y)
{
    BnGeom g;
    g.C = C;
    g.HW = HW;
    g.HWv = HW / vec;
    g.div_hwv = make_fastdiv((uint32_t)g.HWv);
    g.units = N * g.HWv;
    g.grid_y = grid_y;
    g.upb = (int)ceil_div(g.units, grid_y);
    return g;
}

struct BnCall {
    int io;              // 0 fp32, 1 bf16
    int N, C, HW;
    int vec;             // vector width in elements (1, 4 or 8)
    int grid_y;          // blocks per channel of the reduction and elementwise passes
    int separate_finalize;  // 1: finalize as its own kernel; 0: in the elementwise prologue
    int inference;       // forward only: apply with the running statistics, no reduction
    int act;             // 0 none, 1 ReLU, 2 LeakyReLU
    float slope;         // LeakyReLU negative slope
    const void *x;
    const void *dy;      // backward only
    void *out;           // y (forward) or dx (backward; may be NULL)
    const float *gamma, *beta;         // beta is also read by the backward with an activation
    float *running_mean, *running_var;
    float momentum, eps;
    float *stats;        // [4, C]
    float *grads;        // [4, C] (backward)
    float *partials;     // [2, grid_y, C]
};

hipError_t bn_forward_launch(const BnCall &a, hipStream_t s);
hipError_t bn_backward_launch(const BnCall &a, hipStream_t s);

// ---- LayerNorm / RMSNorm rows -------------------------------------------------
struct RowsCall {
    int kind;            // 0 LayerNorm, 1 RMSNorm, 2 bias + dropout + add + LayerNorm
    int x_t, dy_t, w_t, dx_t;
    int rows, cols;
    int blocks;          // G: column-partial rows
    int maxg;            // 16-byte groups per thread per row (vector path); 0 = generic path
    int vec;             // elements per group
    const void *x, *dy, *w;
    const float *mean, *rstd;  // LayerNorm
    const float *rms;          // RMSNorm (NULL: recompute)
    float eps;
    void *dx, *dweight, *dbias;  // kind 2: dx is da (dtype dy_t)
    const float *dresidual;      // kind 2: fp32 [rows, cols] or NULL
    const uint8_t *mask;         // kind 2: 0/1 bytes [rows, cols] or NULL
    float scale;                 // kind 2: dropout scale
    float *dh;                   // kind 2: fp32 [rows, cols] out or NULL
    void *dbias_in;              // kind 2: [cols] of w_t out or NULL
    float *partials;     // [Q, G, cols]
    int depth;           // row-pipeline depth of the vector path (0 = the kernel's default)
    int colsum_cols;     // columns per column-finalize block (0 = default)
    int *occupancy_out;  // non-NULL: report resident 256-thread blocks per CU
                         // of the selected row kernel instead of launching
};

hipError_t rows_backward_launch(const RowsCall &a, hipStream_t s);
hipError_t bda_backward_launch(const RowsCall &a, hipStream_t s);
// Column finalize of the Q = rows_q(kind) partial rows into dweight, dbias, dbias_in.
hipError_t rows_colsum_launch(const RowsCall &a, int kid, hipStream_t s);
// Column sums per kind: LayerNorm dweight, dbias; RMSNorm dweight;
// bias + dropout + add + LayerNorm dweight, dbias, dbias_in.
constexpr int rows_q(int kind) { return kind == 0 ? 2 : (kind == 1 ? 1 : 3); }

// Block-size bound of a vector forward row-kernel variant: 1024 threads
// (128 VGPRs per thread) when a thread holds at most 8 elements of a row,
// else 512 (256 VGPRs).  The forward fills the device with blocks, so it
// keeps registers low.
constexpr int rows_max_threads(int maxg, int vec) { return maxg * vec <= 8 ? 1024 : 512; }
// The backward row kernels run one 256-thread team per block at no more
// than kRowsMaxBlocksPerCu blocks per CU, i.e. 2 waves per SIMD: each wave
// may use up to 256 VGPRs for its pipelined rows, weights and column sums.
constexpr int kRowsBwdWavesPerSimd = 2;
// Row-kernel blocks per CU, at most: more blocks shorten the row kernel a
// little but every block adds a partial row that the column finalize reads
// back (measured on MI355X: 2 per CU is the best total for 1600..8192 wide
// rows).
constexpr int kRowsMaxBlocksPerCu = 2;
// Per kind: RMSNorm's wide rows (8192) keep enough rows in flight with one
// block per CU, and halving the partial rows saves more than the second
// block gains (27.9 -> 26.1 us bf16, 44.4 -> 41.0 us fp32 at 2048 x 8192);
// LayerNorm and the bias+dropout+add backward at 1600 columns need two.
constexpr int rows_blocks_per_cu(int kind) { return kind == 1 ? 1 : kRowsMaxBlocksPerCu; }
constexpr int kRowsMaxBlocks = 2048;
// Row elements a thread holds in the vector row kernels: 32 for LayerNorm and
// RMSNorm; 16 for the bias + dropout + add + LayerNorm backward, whose row
// also carries the incoming gradient and the mask (32 would spill).
constexpr int kRowsMaxRowElems = 32;
constexpr int kBdaMaxRowElems = 16;

// ---- LayerNorm / RMSNorm forward ---------------------------------------------------
struct FwdCall {
    int kind;            // 0 LayerNorm, 1 RMSNorm
    int x_t, y_t, w_t;
    int rows, cols;
    int blocks;
    int maxg;            // 16-byte groups per thread per row (vector path); 0 = generic path
    int vec;
    const void *x, *w, *b;
    float eps;
    void *y;
    float *stat0, *stat1;  // LayerNorm: mean, rstd; RMSNorm: rms
    int depth;             // row-pipeline depth of the vector path (0 = the kernel's default)
    int *occupancy_out;    // non-NULL: report blocks per CU instead of launching
};

hipError_t rows_forward_launch(const FwdCall &a, hipStream_t s);

// ---- calibration --------------------------------------------------------------
hipError_t calib_copy_launch(const void *src, void *dst, size_t bytes, int slots, hipStream_t s);
hipError_t calib_add_launch(const float *a, const float *b, float *o, int64_t n, int slots, hipStream_t s);

} // namespace nh
