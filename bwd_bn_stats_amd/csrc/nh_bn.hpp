// Host/device interface of the BatchNorm kernels (bn_kernels.hip): launch
// geometry, the unit-to-address map shared with the host self test, and the
// call record api.cpp fills.
#pragma once

#include "nh_internal.hpp"

namespace nh {

// ---- BatchNorm -------------------------------------------------------------
constexpr int kBnThreads = 256;
constexpr int kBnUnroll = 4;     // vector units in flight per thread

constexpr int64_t kBnMinUnits = (int64_t)kBnThreads * kBnUnroll;  // one full unrolled sweep

// Waves per SIMD the split passes are compiled for: 8 blocks of 256 threads
// per CU, the resident slots the grid plan fills (at most 64 VGPRs each).
// Measured on MI355X: the fused dx pass at 68 VGPRs ran 7 blocks per CU and
// left an eighth of the grid for a second round ((64,256,56,56) bf16 dx
// 42.3 -> 43.2 us).
constexpr int kBnWavesPerSimd = 8;

// Blocks per channel for a channel of `units` vector units: enough blocks
// that all C*grid_y blocks fill the device's resident slots once, but no
// block gets less than kBnGridMinUnits units (two per thread).  Measured on
// MI355X against a minimum of one full unrolled sweep (1024 units) per
// block, fwd+bwd step: (32,64,32,32) bf16 19.7 -> 17.2 us, (64,256,28,28)
// bf16 42.4 -> 39.7 us, but (16,32,32,32) fp32 15.0 -> 15.8 us and
// (128,64,16,16) fp32 18.6 -> 19.3 us; the configs' grids (bound by the
// slots) do not change.
//
// The reductions and the elementwise passes use the same split: an
// elementwise block then reads exactly the units that the reduction block of
// the same index read.  Measured on MI355X with contiguous ranges and the
// partial slots stored block-index-major, splitting them differently (for
// example 64 reduction blocks per channel, 32 elementwise) made apply and dx
// 25-40% slower, although no L2 line survives from one kernel to the next;
// with the current layout, elementwise blocks of one whole sweep each
// measured from 3.5% faster ((256,32,32,32) bf16) to 5% slower
// ((64,256,14,14) fp32) per fwd+bwd step.
//
// Interleaved unit assignment (bn_range) where the channel holds at least
// one whole sweep per block of that grid: then up to twice the resident
// slots per channel, as many as give every block a whole sweep.  Measured on
// MI355X, cold per call, fwd+bwd step, contiguous at the one-round grid ->
// interleaved at the same grid -> interleaved at the larger grid:
//   (64,256,56,56) bf16    124.6 -> 123.3 -> 121.8 us (16 blocks per channel)
//   (64,64,112,112) bf16   125.5 -> 123.1 -> 120.8 us (64)
//   (128,256,28,28) fp32   137.0 -> 135.4 -> 132.7 us (16)
//   (32,128,56,56) fp32     61.0 ->  60.1 ->  59.6 us (24)
//   (64,512,28,28) bf16     71.3 ->  71.2 ->  70.7 us (6)
// and inference + ReLU at (64,64,112,112) bf16 38.5 -> 35.5 -> 34.5 us.
// More blocks per channel lose again: (64,256,56,56) bf16 at 32 blocks per
// channel 122.6 us.  The one-round grid is what the Aether-ML PR's
// "Reduction grid" rule gives; the second round only pays with the
// interleaved order, and only while a channel has at most
// kBnTwoRoundMaxGrid blocks: every elementwise block first sums its
// channel's partial slots, and with two rounds that prologue's latency is
// paid twice.  Fewer channels keep the one-round grid, interleaved.
// Measured, contiguous / interleaved one round / interleaved two rounds:
//   (256,4,128,128) fp32    78.7 / 78.5 / 84.9 us (512 -> 1024 blocks per channel)
//   (64,3,224,224) fp32     52.3 / 47.8 / 48.7 us (682 -> 784)
//   (32,16,224,224) fp32   123.0 / 121.8 / 121.1 us (128 -> 256)
//   (128,32,112,112) bf16  124.8 / 122.5 / 121.2 us (64 -> 128)
constexpr int64_t kBnGridMinUnits = (int64_t)kBnThreads * 2;
constexpr int64_t kBnTwoRoundMaxGrid = 256;
inline int64_t bn_auto_grid_y(int64_t units, int64_t C, int64_t slots, bool interleave)
{
    int64_t per_channel = slots / (C > 0 ? C : 1);
    if (per_channel < 1) per_channel = 1;
    int64_t want = ceil_div(units, kBnGridMinUnits);
    if (want < 1) want = 1;
    const int64_t one_round = want < per_channel ? want : per_channel;
    if (interleave && units >= one_round * kBnMinUnits) {
        const int64_t whole = units / kBnMinUnits;
        const int64_t cap = 2 * per_channel <= kBnTwoRoundMaxGrid ? 2 * per_channel : one_round;
        return whole < cap ? whole : cap;
    }
    return one_round;
}

// Channels of at most kBnChannelMaxUnits units (twice that with enough
// channels to fill the device) take the one-block-per-channel fused kernels:
// a block covers the channel in a few unrolled sweeps per pass, so the
// launches it saves outweigh the lost split, and each fp32 per-thread sum
// takes at most four units (the split path's fp64 combine of block sums keeps
// large channels accurate; one block over a channel of a few hundred
// thousand elements would not).
constexpr int64_t kBnChannelMaxUnits = 2 * kBnMinUnits;
constexpr int kBnChannelBigBlock = 1024;  // threads of the larger fused-kernel block

// Geometry of a BatchNorm launch: channel c's M elements in units of V
// consecutive elements inside one plane, block (c, yb) owning either the
// units [yb*upb, min((yb+1)*upb, units)) or every grid_y-th sweep of the
// channel (bn_range).
struct BnGeom {
    int C;
    int HW;
    int HWv;        // units per plane
    FastDiv div_hwv;
    int units;      // units per channel (N * HWv)
    int upb;        // units per block
    int grid_y;
    int chan_fast;  // block numbering: 0 channel-major, 1 channel-fastest (bn_block)
    int ilv;        // unit assignment: 0 contiguous ranges, 1 interleaved sweeps (bn_range)
};

// Block id -> (channel c, block yb of that channel).  Channel-major: the
// grid_y blocks of a channel have consecutive ids.  Channel-fastest:
// consecutive ids take consecutive channels at the same yb, so the blocks
// dispatched first cover the first planes of every channel, one contiguous
// stretch of the tensor, and the launch walks memory in address order.
// Every pass of one call uses the same numbering, so an elementwise block
// still re-reads the units that the reduction block of its id read.
//
// One division and two value selects: assigning c and yb in the two arms of
// a branch let the compiler merge the arms into stores through a selected
// address, which put both in scratch memory and made every address that
// depends on them a per-lane value.
struct BnBlock {
    int c, yb;
};
__device__ __forceinline__ BnBlock bn_block(const BnGeom &g)
{
    const int b = (int)blockIdx.x;
    const int d = g.chan_fast ? g.C : g.grid_y;
    const int q = b / d;
    const int r = b - q * d;
    return {g.chan_fast ? r : q, g.chan_fast ? q : r};
}

// The units of block yb: sweeps of kBnMinUnits units (one unrolled pass of
// the block's threads) starting at u0, u0 + step, ..., each cut at u1.
// Contiguous: one range of upb units, step one sweep.  Interleaved: sweep s
// of the channel goes to block s mod grid_y, so at any moment the blocks of
// a channel read neighbouring sweeps and, with the channels side by side in
// memory, the whole grid reads one compact stretch of the tensor.  Every
// pass of one call uses the same assignment, so an elementwise block still
// re-reads the units that the reduction block of its id read.  Value selects,
// as in bn_block.
struct BnRange {
    uint32_t u0, u1, step;
};
__device__ __forceinline__ BnRange bn_range(const BnGeom &g, int yb)
{
    constexpr uint32_t S = (uint32_t)kBnMinUnits;
    const uint32_t c0 = (uint32_t)yb * (uint32_t)g.upb;
    const uint32_t c1 = min(c0 + (uint32_t)g.upb, (uint32_t)g.units);
    return {g.ilv ? (uint32_t)yb * S : c0, g.ilv ? (uint32_t)g.units : c1, g.ilv ? (uint32_t)g.grid_y * S : S};
}

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

inline BnGeom make_bn_geom(int N, int C, int HW, int vec, int grid_y, int chan_fast, int ilv)
{
    BnGeom g;
    g.chan_fast = chan_fast;
    g.ilv = ilv;
    g.C = C;
    g.HW = HW;
    g.HWv = HW / vec;
    g.div_hwv = make_fastdiv((uint32_t)g.HWv);
    g.units = N * g.HWv;
    g.grid_y = grid_y;
    g.upb = (int)ceil_div(g.units, grid_y);
    return g;
}

// Small planes: the tensor viewed as [N, L] rows, L = C*HW, column j in
// channel j/HW.  A block is 2^cl_log2 column lanes (the power of two covering
// the row's groups of `vec` elements, at most kBnColLanes) by rl =
// kBnThreads / 2^cl_log2 row lanes over one chunk of rpc rows, so every lane
// has columns even when the row holds fewer than kBnColLanes groups.  A launch
// is a 1-D grid of strips x rb blocks (bn_col_work maps a block to its strip
// and chunk).  The reduction passes write partials[2, rb, L].
constexpr int kBnColLanes = 64;              // column lanes per block, at most: one wave
constexpr int64_t kBnColMaxChunks = 256;     // row chunks, at most
constexpr int64_t kBnColMinChunkRows = 16;   // rows per chunk, at least (and at least the row lanes)
constexpr int64_t kBnColTargetBlocks = 2048; // blocks aimed at: the resident 256-thread slots
constexpr int kBnColMaxVec = 8;              // widest unit (bf16, 16 bytes)
constexpr int kXcds = 8;                     // XCDs of the device; blocks are dealt to them by id
struct BnColGeom {
    int N, C, HW, L;
    int strips, rb, rpc;
    int cl_log2, rl;  // column lanes per block = 1 << cl_log2; row lanes = kBnThreads >> cl_log2
    FastDiv div_hw;   // column -> channel
};

// Row chunks the workspace holds for N rows of L columns, for every unit
// width: at most one per kBnColMinChunkRows rows, at most kBnColMaxChunks,
// and at most kBnColTargetBlocks over the fewest strips any unit width gives
// (kBnColLanes groups of kBnColMaxVec elements to a strip).
inline int64_t bn_col_chunks_max(int64_t N, int64_t L)
{
    int64_t c = ceil_div(N, kBnColMinChunkRows);
    int64_t s = ceil_div(L, (int64_t)kBnColMaxVec * kBnColLanes);
    if (s < 1) s = 1;
    const int64_t t = ceil_div(kBnColTargetBlocks, s);
    if (c > t) c = t;
    if (c > kBnColMaxChunks) c = kBnColMaxChunks;
    return c < 1 ? 1 : c;
}

inline BnColGeom make_bn_col_geom(int N, int C, int HW, int vec)
{
    BnColGeom g;
    g.N = N;
    g.C = C;
    g.HW = HW;
    g.L = C * HW;
    g.div_hw = make_fastdiv((uint32_t)HW);
    const int64_t groups = g.L / vec;
    int lg = 0;
    while ((1 << lg) < groups && (1 << lg) < kBnColLanes) ++lg;
    g.cl_log2 = lg;
    g.rl = kBnThreads >> lg;
    g.strips = (int)ceil_div(groups, (int64_t)1 << lg);
    int64_t rb = ceil_div(kBnColTargetBlocks, g.strips);
    const int64_t by_rows = ceil_div(N, g.rl > kBnColMinChunkRows ? (int64_t)g.rl : kBnColMinChunkRows);
    if (rb > by_rows) rb = by_rows;
    if (rb > bn_col_chunks_max(N, g.L)) rb = bn_col_chunks_max(N, g.L);
    if (rb < 1) rb = 1;
    g.rpc = (int)ceil_div(N, rb);
    g.rb = (int)ceil_div(N, g.rpc);
    return g;
}

// Block id -> (strip, chunk) of the row layout's 1-D grid.  Work items are
// numbered strip-fastest.  With at least kBnColXcdMinChunks chunks, the
// blocks that land on one XCD (ids k, k + 8, ...) take consecutive work items,
// so each XCD streams one contiguous part of the tensor (measured on MI355X:
// (16384, 2048) bf16 fwd+bwd 123 -> 106 us); with fewer, block id = work
// item, which is faster there ((64, 2048, 7, 7) bf16).  Every row-layout pass
// uses this mapping, so an elementwise block re-reads the rows that the
// reduction block of its id read, on the same XCD.  A bijection on
// [0, strips * rb).
constexpr int kBnColXcdMinChunks = 64;
struct BnColWork {
    int strip, chunk;
};
__host__ __device__ inline BnColWork bn_col_work(const BnColGeom &g, int id)
{
    if (g.rb < kBnColXcdMinChunks) return {id % g.strips, id / g.strips};
    const int total = g.strips * g.rb;
    const int k = id % kXcds, s = id / kXcds;
    const int q = total / kXcds, rem = total % kXcds;
    const int w = k * q + (k < rem ? k : rem) + s;
    return {w % g.strips, w / g.strips};
}

struct BnCall {
    int io;              // 0 fp32, 1 bf16
    int N, C, HW;
    int vec;             // unit width in elements: fp32 4 or 1; bf16 8, 4 or 1
    int grid_y;          // blocks per channel of the reduction passes (stats, grad_sums)
    int ew_grid_y;       // blocks per channel of the elementwise passes (apply, dx)
    int chan_fast;       // block numbering of the split passes (BnGeom::chan_fast)
    int ilv;             // unit assignment of the split passes (BnGeom::ilv)
    int separate_finalize;  // 1: finalize as its own kernel; 0: in the elementwise prologue
    int inference;       // forward only: apply with the running statistics, no reduction
    int channel_fused;   // 1: one block per channel, reduction + finalize + elementwise in one kernel
    int channel_threads; // threads of that block: kBnThreads or kBnChannelBigBlock
    int col;             // 1: small planes, the [N, C*HW] row layout (colg; vec along the rows)
    BnColGeom colg;
    int stage;           // 0 the whole operation; 1 its reduction pass only (partials into the
                         // workspace); 2 the rest (finalize + elementwise pass, from those partials)
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

} // namespace nh
