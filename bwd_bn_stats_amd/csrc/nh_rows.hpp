// Host interface of the LayerNorm / RMSNorm row kernels (rows_kernels.hip,
// rows_bda_kernels.hip, rows_fwd_kernels.hip): call records and planning
// constants.
#pragma once

#include "nh_internal.hpp"

namespace nh {

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
    int team;            // threads per row team / block of the vector path (256 or 512)
    int depth;           // row-pipeline depth of the vector path (0 = the kernel's default)
    int colsum_cols;     // columns per column-finalize block (0 = default)
    int teams;           // RMSNorm vector path: row teams per block (1 or 2; 0 = by row size)
    int *occupancy_out;  // non-NULL: report resident 256-thread blocks per CU
                         // of the selected row kernel instead of launching
    // Generic path (maxg == 0; vec is then 1 or the vector width):
    int gen_ct;          // lanes per row of rows_narrow_kernel; 0 = coefficient + strip kernels
    int gen_rpc;         // rows_strip_kernel: rows per chunk (blocks = number of chunks)
    int gen_coef_waves;  // rows_coef_kernel: waves per row segment (1 or kGenCoefTeamWaves)
    int gen_coef_segs;   // rows_coef_kernel: column segments per row (1 with one wave per row)
    float *coef;         // [rows, gen_coef_segs, 2] row-segment sums (strip path)
};

hipError_t rows_backward_launch(const RowsCall &a, hipStream_t s);
hipError_t bda_backward_launch(const RowsCall &a, hipStream_t s);
// Row kernels of the generic path (any kind), without the column finalize.
hipError_t rows_generic_launch(const RowsCall &a, hipStream_t s);
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
// Per kind, row size (row_bytes: bytes of x and dy a thread holds per row)
// and row groups.  Rows of at least 128 B per thread (8192 columns) keep
// enough rows in flight with one block per CU, and halving the partial rows
// saves more than the second block gains -- RMSNorm at 2048 x 8192: 27.9 ->
// 26.1 us bf16, 44.4 -> 41.0 us fp32; LayerNorm: 33.8 -> 29.7 us bf16, 51.2
// -> 49.1 us fp32.  RMSNorm keeps one block per CU (of two row teams) for
// rows of 256 groups too (16384 x 1024 fp32: 38.5 vs 41.8 us), but rows of
// at most 128 groups leave half of each team idle and want two blocks
// (32768 x 512 fp32: 53.2 -> 41.0 us, 16384 x 1024 bf16: 34.7 -> 28.8 us).
// LayerNorm at 33..64 B runs one block of two row teams per CU: as many
// rows in flight as two one-team blocks, half the partial rows (8192 x 1600
// x fp32 / dy bf16: 29.4 -> 28.5 us; 4096 x 4096 bf16: 30.2 -> 27.1 us;
// 4096 x 2048 fp32: 25.5 -> 23.7 us).  LayerNorm at <= 32 B (two teams per
// block, two blocks) and at 96 B, and the bias+dropout+add backward, use two.
constexpr int rows_blocks_per_cu(int kind, int row_bytes, int64_t groups)
{
    if (kind == 1) return groups <= 128 ? kRowsMaxBlocksPerCu : 1;
    if (kind == 0 && (row_bytes >= 128 || (row_bytes > 32 && row_bytes <= 64))) return 1;
    return kRowsMaxBlocksPerCu;
}
constexpr int kRowsMaxBlocks = 2048;
// Row elements a thread holds in the vector row kernels: 32 for LayerNorm and
// RMSNorm; 16 for the bias + dropout + add + LayerNorm backward, whose row
// also carries the incoming gradient and the mask (32 would spill).
constexpr int kRowsMaxRowElems = 32;
constexpr int kBdaMaxRowElems = 16;
// Threads of a row team (one block): 256, or kWideTeam for rows too wide for
// 256 threads at the element limit above (up to twice as wide).
constexpr int kTeam = 256;
constexpr int kWideTeam = 512;

// Generic path (widths the vector kernels do not take, misaligned tensors).
// Rows of at most kGenNarrowGroups groups take rows_narrow_kernel (a
// subgroup of lanes per row); wider rows take rows_coef_kernel and
// rows_strip_kernel, whose blocks cover kGenStripGroups column groups (one
// wave) by 4 row lanes.  The strip grid aims at kGenTargetBlocks blocks (8
// per CU) with chunks of at least kGenMinChunkRows rows, so that a chunk's
// partial row costs little next to the rows it sums.  Row sums are reduced
// by one wave per row, or by a 256-thread team for rows of at least
// kGenTeamCoefGroups groups; with fewer than kGenCoefTargetBlocks such rows,
// each row is cut into up to kGenCoefMaxSegs segments of at least
// kGenCoefMinSegGroups groups, one team each, so that enough teams run.
constexpr int kGenNarrowGroups = 64;
constexpr int kGenNarrowMaxCols = 8 * kGenNarrowGroups;  // widest narrow row: 64 groups of 8
constexpr int kGenNarrowRowsInFlight = 8;  // rows a narrow row slot loads at once
constexpr int kGenStripGroups = 64;
constexpr int64_t kGenTargetBlocks = 2048;
constexpr int64_t kGenMinChunkRows = 32;
constexpr int kGenTeamCoefGroups = 1024;
constexpr int kGenCoefTeamWaves = kTeam / 64;
constexpr int64_t kGenCoefTargetBlocks = 1024;
constexpr int kGenCoefMaxSegs = 8;
constexpr int kGenCoefMinSegGroups = 512;
// Row-segment sum slots per row that the workspace holds for `rows` rows.
constexpr int64_t gen_coef_slots(int64_t rows)
{
    return rows >= kGenCoefTargetBlocks ? 1
         : ((kGenCoefTargetBlocks + rows - 1) / rows < kGenCoefMaxSegs ? (kGenCoefTargetBlocks + rows - 1) / rows
                                                                      : kGenCoefMaxSegs);
}

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
    int team;              // threads per row team / block: vector path 256 or 512, generic path 256 or 1024
    int depth;             // row-pipeline depth of the vector path (0 = the kernel's default)
    int *occupancy_out;    // non-NULL: report blocks per CU instead of launching
    int gen_ct;            // generic path: lanes per row of the narrow kernel (0 = a team per row)
};

// Forward generic path: rows of at most kGenNarrowGroups columns take a
// lane subgroup per row; wider rows a team per row that reads the row twice
// (the second time from the caches), kGenFwdBigTeam threads wide when there
// are too few rows to fill the device with 256-thread teams and each thread
// still gets at least kGenFwdMinGroupsPerThread groups.
constexpr int kGenFwdBigTeam = 1024;
constexpr int kGenFwdMinGroupsPerThread = 2;

hipError_t rows_forward_launch(const FwdCall &a, hipStream_t s);

} // namespace nh
