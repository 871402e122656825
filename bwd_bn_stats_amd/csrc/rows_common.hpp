// Helpers shared by the row kernels (LayerNorm / RMSNorm forward and
// backward): the 256-thread team that owns one row at a time, its weights
// and its fixed-order row sums.
#pragma once

#include <type_traits>

#include "nh_rows.hpp"

namespace nh {

constexpr int kTeamWaves = kTeam / kWave;
constexpr int kRedFloats = 2 * kTeamWaves * 2;  // double-buffered row sums, 256-thread team

__device__ __forceinline__ float load_param(const void *w, int w_bf16, int col)
{
    return w_bf16 ? to_f32(static_cast<const uint16_t *>(w)[col]) : static_cast<const float *>(w)[col];
}

// The weight group of a thread, widened to fp32 once per kernel (NULL: 1.0).
template <int VEC>
struct WeightGroup {
    float v[VEC];
    __device__ __forceinline__ void load(const void *w, int w_bf16, int col)
    {
        if (w == nullptr) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[e] = 1.f;
        } else if (w_bf16) {
            load_vec<uint16_t, VEC>(static_cast<const uint16_t *>(w) + col, v);
        } else {
            load_vec<float, VEC>(static_cast<const float *>(w) + col, v);
        }
    }
    __device__ __forceinline__ float get(int e) const { return v[e]; }
};

// LayerNorm-type row kernels keep xhat and g = dy*w from the row sums for
// rows of at most this many elements per thread.
constexpr int kLnKeepMaxElems = 16;

// LDS floats of a team's double-buffered row sums (two quantities per wave;
// red3_floats: three).
constexpr int red_floats(int team) { return 2 * (team / kWave) * 2; }
constexpr int red3_floats(int team) { return 2 * (team / kWave) * 3; }

// The DPP wave sums (dpp_pair_add, wave_total) live in nh_device.hpp.

// Fixed-order sum of the WAVES wave results of a team for two quantities.
// Called by every thread of the block.
template <int WAVES = kTeamWaves>
__device__ __forceinline__ void team_sum2(float *red, int wave, int lane, float &a, float &b)
{
    a = wave_total(a);
    b = wave_total(b);
    if (lane == 0) {
        red[wave * 2 + 0] = a;
        red[wave * 2 + 1] = b;
    }
    lds_barrier();
    float sa = red[0];
    float sb = red[1];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) {
        sa += red[w * 2 + 0];
        sb += red[w * 2 + 1];
    }
    a = sa;
    b = sb;
}

// The same for three quantities.
template <int WAVES = kTeamWaves>
__device__ __forceinline__ void team_sum3(float *red, int wave, int lane, float &a, float &b, float &c)
{
    a = wave_total(a);
    b = wave_total(b);
    c = wave_total(c);
    if (lane == 0) {
        red[wave * 3 + 0] = a;
        red[wave * 3 + 1] = b;
        red[wave * 3 + 2] = c;
    }
    lds_barrier();
    float sa = red[0];
    float sb = red[1];
    float sc = red[2];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) {
        sa += red[w * 3 + 0];
        sb += red[w * 3 + 1];
        sc += red[w * 3 + 2];
    }
    a = sa;
    b = sb;
    c = sc;
}

// Sum over the ct lanes of a subgroup (ct a power of two, subgroups aligned
// to ct inside the wave).  Each step adds a partner lane, so every lane of
// the subgroup ends with the same bits, in a fixed order: xor 32 and xor 16
// across rows of 16 lanes (lane permutes through the LDS crossbar), then
// row_mirror, row_half_mirror, xor 2 and xor 1 inside a row as DPP operand
// selections, which cost no LDS round trip.  The steps a subgroup needs are
// uniform branches on ct.
__device__ __forceinline__ float sub_sum(float v, int ct)
{
    if (ct > 32) v += __shfl_xor(v, 32, kWave);
    if (ct > 16) v += __shfl_xor(v, 16, kWave);
    if (ct > 8) v = dpp_pair_add<kDppRowMirror>(v);
    if (ct > 4) v = dpp_pair_add<kDppRowHalfMirror>(v);
    if (ct > 2) v = dpp_pair_add<kDppQuadXor2>(v);
    if (ct > 1) v = dpp_pair_add<kDppQuadXor1>(v);
    return v;
}

// Software-pipelined walk over a team's rows with D row buffers in
// registers: while row i is reduced and written, the loads of rows i+1 ..
// i+D-1 are in flight.  Buffers rotate by unrolling, so each stays in fixed
// registers.  load_row(buf, it) must be branch-free and accept any it (rows
// past the end load nothing); do_row(buf, it) handles row iteration it.
template <int D, typename RowBuf, typename Load, typename Do>
__device__ __forceinline__ void pipeline_rows(int iters, Load &&load_row, Do &&do_row)
{
    RowBuf buf[D];
#pragma unroll
    for (int d = 0; d < D - 1; ++d) load_row(buf[d], d);
    for (int it = 0; it < iters; it += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (it + d >= iters) return;
            load_row(buf[(d + D - 1) % D], it + d + D - 1);
            do_row(buf[d], it + d);
        }
    }
}

// Default pipeline depth of a backward row kernel (2 waves per SIMD) from
// the bytes of one row buffer per thread.  Measured on MI355X: LayerNorm at
// 1600 columns (48 B) is best at 3, RMSNorm at 8192 columns (128 B bf16,
// 256 B fp32) and the bias+dropout+add backward (88 B) at 2; deeper
// pipelines gain nothing and cost registers.
constexpr int rows_depth(int row_bytes_per_thread)
{
    return row_bytes_per_thread <= 32 ? 4 : (row_bytes_per_thread <= 64 ? 3 : (row_bytes_per_thread <= 256 ? 2 : 1));
}
// The 512-thread wide-row teams hold 32 elements per thread (16 for the
// bias+dropout+add backward) at 2 waves per SIMD: depth 2 fits in 256 VGPRs
// up to 192 bytes of row buffer per thread, beyond that depth 1.
constexpr int rows_depth_wide(int row_bytes_per_thread) { return row_bytes_per_thread <= 192 ? 2 : 1; }
// The forward kernels run up to 8 blocks per CU, so many rows are in flight
// per CU already: depth 2 measured best (LayerNorm 1600, RMSNorm 8192).
constexpr int kFwdDepth = 2;

// Two row teams per block: adds team 1's column sums into team 0's through
// LDS, one quantity at a time, in a fixed order.  Returns true for the
// threads that then hold the block's sums (team 0; every thread with one
// team).  Every thread of the block must call it.
template <int Q, int MAXG, int VEC, int TEAM, int TEAMS>
__device__ __forceinline__ bool combine_teams(float (&p)[Q][MAXG][VEC], int team, int tt)
{
    static_assert(TEAMS == 1 || TEAMS == 2, "one or two row teams per block");
    if constexpr (TEAMS == 1) {
        return true;
    } else {
        __shared__ float comb[MAXG * VEC * TEAM];
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            if (q > 0) __syncthreads();  // team 0 has read the previous quantity
            if (team == 1)
#pragma unroll
                for (int k = 0; k < MAXG; ++k)
#pragma unroll
                    for (int e = 0; e < VEC; ++e) comb[(k * VEC + e) * TEAM + tt] = p[q][k][e];
            __syncthreads();
            if (team == 0)
#pragma unroll
                for (int k = 0; k < MAXG; ++k)
#pragma unroll
                    for (int e = 0; e < VEC; ++e) p[q][k][e] += comb[(k * VEC + e) * TEAM + tt];
        }
        return team == 0;
    }
}

// Writes a block's column sums (Q quantities) as its row of partials[Q, G, H].
template <int VEC, int MAXG, int Q, int TEAM>
__device__ __forceinline__ void write_partials(const float (&p)[Q][MAXG][VEC], int tt, int Gr, int H,
                                               int G, float *__restrict__ partials)
{
#pragma unroll
    for (int k = 0; k < MAXG; ++k) {
        const int grp = tt + k * TEAM;
        if (grp < Gr)
#pragma unroll
            for (int q = 0; q < Q; ++q)
                store_vec<float, VEC>(partials + ((size_t)q * G + blockIdx.x) * H + grp * VEC, p[q][k]);
    }
}

} // namespace nh
