// LayerNorm and RMSNorm backward over the last dimension of [rows, H].
//
// Definitions: NVIDIA/Fuser issue #1473 ("Why is LayerNorm Backward
// Segmenting?", the layer_norm backward definition) and NVIDIA/Fuser issue
// #3629 ("Performance gap between manual nvfuser definition and thunder.jit
// for rmsnorm", rmsnorm_bwd_fusion):
//   LayerNorm: xhat = (x - mean)*rstd, g = dy*w,
//              dx = rstd*(g - sum g/H - xhat*sum(g*xhat)/H),
//              dweight_j = sum_rows dy*xhat, dbias_j = sum_rows dy
//   RMSNorm:   rinv = 1/rms, g = dy*w,
//              dx = rinv*g - x*rinv^3*sum(g*x)/H, dweight_j = sum_rows dy*x*rinv
//
// Design (one pass over x and dy; the row stays in registers):
//   * A team of 256 threads (4 waves) owns one row at a time.  Thread t of a
//     team owns the 16-byte column groups t, t+256, ... (at most MAXG of
//     them), the same columns for every row it visits, so it keeps the
//     weight and its share of the column sums (the dweight/dbias split over
//     rows) in registers across rows.
//   * A block is one team; block b takes rows it*G + b for it = 0, 1, ...,
//     keeping D of them in flight (software pipeline).  Row sums are wave
//     butterflies followed by a fixed-order add of the 4 wave results
//     through LDS, one block barrier per row.
//   * After its last row, the block writes its column sums as one row of
//     partials[Q, G, H].
//   * rows_colsum_kernel sums the G partial rows of each column in fp64, in
//     index order, and rounds to the weight's dtype.
// No atomics: every output has one writer and a fixed summation order.
//
// Rows whose width is not a multiple of the group, misaligned pointers, or
// rows wider than the vector path's register budget take the generic kernels
// (rows_generic_kernels.hip).
#include "rows_common.hpp"

namespace nh {

// ---- LayerNorm, vector path ----------------------------------------------------
// D: software-pipeline depth.  While a team reduces and writes row i, the
// loads of its rows i+1 .. i+D-1 are already in flight (D register sets,
// used in rotation), so each team keeps D rows of HBM traffic outstanding
// across the block barrier of the row sum.
//
// TEAMS row teams per block (1 or 2).  With 2, the teams take interleaved
// rows and keep their own column sums, which meet in LDS at the end: twice
// the rows in flight per block for the same number of partial rows.  Both
// teams pass every row-sum barrier (a block barrier) the same number of
// times, since they share the iteration count.
template <typename TX, typename TDY, typename TDX, int VEC, int MAXG, int TEAM, int D, int TEAMS = 1>
__global__ void __launch_bounds__(TEAM * TEAMS, kRowsBwdWavesPerSimd)
ln_rows_kernel(const TDY *__restrict__ dy, const TX *__restrict__ x,
               const float *__restrict__ mean, const float *__restrict__ rstd,
               const void *__restrict__ w, int w_bf16, int rows, int H,
               TDX *__restrict__ dx, float *__restrict__ partials, int want_cols)
{
    __shared__ float red_all[TEAMS * red_floats(TEAM)];
    const int team = TEAMS > 1 ? (int)threadIdx.x / TEAM : 0;
    const int tt = (int)threadIdx.x - team * TEAM;
    float *red = red_all + team * red_floats(TEAM);
    const int wave = tt / kWave;
    const int lane = tt & (kWave - 1);
    const int G = gridDim.x;
    const int Gr = H / VEC;
    const float invH = 1.0f / (float)H;

    WeightGroup<VEC> wv[MAXG];
    float p[2][MAXG][VEC];
#pragma unroll
    for (int k = 0; k < MAXG; ++k) {
        const int grp = tt + k * TEAM;
        if (grp < Gr) wv[k].load(w, w_bf16, grp * VEC);
#pragma unroll
        for (int e = 0; e < VEC; ++e) { p[0][k][e] = 0.f; p[1][k][e] = 0.f; }
    }

    const int iters = (int)ceil_div(rows, (int64_t)G * TEAMS);
    auto row_of = [&](int it) { return (it * G + (int)blockIdx.x) * TEAMS + team; };

    // One row in flight: its x/dy groups and its saved statistics.  The row
    // is read through buffer resources sized to the row (empty past the last
    // row), so the loads need no branches: out-of-range groups and rows read
    // as zeros without memory traffic, and the compiler can wait for exactly
    // the older row's loads while the next row's are in flight.
    struct RowBuf {
        Raw<TX, VEC> x[MAXG];
        Raw<TDY, VEC> d[MAXG];
        float mu, rs;
    };
    auto load_row = [&](RowBuf &b, int it) {
        const int r = __builtin_amdgcn_readfirstlane(row_of(it));
        const bool live = r < rows;
        const int rc = live ? r : rows - 1;
        const size_t rowoff = (size_t)rc * H;
        const auto rx = make_rsrc(x + rowoff, live ? (uint32_t)(H * sizeof(TX)) : 0u);
        const auto rd = make_rsrc(dy + rowoff, live ? (uint32_t)(H * sizeof(TDY)) : 0u);
#pragma unroll
        for (int k = 0; k < MAXG; ++k) {
            const int grp = tt + k * TEAM;
            b.x[k].load_buf(rx, grp * VEC * (int)sizeof(TX));
            b.d[k].load_buf(rd, grp * VEC * (int)sizeof(TDY));
        }
        b.mu = mean[rc];
        b.rs = rstd[rc];
    };

    // Rows of at most kLnKeepMaxElems elements per thread keep xhat and
    // g = dy*w from the row sums for dx instead of recomputing them (same
    // values, so the same results bit for bit).
    constexpr bool KEEP = MAXG * VEC <= kLnKeepMaxElems;
    auto do_row = [&](const RowBuf &b, int it) {
        const int r = row_of(it);
        const bool active = r < rows;
        const float mu = b.mu, rs = b.rs;
        float a = 0.f, bb = 0.f;
        float kx[KEEP ? MAXG : 1][VEC], kg[KEEP ? MAXG : 1][VEC];
#pragma unroll
        for (int k = 0; k < MAXG; ++k) {
            const int grp = tt + k * TEAM;
            if (active && grp < Gr) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float d = b.d[k].get(e);
                    const float xh = (b.x[k].get(e) - mu) * rs;
                    const float g = d * wv[k].get(e);
                    if constexpr (KEEP) {
                        kx[k][e] = xh;
                        kg[k][e] = g;
                    }
                    a += g;
                    bb = fmaf(g, xh, bb);
                    p[0][k][e] = fmaf(d, xh, p[0][k][e]);
                    p[1][k][e] += d;
                }
            } else if constexpr (KEEP) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    kx[k][e] = 0.f;
                    kg[k][e] = 0.f;
                }
            }
        }
        team_sum2<TEAM / kWave>(red + (it & 1) * (red_floats(TEAM) / 2), wave, lane, a, bb);
        if (active && dx != nullptr) {
            const float ca = a * invH, cb = bb * invH;
            const size_t rowoff = (size_t)r * H;
#pragma unroll
            for (int k = 0; k < MAXG; ++k) {
                const int grp = tt + k * TEAM;
                if (grp < Gr) {
                    float o[VEC];
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        float xh, g;
                        if constexpr (KEEP) {
                            xh = kx[k][e];
                            g = kg[k][e];
                        } else {
                            xh = (b.x[k].get(e) - mu) * rs;
                            g = b.d[k].get(e) * wv[k].get(e);
                        }
                        o[e] = rs * fmaf(-xh, cb, g - ca);
                    }
                    st<true, TDX, VEC>(dx + rowoff + grp * VEC, o);
                }
            }
        }
    };

    pipeline_rows<D, RowBuf>(iters, load_row, do_row);
    if (want_cols && combine_teams<2, MAXG, VEC, TEAM, TEAMS>(p, team, tt))
        write_partials<VEC, MAXG, 2, TEAM>(p, tt, Gr, H, G, partials);
}

// ---- RMSNorm, vector path ----------------------------------------------------
constexpr int kRmsKeepGMinGroups = 4;      // groups per thread (see do_row)
constexpr int kRmsKeepGMaxRowBytes = 128;  // x and dy bytes per thread and row
// TEAMS row teams per block (1 or 2), as in the LayerNorm kernel.
template <typename T, int VEC, int MAXG, int TEAM, int D, int TEAMS = 1>
__global__ void __launch_bounds__(TEAM * TEAMS, kRowsBwdWavesPerSimd)
rms_rows_kernel(const T *__restrict__ dy, const T *__restrict__ x,
                const float *__restrict__ rms, float eps, const void *__restrict__ w,
                int w_bf16, int rows, int H, T *__restrict__ dx,
                float *__restrict__ partials, int want_cols)
{
    __shared__ float red_all[TEAMS * red_floats(TEAM)];
    const int team = TEAMS > 1 ? (int)threadIdx.x / TEAM : 0;
    const int tt = (int)threadIdx.x - team * TEAM;
    float *red = red_all + team * red_floats(TEAM);
    const int wave = tt / kWave;
    const int lane = tt & (kWave - 1);
    const int G = gridDim.x;
    const int Gr = H / VEC;
    const float invH = 1.0f / (float)H;

    WeightGroup<VEC> wv[MAXG];
    float p[1][MAXG][VEC];
#pragma unroll
    for (int k = 0; k < MAXG; ++k) {
        const int grp = tt + k * TEAM;
        if (grp < Gr) wv[k].load(w, w_bf16, grp * VEC);
#pragma unroll
        for (int e = 0; e < VEC; ++e) p[0][k][e] = 0.f;
    }

    const int iters = (int)ceil_div(rows, (int64_t)G * TEAMS);
    auto row_of = [&](int it) { return (it * G + (int)blockIdx.x) * TEAMS + team; };

    // One row in flight (see the LayerNorm kernel: branch-free buffer loads).
    struct RowBuf {
        Raw<T, VEC> x[MAXG];
        Raw<T, VEC> d[MAXG];
        float rms;
    };
    auto load_row = [&](RowBuf &b, int it) {
        const int r = __builtin_amdgcn_readfirstlane(row_of(it));
        const bool live = r < rows;
        const int rc = live ? r : rows - 1;
        const size_t rowoff = (size_t)rc * H;
        const uint32_t nbytes = live ? (uint32_t)(H * sizeof(T)) : 0u;
        const auto rx = make_rsrc(x + rowoff, nbytes);
        const auto rd = make_rsrc(dy + rowoff, nbytes);
#pragma unroll
        for (int k = 0; k < MAXG; ++k) {
            const int grp = tt + k * TEAM;
            b.x[k].load_buf(rx, grp * VEC * (int)sizeof(T));
            b.d[k].load_buf(rd, grp * VEC * (int)sizeof(T));
        }
        b.rms = rms != nullptr ? rms[rc] : 0.f;
    };

    // Rows of at least kRmsKeepGMinGroups groups per thread, whose x and dy
    // take at most kRmsKeepGMaxRowBytes bytes of registers per thread, keep
    // g = dy*w from the row sums for dx and skip sum x^2 when rms is given (a
    // uniform branch: two copies of the loop).  Other rows recompute g: short
    // rows gain nothing from it, and larger row buffers spill.  Measured on
    // MI355X, same results bit for bit: 2048x8192 bf16 26.2 -> 25.3 us and
    // 4096x4096 fp32 37.0 -> 36.4 us, but 8192x1600 bf16 20.4 -> 21.2 us and
    // 2048x8192 fp32 40.0 -> 58.5 us.
    constexpr bool KEEP_G =
        MAXG >= kRmsKeepGMinGroups && MAXG * VEC * 2 * (int)sizeof(T) <= kRmsKeepGMaxRowBytes;
    auto do_row = [&](const RowBuf &b, int it) {
        const int r = row_of(it);
        const bool active = r < rows;
        float g[KEEP_G ? MAXG : 1][VEC];
        float sgx = 0.f, q = 0.f;  // sum g*x, sum x^2
        if constexpr (KEEP_G) {
            auto row_sums = [&](auto with_q) {
#pragma unroll
                for (int k = 0; k < MAXG; ++k) {
                    const int grp = tt + k * TEAM;
                    const bool live = active && grp < Gr;
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        const float xe = b.x[k].get(e);
                        g[k][e] = live ? b.d[k].get(e) * wv[k].get(e) : 0.f;
                        sgx = fmaf(g[k][e], xe, sgx);
                        if constexpr (decltype(with_q)::value) q = fmaf(xe, xe, q);
                    }
                }
            };
            if (rms != nullptr)
                row_sums(std::false_type{});
            else
                row_sums(std::true_type{});
        } else {
#pragma unroll
            for (int k = 0; k < MAXG; ++k) {
                const int grp = tt + k * TEAM;
                if (active && grp < Gr) {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        const float xe = b.x[k].get(e);
                        sgx = fmaf(b.d[k].get(e) * wv[k].get(e), xe, sgx);
                        q = fmaf(xe, xe, q);
                    }
                }
            }
        }
        team_sum2<TEAM / kWave>(red + (it & 1) * (red_floats(TEAM) / 2), wave, lane, sgx, q);
        if (active) {
            const float rinv = rms != nullptr ? 1.0f / b.rms : 1.0f / sqrtf(fmaf(q, invH, eps));
            const float c = rinv * rinv * rinv * sgx * invH;
            const size_t rowoff = (size_t)r * H;
#pragma unroll
            for (int k = 0; k < MAXG; ++k) {
                const int grp = tt + k * TEAM;
                if (grp < Gr) {
                    float o[VEC];
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        const float xe = b.x[k].get(e);
                        const float d = b.d[k].get(e);
                        float gk;
                        if constexpr (KEEP_G)
                            gk = g[k][e];
                        else
                            gk = d * wv[k].get(e);
                        o[e] = fmaf(-xe, c, rinv * gk);
                        p[0][k][e] = fmaf(d * xe, rinv, p[0][k][e]);
                    }
                    if (dx != nullptr) st<true, T, VEC>(dx + rowoff + grp * VEC, o);
                }
            }
        }
    };

    pipeline_rows<D, RowBuf>(iters, load_row, do_row);
    if (want_cols && combine_teams<1, MAXG, VEC, TEAM, TEAMS>(p, team, tt))
        write_partials<VEC, MAXG, 1, TEAM>(p, tt, Gr, H, G, partials);
}

// ---- column finalize: fp64 fixed-order sum of the G partial rows -------------
// Block = CX columns x (1024/CX) slices; slice ty sums partial rows
// ty, ty + CY, ... in order, then the slices are combined in slice order
// through LDS.  The partials were just written and sit in L2 / the Infinity
// Cache, so the kernel is latency-bound: a thread issues NL loads at once
// (rows past G re-read row G-1 and are added as zero, so the loads need no
// branch), one round trip per NL*CY partial rows.
constexpr int kColThreads = 1024;
template <typename TOUT, int CX, int NL>
__global__ void __launch_bounds__(kColThreads)
rows_colsum_kernel(const float *__restrict__ partials, int G, int H, TOUT *__restrict__ out0,
                   TOUT *__restrict__ out1, TOUT *__restrict__ out2)
{
    constexpr int CY = kColThreads / CX;
    __shared__ double acc[CY][CX];
    const int q = blockIdx.y;
    TOUT *out = q == 0 ? out0 : (q == 1 ? out1 : out2);
    if (out == nullptr) return;  // uniform across the block
    const int tx = threadIdx.x % CX;
    const int ty = threadIdx.x / CX;
    const int j = blockIdx.x * CX + tx;
    double s = 0.0;
    if (j < H) {
        const float *col = partials + (size_t)q * G * H + j;
        for (int b0 = ty; b0 < G; b0 += NL * CY) {
            float v[NL];
#pragma unroll
            for (int i = 0; i < NL; ++i) v[i] = col[(size_t)min(b0 + i * CY, G - 1) * H];
#pragma unroll
            for (int i = 0; i < NL; ++i) s += b0 + i * CY < G ? (double)v[i] : 0.0;
        }
    }
    acc[ty][tx] = s;
    __syncthreads();
    if (ty == 0 && j < H) {
        double t = acc[0][tx];
#pragma unroll 8
        for (int y = 1; y < CY; ++y) t += acc[y][tx];
        out[j] = from_f32<TOUT>((float)t);
    }
}

// ---- host dispatch ---------------------------------------------------------------
// With a.occupancy_out set, report how many blocks of `kernel` (of `team`
// threads) fit on a CU (registers, LDS) instead of launching it.
template <typename K>
static hipError_t occupancy(const RowsCall &a, K kernel, int team = kTeam)
{
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(a.occupancy_out, kernel, team, 0);
}

template <typename TX, typename TDY, typename TDX, int VEC, int MAXG, int TEAM, int D, int TEAMS>
static hipError_t ln_vec_dt(const RowsCall &a, hipStream_t s)
{
    auto kern = ln_rows_kernel<TX, TDY, TDX, VEC, MAXG, TEAM, D, TEAMS>;
    if (a.occupancy_out) return occupancy(a, kern, TEAM * TEAMS);
    return launch(NH_K_LN_ROWS, kern, dim3(a.blocks), dim3(TEAM * TEAMS), 0u, s,
                  static_cast<const TDY *>(a.dy), static_cast<const TX *>(a.x), a.mean, a.rstd,
                  a.w, a.w_t, a.rows, a.cols, static_cast<TDX *>(a.dx), a.partials,
                  (int)(a.dweight != nullptr || a.dbias != nullptr));
}

// Row teams per block: 2 when a thread's row buffer is at most 64 bytes
// (rows of up to 4096 bf16 / 2048 fp32 columns), else 1.  Measured on
// MI355X: at <= 32 B (two such blocks per CU) 8192x1600 bf16 23.3 -> 22.1 us,
// 16384x1024 bf16 33.7 -> 27.5 us; at 48 and 64 B one two-team block per CU
// beats two one-team blocks (8192x1600 x fp32 / dy bf16 29.4 -> 28.5 us,
// 4096x4096 bf16 30.2 -> 27.1 us), while two two-team blocks per CU are
// slower than either (30.2, 31.1 us).
template <typename TX, typename TDY, typename TDX, int VEC, int MAXG, int TEAM, int D>
static hipError_t ln_vec_d(const RowsCall &a, hipStream_t s)
{
    constexpr int BYTES = MAXG * VEC * (int)(sizeof(TX) + sizeof(TDY));
    if constexpr (TEAM == kTeam) {
        const int teams = a.teams > 0 ? a.teams : (BYTES <= 64 ? 2 : 1);
        if (teams == 2) return ln_vec_dt<TX, TDY, TDX, VEC, MAXG, TEAM, D, 2>(a, s);
    }
    return ln_vec_dt<TX, TDY, TDX, VEC, MAXG, TEAM, D, 1>(a, s);
}

// Pipeline depth: the kernel's default, or the rows_depth override (256-thread
// teams; the 512-thread wide-row teams always run their default).
template <typename TX, typename TDY, typename TDX, int VEC, int MAXG, int TEAM = kTeam>
static hipError_t ln_vec(const RowsCall &a, hipStream_t s)
{
    constexpr int BYTES = MAXG * VEC * (int)(sizeof(TX) + sizeof(TDY));
    if constexpr (TEAM != kTeam) {
        return ln_vec_d<TX, TDY, TDX, VEC, MAXG, TEAM, rows_depth_wide(BYTES)>(a, s);
    } else {
        switch (a.depth > 0 ? a.depth : rows_depth(BYTES)) {
        case 1: return ln_vec_d<TX, TDY, TDX, VEC, MAXG, TEAM, 1>(a, s);
        case 2: return ln_vec_d<TX, TDY, TDX, VEC, MAXG, TEAM, 2>(a, s);
        case 3: return ln_vec_d<TX, TDY, TDX, VEC, MAXG, TEAM, 3>(a, s);
        default: return ln_vec_d<TX, TDY, TDX, VEC, MAXG, TEAM, 4>(a, s);
        }
    }
}

template <typename T, int VEC, int MAXG, int TEAM, int D, int TEAMS>
static hipError_t rms_vec_dt(const RowsCall &a, hipStream_t s)
{
    auto kern = rms_rows_kernel<T, VEC, MAXG, TEAM, D, TEAMS>;
    if (a.occupancy_out) return occupancy(a, kern, TEAM * TEAMS);
    return launch(NH_K_RMS_ROWS, kern, dim3(a.blocks), dim3(TEAM * TEAMS), 0u, s,
                  static_cast<const T *>(a.dy), static_cast<const T *>(a.x), a.rms, a.eps, a.w,
                  a.w_t, a.rows, a.cols, static_cast<T *>(a.dx), a.partials,
                  (int)(a.dweight != nullptr));
}

// Row teams per block: 2 when a thread's row buffer is at most 64 bytes
// (rows of up to 4096 bf16 / 2048 fp32 columns), else 1.  Measured on
// MI355X with one block per CU: short rows leave one team per CU latency
// bound (8192x1600 bf16: 31.6 -> 23.0 us with two teams; 4096x4096 bf16:
// 26.3 -> 24.4 us), while at 8192 columns the second team only costs
// registers (2048x8192 fp32: 40.6 -> 44.2 us).
template <typename T, int VEC, int MAXG, int TEAM, int D>
static hipError_t rms_vec_d(const RowsCall &a, hipStream_t s)
{
    constexpr int BYTES = MAXG * VEC * 2 * (int)sizeof(T);
    if constexpr (TEAM == kTeam) {
        const int teams = a.teams > 0 ? a.teams : (BYTES <= 64 ? 2 : 1);
        if (teams == 2) return rms_vec_dt<T, VEC, MAXG, TEAM, D, 2>(a, s);
    }
    return rms_vec_dt<T, VEC, MAXG, TEAM, D, 1>(a, s);
}

template <typename T, int VEC, int MAXG, int TEAM = kTeam>
static hipError_t rms_vec(const RowsCall &a, hipStream_t s)
{
    constexpr int BYTES = MAXG * VEC * 2 * (int)sizeof(T);
    if constexpr (TEAM != kTeam) {
        return rms_vec_d<T, VEC, MAXG, TEAM, rows_depth_wide(BYTES)>(a, s);
    } else {
        switch (a.depth > 0 ? a.depth : rows_depth(BYTES)) {
        case 1: return rms_vec_d<T, VEC, MAXG, TEAM, 1>(a, s);
        case 2: return rms_vec_d<T, VEC, MAXG, TEAM, 2>(a, s);
        case 3: return rms_vec_d<T, VEC, MAXG, TEAM, 3>(a, s);
        default: return rms_vec_d<T, VEC, MAXG, TEAM, 4>(a, s);
        }
    }
}

// A 256-thread team holds at most 32 row elements per thread (MAXG = 8 only
// with 4-element groups); rows up to twice as wide take a 512-thread team at
// 32 elements per thread (a.team == kWideTeam); wider rows take the generic
// path.
template <typename TX, typename TDY, typename TDX, int VEC>
static hipError_t ln_maxg(const RowsCall &a, hipStream_t s)
{
    if (a.team == kWideTeam) return ln_vec<TX, TDY, TDX, VEC, kRowsMaxRowElems / VEC, kWideTeam>(a, s);
    switch (a.maxg) {
    case 1: return ln_vec<TX, TDY, TDX, VEC, 1>(a, s);
    case 2: return ln_vec<TX, TDY, TDX, VEC, 2>(a, s);
    case 4: return ln_vec<TX, TDY, TDX, VEC, 4>(a, s);
    default:
        if constexpr (VEC == 4) return ln_vec<TX, TDY, TDX, VEC, 8>(a, s);
        return hipErrorInvalidValue;
    }
}

template <typename T, int VEC>
static hipError_t rms_maxg(const RowsCall &a, hipStream_t s)
{
    if (a.team == kWideTeam) return rms_vec<T, VEC, kRowsMaxRowElems / VEC, kWideTeam>(a, s);
    switch (a.maxg) {
    case 1: return rms_vec<T, VEC, 1>(a, s);
    case 2: return rms_vec<T, VEC, 2>(a, s);
    case 4: return rms_vec<T, VEC, 4>(a, s);
    default:
        if constexpr (VEC == 4) return rms_vec<T, VEC, 8>(a, s);
        return hipErrorInvalidValue;
    }
}

template <typename TX, typename TDY, typename TDX>
static hipError_t ln_dispatch_vec(const RowsCall &a, hipStream_t s)
{
    return a.vec == 4 ? ln_maxg<TX, TDY, TDX, 4>(a, s) : ln_maxg<TX, TDY, TDX, 8>(a, s);
}

// dtype code 0 = float, 1 = bf16 (uint16_t)
template <template <typename, typename, typename> class F>
static hipError_t by_types(int tx, int tdy, int tdx, const RowsCall &a, hipStream_t s)
{
    const int code = tx * 4 + tdy * 2 + tdx;
    switch (code) {
    case 0: return F<float, float, float>::run(a, s);
    case 1: return F<float, float, uint16_t>::run(a, s);
    case 2: return F<float, uint16_t, float>::run(a, s);
    case 3: return F<float, uint16_t, uint16_t>::run(a, s);
    case 4: return F<uint16_t, float, float>::run(a, s);
    case 5: return F<uint16_t, float, uint16_t>::run(a, s);
    case 6: return F<uint16_t, uint16_t, float>::run(a, s);
    default: return F<uint16_t, uint16_t, uint16_t>::run(a, s);
    }
}

template <typename TX, typename TDY, typename TDX> struct LnVecF {
    static hipError_t run(const RowsCall &a, hipStream_t s) { return ln_dispatch_vec<TX, TDY, TDX>(a, s); }
};

template <typename TOUT, int CX>
static hipError_t colsum_cx(const RowsCall &a, int kid, hipStream_t s)
{
    const int Q = rows_q(a.kind);
    const dim3 grid((unsigned)ceil_div(a.cols, CX), (unsigned)Q);
    constexpr int CY = kColThreads / CX;
    // All of a thread's partial rows in one round when they fit 16 loads.
    auto kern = a.blocks > 8 * CY ? rows_colsum_kernel<TOUT, CX, 16> : rows_colsum_kernel<TOUT, CX, 8>;
    return launch(kid, kern, grid, dim3(kColThreads), 0u, s,
                  (const float *)a.partials, a.blocks, a.cols, static_cast<TOUT *>(a.dweight),
                  static_cast<TOUT *>(a.kind != 1 ? a.dbias : nullptr),
                  static_cast<TOUT *>(a.kind == 2 ? a.dbias_in : nullptr));
}

template <typename TOUT>
static hipError_t colsum(const RowsCall &a, int kid, hipStream_t s)
{
    // Columns per block, measured on MI355X: 64 when there are at most 16
    // partial rows (fewer, fuller blocks: 4.2 vs 6.5 us at 32768 columns),
    // 16 for rows of at most 64 columns (more threads per column: 4.5 vs 14 us
    // over 2048 partial rows), else 32.
    const int cx = a.colsum_cols > 0 ? a.colsum_cols
                 : (a.blocks <= 16 ? 64 : (a.cols <= kGenNarrowGroups ? 16 : 32));
    switch (cx) {
    case 8: return colsum_cx<TOUT, 8>(a, kid, s);
    case 16: return colsum_cx<TOUT, 16>(a, kid, s);
    case 64: return colsum_cx<TOUT, 64>(a, kid, s);
    default: return colsum_cx<TOUT, 32>(a, kid, s);
    }
}

hipError_t rows_colsum_launch(const RowsCall &a, int kid, hipStream_t s)
{
    return a.w_t == 0 ? colsum<float>(a, kid, s) : colsum<uint16_t>(a, kid, s);
}

hipError_t rows_backward_launch(const RowsCall &a, hipStream_t s)
{
    if (a.kind == 2) return bda_backward_launch(a, s);
    // The dx dtype of a skipped dx is irrelevant: use the dy dtype.
    const int dxt = a.dx != nullptr ? a.dx_t : a.dy_t;
    hipError_t e = hipSuccess;
    if (a.rows == 0) {
        // nothing to launch for the rows; the finalize writes zero sums
    } else if (a.maxg == 0) {
        e = rows_generic_launch(a, s);
    } else if (a.kind == 0) {
        e = by_types<LnVecF>(a.x_t, a.dy_t, dxt, a, s);
    } else {
        e = a.x_t == 0 ? rms_maxg<float, 4>(a, s) : rms_maxg<uint16_t, 8>(a, s);
    }
    if (e != hipSuccess || a.occupancy_out) return e;
    const bool cols = a.kind == 0 ? (a.dweight != nullptr || a.dbias != nullptr) : a.dweight != nullptr;
    if (!cols) return hipSuccess;
    const int kid = a.kind == 0 ? NH_K_LN_COLSUM : NH_K_RMS_COLSUM;
    return rows_colsum_launch(a, kid, s);
}

} // namespace nh
