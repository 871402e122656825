// Backward of bias + dropout + add + LayerNorm over the last dimension of
// [rows, H]: NVIDIA/Fuser issue #1473, the one-kernel fusion of its first
// example.  The forward is h = residual + dropout(a + bias), y =
// LayerNorm(h); with xhat = (h - mean)*rstd and g = dy*w,
//   dx_ln     = rstd*(g - sum g/H - xhat*sum(g*xhat)/H)    (LayerNorm backward)
//   dh        = dresidual + dx_ln                         (fp32 out)
//   da        = dh * scale * mask                         (dy's dtype out)
//   dweight_j = sum_rows dy*xhat,  dbias_j = sum_rows dy,  dbias_in_j = sum_rows da.
//
// The LayerNorm backward row kernel extended by the fused epilogue: the
// incoming gradient and the keep-mask of a row are read with its x and dy
// (one row ahead, through range-checked buffer loads; a NULL input is an
// empty buffer that reads as zeros), the epilogue writes dh and da, and a
// third column accumulator carries dbias_in through the same split-over-rows
// partials and fixed-order column finalize.  Every element of every input
// is read once and every output written once.
#include "rows_common.hpp"

namespace nh {

// A group of V keep-mask bytes (V = 4 or 8), packed four to a register.
template <int V>
struct MaskGroup {
    static_assert(V == 4 || V == 8, "mask groups hold 4 or 8 bytes");
    uint32_t u[V / 4];
    __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r, int off)
    {
        if constexpr (V == 8) {
            u32x2_t t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kBufferNT);
            u[0] = t.x;
            u[1] = t.y;
        } else {
            u[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kBufferNT);
        }
    }
    __device__ __forceinline__ float get(int e) const
    {
        return ((u[e >> 2] >> (8 * (e & 3))) & 0xffu) != 0u ? 1.f : 0.f;
    }
};

template <typename TX, typename TDY, int VEC, int MAXG, int TEAM, int D>
__global__ void __launch_bounds__(TEAM, kRowsBwdWavesPerSimd)
bda_rows_kernel(const TDY *__restrict__ dy, const TX *__restrict__ x,
                const float *__restrict__ mean, const float *__restrict__ rstd,
                const void *__restrict__ w, int w_bf16, const float *__restrict__ dres,
                const uint8_t *__restrict__ mask, float scale, int rows, int H,
                float *__restrict__ dh, TDY *__restrict__ da, float *__restrict__ partials,
                int want_cols)
{
    __shared__ float red[red_floats(TEAM)];
    const int tt = threadIdx.x;
    const int wave = tt / kWave;
    const int lane = tt & (kWave - 1);
    const int G = gridDim.x;
    const int Gr = H / VEC;
    const float invH = 1.0f / (float)H;
    const bool has_mask = mask != nullptr;

    WeightGroup<VEC> wv[MAXG];
    float p[3][MAXG][VEC];
#pragma unroll
    for (int k = 0; k < MAXG; ++k) {
        const int grp = tt + k * TEAM;
        if (grp < Gr) wv[k].load(w, w_bf16, grp * VEC);
#pragma unroll
        for (int e = 0; e < VEC; ++e) { p[0][k][e] = 0.f; p[1][k][e] = 0.f; p[2][k][e] = 0.f; }
    }

    const int iters = (int)ceil_div(rows, (int64_t)G);
    auto row_of = [&](int it) { return it * G + (int)blockIdx.x; };

    struct RowBuf {
        Raw<TX, VEC> x[MAXG];
        Raw<TDY, VEC> d[MAXG];
        Raw<float, VEC> r[MAXG];
        MaskGroup<VEC> m[MAXG];
        float mu, rs;
    };
    auto load_row = [&](RowBuf &b, int it) {
        const int r = __builtin_amdgcn_readfirstlane(row_of(it));
        const bool live = r < rows;
        const int rc = live ? r : rows - 1;
        const size_t rowoff = (size_t)rc * H;
        const auto rx = make_rsrc(x + rowoff, live ? (uint32_t)(H * sizeof(TX)) : 0u);
        const auto rd = make_rsrc(dy + rowoff, live ? (uint32_t)(H * sizeof(TDY)) : 0u);
        const auto rr = make_rsrc(dres ? dres + rowoff : nullptr,
                                  live && dres ? (uint32_t)(H * sizeof(float)) : 0u);
        const auto rm = make_rsrc(mask ? mask + rowoff : nullptr, live && mask ? (uint32_t)H : 0u);
#pragma unroll
        for (int k = 0; k < MAXG; ++k) {
            const int grp = tt + k * TEAM;
            b.x[k].load_buf(rx, grp * VEC * (int)sizeof(TX));
            b.d[k].load_buf(rd, grp * VEC * (int)sizeof(TDY));
            b.r[k].load_buf(rr, grp * VEC * (int)sizeof(float));
            b.m[k].load_buf(rm, grp * VEC);
        }
        b.mu = mean[rc];
        b.rs = rstd[rc];
    };

    // As in the LayerNorm kernel: rows of at most kLnKeepMaxElems elements per
    // thread keep xhat and g = dy*w from the row sums, so dh rounds exactly as
    // layernorm_backward's dx does.
    constexpr bool KEEP = MAXG * VEC <= kLnKeepMaxElems;
    auto do_row = [&](const RowBuf &b, int it) {
        const int r = row_of(it);
        const bool active = r < rows;
        const float mu = b.mu, rs = b.rs;
        float sa = 0.f, sb = 0.f;
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
                    sa += g;
                    sb = fmaf(g, xh, sb);
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
        team_sum2<TEAM / kWave>(red + (it & 1) * (red_floats(TEAM) / 2), wave, lane, sa, sb);
        if (!active) return;
        const float ca = sa * invH, cb = sb * invH;
        const size_t rowoff = (size_t)r * H;
#pragma unroll
        for (int k = 0; k < MAXG; ++k) {
            const int grp = tt + k * TEAM;
            if (grp < Gr) {
                float hv[VEC], av[VEC];
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
                    hv[e] = rs * fmaf(-xh, cb, g - ca) + b.r[k].get(e);
                    av[e] = hv[e] * scale * (has_mask ? b.m[k].get(e) : 1.f);
                    p[2][k][e] += av[e];
                }
                if (dh != nullptr) st<true, float, VEC>(dh + rowoff + grp * VEC, hv);
                if (da != nullptr) st<true, TDY, VEC>(da + rowoff + grp * VEC, av);
            }
        }
    };

    pipeline_rows<D, RowBuf>(iters, load_row, do_row);
    if (want_cols) write_partials<VEC, MAXG, 3, TEAM>(p, tt, Gr, H, G, partials);
}

// ---- host dispatch ---------------------------------------------------------------
template <typename TX, typename TDY, int VEC, int MAXG, int TEAM, int D>
static hipError_t bda_vec_d(const RowsCall &a, hipStream_t s)
{
    auto kern = bda_rows_kernel<TX, TDY, VEC, MAXG, TEAM, D>;
    if (a.occupancy_out)
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(a.occupancy_out, kern, TEAM, 0);
    return launch(NH_K_BDA_ROWS, kern, dim3(a.blocks), dim3(TEAM), 0u, s, static_cast<const TDY *>(a.dy),
                  static_cast<const TX *>(a.x), a.mean, a.rstd, a.w, a.w_t, a.dresidual, a.mask,
                  a.scale, a.rows, a.cols, a.dh, static_cast<TDY *>(a.dx), a.partials,
                  (int)(a.dweight != nullptr || a.dbias != nullptr || a.dbias_in != nullptr));
}

template <typename TX, typename TDY, int VEC, int MAXG, int TEAM = kTeam>
static hipError_t bda_vec(const RowsCall &a, hipStream_t s)
{
    // Row buffer: x, dy, the fp32 incoming gradient and the mask byte.
    constexpr int BYTES = MAXG * VEC * (int)(sizeof(TX) + sizeof(TDY) + 5);
    if constexpr (TEAM != kTeam) {
        return bda_vec_d<TX, TDY, VEC, MAXG, TEAM, rows_depth_wide(BYTES)>(a, s);
    } else {
        switch (a.depth > 0 ? a.depth : rows_depth(BYTES)) {
        case 1: return bda_vec_d<TX, TDY, VEC, MAXG, TEAM, 1>(a, s);
        case 2: return bda_vec_d<TX, TDY, VEC, MAXG, TEAM, 2>(a, s);
        case 3: return bda_vec_d<TX, TDY, VEC, MAXG, TEAM, 3>(a, s);
        default: return bda_vec_d<TX, TDY, VEC, MAXG, TEAM, 4>(a, s);
        }
    }
}

template <typename TX, typename TDY>
static hipError_t bda_types(const RowsCall &a, hipStream_t s)
{
    // At most kBdaMaxRowElems row elements per thread: a 256-thread team, or
    // a 512-thread team for rows up to twice as wide; the planner sends wider
    // rows to the generic path.
    if (a.team == kWideTeam) {
        if (a.vec == 4) return bda_vec<TX, TDY, 4, kBdaMaxRowElems / 4, kWideTeam>(a, s);
        return bda_vec<TX, TDY, 8, kBdaMaxRowElems / 8, kWideTeam>(a, s);
    }
    if (a.vec == 4) {
        switch (a.maxg) {
        case 1: return bda_vec<TX, TDY, 4, 1>(a, s);
        case 2: return bda_vec<TX, TDY, 4, 2>(a, s);
        case 4: return bda_vec<TX, TDY, 4, 4>(a, s);
        default: return hipErrorInvalidValue;
        }
    }
    switch (a.maxg) {
    case 1: return bda_vec<TX, TDY, 8, 1>(a, s);
    case 2: return bda_vec<TX, TDY, 8, 2>(a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t bda_backward_launch(const RowsCall &a, hipStream_t s)
{
    hipError_t e = hipSuccess;
    if (a.rows > 0 && a.maxg == 0) {
        e = rows_generic_launch(a, s);
    } else if (a.rows > 0) {
        switch (a.x_t * 2 + a.dy_t) {
        case 0: e = bda_types<float, float>(a, s); break;
        case 1: e = bda_types<float, uint16_t>(a, s); break;
        case 2: e = bda_types<uint16_t, float>(a, s); break;
        default: e = bda_types<uint16_t, uint16_t>(a, s); break;
        }
    }
    if (e != hipSuccess || a.occupancy_out) return e;
    if (a.dweight == nullptr && a.dbias == nullptr && a.dbias_in == nullptr) return hipSuccess;
    return rows_colsum_launch(a, NH_K_BDA_COLSUM, s);
}

} // namespace nh
