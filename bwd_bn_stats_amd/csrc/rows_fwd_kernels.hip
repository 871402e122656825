// LayerNorm and RMSNorm training forward over the last dimension of [rows, H],
// writing the statistics their backward passes consume.
//
//   LayerNorm: the statistics NVIDIA/Fuser issue #1473's layer_norm backward
//     takes as inputs (mean and rstd per row).  The variance comes from the
//     one-pass shifted sums of Aether-ML PR #18 ("One-pass statistics")
//     applied per row: with K = the row's first element, d = x - K and
//     md = sum d / H,
//       var = sum d^2 / H - md^2 (clamped at 0),  rstd = 1/sqrt(var + eps),
//       y = ((x - K) - md)*rstd*w + b:
//     x - (K + md) would round the mean before a subtraction that rstd (up
//     to 1/sqrt(eps)) amplifies on nearly constant rows.  The stored mean is
//     K + md or sum x / H, whichever sums the smaller terms: an fp32 sum errs
//     in proportion to the magnitude of its terms, |x - K| for the one and
//     |x| for the other, and |md| < |sum x / H| says the first are smaller
//     (rows far from zero relative to their spread; rows around zero take
//     the plain sum, which K + md would lose to cancellation).
//   RMSNorm: NVIDIA/Fuser issue #3629's rmsnorm_prims,
//       rms = sqrt(sum x^2 / H + eps),  y = w*(x/rms)
//     (rms is what that issue's rmsnorm_bwd_fusion takes as its saved input).
//
// Same structure as the backward row kernels: a 256-thread team per row, the
// row in registers (read once, one row ahead, through range-checked buffer
// loads), one fixed-order team sum per row, nontemporal y stores.
#include "rows_common.hpp"

namespace nh {

// A parameter group widened to fp32 once; NULL reads as `dflt`.
template <int VEC>
struct ParamGroup {
    float v[VEC];
    __device__ __forceinline__ void load(const void *p, int bf16, int col, float dflt)
    {
        if (p == nullptr) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[e] = dflt;
        } else if (bf16) {
            load_vec<uint16_t, VEC>(static_cast<const uint16_t *>(p) + col, v);
        } else {
            load_vec<float, VEC>(static_cast<const float *>(p) + col, v);
        }
    }
};

// A row's statistics from its sums (LayerNorm: plain sum s0, shifted sum s1
// and sum of squares s2 of d = x - K; RMSNorm: sum of squares s2 of x), and
// the two numbers its output takes: a = rstd (LayerNorm) or 1/rms (RMSNorm),
// md = s1 / H (LayerNorm) or 0.  Writes the statistics if `writer`.
template <int KIND>
__device__ __forceinline__ void fwd_row_stats(float s0, float s1, float s2, float K, float invH, float eps,
                                              int64_t r, bool writer, float *stat0, float *stat1, float &a,
                                              float &md)
{
    if constexpr (KIND == 0) {
        md = s1 * invH;
        const float var = fmaxf(s2 * invH - md * md, 0.f);
        a = 1.0f / sqrtf(var + eps);
        if (writer) {
            const float mp = s0 * invH;
            stat0[r] = fabsf(md) < fabsf(mp) ? K + md : mp;
            if (stat1 != nullptr) stat1[r] = a;
        }
    } else {
        const float rms = sqrtf(fmaf(s2, invH, eps));
        a = 1.0f / rms;
        md = 0.f;
        if (writer && stat0 != nullptr) stat0[r] = rms;
    }
}

// One output element: ((x - K) - md)*rstd*w + b (LayerNorm), w*(x/rms) (RMSNorm).
template <int KIND>
__device__ __forceinline__ float fwd_out(float v, float K, float md, float a, float w, float b)
{
    if constexpr (KIND == 0) return fmaf(((v - K) - md) * a, w, b);
    else return w * (v * a);
}

// LDS floats of a team's double-buffered row sums: three for LayerNorm, two
// for RMSNorm (only the second is used).
template <int KIND>
constexpr int fwd_red_floats(int team) { return KIND == 0 ? red3_floats(team) : red_floats(team); }

// KIND 0: LayerNorm (stat0 = mean, stat1 = rstd); KIND 1: RMSNorm (stat0 = rms).
template <int KIND, typename TX, typename TY, int VEC, int MAXG, int MT, int D, int TEAM>
__global__ void __launch_bounds__(MT)
norm_fwd_rows_kernel(const TX *__restrict__ x, const void *__restrict__ w,
                     const void *__restrict__ b, int w_bf16, int rows, int H, float eps,
                     TY *__restrict__ y, float *__restrict__ stat0, float *__restrict__ stat1)
{
    constexpr int kRed = fwd_red_floats<KIND>(TEAM);
    __shared__ float red[kRed];
    const int tt = threadIdx.x;
    const int wave = tt / kWave;
    const int lane = tt & (kWave - 1);
    const int G = gridDim.x;
    const int Gr = H / VEC;
    const float invH = 1.0f / (float)H;

    ParamGroup<VEC> wv[MAXG];
    ParamGroup<VEC> bv[KIND == 0 ? MAXG : 1];
#pragma unroll
    for (int k = 0; k < MAXG; ++k) {
        const int grp = tt + k * TEAM;
        if (grp < Gr) {
            wv[k].load(w, w_bf16, grp * VEC, 1.f);
            if constexpr (KIND == 0) bv[k].load(b, w_bf16, grp * VEC, 0.f);
        }
    }

    const int iters = (int)ceil_div(rows, (int64_t)G);
    struct RowBuf {
        Raw<TX, VEC> x[MAXG];
        float K;
    };
    auto load_row = [&](RowBuf &rb, int it) {
        const int r = __builtin_amdgcn_readfirstlane(it * G + (int)blockIdx.x);
        const bool live = r < rows;
        const int rc = live ? r : rows - 1;
        const size_t rowoff = (size_t)rc * H;
        const auto rx = make_rsrc(x + rowoff, live ? (uint32_t)(H * sizeof(TX)) : 0u);
#pragma unroll
        for (int k = 0; k < MAXG; ++k) rb.x[k].load_buf(rx, (tt + k * TEAM) * VEC * (int)sizeof(TX));
        rb.K = KIND == 0 ? to_f32(x[rowoff]) : 0.f;
    };
    auto do_row = [&](const RowBuf &rb, int it) {
        const int r = it * G + (int)blockIdx.x;
        const bool active = r < rows;
        float s0 = 0.f, s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int k = 0; k < MAXG; ++k) {
            const int grp = tt + k * TEAM;
            if (active && grp < Gr) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float v = rb.x[k].get(e);
                    if constexpr (KIND == 0) {
                        const float d = v - rb.K;
                        s0 += v;
                        s1 += d;
                        s2 = fmaf(d, d, s2);
                    } else {
                        s2 = fmaf(v, v, s2);
                    }
                }
            }
        }
        if constexpr (KIND == 0)
            team_sum3<TEAM / kWave>(red + (it & 1) * (kRed / 2), wave, lane, s0, s1, s2);
        else
            team_sum2<TEAM / kWave>(red + (it & 1) * (kRed / 2), wave, lane, s1, s2);
        if (!active) return;
        float a, md;
        fwd_row_stats<KIND>(s0, s1, s2, rb.K, invH, eps, r, tt == 0, stat0, stat1, a, md);
        const size_t rowoff = (size_t)r * H;
#pragma unroll
        for (int k = 0; k < MAXG; ++k) {
            const int grp = tt + k * TEAM;
            if (grp < Gr) {
                float o[VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    float bias = 0.f;
                    if constexpr (KIND == 0) bias = bv[k].v[e];
                    o[e] = fwd_out<KIND>(rb.x[k].get(e), rb.K, md, a, wv[k].v[e], bias);
                }
                st<true, TY, VEC>(y + rowoff + grp * VEC, o);
            }
        }
    };

    pipeline_rows<D, RowBuf>(iters, load_row, do_row);
}

// ---- generic path ------------------------------------------------------------------
// Rows of at most 64 groups of VEC elements (VEC = 1 for any alignment, or
// the vector width for aligned rows): a subgroup of ct lanes (the power of
// two covering the groups) per row, U rows of a slot loaded at once, the row
// sums reduced by lane exchanges inside the subgroup.
template <int KIND, typename TX, typename TY, int VEC>
__global__ void __launch_bounds__(kTeam)
norm_fwd_narrow_kernel(const TX *__restrict__ x, const void *__restrict__ w,
                       const void *__restrict__ b, int w_bf16, int rows, int H, float eps,
                       TY *__restrict__ y, float *__restrict__ stat0, float *__restrict__ stat1, int ct)
{
    constexpr int U = VEC == 1 ? kGenNarrowRowsInFlight : 4;
    const int tt = threadIdx.x;
    const int lane = tt & (ct - 1);
    const int slot = tt >> __builtin_ctz((unsigned)ct);
    const int slots = kTeam / ct;
    const bool col_ok = lane < H / VEC;
    const int col = (col_ok ? lane : 0) * VEC;  // dead lanes read group 0 and drop it
    const float invH = 1.0f / (float)H;
    ParamGroup<VEC> wv, bv;
    wv.load(w, w_bf16, col, 1.f);
    bv.load(KIND == 0 ? b : nullptr, w_bf16, col, 0.f);
    const int64_t stride = (int64_t)gridDim.x * slots;
    for (int64_t r0 = (int64_t)blockIdx.x * slots + slot; r0 < rows; r0 += U * stride) {
        float v[U][VEC], K[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t rk = r0 + k * stride;
            const size_t rowoff = (size_t)(rk < rows ? rk : rows - 1) * H;
            ld<true, TX, VEC>(x + rowoff + col, v[k]);
            K[k] = KIND == 0 ? to_f32(x[rowoff]) : 0.f;
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            float s0 = 0.f, s1 = 0.f, s2 = 0.f;
            if (col_ok) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float d = v[k][e] - K[k];
                    if constexpr (KIND == 0) {
                        s0 += v[k][e];
                        s1 += d;
                    }
                    s2 = fmaf(d, d, s2);
                }
            }
            if constexpr (KIND == 0) {
                s0 = sub_sum(s0, ct);
                s1 = sub_sum(s1, ct);
            }
            s2 = sub_sum(s2, ct);
            const int64_t rk = r0 + k * stride;
            if (rk < rows) {
                float a, md;
                fwd_row_stats<KIND>(s0, s1, s2, K[k], invH, eps, rk, lane == 0, stat0, stat1, a, md);
                if (col_ok) {
                    float o[VEC];
#pragma unroll
                    for (int e = 0; e < VEC; ++e) o[e] = fwd_out<KIND>(v[k][e], K[k], md, a, wv.v[e], bv.v[e]);
                    st<true, TY, VEC>(y + (size_t)rk * H + col, o);
                }
            }
        }
    }
}

// Wider rows, any alignment (VEC = 1) or too wide for the register-resident
// kernel (VEC = the vector width): a TEAM-thread block per row, two reads of
// the row -- the first (cacheable) for the sums, U groups of a thread in
// flight, the second from the caches for the output.  The plan counts on two
// 1024-thread blocks per CU (8 waves per SIMD); the one variant the compiler
// otherwise gives more than 64 VGPRs (bf16 rows in 8-byte groups, fp32
// output) is held to that explicitly -- bounding the others makes them spill.
template <int KIND, typename TX, typename TY, int VEC, int TEAM>
constexpr int fwd_team_min_waves()
{
    return TEAM == kGenFwdBigTeam && sizeof(TX) == 2 && sizeof(TY) == 4 && VEC == 4 ? 8 : 1;
}

template <int KIND, typename TX, typename TY, int VEC, int TEAM>
__global__ void __launch_bounds__(TEAM, (fwd_team_min_waves<KIND, TX, TY, VEC, TEAM>()))
norm_fwd_team_kernel(const TX *__restrict__ x, const void *__restrict__ w,
                     const void *__restrict__ b, int w_bf16, int rows, int H, float eps,
                     TY *__restrict__ y, float *__restrict__ stat0, float *__restrict__ stat1)
{
    constexpr int WAVES = TEAM / kWave;
    constexpr int U = VEC == 8 ? 4 : 8;
    constexpr int kRed = fwd_red_floats<KIND>(TEAM);
    __shared__ float red[kRed];
    const int tt = threadIdx.x;
    const int wave = tt / kWave;
    const int lane = tt & (kWave - 1);
    const int groups = H / VEC;
    const float invH = 1.0f / (float)H;
    int it = 0;
    // 64-bit row index: r + gridDim.x must not wrap.
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x, ++it) {
        const TX *xr = x + (size_t)r * H;
        const float K = KIND == 0 ? to_f32(xr[0]) : 0.f;
        float s0 = 0.f, s1 = 0.f, s2 = 0.f;
        auto add = [&](const float (&v)[VEC]) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float d = v[e] - K;
                if constexpr (KIND == 0) {
                    s0 += v[e];
                    s1 += d;
                }
                s2 = fmaf(d, d, s2);
            }
        };
        int gi = tt;
        for (; gi + (U - 1) * TEAM < groups; gi += U * TEAM) {
            float v[U][VEC];
#pragma unroll
            for (int k = 0; k < U; ++k) ld<false, TX, VEC>(xr + (size_t)(gi + k * TEAM) * VEC, v[k]);
#pragma unroll
            for (int k = 0; k < U; ++k) add(v[k]);
        }
        for (; gi < groups; gi += TEAM) {
            float v[VEC];
            ld<false, TX, VEC>(xr + (size_t)gi * VEC, v);
            add(v);
        }
        if constexpr (KIND == 0)
            team_sum3<WAVES>(red + (it & 1) * (kRed / 2), wave, lane, s0, s1, s2);
        else
            team_sum2<WAVES>(red + (it & 1) * (kRed / 2), wave, lane, s1, s2);
        float a, md;
        fwd_row_stats<KIND>(s0, s1, s2, K, invH, eps, r, tt == 0, stat0, stat1, a, md);
        TY *yr = y + (size_t)r * H;
        auto out = [&](int grp, const float (&v)[VEC]) {
            ParamGroup<VEC> wv, bv;
            wv.load(w, w_bf16, grp * VEC, 1.f);
            if constexpr (KIND == 0) bv.load(b, w_bf16, grp * VEC, 0.f);
            float o[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) o[e] = fwd_out<KIND>(v[e], K, md, a, wv.v[e], KIND == 0 ? bv.v[e] : 0.f);
            st<true, TY, VEC>(yr + (size_t)grp * VEC, o);
        };
        gi = tt;
        for (; gi + (U - 1) * TEAM < groups; gi += U * TEAM) {
            float v[U][VEC];
#pragma unroll
            for (int k = 0; k < U; ++k) ld<true, TX, VEC>(xr + (size_t)(gi + k * TEAM) * VEC, v[k]);
#pragma unroll
            for (int k = 0; k < U; ++k) out(gi + k * TEAM, v[k]);
        }
        for (; gi < groups; gi += TEAM) {
            float v[VEC];
            ld<true, TX, VEC>(xr + (size_t)gi * VEC, v);
            out(gi, v);
        }
    }
}

// ---- host dispatch ------------------------------------------------------------------
template <int KIND, typename TX, typename TY, int VEC, int MAXG, int D, int TEAM>
static hipError_t fwd_vec_d(const FwdCall &a, hipStream_t s)
{
    constexpr int MT = rows_max_threads(MAXG, VEC) > TEAM ? rows_max_threads(MAXG, VEC) : TEAM;
    auto kern = norm_fwd_rows_kernel<KIND, TX, TY, VEC, MAXG, MT, D, TEAM>;
    if (a.occupancy_out)
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(a.occupancy_out, kern, TEAM, 0);
    return launch(KIND == 0 ? NH_K_LN_FWD : NH_K_RMS_FWD, kern, dim3(a.blocks), dim3(TEAM), 0u, s,
                  static_cast<const TX *>(a.x), a.w, a.b, a.w_t, a.rows, a.cols, a.eps,
                  static_cast<TY *>(a.y), a.stat0, a.stat1);
}

template <int KIND, typename TX, typename TY, int VEC, int MAXG, int TEAM = kTeam>
static hipError_t fwd_vec(const FwdCall &a, hipStream_t s)
{
    if constexpr (TEAM != kTeam) {
        return fwd_vec_d<KIND, TX, TY, VEC, MAXG, kFwdDepth, TEAM>(a, s);
    } else {
        switch (a.depth > 0 ? a.depth : kFwdDepth) {
        case 1: return fwd_vec_d<KIND, TX, TY, VEC, MAXG, 1, TEAM>(a, s);
        case 2: return fwd_vec_d<KIND, TX, TY, VEC, MAXG, 2, TEAM>(a, s);
        case 3: return fwd_vec_d<KIND, TX, TY, VEC, MAXG, 3, TEAM>(a, s);
        default: return fwd_vec_d<KIND, TX, TY, VEC, MAXG, 4, TEAM>(a, s);
        }
    }
}

template <int KIND, typename TX, typename TY, int VEC>
static hipError_t fwd_team(const FwdCall &a, hipStream_t s)
{
    const int kid = KIND == 0 ? NH_K_LN_FWD : NH_K_RMS_FWD;
    if (a.team == kGenFwdBigTeam)
        return launch(kid, norm_fwd_team_kernel<KIND, TX, TY, VEC, kGenFwdBigTeam>, dim3(a.blocks),
                      dim3(kGenFwdBigTeam), 0u, s, static_cast<const TX *>(a.x), a.w, a.b, a.w_t, a.rows,
                      a.cols, a.eps, static_cast<TY *>(a.y), a.stat0, a.stat1);
    return launch(kid, norm_fwd_team_kernel<KIND, TX, TY, VEC, kTeam>, dim3(a.blocks), dim3(kTeam), 0u, s,
                  static_cast<const TX *>(a.x), a.w, a.b, a.w_t, a.rows, a.cols, a.eps,
                  static_cast<TY *>(a.y), a.stat0, a.stat1);
}

// Generic path: the plan (gen_ct, team, vec, blocks) comes from the host.
template <int KIND, typename TX, typename TY>
static hipError_t fwd_generic(const FwdCall &a, hipStream_t s)
{
    if (a.occupancy_out) { *a.occupancy_out = 1; return hipSuccess; }  // not used by the generic plan
    // The vector width of a type mix: 8 when x and y are both bf16, else 4.
    constexpr int V = sizeof(TX) == 2 && sizeof(TY) == 2 ? 8 : 4;
    if (a.vec != 1 && a.vec != V) return hipErrorInvalidValue;
    const int kid = KIND == 0 ? NH_K_LN_FWD : NH_K_RMS_FWD;
    if (a.gen_ct > 0) {
        if (a.vec == 1)
            return launch(kid, norm_fwd_narrow_kernel<KIND, TX, TY, 1>, dim3(a.blocks), dim3(kTeam), 0u, s,
                          static_cast<const TX *>(a.x), a.w, a.b, a.w_t, a.rows, a.cols, a.eps,
                          static_cast<TY *>(a.y), a.stat0, a.stat1, a.gen_ct);
        return launch(kid, norm_fwd_narrow_kernel<KIND, TX, TY, V>, dim3(a.blocks), dim3(kTeam), 0u, s,
                      static_cast<const TX *>(a.x), a.w, a.b, a.w_t, a.rows, a.cols, a.eps,
                      static_cast<TY *>(a.y), a.stat0, a.stat1, a.gen_ct);
    }
    if (a.vec == 1) return fwd_team<KIND, TX, TY, 1>(a, s);
    return fwd_team<KIND, TX, TY, V>(a, s);
}

template <int KIND, typename TX, typename TY, int VEC>
static hipError_t fwd_maxg(const FwdCall &a, hipStream_t s)
{
    if (a.team == kWideTeam) return fwd_vec<KIND, TX, TY, VEC, kRowsMaxRowElems / VEC, kWideTeam>(a, s);
    switch (a.maxg) {
    case 1: return fwd_vec<KIND, TX, TY, VEC, 1>(a, s);
    case 2: return fwd_vec<KIND, TX, TY, VEC, 2>(a, s);
    case 4: return fwd_vec<KIND, TX, TY, VEC, 4>(a, s);
    default:
        if constexpr (VEC == 4) return fwd_vec<KIND, TX, TY, VEC, 8>(a, s);
        return hipErrorInvalidValue;
    }
}

template <int KIND, typename TX, typename TY>
static hipError_t fwd_types(const FwdCall &a, hipStream_t s)
{
    if (a.maxg == 0) return fwd_generic<KIND, TX, TY>(a, s);
    return a.vec == 4 ? fwd_maxg<KIND, TX, TY, 4>(a, s) : fwd_maxg<KIND, TX, TY, 8>(a, s);
}

hipError_t rows_forward_launch(const FwdCall &a, hipStream_t s)
{
    if (a.kind == 1) return a.x_t == 0 ? fwd_types<1, float, float>(a, s) : fwd_types<1, uint16_t, uint16_t>(a, s);
    switch (a.x_t * 2 + a.y_t) {
    case 0: return fwd_types<0, float, float>(a, s);
    case 1: return fwd_types<0, float, uint16_t>(a, s);
    case 2: return fwd_types<0, uint16_t, float>(a, s);
    default: return fwd_types<0, uint16_t, uint16_t>(a, s);
    }
}

} // namespace nh
