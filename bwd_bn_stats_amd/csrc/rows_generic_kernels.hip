// Backward row kernels for the shapes that the register-resident team
// kernels do not take -- rows wider than a 512-thread team holds, widths that
// are not a multiple of the 16-byte group, tensors at misaligned addresses --
// and for short rows (at most 64 groups), which a 256-thread team per row
// would run with most of its threads idle.  The arithmetic is that of the
// vector kernels -- LayerNorm and RMSNorm backward (NVIDIA/Fuser issues
// #1473 and #3629) and the bias + dropout + add + LayerNorm backward (issue
// #1473, first example):
//   LayerNorm: xhat = (x - mean)*rstd, g = dy*w,
//              dx = rstd*(g - sum g/H - xhat*sum(g*xhat)/H)
//   RMSNorm:   rinv = 1/rms, g = dy*w, dx = rinv*g - x*rinv^3*sum(g*x)/H
//   bias+dropout+add: dh = dresidual + dx_ln, da = dh*scale*mask
// with the column sums dweight, dbias (and dbias_in) split over rows into
// partials[Q, G, H] and reduced by rows_colsum_kernel as for the vector path.
// Only the mapping of rows and columns to threads differs.
//
// Short rows (at most 64 groups of VEC elements: H <= 64 with scalar
// accesses, or up to 64 vector groups when the tensors are aligned):
// rows_narrow_kernel.  A subgroup of ct lanes of a wave (ct = the power of
// two covering the groups) owns one row at a time, so a 256-thread block
// works on 256/ct rows at once.  The row sums are lane exchanges inside the
// subgroup, with no barrier; every lane keeps its columns' sums in registers
// across rows, and the block's row slots add theirs through LDS, in slot
// order, once at the end.
//
// Wider rows: rows_coef_kernel, then rows_strip_kernel.  The first reduces
// each row (one wave, a 256-thread team for long rows, or several teams for
// few long rows) to the two sums its gradient needs, 8 bytes per row
// segment.  The second cuts [rows, H] into strips of 64 column groups by
// chunks of rows.  A 256-thread block takes one strip of one chunk as 64
// column lanes by 4 row lanes, walks the chunk's rows writing the outputs,
// keeps its columns' sums in registers and writes them once as the chunk's
// partial row (the 4 row lanes meet in LDS).  x and dy are read twice; the
// second read comes from the Infinity Cache when the tensors fit it.  No
// partial row is read back while rows are walked, and every output element
// has one writer.
#include "rows_common.hpp"

namespace nh {

static_assert(kGenStripGroups == kWave, "a strip block's column lanes are one wave");
static_assert(kGenCoefTeamWaves == kTeamWaves, "team-per-row coefficients use the whole block");

// Arguments of the generic kernels, passed by value.
struct GenArgs {
    const void *x, *dy, *w;     // w NULL: all ones
    const float *mean, *rstd;   // LayerNorm and bias+dropout+add
    const float *rms;           // RMSNorm (NULL: recompute with eps)
    const float *dres;          // bias+dropout+add: incoming gradient of the residual, or NULL
    const uint8_t *mask;        // bias+dropout+add: keep-mask bytes, or NULL (all kept)
    float *dh;                  // bias+dropout+add: fp32 output, or NULL
    void *dx;                   // dx (LayerNorm, RMSNorm) or da (bias+dropout+add), or NULL
    float *partials;            // [Q, G, H]
    float *coef;                // [rows, nseg, 2] row-segment sums (strip path)
    float eps, scale;
    int rows, cols;
    int w_bf16;
    int want_cols;
    int ct;                     // narrow: lanes per row
    int rpc;                    // strip: rows per chunk
    int nseg;                   // strip: column segments per row in the row-sum pass
};

// One group of VEC consecutive elements of a row, widened to fp32: x, dy and,
// for the bias+dropout+add backward, the incoming gradient and the mask.
template <int VEC>
struct GroupIn {
    float x[VEC], d[VEC], r[VEC], m[VEC];
};

template <int VEC>
__device__ __forceinline__ void load_mask(const uint8_t *p, float (&m)[VEC])
{
    if constexpr (VEC == 1) {
        m[0] = __builtin_nontemporal_load(p) != 0 ? 1.f : 0.f;
    } else if constexpr (VEC == 4) {
        const uint32_t u = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
#pragma unroll
        for (int e = 0; e < 4; ++e) m[e] = ((u >> (8 * e)) & 0xffu) != 0u ? 1.f : 0.f;
    } else {
        const u32x2_t u = nt_load(reinterpret_cast<const u32x2_t *>(p));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            m[e] = ((u.x >> (8 * e)) & 0xffu) != 0u ? 1.f : 0.f;
            m[e + 4] = ((u.y >> (8 * e)) & 0xffu) != 0u ? 1.f : 0.f;
        }
    }
}

// Loads the group at element offset `off`.  EXTRAS: also the incoming
// gradient (zeros when NULL) and the mask (ones when NULL).  NT: streaming
// loads (the data is not read again).
template <bool EXTRAS, bool NT, typename TX, typename TDY, int VEC>
__device__ __forceinline__ void load_group(const GenArgs &a, size_t off, GroupIn<VEC> &g)
{
    ld<NT, TX, VEC>(static_cast<const TX *>(a.x) + off, g.x);
    ld<NT, TDY, VEC>(static_cast<const TDY *>(a.dy) + off, g.d);
    if constexpr (EXTRAS) {
        if (a.dres != nullptr) {
            ld<NT, float, VEC>(a.dres + off, g.r);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) g.r[e] = 0.f;
        }
        if (a.mask != nullptr) {
            load_mask<VEC>(a.mask + off, g.m);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) g.m[e] = 1.f;
        }
    }
}

// A group's share of the two row sums: LayerNorm (KIND 0, 2) sum g and
// sum g*xhat; RMSNorm (KIND 1) sum g*x and sum x^2.
//
// Here and in group_out the products g = dy*w are rounded before they are
// added (no implicit multiply-add contraction), so that the row sum and the
// g - sum g/H of the output see the same g: a row of one column then gets
// dx = 0 exactly, as the definition gives.
template <int KIND, int VEC>
__device__ __forceinline__ void add_row_sums(const GroupIn<VEC> &g, const float (&w)[VEC], float mu,
                                             float rs, float &s0, float &s1)
{
#pragma clang fp contract(off)
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        const float gg = g.d[e] * w[e];
        if constexpr (KIND == 1) {
            s0 = fmaf(gg, g.x[e], s0);
            s1 = fmaf(g.x[e], g.x[e], s1);
        } else {
            s0 += gg;
            s1 = fmaf(gg, (g.x[e] - mu) * rs, s1);
        }
    }
}

// The row's gradient coefficients from its two sums: LayerNorm (sum g/H,
// sum g*xhat/H); RMSNorm (rinv, rinv^3*sum(g*x)/H).
template <int KIND>
__device__ __forceinline__ float2 row_coefs(const GenArgs &a, int64_t r, float s0, float s1)
{
    const float invH = 1.0f / (float)a.cols;
    if constexpr (KIND == 1) {
        const float rinv = a.rms != nullptr ? 1.0f / a.rms[r] : 1.0f / sqrtf(fmaf(s1, invH, a.eps));
        return make_float2(rinv, rinv * rinv * rinv * s0 * invH);
    } else {
        return make_float2(s0 * invH, s1 * invH);
    }
}

// Outputs of one group of row elements at element offset `off`, and its
// contribution to the column sums p.
template <int KIND, typename TDX, int VEC, int Q>
__device__ __forceinline__ void group_out(const GenArgs &a, size_t off, const GroupIn<VEC> &g,
                                          const float (&w)[VEC], float mu, float rs, float2 c,
                                          float (&p)[Q][VEC])
{
#pragma clang fp contract(off)
    float o[VEC];
    if constexpr (KIND == 1) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            o[e] = fmaf(-g.x[e], c.y, c.x * (g.d[e] * w[e]));
            p[0][e] = fmaf(g.d[e] * g.x[e], c.x, p[0][e]);
        }
    } else {
        float hv[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float xh = (g.x[e] - mu) * rs;
            o[e] = rs * fmaf(-xh, c.y, g.d[e] * w[e] - c.x);
            p[0][e] = fmaf(g.d[e], xh, p[0][e]);
            p[1][e] += g.d[e];
            if constexpr (KIND == 2) {
                hv[e] = o[e] + g.r[e];
                o[e] = hv[e] * a.scale * g.m[e];
                p[2][e] += o[e];
            }
        }
        if constexpr (KIND == 2)
            if (a.dh != nullptr) st<true, float, VEC>(a.dh + off, hv);
    }
    if (a.dx != nullptr) st<true, TDX, VEC>(static_cast<TDX *>(a.dx) + off, o);
}

// ---- narrow rows: a subgroup of lanes per row ----------------------------------
// VEC elements per lane (1, or the vector width when the tensors allow it);
// a row holds at most kGenNarrowGroups groups.
template <int KIND, typename TX, typename TDY, typename TDX, int VEC>
__global__ void __launch_bounds__(kTeam)
rows_narrow_kernel(GenArgs a)
{
    constexpr int Q = rows_q(KIND);
    // rows of a slot in flight: fewer for wide groups, to stay within registers
    constexpr int U = VEC == 1 ? kGenNarrowRowsInFlight : (KIND == 2 && VEC == 8 ? 2 : 4);
    __shared__ float red[Q * VEC * kTeam];
    const int tt = threadIdx.x;
    const int ct = a.ct;
    const int lane = tt & (ct - 1);        // the lane's column group
    const int slot = tt >> __builtin_ctz((unsigned)ct);
    const int slots = kTeam / ct;
    const int H = a.cols;
    const bool col_ok = lane < H / VEC;
    const int col = (col_ok ? lane : 0) * VEC;  // dead lanes read group 0 and drop it
    const int64_t rows = a.rows;
    WeightGroup<VEC> w;
    w.load(a.w, a.w_bf16, col);
    float p[Q][VEC];
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int e = 0; e < VEC; ++e) p[q][e] = 0.f;

    const int64_t stride = (int64_t)gridDim.x * slots;
    for (int64_t r0 = (int64_t)blockIdx.x * slots + slot; r0 < rows; r0 += U * stride) {
        GroupIn<VEC> g[U];
        float mu[U], rs[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t rk = r0 + k * stride;
            const int64_t rc = rk < rows ? rk : rows - 1;  // in bounds; results dropped below
            load_group<KIND == 2, true, TX, TDY, VEC>(a, (size_t)rc * H + col, g[k]);
            mu[k] = KIND != 1 ? a.mean[rc] : 0.f;
            rs[k] = KIND != 1 ? a.rstd[rc] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            float s0 = 0.f, s1 = 0.f;
            if (col_ok) add_row_sums<KIND, VEC>(g[k], w.v, mu[k], rs[k], s0, s1);
            s0 = sub_sum(s0, ct);
            s1 = sub_sum(s1, ct);
            const int64_t rk = r0 + k * stride;
            if (rk < rows && col_ok) {
                const float2 c = row_coefs<KIND>(a, rk, s0, s1);
                group_out<KIND, TDX, VEC, Q>(a, (size_t)rk * H + col, g[k], w.v, mu[k], rs[k], c, p);
            }
        }
    }
    if (!a.want_cols) return;
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int e = 0; e < VEC; ++e) red[(q * VEC + e) * kTeam + tt] = p[q][e];
    __syncthreads();
    if (tt < ct && col_ok) {
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            float sv[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                float acc = 0.f;
                for (int k = 0; k < slots; ++k) acc += red[(q * VEC + e) * kTeam + k * ct + tt];
                sv[e] = acc;
            }
            store_vec<float, VEC>(a.partials + ((size_t)q * gridDim.x + blockIdx.x) * H + col, sv);
        }
    }
}

// ---- wide rows, pass 1: per-row sums ----------------------------------------------
// A unit is one of the a.nseg equal column segments of a row (a.nseg > 1
// only for few, long rows, so that enough blocks run); it gets W waves: 1
// (four units per block) or the whole block.  The unit's two sums go to
// coef[unit] = coef[row*nseg + segment]; the strip pass adds a row's
// segments in order.  Cacheable loads, so that the strip pass finds the rows
// in the caches.
template <int KIND, typename TX, typename TDY, int VEC, int W>
__global__ void __launch_bounds__(kTeam)
rows_coef_kernel(GenArgs a)
{
    constexpr int RPB = kTeamWaves / W;
    constexpr int LANES = W * kWave;
    constexpr int U = VEC == 8 ? 4 : 8;  // groups of a lane in flight
    __shared__ float red[2 * kTeamWaves];
    const int tt = threadIdx.x;
    const int wave = tt / kWave;
    const int slot = wave / W;
    const int li = tt - slot * LANES;
    const int64_t unit = (int64_t)blockIdx.x * RPB + slot;
    const int64_t r = unit / a.nseg;
    const int seg = (int)(unit - r * a.nseg);
    const bool live = r < a.rows;
    const int groups = a.cols / VEC;
    const int per_seg = (int)ceil_div(groups, a.nseg);
    const int g1 = (seg + 1) * per_seg < groups ? (seg + 1) * per_seg : groups;
    float s0 = 0.f, s1 = 0.f;
    if (live) {
        const size_t rowoff = (size_t)r * a.cols;
        const float mu = KIND != 1 ? a.mean[r] : 0.f;
        const float rs = KIND != 1 ? a.rstd[r] : 0.f;
        int gi = seg * per_seg + li;
        for (; gi + (U - 1) * LANES < g1; gi += U * LANES) {
            GroupIn<VEC> g[U];
            WeightGroup<VEC> w[U];
#pragma unroll
            for (int k = 0; k < U; ++k) {
                const int c = (gi + k * LANES) * VEC;
                load_group<false, false, TX, TDY, VEC>(a, rowoff + c, g[k]);
                w[k].load(a.w, a.w_bf16, c);
            }
#pragma unroll
            for (int k = 0; k < U; ++k) add_row_sums<KIND, VEC>(g[k], w[k].v, mu, rs, s0, s1);
        }
        for (; gi < g1; gi += LANES) {
            GroupIn<VEC> g;
            WeightGroup<VEC> w;
            load_group<false, false, TX, TDY, VEC>(a, rowoff + (size_t)gi * VEC, g);
            w.load(a.w, a.w_bf16, gi * VEC);
            add_row_sums<KIND, VEC>(g, w.v, mu, rs, s0, s1);
        }
    }
    s0 = wave_sum(s0);
    s1 = wave_sum(s1);
    if constexpr (W > 1) {
        if ((tt & (kWave - 1)) == 0) {
            red[wave * 2 + 0] = s0;
            red[wave * 2 + 1] = s1;
        }
        __syncthreads();
        const int w0 = slot * W;
        s0 = red[w0 * 2 + 0];
        s1 = red[w0 * 2 + 1];
#pragma unroll
        for (int k = 1; k < W; ++k) {
            s0 += red[(w0 + k) * 2 + 0];
            s1 += red[(w0 + k) * 2 + 1];
        }
    }
    if (live && li == 0) reinterpret_cast<float2 *>(a.coef)[unit] = make_float2(s0, s1);
}

// The coefficients of row r from its segments' sums, added in segment order.
template <int KIND>
__device__ __forceinline__ float2 strip_coefs(const GenArgs &a, int64_t r)
{
    const float2 *c = reinterpret_cast<const float2 *>(a.coef) + r * a.nseg;
    float s0 = c[0].x, s1 = c[0].y;
    for (int k = 1; k < a.nseg; ++k) {
        s0 += c[k].x;
        s1 += c[k].y;
    }
    return row_coefs<KIND>(a, r, s0, s1);
}

// ---- wide rows, pass 2: column strips by row chunks --------------------------------
template <int KIND, typename TX, typename TDY, typename TDX, int VEC>
__global__ void __launch_bounds__(kTeam)
rows_strip_kernel(GenArgs a)
{
    constexpr int Q = rows_q(KIND);
    constexpr int CT = kGenStripGroups;   // column lanes (one wave)
    constexpr int RT = kTeam / CT;        // row lanes
    constexpr int U = VEC == 1 ? 8 : (VEC == 4 ? 4 : 2);  // rows of a lane in flight
    __shared__ float red[(RT - 1) * Q * VEC * CT];
    const int tt = threadIdx.x;
    const int cl = tt & (CT - 1);
    const int rl = __builtin_amdgcn_readfirstlane(tt / CT);  // one row lane per wave
    const int groups = a.cols / VEC;
    const int grp = (int)blockIdx.x * CT + cl;
    const bool col_ok = grp < groups;
    const int col = grp * VEC;
    const int64_t r0 = (int64_t)blockIdx.y * a.rpc;
    const int64_t r1 = r0 + a.rpc < a.rows ? r0 + a.rpc : a.rows;
    float p[Q][VEC];
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int e = 0; e < VEC; ++e) p[q][e] = 0.f;

    if (col_ok) {
        WeightGroup<VEC> w;
        w.load(a.w, a.w_bf16, col);
        int64_t r = r0 + rl;
        for (; r + (U - 1) * RT < r1; r += U * RT) {
            GroupIn<VEC> g[U];
            float2 c[U];
            float mu[U], rs[U];
#pragma unroll
            for (int k = 0; k < U; ++k) {
                const int64_t rk = r + k * RT;
                load_group<KIND == 2, true, TX, TDY, VEC>(a, (size_t)rk * a.cols + col, g[k]);
                c[k] = strip_coefs<KIND == 2 ? 0 : KIND>(a, rk);
                mu[k] = KIND != 1 ? a.mean[rk] : 0.f;
                rs[k] = KIND != 1 ? a.rstd[rk] : 0.f;
            }
#pragma unroll
            for (int k = 0; k < U; ++k)
                group_out<KIND, TDX, VEC, Q>(a, (size_t)(r + k * RT) * a.cols + col, g[k], w.v, mu[k],
                                             rs[k], c[k], p);
        }
        for (; r < r1; r += RT) {
            GroupIn<VEC> g;
            load_group<KIND == 2, true, TX, TDY, VEC>(a, (size_t)r * a.cols + col, g);
            const float mu = KIND != 1 ? a.mean[r] : 0.f;
            const float rs = KIND != 1 ? a.rstd[r] : 0.f;
            group_out<KIND, TDX, VEC, Q>(a, (size_t)r * a.cols + col, g, w.v, mu, rs,
                                         strip_coefs<KIND == 2 ? 0 : KIND>(a, r), p);
        }
    }
    if (!a.want_cols) return;
    if (rl > 0)
#pragma unroll
        for (int q = 0; q < Q; ++q)
#pragma unroll
            for (int e = 0; e < VEC; ++e) red[(((rl - 1) * Q + q) * VEC + e) * CT + cl] = p[q][e];
    __syncthreads();
    if (rl == 0 && col_ok) {
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            float s[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                s[e] = p[q][e];
#pragma unroll
                for (int k = 1; k < RT; ++k) s[e] += red[(((k - 1) * Q + q) * VEC + e) * CT + cl];
            }
            store_vec<float, VEC>(a.partials + ((size_t)q * gridDim.y + blockIdx.y) * a.cols + col, s);
        }
    }
}

// ---- host dispatch ---------------------------------------------------------------
template <int KIND, typename TX, typename TDY, typename TDX, int VEC>
static hipError_t strip_launch(const RowsCall &a, const GenArgs &g, int kid, hipStream_t s)
{
    constexpr int CK = KIND == 2 ? 0 : KIND;  // the bias+dropout+add rows reduce as LayerNorm's
    hipError_t e;
    const int64_t units = (int64_t)a.rows * a.gen_coef_segs;
    if (a.gen_coef_waves == 1)
        e = launch(NH_K_ROWS_COEF, rows_coef_kernel<CK, TX, TDY, VEC, 1>,
                   dim3((unsigned)ceil_div(units, kTeamWaves)), dim3(kTeam), 0u, s, g);
    else
        e = launch(NH_K_ROWS_COEF, rows_coef_kernel<CK, TX, TDY, VEC, kTeamWaves>, dim3((unsigned)units),
                   dim3(kTeam), 0u, s, g);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)ceil_div(a.cols / VEC, kGenStripGroups), (unsigned)a.blocks);
    return launch(kid, rows_strip_kernel<KIND, TX, TDY, TDX, VEC>, grid, dim3(kTeam), 0u, s, g);
}

template <int KIND, typename TX, typename TDY, typename TDX>
static hipError_t generic_types(const RowsCall &a, const GenArgs &g, hipStream_t s)
{
    const int kid = KIND == 0 ? NH_K_LN_ROWS : (KIND == 1 ? NH_K_RMS_ROWS : NH_K_BDA_ROWS);
    // The vector width of a type mix: 8 when every row tensor is bf16, else 4.
    constexpr int V = sizeof(TX) == 2 && sizeof(TDY) == 2 && sizeof(TDX) == 2 ? 8 : 4;
    if (a.vec != 1 && a.vec != V) return hipErrorInvalidValue;
    if (a.gen_ct > 0) {
        if (a.vec == 1)
            return launch(kid, rows_narrow_kernel<KIND, TX, TDY, TDX, 1>, dim3((unsigned)a.blocks),
                          dim3(kTeam), 0u, s, g);
        return launch(kid, rows_narrow_kernel<KIND, TX, TDY, TDX, V>, dim3((unsigned)a.blocks), dim3(kTeam),
                      0u, s, g);
    }
    if (a.vec == 1) return strip_launch<KIND, TX, TDY, TDX, 1>(a, g, kid, s);
    return strip_launch<KIND, TX, TDY, TDX, V>(a, g, kid, s);
}

template <int KIND>
static hipError_t generic_kind(const RowsCall &a, const GenArgs &g, hipStream_t s)
{
    if constexpr (KIND == 1) {
        // RMSNorm: one dtype for x, dy and dx
        return a.x_t == 0 ? generic_types<1, float, float, float>(a, g, s)
                          : generic_types<1, uint16_t, uint16_t, uint16_t>(a, g, s);
    } else if constexpr (KIND == 2) {
        // da has dy's dtype
        switch (a.x_t * 2 + a.dy_t) {
        case 0: return generic_types<2, float, float, float>(a, g, s);
        case 1: return generic_types<2, float, uint16_t, uint16_t>(a, g, s);
        case 2: return generic_types<2, uint16_t, float, float>(a, g, s);
        default: return generic_types<2, uint16_t, uint16_t, uint16_t>(a, g, s);
        }
    } else {
        // The dx dtype of a skipped dx is irrelevant: use the dy dtype.
        const int dxt = a.dx != nullptr ? a.dx_t : a.dy_t;
        switch (a.x_t * 4 + a.dy_t * 2 + dxt) {
        case 0: return generic_types<0, float, float, float>(a, g, s);
        case 1: return generic_types<0, float, float, uint16_t>(a, g, s);
        case 2: return generic_types<0, float, uint16_t, float>(a, g, s);
        case 3: return generic_types<0, float, uint16_t, uint16_t>(a, g, s);
        case 4: return generic_types<0, uint16_t, float, float>(a, g, s);
        case 5: return generic_types<0, uint16_t, float, uint16_t>(a, g, s);
        case 6: return generic_types<0, uint16_t, uint16_t, float>(a, g, s);
        default: return generic_types<0, uint16_t, uint16_t, uint16_t>(a, g, s);
        }
    }
}

hipError_t rows_generic_launch(const RowsCall &a, hipStream_t s)
{
    if (a.rows == 0) return hipSuccess;
    GenArgs g{};
    g.x = a.x;
    g.dy = a.dy;
    g.w = a.w;
    g.mean = a.mean;
    g.rstd = a.rstd;
    g.rms = a.rms;
    g.dres = a.dresidual;
    g.mask = a.mask;
    g.dh = a.dh;
    g.dx = a.dx;
    g.partials = a.partials;
    g.coef = a.coef;
    g.eps = a.eps;
    g.scale = a.scale;
    g.rows = a.rows;
    g.cols = a.cols;
    g.w_bf16 = a.w_t;
    g.want_cols = a.kind == 1 ? a.dweight != nullptr
                              : (a.dweight != nullptr || a.dbias != nullptr ||
                                 (a.kind == 2 && a.dbias_in != nullptr));
    g.ct = a.gen_ct;
    g.rpc = a.gen_rpc;
    g.nseg = a.gen_coef_segs;
    if (a.gen_ct <= 0 && (a.coef == nullptr || a.gen_rpc <= 0 || a.gen_coef_segs < 1 ||
                          (a.gen_coef_segs > 1 && a.gen_coef_waves == 1)))
        return hipErrorInvalidValue;
    switch (a.kind) {
    case 0: return generic_kind<0>(a, g, s);
    case 1: return generic_kind<1>(a, g, s);
    default: return generic_kind<2>(a, g, s);
    }
}

} // namespace nh
