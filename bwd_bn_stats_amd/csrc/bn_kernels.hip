// BatchNorm2d training forward/backward kernels (NCHW, statistics per channel).
//
// Follows Aether-ML PR #18, "perf(batchnorm): device-sized grid, one-pass
// statistics, finalize kernels" (its "Reduction grid", "One-pass statistics"
// and "Backward finalize" sections), re-designed for gfx950:
//
//   forward : bn_stats_kernel      one read of x: shifted sums
//                                  (sum d, sum d^2), d = x - x[0,c,0,0],
//                                  one slot of partials[2, grid_y, C] per block
//             bn_fwd_finalize      fixed-order fp64 combine of the partials ->
//                                  stats[4, C]; running statistics in place
//             bn_apply_kernel      y = fmaf(x - mean, scale, beta)
//   backward: bn_grad_sums_kernel  (sum dy, sum dy*(x - mean)) -> partials
//             bn_bwd_finalize      -> grads[4, C] = (dgamma, dbeta, k1, k2)
//             bn_dx_kernel         dx = dy*scale + (x - mean)*k1 + k2
//
// Work split: channel c owns N planes of HW contiguous elements (one per
// image n, stride C*HW).  Its M = N*HW elements are cut into `units` of `V`
// consecutive elements inside one plane (V = 16 bytes of data when the
// plane length and pointers allow it, else 1), numbered plane-major.  The
// launch has C*grid_y blocks; block (c, yb) takes the contiguous unit range
// [yb*upb, (yb+1)*upb) of channel c, so every block touches one channel
// only and reads its per-channel constants once into scalar registers.  The
// elementwise passes use the same split as the reductions.
//
// No atomics anywhere: each reduction block writes its own partial slot, the
// finalize kernels combine slots in index order, so results are
// bit-identical run to run and the workspace needs no zeroing.
#include "nh_internal.hpp"

namespace nh {

struct BnGeom {
    int C;
    int HW;
    int HWv;        // units per plane
    FastDiv div_hwv;
    int units;      // units per channel (N * HWv)
    int upb;        // units per block
    int grid_y;
};

// Element offset of unit u of channel c.
template <int V>
__device__ __forceinline__ int bn_unit_offset(const BnGeom &g, int c, int u)
{
    int n = (int)g.div_hwv.div((uint32_t)u);
    int j = u - n * g.HWv;
    return (n * g.C + c) * g.HW + j * V;
}

// Sums of (a, b) over a 256-thread block; the result is valid in thread 0.
__device__ __forceinline__ void block_sum2(float &a, float &b)
{
    __shared__ float red[kBnThreads / kWave][2];
    a = wave_sum(a);
    b = wave_sum(b);
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) {
        red[wave][0] = a;
        red[wave][1] = b;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float sa = red[0][0], sb = red[0][1];
#pragma unroll
        for (int w = 1; w < kBnThreads / kWave; ++w) {
            sa += red[w][0];
            sb += red[w][1];
        }
        a = sa;
        b = sb;
    }
}

// ---- forward reduction: shifted one-pass sums ------------------------------
template <typename T, int V>
__global__ void __launch_bounds__(kBnThreads)
bn_stats_kernel(const T *__restrict__ x, BnGeom g, float *__restrict__ partials)
{
    const int c = blockIdx.x / g.grid_y;
    const int yb = blockIdx.x - c * g.grid_y;
    const int u0 = yb * g.upb;
    const int u1 = min(u0 + g.upb, g.units);
    // The shift: the channel's first element, x[0, c, 0, 0].
    const float K = to_f32(x[c * g.HW]);

    float s1[kBnUnroll], s2[kBnUnroll];
#pragma unroll
    for (int k = 0; k < kBnUnroll; ++k) { s1[k] = 0.f; s2[k] = 0.f; }

    for (int base = u0 + (int)threadIdx.x; base < u1; base += kBnThreads * kBnUnroll) {
        float v[kBnUnroll][V];
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const int u = base + k * kBnThreads;
            if (u < u1) load_vec<T, V>(x + bn_unit_offset<V>(g, c, u), v[k]);
        }
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const int u = base + k * kBnThreads;
            if (u < u1) {
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float d = v[k][e] - K;
                    s1[k] += d;
                    s2[k] = fmaf(d, d, s2[k]);
                }
            }
        }
    }
    float a = s1[0], b = s2[0];
#pragma unroll
    for (int k = 1; k < kBnUnroll; ++k) { a += s1[k]; b += s2[k]; }
    block_sum2(a, b);
    if (threadIdx.x == 0) {
        partials[(0 * g.grid_y + yb) * g.C + c] = a;
        partials[(1 * g.grid_y + yb) * g.C + c] = b;
    }
}

// ---- backward reduction: sum dy, sum dy*(x - mean) ----------------------------
template <typename T, int V>
__global__ void __launch_bounds__(kBnThreads)
bn_grad_sums_kernel(const T *__restrict__ dy, const T *__restrict__ x,
                    const float *__restrict__ stats, BnGeom g, float *__restrict__ partials)
{
    const int c = blockIdx.x / g.grid_y;
    const int yb = blockIdx.x - c * g.grid_y;
    const int u0 = yb * g.upb;
    const int u1 = min(u0 + g.upb, g.units);
    const float mean = stats[c];

    float s1[kBnUnroll], s2[kBnUnroll];
#pragma unroll
    for (int k = 0; k < kBnUnroll; ++k) { s1[k] = 0.f; s2[k] = 0.f; }

    for (int base = u0 + (int)threadIdx.x; base < u1; base += kBnThreads * kBnUnroll) {
        float vx[kBnUnroll][V], vd[kBnUnroll][V];
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const int u = base + k * kBnThreads;
            if (u < u1) {
                const int off = bn_unit_offset<V>(g, c, u);
                load_vec<T, V>(x + off, vx[k]);
                load_vec<T, V>(dy + off, vd[k]);
            }
        }
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const int u = base + k * kBnThreads;
            if (u < u1) {
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    s1[k] += vd[k][e];
                    s2[k] = fmaf(vd[k][e], vx[k][e] - mean, s2[k]);
                }
            }
        }
    }
    float a = s1[0], b = s2[0];
#pragma unroll
    for (int k = 1; k < kBnUnroll; ++k) { a += s1[k]; b += s2[k]; }
    block_sum2(a, b);
    if (threadIdx.x == 0) {
        partials[(0 * g.grid_y + yb) * g.C + c] = a;
        partials[(1 * g.grid_y + yb) * g.C + c] = b;
    }
}

// ---- finalize kernels: one wave per channel, fp64 fixed-order combine -------
// Lane l sums slots l, l+64, ... in order; the butterfly then combines lanes.
__device__ __forceinline__ void sum_partials(const float *__restrict__ partials, int grid_y,
                                             int C, int c, double &s1, double &s2)
{
    const int lane = threadIdx.x & (kWave - 1);
    double a = 0.0, b = 0.0;
    for (int yb = lane; yb < grid_y; yb += kWave) {
        a += (double)partials[(0 * grid_y + yb) * C + c];
        b += (double)partials[(1 * grid_y + yb) * C + c];
    }
    s1 = wave_sum(a);
    s2 = wave_sum(b);
}

template <typename T>
__global__ void __launch_bounds__(kBnThreads)
bn_fwd_finalize(const T *__restrict__ x, const float *__restrict__ partials, int grid_y,
                int C, int HW, int64_t M, const float *__restrict__ gamma,
                float *__restrict__ running_mean, float *__restrict__ running_var,
                float momentum, float eps, float *__restrict__ stats)
{
    const int c = blockIdx.x * (kBnThreads / kWave) + (int)threadIdx.x / kWave;
    if (c >= C) return;  // whole wave exits together
    double S1, S2;
    sum_partials(partials, grid_y, C, c, S1, S2);
    if ((threadIdx.x & (kWave - 1)) != 0) return;
    const double Md = (double)M;
    const double K = (double)to_f32(x[c * HW]);
    const double md = S1 / Md;                    // mean of the shifted values
    double var = S2 / Md - md * md;               // biased variance
    if (var < 0.0) var = 0.0;
    const double mean = K + md;
    const double inv_std = 1.0 / sqrt(var + (double)eps);
    const double gm = gamma ? (double)gamma[c] : 1.0;
    stats[0 * C + c] = (float)mean;
    stats[1 * C + c] = (float)var;
    stats[2 * C + c] = (float)inv_std;
    stats[3 * C + c] = (float)(gm * inv_std);
    const double m = (double)momentum;
    if (running_mean)
        running_mean[c] = (float)((1.0 - m) * (double)running_mean[c] + m * mean);
    if (running_var)
        running_var[c] = (float)((1.0 - m) * (double)running_var[c] + m * var * Md / (Md - 1.0));
}

__global__ void __launch_bounds__(kBnThreads)
bn_bwd_finalize(const float *__restrict__ partials, int grid_y, int C, int64_t M,
                const float *__restrict__ stats, float *__restrict__ grads)
{
    const int c = blockIdx.x * (kBnThreads / kWave) + (int)threadIdx.x / kWave;
    if (c >= C) return;
    double Sdy, Sdyxc;
    sum_partials(partials, grid_y, C, c, Sdy, Sdyxc);
    if ((threadIdx.x & (kWave - 1)) != 0) return;
    const double Md = (double)M;
    const double inv_std = (double)stats[2 * C + c];
    const double scale = (double)stats[3 * C + c];
    grads[0 * C + c] = (float)(inv_std * Sdyxc);                       // dgamma
    grads[1 * C + c] = (float)Sdy;                                     // dbeta
    grads[2 * C + c] = (float)(-scale * inv_std * inv_std * Sdyxc / Md); // k1
    grads[3 * C + c] = (float)(-scale * Sdy / Md);                     // k2
}

// ---- elementwise passes ------------------------------------------------------
template <typename T, int V>
__global__ void __launch_bounds__(kBnThreads)
bn_apply_kernel(const T *__restrict__ x, T *__restrict__ y, const float *__restrict__ stats,
                const float *__restrict__ beta, BnGeom g)
{
    const int c = blockIdx.x / g.grid_y;
    const int yb = blockIdx.x - c * g.grid_y;
    const int u0 = yb * g.upb;
    const int u1 = min(u0 + g.upb, g.units);
    const float mean = stats[c];
    const float scale = stats[3 * g.C + c];
    const float b = beta ? beta[c] : 0.f;

    for (int base = u0 + (int)threadIdx.x; base < u1; base += kBnThreads * kBnUnroll) {
        float v[kBnUnroll][V];
        int off[kBnUnroll];
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const int u = base + k * kBnThreads;
            off[k] = bn_unit_offset<V>(g, c, u);
            if (u < u1) load_vec<T, V>(x + off[k], v[k]);
        }
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const int u = base + k * kBnThreads;
            if (u < u1) {
                float o[V];
#pragma unroll
                for (int e = 0; e < V; ++e) o[e] = fmaf(v[k][e] - mean, scale, b);
                store_vec<T, V>(y + off[k], o);
            }
        }
    }
}

template <typename T, int V>
__global__ void __launch_bounds__(kBnThreads)
bn_dx_kernel(const T *__restrict__ dy, const T *__restrict__ x, T *__restrict__ dx,
             const float *__restrict__ stats, const float *__restrict__ grads, BnGeom g)
{
    const int c = blockIdx.x / g.grid_y;
    const int yb = blockIdx.x - c * g.grid_y;
    const int u0 = yb * g.upb;
    const int u1 = min(u0 + g.upb, g.units);
    const float mean = stats[c];
    const float scale = stats[3 * g.C + c];
    const float k1 = grads[2 * g.C + c];
    const float k2 = grads[3 * g.C + c];

    for (int base = u0 + (int)threadIdx.x; base < u1; base += kBnThreads * kBnUnroll) {
        float vx[kBnUnroll][V], vd[kBnUnroll][V];
        int off[kBnUnroll];
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const int u = base + k * kBnThreads;
            off[k] = bn_unit_offset<V>(g, c, u);
            if (u < u1) {
                load_vec<T, V>(x + off[k], vx[k]);
                load_vec<T, V>(dy + off[k], vd[k]);
            }
        }
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const int u = base + k * kBnThreads;
            if (u < u1) {
                float o[V];
#pragma unroll
                for (int e = 0; e < V; ++e)
                    o[e] = fmaf(vd[k][e], scale, fmaf(vx[k][e] - mean, k1, k2));
                store_vec<T, V>(dx + off[k], o);
            }
        }
    }
}

// ---- host launchers -----------------------------------------------------------
static BnGeom make_geom(const BnCall &a)
{
    BnGeom g;
    g.C = a.C;
    g.HW = a.HW;
    g.HWv = a.HW / a.vec;
    g.div_hwv = make_fastdiv((uint32_t)g.HWv);
    g.units = a.N * g.HWv;
    g.grid_y = a.grid_y;
    g.upb = (int)ceil_div(g.units, a.grid_y);
    return g;
}

template <typename T, int V>
static hipError_t bn_forward_t(const BnCall &a, hipStream_t s)
{
    const BnGeom g = make_geom(a);
    const T *x = static_cast<const T *>(a.x);
    const dim3 grid((unsigned)(a.C * a.grid_y)), block(kBnThreads);
    hipError_t e = launch(NH_K_BN_STATS, bn_stats_kernel<T, V>, grid, block, 0, s, x, g, a.partials);
    if (e != hipSuccess) return e;
    const dim3 fgrid((unsigned)ceil_div(a.C, kBnThreads / kWave));
    e = launch(NH_K_BN_FWD_FINALIZE, bn_fwd_finalize<T>, fgrid, block, 0, s, x, a.partials,
               a.grid_y, a.C, a.HW, (int64_t)a.N * a.HW, a.gamma, a.running_mean,
               a.running_var, a.momentum, a.eps, a.stats);
    if (e != hipSuccess) return e;
    return launch(NH_K_BN_APPLY, bn_apply_kernel<T, V>, grid, block, 0, s, x,
                  static_cast<T *>(a.out), a.stats, a.beta, g);
}

template <typename T, int V>
static hipError_t bn_backward_t(const BnCall &a, hipStream_t s)
{
    const BnGeom g = make_geom(a);
    const T *x = static_cast<const T *>(a.x);
    const T *dy = static_cast<const T *>(a.dy);
    const dim3 grid((unsigned)(a.C * a.grid_y)), block(kBnThreads);
    hipError_t e = launch(NH_K_BN_GRAD_SUMS, bn_grad_sums_kernel<T, V>, grid, block, 0, s, dy, x,
                          a.stats, g, a.partials);
    if (e != hipSuccess) return e;
    const dim3 fgrid((unsigned)ceil_div(a.C, kBnThreads / kWave));
    e = launch(NH_K_BN_BWD_FINALIZE, bn_bwd_finalize, fgrid, block, 0, s, a.partials, a.grid_y,
               a.C, (int64_t)a.N * a.HW, a.stats, a.grads);
    if (e != hipSuccess || a.out == nullptr) return e;
    return launch(NH_K_BN_DX, bn_dx_kernel<T, V>, grid, block, 0, s, dy, x,
                  static_cast<T *>(a.out), a.stats, a.grads, g);
}

hipError_t bn_forward_launch(const BnCall &a, hipStream_t s)
{
    if (a.io == 0) return a.vec == 4 ? bn_forward_t<float, 4>(a, s) : bn_forward_t<float, 1>(a, s);
    return a.vec == 8 ? bn_forward_t<uint16_t, 8>(a, s) : bn_forward_t<uint16_t, 1>(a, s);
}

hipError_t bn_backward_launch(const BnCall &a, hipStream_t s)
{
    if (a.io == 0) return a.vec == 4 ? bn_backward_t<float, 4>(a, s) : bn_backward_t<float, 1>(a, s);
    return a.vec == 8 ? bn_backward_t<uint16_t, 8>(a, s) : bn_backward_t<uint16_t, 1>(a, s);
}

} // namespace nh
