// BatchNorm2d training forward/backward kernels (NCHW, statistics per channel).
//
// Follows Aether-ML PR #18, "perf(batchnorm): device-sized grid, one-pass
// statistics, finalize kernels" (its "Reduction grid", "One-pass statistics"
// and "Backward finalize" sections), re-designed for gfx950:
//
//   forward : bn_stats_kernel      one read of x: shifted sums
//                                  (sum d, sum d^2), d = x - x[0,c,0,0],
//                                  one slot of partials[C, 2, grid_y] per block
//             finalize             fixed-order fp64 combine of the partials ->
//                                  stats[4, C]; running statistics in place
//             bn_apply_kernel      y = fmaf(x - mean, scale, beta)
//   backward: bn_grad_sums_kernel  (sum dy, sum dy*(x - mean)) -> partials
//             finalize             -> grads[4, C] = (dgamma, dbeta, k1, k2)
//             bn_dx_kernel         dx = dy*scale + (x - mean)*k1 + k2
//
// The finalize step runs either as its own small kernel (bn_fwd_finalize /
// bn_bwd_finalize, the pages' three-launch structure) or, by default, in the
// prologue of the elementwise kernel that consumes it: on MI355X a dependent
// launch of a few-KB kernel costs about 4 us, a sizeable share of a 50 us
// forward+backward step, while re-reading a channel's partials per block
// costs a few hundred bytes of L2 traffic.
//
// Workspace: partials[C, 2, grid_y] followed by the shifts K[C].  A
// channel's slots are contiguous, so the wave that combines them reads a
// few cache lines, and blocks of different channels that finish together
// write different lines.  With the slots of one block index side by side
// ([2, grid_y, C]) every lane's load touched its own line (256 lines per
// block at 64 slots, as many L2 requests as the pass's own data) and
// neighbouring channels' blocks, on different XCDs, wrote into one line.
// Measured on MI355X, cold per call, fwd+bwd: (256,32,32,32) fp32 40.10 ->
// 39.46 us, bf16 26.76 -> 26.05 us, (64,256,56,56) bf16 121.43 -> 120.56 us
// (the reductions faster as well as the elementwise passes).
//
// Work split: channel c owns N planes of HW contiguous elements (one per
// image n, stride C*HW).  Its M = N*HW elements are cut into `units` of `V`
// consecutive elements inside one plane (V = 16 bytes of data when the
// plane length and pointers allow it; 8 bytes for bf16 planes of 4k
// elements; else 1), numbered plane-major.  The
// launch has C*grid_y blocks; block (c, yb) takes units of channel c only
// (the contiguous range [yb*upb, (yb+1)*upb), or every grid_y-th sweep of
// the channel: bn_range), so it reads its per-channel constants once into
// scalar registers.  The elementwise passes use the same split as the
// reductions.
//
// Activation (the BatchNorm + ReLU/LeakyReLU fusion the PR lists as its
// follow-up): with z = fmaf(x - mean, scale, beta) the forward stores act(z),
// and the backward multiplies dy by act'(z) before both of its passes use it.
// The backward recomputes z from x, which it reads anyway, and from the same
// fp32 mean/scale/beta the forward used, so its mask is bit-for-bit the
// forward's and the fusion adds no memory traffic.  act'(0) is taken from the
// left (ReLU 0, LeakyReLU slope).
//
// Inference applies the same centred step with the running statistics in
// place of the batch statistics (mean = running_mean, scale =
// gamma/sqrt(running_var + eps)): one elementwise pass, no workspace.
//
// Small channels (few units each) take one fused kernel per direction
// instead: a block per channel reduces, finalizes and writes the elementwise
// pass (bn_fwd_channel_kernel, bn_bwd_channel_kernel).  Small planes (a few
// elements per image and channel) take the row layout: the tensor as
// [N, C*HW] rows, column sums over row chunks (bn_col_* kernels below).
// Which path runs is the host plan's choice (api.cpp).
//
// No atomics anywhere: each reduction block writes its own partial slot, the
// finalize kernels combine slots in index order, so results are
// bit-identical run to run and the workspace needs no zeroing.
#include "nh_bn.hpp"

namespace nh {

// Cache policy of the BatchNorm streams: which accesses carry the
// nontemporal hint.  Measured on MI355X over cold 33-103 MB tensors, the best
// of the eight combinations keeps the reduction passes' loads cacheable (the
// elementwise pass re-reads the same x and dy right after, and finds them in
// the 256 MB Infinity Cache), streams the elementwise passes' loads (last
// use) and streams every store.  No setting of a load's cache-policy bits
// (sc0, nt, sc1) both reads at the nontemporal rate and leaves the data in
// the Infinity Cache: the nt bit decides both.
enum : int { kNtReduceLoads = 1, kNtEwLoads = 2, kNtStores = 4 };
#ifndef NH_BN_NT_POLICY
#define NH_BN_NT_POLICY (kNtEwLoads | kNtStores)
#endif
constexpr int kBnNtPolicy = NH_BN_NT_POLICY;

// Loads a unit into its storage form (bf16 stays packed, two per register):
// the widening to fp32 happens where the values are used, so a conditional
// load's block holds the load alone and the unit's loads of a sweep all stay
// in flight together, instead of each waiting for its data before the next
// one issues.
template <bool NT, typename T, int V>
__device__ __forceinline__ void ldr(Raw<T, V> &r, const T *p)
{
    if constexpr (NT) r.load_nt(p);
    else r.load(p);
}

// Activations: 0 none, 1 ReLU, 2 LeakyReLU.
template <int ACT>
__device__ __forceinline__ float act_fwd(float z, float slope)
{
    if constexpr (ACT == 1) return z > 0.f ? z : 0.f;
    else if constexpr (ACT == 2) return z > 0.f ? z : z * slope;
    else return z;
}

// dy * act'(z).
template <int ACT>
__device__ __forceinline__ float act_bwd(float dy, float z, float slope)
{
    if constexpr (ACT == 1) return z > 0.f ? dy : 0.f;
    else if constexpr (ACT == 2) return z > 0.f ? dy : dy * slope;
    else return dy;
}

// Sums of (a, b) over a 256-thread block; the result is valid in thread 0.
// The wave sums are DPP steps (wave_total), then the waves in index order.
__device__ __forceinline__ void block_sum2(float &a, float &b)
{
    __shared__ float red[kBnThreads / kWave][2];
    a = wave_total(a);
    b = wave_total(b);
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

// Sums of (a, b) over a TB-thread block, in the order of block_sum2 (wave
// sums, then the waves in index order); the result is valid in thread 0.
template <int TB>
__device__ __forceinline__ void block_sum2_tb(float &a, float &b)
{
    if constexpr (TB == kBnThreads) {
        block_sum2(a, b);
    } else {
        __shared__ float red[TB / kWave][2];
        a = wave_total(a);
        b = wave_total(b);
        const int wave = threadIdx.x / kWave;
        if ((threadIdx.x & (kWave - 1)) == 0) {
            red[wave][0] = a;
            red[wave][1] = b;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            float sa = red[0][0], sb = red[0][1];
#pragma unroll
            for (int w = 1; w < TB / kWave; ++w) {
                sa += red[w][0];
                sb += red[w][1];
            }
            a = sa;
            b = sb;
        }
    }
}

// The shift x[0, c, 0, 0] of the forward reductions, read with a vector
// memory load: as a scalar load it would be waited for, together with the
// kernel arguments loaded after it, before the block's first loads of x were
// issued, putting one more memory round trip in every block's path.
__device__ __forceinline__ float load_shift(const float *p)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(p, 4u), 0, 0, 0));
}

// A per-channel fp32 value (stats, gamma, beta, a shift, running
// statistics) read with a vector memory load, for the same reason: issued
// right after a pass's first loads of x, it arrives with them, where a
// scalar load would add a memory round trip before the elementwise work.
__device__ __forceinline__ float ldv(const float *p) { return load_shift(p); }

// p[i] by a vector memory load, or 0 when `on` is false or p is NULL: the
// buffer range is then empty and the load touches no memory.  No branch
// surrounds the load, so the compiler keeps it in flight with the caller's
// other loads (a load under a branch is waited for where the branches meet).
__device__ __forceinline__ float ldv_if(const float *p, int i, bool on)
{
    const bool live = on && p != nullptr;
    return __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(live ? p + i : p, live ? 4u : 0u), 0, 0, 0));
}
__device__ __forceinline__ float load_shift(const uint16_t *p)
{
    // the bf16 bits straight into the high half of a zeroed register: the
    // fp32 value with no instruction between the load and its first use
    typedef short short2_t __attribute__((ext_vector_type(2)));
    short2_t t = {0, 0};
    t.y = (short)__builtin_amdgcn_raw_buffer_load_b16(make_rsrc(p, 2u), 0, 0, 0);
    return __builtin_bit_cast(float, t);
}

// ---- forward reduction: shifted one-pass sums ------------------------------
template <typename T, int V, int NT>
__global__ void __launch_bounds__(kBnThreads, kBnWavesPerSimd)
bn_stats_kernel(const T *__restrict__ x, BnGeom g, float *__restrict__ partials)
{
    const BnBlock blk = bn_block(g);
    const int c = blk.c, yb = blk.yb;
    // Unit indices are unsigned: a channel may hold up to 2^31 - 1 units,
    // and the loop index runs up to a step past the last one.
    const BnRange rg = bn_range(g, yb);
    const uint32_t u0 = rg.u0, u1 = rg.u1, step = rg.step;

    float s1[kBnUnroll], s2[kBnUnroll];
#pragma unroll
    for (int k = 0; k < kBnUnroll; ++k) { s1[k] = 0.f; s2[k] = 0.f; }

    // The first sweep's loads go out before the shift's, so that no load of
    // x waits for the shift (loads complete in issue order).
    uint32_t base = u0 + threadIdx.x;
    Raw<T, V> v[kBnUnroll];
#pragma unroll
    for (int k = 0; k < kBnUnroll; ++k) {
        const uint32_t u = base + k * kBnThreads;
        if (u < u1) ldr<(NT & kNtReduceLoads) != 0>(v[k], x + bn_unit_offset<V>(g, c, u));
    }
    // The shift: the channel's first element, x[0, c, 0, 0].
    const float K = load_shift(x + c * g.HW);
    while (base < u1) {
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const uint32_t u = base + k * kBnThreads;
            if (u < u1) {
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float d = v[k].get(e) - K;
                    s1[k] += d;
                    s2[k] = fmaf(d, d, s2[k]);
                }
            }
        }
        base += step;
        if (base >= u1) break;
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const uint32_t u = base + k * kBnThreads;
            if (u < u1) ldr<(NT & kNtReduceLoads) != 0>(v[k], x + bn_unit_offset<V>(g, c, u));
        }
    }
    float a = s1[0], b = s2[0];
#pragma unroll
    for (int k = 1; k < kBnUnroll; ++k) { a += s1[k]; b += s2[k]; }
    block_sum2(a, b);
    if (threadIdx.x == 0) {
        partials[((size_t)c * 2 + 0) * g.grid_y + yb] = a;
        partials[((size_t)c * 2 + 1) * g.grid_y + yb] = b;
        // The shift itself, kept beside the partials: with y == x the apply
        // pass may overwrite x[0, c, 0, 0] before every block has read it.
        if (yb == 0) partials[(size_t)2 * g.grid_y * g.C + c] = K;
    }
}

// ---- backward reduction: sum dy, sum dy*(x - mean) ----------------------------
// With an activation, dy is first replaced by dz = dy * act'(z).
template <typename T, int V, int NT, int ACT>
__global__ void __launch_bounds__(kBnThreads, kBnWavesPerSimd)
bn_grad_sums_kernel(const T *__restrict__ dy, const T *__restrict__ x,
                    const float *__restrict__ stats, const float *__restrict__ beta, float slope,
                    BnGeom g, float *__restrict__ partials)
{
    const BnBlock blk = bn_block(g);
    const int c = blk.c, yb = blk.yb;
    // Unit indices are unsigned: a channel may hold up to 2^31 - 1 units,
    // and the loop index runs up to a step past the last one.
    const BnRange rg = bn_range(g, yb);
    const uint32_t u0 = rg.u0, u1 = rg.u1, step = rg.step;
    const float mean = stats[c];
    const float scale = ACT != 0 ? stats[3 * g.C + c] : 0.f;
    const float bz = (ACT != 0 && beta) ? beta[c] : 0.f;

    float s1[kBnUnroll], s2[kBnUnroll];
#pragma unroll
    for (int k = 0; k < kBnUnroll; ++k) { s1[k] = 0.f; s2[k] = 0.f; }

    for (uint32_t base = u0 + threadIdx.x; base < u1; base += step) {
        Raw<T, V> vx[kBnUnroll], vd[kBnUnroll];
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const uint32_t u = base + k * kBnThreads;
            if (u < u1) {
                const int off = bn_unit_offset<V>(g, c, u);
                ldr<(NT & kNtReduceLoads) != 0>(vx[k], x + off);
                ldr<(NT & kNtReduceLoads) != 0>(vd[k], dy + off);
            }
        }
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const uint32_t u = base + k * kBnThreads;
            if (u < u1) {
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float xc = vx[k].get(e) - mean;
                    const float dz = act_bwd<ACT>(vd[k].get(e), fmaf(xc, scale, bz), slope);
                    s1[k] += dz;
                    s2[k] = fmaf(dz, xc, s2[k]);
                }
            }
        }
    }
    float a = s1[0], b = s2[0];
#pragma unroll
    for (int k = 1; k < kBnUnroll; ++k) { a += s1[k]; b += s2[k]; }
    block_sum2(a, b);
    if (threadIdx.x == 0) {
        partials[((size_t)c * 2 + 0) * g.grid_y + yb] = a;
        partials[((size_t)c * 2 + 1) * g.grid_y + yb] = b;
    }
}

// ---- finalize: one wave per channel, fp64 fixed-order combine -----------------
// Lane l sums slots l, l+64, ... in order; the DPP wave total then combines
// the lanes.  The loads (load) are separate from the sums (sum) so that an
// elementwise pass issues them together with its first loads of x: they
// arrive with that data instead of a memory round trip after it.  Lanes hold
// up to S slots in registers (grid_y <= 64*S); the rest are read in the sum.
// The elementwise prologues hold 2 (the one-round grid of every channel
// count of at least 16 at 2048 resident blocks; two rounds and fewer
// channels read the rest in batches), which keeps the fused dx pass within
// the 64 VGPRs of 8 waves per SIMD; the finalize kernels hold 4.
constexpr int kFinSlotsEw = 2;
constexpr int kFinSlotsKernel = 4;
// Slots per lane loaded together past the register-held ones
// (PartialSlots::sum): 4 in the elementwise prologues (8 would push the
// fused dx pass past 64 VGPRs), 8 in the finalize kernels.
constexpr int kFinBatchEw = 4;
constexpr int kFinBatchKernel = 8;
template <int S, int B>
struct PartialSlots {
    float a[S], b[S];

    // BUF: through buffer resources over the channel's two rows of slots, so
    // that a slot past grid_y reads 0 without a branch or a memory access and
    // the loads stay in flight with the caller's (byte offsets yb*4: the host
    // plan keeps grid_y*4 below 2^31 for this form).  Else plain loads.
    template <bool BUF>
    __device__ __forceinline__ void load(const float *__restrict__ partials, int grid_y, int C, int c)
    {
        const int lane = threadIdx.x & (kWave - 1);
        if constexpr (BUF) {
            const uint32_t span = (uint32_t)grid_y * 4u;
            const auto r0 = make_rsrc(partials + (size_t)c * 2 * grid_y, span);
            const auto r1 = make_rsrc(partials + ((size_t)c * 2 + 1) * grid_y, span);
#pragma unroll
            for (int k = 0; k < S; ++k) {
                const int yb = lane + k * kWave;
                const uint32_t off = yb < grid_y ? (uint32_t)yb * 4u : span;
                a[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r0, off, 0, 0));
                b[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r1, off, 0, 0));
            }
        } else {
#pragma unroll
            for (int k = 0; k < S; ++k) {
                const int yb = lane + k * kWave;
                a[k] = yb < grid_y ? partials[((size_t)c * 2 + 0) * grid_y + yb] : 0.f;
                b[k] = yb < grid_y ? partials[((size_t)c * 2 + 1) * grid_y + yb] : 0.f;
            }
        }
    }
    // Called by all 64 lanes of a wave (the wave total needs every lane).
    __device__ __forceinline__ void sum(const float *__restrict__ partials, int grid_y, int C, int c, double &s1,
                                        double &s2) const
    {
        const int lane = threadIdx.x & (kWave - 1);
        double x = 0.0, y = 0.0;
#pragma unroll
        for (int k = 0; k < S; ++k) {
            if (lane + k * kWave < grid_y) {
                x += (double)a[k];
                y += (double)b[k];
            }
        }
        // The rest in batches of B slots per lane, every load of a
        // batch in flight at once (one round trip per batch instead of per
        // slot): a slot past grid_y loads slot grid_y - 1 and adds 0, so no
        // branch separates the loads.  Each lane still adds its slots in
        // index order.
        for (int y0 = lane + S * kWave; y0 < grid_y; y0 += B * kWave) {
            float ra[B], rb[B];
#pragma unroll
            for (int j = 0; j < B; ++j) {
                const int yb = min(y0 + j * kWave, grid_y - 1);
                ra[j] = partials[((size_t)c * 2 + 0) * grid_y + yb];
                rb[j] = partials[((size_t)c * 2 + 1) * grid_y + yb];
            }
#pragma unroll
            for (int j = 0; j < B; ++j) {
                const bool live = y0 + j * kWave < grid_y;
                x += live ? (double)ra[j] : 0.0;
                y += live ? (double)rb[j] : 0.0;
            }
        }
        s1 = wave_total(x);
        s2 = wave_total(y);
    }
};

__device__ __forceinline__ void sum_partials(const float *__restrict__ partials, int grid_y, int C, int c,
                                             double &s1, double &s2)
{
    PartialSlots<kFinSlotsKernel, kFinBatchKernel> ps;
    ps.load<false>(partials, grid_y, C, c);
    ps.sum(partials, grid_y, C, c, s1, s2);
}

// Forward finalize of channel c from its shifted sums, every input given:
// gm = gamma[c] (or 1), rm / rv = the running statistics before the update
// (used only when write).  stats[4, C] = (mean, var, inv_std, scale) and the
// running statistics are written when `write` (one lane of the grid per
// channel).  Returns mean and scale for the caller's apply.
__device__ __forceinline__ void fwd_finalize_core(double S1, double S2, float K, int C, int c, int64_t M,
                                                  double gm, float rm, float rv, float *__restrict__ running_mean,
                                                  float *__restrict__ running_var, float momentum, float eps,
                                                  bool write, float *__restrict__ stats, float &mean_out,
                                                  float &scale_out)
{
    const double Md = (double)M;
    const double md = S1 / Md;                    // mean of the shifted values
    double var = S2 / Md - md * md;               // biased variance
    if (var < 0.0) var = 0.0;
    const double mean = (double)K + md;
    const double inv_std = 1.0 / sqrt(var + (double)eps);
    const float meanf = (float)mean, scalef = (float)(gm * inv_std);
    mean_out = meanf;
    scale_out = scalef;
    if (!write) return;
    stats[0 * C + c] = meanf;
    stats[1 * C + c] = (float)var;
    stats[2 * C + c] = (float)inv_std;
    stats[3 * C + c] = scalef;
    const double m = (double)momentum;
    if (running_mean) running_mean[c] = (float)((1.0 - m) * (double)rm + m * mean);
    if (running_var) running_var[c] = (float)((1.0 - m) * (double)rv + m * var * Md / (Md - 1.0));
}

// The same, reading gamma and the running statistics itself (called by one
// lane).
__device__ __forceinline__ void fwd_finalize_channel(double S1, double S2, float K, int C, int c,
                                                     int64_t M, const float *__restrict__ gamma,
                                                     float *__restrict__ running_mean,
                                                     float *__restrict__ running_var,
                                                     float momentum, float eps, bool write,
                                                     float *__restrict__ stats, float &mean_out,
                                                     float &scale_out)
{
    const double gm = gamma ? (double)gamma[c] : 1.0;
    const float rm = (write && running_mean) ? running_mean[c] : 0.f;
    const float rv = (write && running_var) ? running_var[c] : 0.f;
    fwd_finalize_core(S1, S2, K, C, c, M, gm, rm, rv, running_mean, running_var, momentum, eps, write, stats,
                      mean_out, scale_out);
}

// Backward finalize of channel c: grads[4, C] = (dgamma, dbeta, k1, k2)
// with k1 = -scale*inv_std^2*S/M, k2 = -scale*dbeta/M, from inv_std and
// scale (stats rows 2 and 3); grads written when `write`.
__device__ __forceinline__ void bwd_finalize_core(double Sdy, double Sdyxc, int C, int c, int64_t M,
                                                  double inv_std, double scale, bool write,
                                                  float *__restrict__ grads, float &k1_out, float &k2_out)
{
    const double Md = (double)M;
    const float k1 = (float)(-scale * inv_std * inv_std * Sdyxc / Md);
    const float k2 = (float)(-scale * Sdy / Md);
    k1_out = k1;
    k2_out = k2;
    if (!write) return;
    grads[0 * C + c] = (float)(inv_std * Sdyxc);  // dgamma
    grads[1 * C + c] = (float)Sdy;                // dbeta
    grads[2 * C + c] = k1;
    grads[3 * C + c] = k2;
}

// The same, reading inv_std and scale from stats (called by one lane).
__device__ __forceinline__ void bwd_finalize_channel(double Sdy, double Sdyxc, int C, int c, int64_t M,
                                                     const float *__restrict__ stats, bool write,
                                                     float *__restrict__ grads, float &k1_out,
                                                     float &k2_out)
{
    bwd_finalize_core(Sdy, Sdyxc, C, c, M, (double)stats[2 * C + c], (double)stats[3 * C + c], write, grads,
                      k1_out, k2_out);
}

__global__ void __launch_bounds__(kBnThreads)
bn_fwd_finalize(const float *__restrict__ partials, int grid_y, int C, int64_t M,
                const float *__restrict__ gamma,
                float *__restrict__ running_mean, float *__restrict__ running_var,
                float momentum, float eps, float *__restrict__ stats)
{
    const int c = blockIdx.x * (kBnThreads / kWave) + (int)threadIdx.x / kWave;
    if (c >= C) return;  // whole wave exits together
    double S1, S2;
    sum_partials(partials, grid_y, C, c, S1, S2);
    if ((threadIdx.x & (kWave - 1)) != 0) return;
    float mean, scale;
    fwd_finalize_channel(S1, S2, partials[(size_t)2 * grid_y * C + c], C, c, M, gamma, running_mean,
                         running_var, momentum, eps, true, stats, mean, scale);
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
    float k1, k2;
    bwd_finalize_channel(Sdy, Sdyxc, C, c, M, stats, true, grads, k1, k2);
}

// ---- elementwise passes ------------------------------------------------------
// FUSED: wave 0 of every block finalizes the block's channel from the
// partials (fixed order, the same arithmetic as the finalize kernels; lane 0
// of block yb == 0 writes stats/grads and the running statistics) and passes
// the two per-channel constants to the other waves through LDS.  All of the
// pass's per-channel inputs -- partial slots, shift, gamma, beta, stats,
// running statistics -- are vector loads issued right after the first loads
// of x, before any is used, so they arrive together with that data: the
// elementwise work starts one memory round trip after the launch, plus the
// fp64 arithmetic.  (Read in a second round trip, as the scalar loads of an
// earlier version were, they cost a round trip per pass.)  One wave per block
// does the fp64 work: with every wave doing it, the eight waves of a SIMD
// ran the same divisions and square roots one after the other, which
// measured 15-28% slower at (256,32,32,32).  This removes the finalize
// launch from the dependency chain at the cost of every block re-reading its
// channel's grid_y partials (L2 hits).
struct FwdFinalizeArgs {
    const float *partials;
    int red_grid_y;  // blocks per channel of the reduction that wrote the partials
    const float *gamma;
    float *running_mean, *running_var;
    float momentum, eps;
    int64_t M;
};

// Where the apply pass takes its per-channel (mean, scale) from.
enum : int {
    kApplyStats = 0,     // stats[4, C] written by a finalize kernel
    kApplyFinalize = 1,  // finalize the channel in the prologue (FUSED above)
    kApplyRunning = 2    // inference: running_mean, gamma/sqrt(running_var + eps)
};

template <typename T, int V, int SRC, int NT, int ACT>
__global__ void __launch_bounds__(kBnThreads, kBnWavesPerSimd)
bn_apply_kernel(const T *__restrict__ x, T *__restrict__ y, float *__restrict__ stats,
                const float *__restrict__ beta, BnGeom g, FwdFinalizeArgs f, float slope)
{
    const BnBlock blk = bn_block(g);
    const int c = blk.c, yb = blk.yb;
    // Unit indices are unsigned: a channel may hold up to 2^31 - 1 units,
    // and the loop index runs up to a step past the last one.
    const BnRange rg = bn_range(g, yb);
    const uint32_t u0 = rg.u0, u1 = rg.u1, step = rg.step;

    uint32_t base = u0 + threadIdx.x;
    Raw<T, V> v[kBnUnroll];
    int off[kBnUnroll];
#pragma unroll
    for (int k = 0; k < kBnUnroll; ++k) {
        const uint32_t u = base + k * kBnThreads;
        off[k] = bn_unit_offset<V>(g, c, u);
        if (u < u1) ldr<(NT & kNtEwLoads) != 0>(v[k], x + off[k]);
    }

    // The per-channel inputs, loaded together with the first units of x.
    // Every load is issued before any result is used (the scheduling barrier):
    // loads complete in issue order, so an early use of one would wait for the
    // loads of x as well, and the later loads would start a round trip after.
    const float b = ldv_if(beta, c, true);
    float mean, scale;
    if constexpr (SRC == kApplyFinalize) {
        __shared__ float sh[2];
        if (threadIdx.x < kWave) {  // wave 0
            PartialSlots<kFinSlotsEw, kFinBatchEw> ps;
            ps.load<true>(f.partials, f.red_grid_y, g.C, c);
            const float K = ldv(f.partials + (size_t)2 * f.red_grid_y * g.C + c);
            const float gv = ldv_if(f.gamma, c, true);
            const float rm = ldv_if(f.running_mean, c, yb == 0);
            const float rv = ldv_if(f.running_var, c, yb == 0);
            __builtin_amdgcn_sched_barrier(0);
            const double gm = f.gamma ? (double)gv : 1.0;
            double S1, S2;
            ps.sum(f.partials, f.red_grid_y, g.C, c, S1, S2);
            float m, sc;
            fwd_finalize_core(S1, S2, K, g.C, c, f.M, gm, rm, rv, f.running_mean, f.running_var, f.momentum,
                              f.eps, yb == 0 && threadIdx.x == 0, stats, m, sc);
            if (threadIdx.x == 0) {
                sh[0] = m;
                sh[1] = sc;
            }
        }
        __syncthreads();
        mean = sh[0];
        scale = sh[1];
    } else if constexpr (SRC == kApplyRunning) {
        const float p0 = ldv(f.running_mean + c);
        const float rv = ldv(f.running_var + c);
        const float gv = ldv_if(f.gamma, c, true);
        __builtin_amdgcn_sched_barrier(0);
        // Same rounding steps as the training finalize: inv_std in fp64,
        // scale rounded once to fp32.
        mean = p0;
        const double gm = f.gamma ? (double)gv : 1.0;
        const double inv_std = 1.0 / sqrt((double)rv + (double)f.eps);
        scale = (float)(gm * inv_std);
    } else {
        mean = ldv(stats + c);
        scale = ldv(stats + 3 * g.C + c);
    }

    for (;;) {
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const uint32_t u = base + k * kBnThreads;
            if (u < u1) {
                float o[V];
#pragma unroll
                for (int e = 0; e < V; ++e) o[e] = act_fwd<ACT>(fmaf(v[k].get(e) - mean, scale, b), slope);
                st<(NT & kNtStores) != 0, T, V>(y + off[k], o);
            }
        }
        base += step;
        if (base >= u1) break;
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const uint32_t u = base + k * kBnThreads;
            off[k] = bn_unit_offset<V>(g, c, u);
            if (u < u1) ldr<(NT & kNtEwLoads) != 0>(v[k], x + off[k]);
        }
    }
}

template <typename T, int V, bool FUSED, int NT, int ACT>
__global__ void __launch_bounds__(kBnThreads, kBnWavesPerSimd)
bn_dx_kernel(const T *__restrict__ dy, const T *__restrict__ x, T *__restrict__ dx,
             const float *__restrict__ stats, float *__restrict__ grads, BnGeom g,
             const float *__restrict__ partials, int red_grid_y, int64_t M,
             const float *__restrict__ beta, float slope)
{
    const BnBlock blk = bn_block(g);
    const int c = blk.c, yb = blk.yb;
    // Unit indices are unsigned: a channel may hold up to 2^31 - 1 units,
    // and the loop index runs up to a step past the last one.
    const BnRange rg = bn_range(g, yb);
    const uint32_t u0 = rg.u0, u1 = rg.u1, step = rg.step;

    // The unit offsets are recomputed for the stores rather than kept: held
    // from the loads to the stores they pushed the bf16 fused pass past the
    // 64 VGPRs of 8 waves per SIMD.
    uint32_t base = u0 + threadIdx.x;
    Raw<T, V> vx[kBnUnroll], vd[kBnUnroll];
#pragma unroll
    for (int k = 0; k < kBnUnroll; ++k) {
        const uint32_t u = base + k * kBnThreads;
        if (u < u1) {
            const int off = bn_unit_offset<V>(g, c, u);
            ldr<(NT & kNtEwLoads) != 0>(vx[k], x + off);
            ldr<(NT & kNtEwLoads) != 0>(vd[k], dy + off);
        }
    }

    // The per-channel inputs, loaded together with the first units of x, dy,
    // every one issued before any is used (as in bn_apply_kernel; wave 0
    // finalizes).
    const float mean = ldv(stats + c);
    const float scale = ldv(stats + 3 * g.C + c);
    const float b = ldv_if(beta, c, ACT != 0);
    float k1, k2;
    if constexpr (FUSED) {
        __shared__ float sh[2];
        if (threadIdx.x < kWave) {  // wave 0
            PartialSlots<kFinSlotsEw, kFinBatchEw> ps;
            ps.load<true>(partials, red_grid_y, g.C, c);
            const float inv_std = ldv(stats + 2 * g.C + c);
            __builtin_amdgcn_sched_barrier(0);
            double Sdy, Sdyxc;
            ps.sum(partials, red_grid_y, g.C, c, Sdy, Sdyxc);
            float a1, a2;
            bwd_finalize_core(Sdy, Sdyxc, g.C, c, M, (double)inv_std, (double)scale, yb == 0 && threadIdx.x == 0,
                              grads, a1, a2);
            if (threadIdx.x == 0) {
                sh[0] = a1;
                sh[1] = a2;
            }
        }
        __syncthreads();
        k1 = sh[0];
        k2 = sh[1];
    } else {
        k1 = ldv(grads + 2 * g.C + c);
        k2 = ldv(grads + 3 * g.C + c);
    }

    for (;;) {
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const uint32_t u = base + k * kBnThreads;
            if (u < u1) {
                float o[V];
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float xc = vx[k].get(e) - mean;
                    const float dz = act_bwd<ACT>(vd[k].get(e), fmaf(xc, scale, b), slope);
                    o[e] = fmaf(dz, scale, fmaf(xc, k1, k2));
                }
                st<(NT & kNtStores) != 0, T, V>(dx + bn_unit_offset<V>(g, c, u), o);
            }
        }
        base += step;
        if (base >= u1) break;
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const uint32_t u = base + k * kBnThreads;
            if (u < u1) {
                const int off = bn_unit_offset<V>(g, c, u);
                ldr<(NT & kNtEwLoads) != 0>(vx[k], x + off);
                ldr<(NT & kNtEwLoads) != 0>(vd[k], dy + off);
            }
        }
    }
}

// ---- small channels: one block per channel ------------------------------------
// When every channel has few units, one block takes a whole channel and the
// step needs no other block's partial sums: the block reduces (the same
// per-thread unrolled sums and block sum as bn_stats_kernel /
// bn_grad_sums_kernel with one block per channel), finalizes in its first
// thread (the same fp64 arithmetic), and runs the elementwise pass over the
// channel again, now from the caches.  One launch per direction instead of
// two; the results equal, bit for bit, those of the two-kernel path with one
// block per channel.  In place (y == x, dx == dy) is safe: the block reads
// the whole channel before it writes any of it, and each thread reads an
// element just before writing it.
template <typename T, int V, int NT, int ACT, int TB>
__global__ void __launch_bounds__(TB)
bn_fwd_channel_kernel(const T *__restrict__ x, T *__restrict__ y, float *__restrict__ stats,
                      const float *__restrict__ beta, BnGeom g, FwdFinalizeArgs f, float slope)
{
    const int c = blockIdx.x;
    const uint32_t u1 = (uint32_t)g.units;
    const float K = to_f32(x[c * g.HW]);
    float s1[kBnUnroll], s2[kBnUnroll];
#pragma unroll
    for (int k = 0; k < kBnUnroll; ++k) { s1[k] = 0.f; s2[k] = 0.f; }
    for (uint32_t base = threadIdx.x; base < u1; base += TB * kBnUnroll) {
        Raw<T, V> v[kBnUnroll];
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const uint32_t u = base + k * TB;
            if (u < u1) ldr<(NT & kNtReduceLoads) != 0>(v[k], x + bn_unit_offset<V>(g, c, u));
        }
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const uint32_t u = base + k * TB;
            if (u < u1) {
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float d = v[k].get(e) - K;
                    s1[k] += d;
                    s2[k] = fmaf(d, d, s2[k]);
                }
            }
        }
    }
    float a = s1[0], b = s2[0];
#pragma unroll
    for (int k = 1; k < kBnUnroll; ++k) { a += s1[k]; b += s2[k]; }
    block_sum2_tb<TB>(a, b);
    __shared__ float sh[2];
    if (threadIdx.x == 0)
        fwd_finalize_channel((double)a, (double)b, K, g.C, c, f.M, f.gamma, f.running_mean, f.running_var,
                             f.momentum, f.eps, true, stats, sh[0], sh[1]);
    __syncthreads();
    const float mean = sh[0], scale = sh[1];
    const float bc = beta ? beta[c] : 0.f;
    for (uint32_t base = threadIdx.x; base < u1; base += TB * kBnUnroll) {
        Raw<T, V> v[kBnUnroll];
        int off[kBnUnroll];
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const uint32_t u = base + k * TB;
            off[k] = bn_unit_offset<V>(g, c, u);
            if (u < u1) ldr<(NT & kNtEwLoads) != 0>(v[k], x + off[k]);
        }
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const uint32_t u = base + k * TB;
            if (u < u1) {
                float o[V];
#pragma unroll
                for (int e = 0; e < V; ++e) o[e] = act_fwd<ACT>(fmaf(v[k].get(e) - mean, scale, bc), slope);
                st<(NT & kNtStores) != 0, T, V>(y + off[k], o);
            }
        }
    }
}

template <typename T, int V, int NT, int ACT, int TB>
__global__ void __launch_bounds__(TB)
bn_bwd_channel_kernel(const T *__restrict__ dy, const T *__restrict__ x, T *__restrict__ dx,
                      const float *__restrict__ stats, float *__restrict__ grads,
                      const float *__restrict__ beta, float slope, BnGeom g, int64_t M)
{
    const int c = blockIdx.x;
    const uint32_t u1 = (uint32_t)g.units;
    const float mean = stats[c];
    const float scale = stats[3 * g.C + c];
    const float bz = (ACT != 0 && beta) ? beta[c] : 0.f;
    float s1[kBnUnroll], s2[kBnUnroll];
#pragma unroll
    for (int k = 0; k < kBnUnroll; ++k) { s1[k] = 0.f; s2[k] = 0.f; }
    for (uint32_t base = threadIdx.x; base < u1; base += TB * kBnUnroll) {
        Raw<T, V> vx[kBnUnroll], vd[kBnUnroll];
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const uint32_t u = base + k * TB;
            if (u < u1) {
                const int off = bn_unit_offset<V>(g, c, u);
                ldr<(NT & kNtReduceLoads) != 0>(vx[k], x + off);
                ldr<(NT & kNtReduceLoads) != 0>(vd[k], dy + off);
            }
        }
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const uint32_t u = base + k * TB;
            if (u < u1) {
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float xc = vx[k].get(e) - mean;
                    const float dz = act_bwd<ACT>(vd[k].get(e), fmaf(xc, ACT != 0 ? scale : 0.f, bz), slope);
                    s1[k] += dz;
                    s2[k] = fmaf(dz, xc, s2[k]);
                }
            }
        }
    }
    float a = s1[0], b = s2[0];
#pragma unroll
    for (int k = 1; k < kBnUnroll; ++k) { a += s1[k]; b += s2[k]; }
    block_sum2_tb<TB>(a, b);
    __shared__ float sh[2];
    if (threadIdx.x == 0) bwd_finalize_channel((double)a, (double)b, g.C, c, M, stats, true, grads, sh[0], sh[1]);
    __syncthreads();
    if (dx == nullptr) return;  // uniform: the caller skipped dx
    const float k1 = sh[0], k2 = sh[1];
    for (uint32_t base = threadIdx.x; base < u1; base += TB * kBnUnroll) {
        Raw<T, V> vx[kBnUnroll], vd[kBnUnroll];
        int off[kBnUnroll];
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const uint32_t u = base + k * TB;
            off[k] = bn_unit_offset<V>(g, c, u);
            if (u < u1) {
                ldr<(NT & kNtEwLoads) != 0>(vx[k], x + off[k]);
                ldr<(NT & kNtEwLoads) != 0>(vd[k], dy + off[k]);
            }
        }
#pragma unroll
        for (int k = 0; k < kBnUnroll; ++k) {
            const uint32_t u = base + k * TB;
            if (u < u1) {
                float o[V];
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float xc = vx[k].get(e) - mean;
                    const float dz = act_bwd<ACT>(vd[k].get(e), fmaf(xc, scale, bz), slope);
                    o[e] = fmaf(dz, scale, fmaf(xc, k1, k2));
                }
                st<(NT & kNtStores) != 0, T, V>(dx + off[k], o);
            }
        }
    }
}

// ---- small planes: the tensor as rows of L = C*HW columns ------------------------
// With small planes a channel's elements lie in short runs C*HW apart, and a
// block per channel reads scattered sectors.  Viewed as [N, L] (column j in
// channel j/HW) the per-channel sums are column sums over the rows, and
// every pass reads whole rows.  A block is 2^cl_log2 column lanes (each a
// group of V consecutive columns) by rl row lanes over one chunk of rows (the
// geometry and the block -> strip/chunk mapping: make_bn_col_geom,
// bn_col_work).  The reduction passes keep their columns' sums in registers
// and write partials[2, rb, L]; the finalize adds each column's rb chunk sums
// and then a channel's HW column sums, in fp64 in a fixed order, and
// finalizes with the arithmetic of the channel path; the elementwise passes load their columns'
// per-channel constants once and stream the rows.  The shift is
// K_c = x[0, c, 0, 0], as in bn_stats_kernel.

// Rows of a column lane in flight.
template <int V>
constexpr int bn_col_unroll() { return V == 8 ? 2 : 4; }

// A thread's place in the row layout: its column lane and row lane, its
// column group, and the rows [r0, r1) of its block's chunk.  Row lanes are
// not wave-uniform when a block has fewer than 64 column lanes.
struct BnColLane {
    int lane, rl, grp, chunk;
    int64_t r0, r1;
};
__device__ __forceinline__ BnColLane bn_col_lane(const BnColGeom &g)
{
    const BnColWork w = bn_col_work(g, (int)blockIdx.x);
    BnColLane c;
    c.lane = (int)threadIdx.x & ((1 << g.cl_log2) - 1);
    c.rl = (int)threadIdx.x >> g.cl_log2;
    c.grp = (w.strip << g.cl_log2) + c.lane;
    c.chunk = w.chunk;
    c.r0 = (int64_t)w.chunk * g.rpc;
    c.r1 = c.r0 + g.rpc < g.N ? c.r0 + g.rpc : g.N;
    return c;
}

// Column sums of the chunk for one column group: the row lanes' sums are
// added pairwise through LDS (for h = rl/2, ..., 1 row lane r < h adds row
// lane r + h), and row lane 0 writes the chunk's two partial rows.  (Adding
// the row lanes in order instead, behind one barrier, measured slower on
// MI355X: (65536, 256) bf16 fwd+bwd 65 -> 80 us.)
template <int V>
__device__ __forceinline__ void bn_col_write_partials(float (&s1)[V], float (&s2)[V], const BnColLane &c, bool ok,
                                                      int j0, const BnColGeom &g, float *__restrict__ partials)
{
    __shared__ float red[2 * V * kBnThreads];
    const int cl = 1 << g.cl_log2;
    auto slot = [&](int r, int q, int e) { return ((r * 2 + q) * V + e) * cl + c.lane; };
    for (int h = g.rl >> 1; h >= 1; h >>= 1) {
        if (c.rl >= h && c.rl < 2 * h)
#pragma unroll
            for (int e = 0; e < V; ++e) {
                red[slot(c.rl, 0, e)] = s1[e];
                red[slot(c.rl, 1, e)] = s2[e];
            }
        __syncthreads();
        if (c.rl < h)
#pragma unroll
            for (int e = 0; e < V; ++e) {
                s1[e] += red[slot(c.rl + h, 0, e)];
                s2[e] += red[slot(c.rl + h, 1, e)];
            }
    }
    if (c.rl != 0 || !ok) return;
    store_vec<float, V>(partials + (size_t)c.chunk * g.L + j0, s1);
    store_vec<float, V>(partials + ((size_t)g.rb + c.chunk) * g.L + j0, s2);
}

template <typename T, int V, int NT>
__global__ void __launch_bounds__(kBnThreads)
bn_col_stats_kernel(const T *__restrict__ x, BnColGeom g, float *__restrict__ partials)
{
    constexpr int U = bn_col_unroll<V>();
    const BnColLane c = bn_col_lane(g);
    const int RL = g.rl;
    const bool ok = c.grp < g.L / V;
    const int j0 = ok ? c.grp * V : 0;
    float K[V], s1[V], s2[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        K[e] = to_f32(x[g.div_hw.div((uint32_t)(j0 + e)) * (uint32_t)g.HW]);
        s1[e] = 0.f;
        s2[e] = 0.f;
    }
    if (ok) {
        int64_t r = c.r0 + c.rl;
        for (; r + (U - 1) * RL < c.r1; r += U * RL) {
            float v[U][V];
#pragma unroll
            for (int k = 0; k < U; ++k)
                ld<(NT & kNtReduceLoads) != 0, T, V>(x + (size_t)(r + k * RL) * g.L + j0, v[k]);
#pragma unroll
            for (int k = 0; k < U; ++k)
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float d = v[k][e] - K[e];
                    s1[e] += d;
                    s2[e] = fmaf(d, d, s2[e]);
                }
        }
        for (; r < c.r1; r += RL) {
            float v[V];
            ld<(NT & kNtReduceLoads) != 0, T, V>(x + (size_t)r * g.L + j0, v);
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const float d = v[e] - K[e];
                s1[e] += d;
                s2[e] = fmaf(d, d, s2[e]);
            }
        }
    }
    bn_col_write_partials<V>(s1, s2, c, ok, j0, g, partials);
}

// Finalize of the row layout.  A block of kBnColLanes x RF threads takes k =
// max(1, kBnColLanes / HW) whole channels, i.e. their k*HW consecutive
// columns, kBnColLanes columns at a time (one pass unless a forced row
// layout has planes of more than kBnColLanes elements), by RF row lanes: row
// lane r adds the chunk sums r, r + RF, ... of its column in fp64, reading
// rows of partials[2, rb, L] coalesced across the lanes.  The row lanes' sums
// meet in LDS in row-lane order, and thread t < k adds the column sums of
// channel c0 + t in column order.  RF = 16 for at least kBnColFinManyChunks
// chunks, else 4.
constexpr int kBnColFinManyChunks = 64;
__host__ __device__ inline int bn_col_fin_channels(const BnColGeom &g)
{
    return g.HW >= kBnColLanes ? 1 : kBnColLanes / g.HW;
}

// Planes of at least kBnColWaveFinalizeHW elements: a wave per channel (four
// channels per block) adds the channel's rb*HW chunk sums chunk-major, lane l
// taking l, l + 64, ... (runs of HW consecutive columns, read coalesced), and
// the butterfly combines the lanes.  RF = 0 selects this team.
constexpr int kBnColWaveFinalizeHW = 16;
__device__ __forceinline__ bool bn_col_wave_sums(const float *__restrict__ partials, const BnColGeom &g, int &c,
                                                 double &s1, double &s2)
{
    c = (int)blockIdx.x * (kBnThreads / kWave) + (int)threadIdx.x / kWave;
    if (c >= g.C) return false;  // a whole wave together; no barrier follows
    const int lane = (int)threadIdx.x & (kWave - 1);
    const int n = g.rb * g.HW;
    double a = 0.0, b = 0.0;
    for (int i = lane; i < n; i += kWave) {
        const int rbi = (int)g.div_hw.div((uint32_t)i);
        const size_t col = (size_t)c * g.HW + (i - rbi * g.HW);
        a += (double)partials[(size_t)rbi * g.L + col];
        b += (double)partials[((size_t)g.rb + rbi) * g.L + col];
    }
    s1 = wave_sum(a);
    s2 = wave_sum(b);
    return lane == 0;
}

// Returns false for the threads that hold no channel; the others get their
// channel c and its two sums.  Every thread passes every barrier.
template <int RF>
__device__ __forceinline__ bool bn_col_channel_sums(const float *__restrict__ partials, const BnColGeom &g, int &c,
                                                    double &s1, double &s2)
{
    constexpr int kBnColFinRows = RF;
    __shared__ double red[2][kBnColFinRows][kBnColLanes];
    const int k = bn_col_fin_channels(g);
    const int c0 = (int)blockIdx.x * k;
    const int kc = g.C - c0 < k ? g.C - c0 : k;
    const int ncol = kc * g.HW;
    const int lane = (int)threadIdx.x & (kBnColLanes - 1);
    const int rf = (int)threadIdx.x / kBnColLanes;
    const int t = (int)threadIdx.x;
    s1 = 0.0;
    s2 = 0.0;
    for (int cb = 0; cb < ncol; cb += kBnColLanes) {
        const int col = cb + lane;
        double a = 0.0, b = 0.0;
        if (col < ncol) {
            const float *p1 = partials + (size_t)c0 * g.HW + col;
            const float *p2 = p1 + (size_t)g.rb * g.L;
            int r = rf;
            for (; r + 3 * kBnColFinRows < g.rb; r += 4 * kBnColFinRows) {
                float u[4], v[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    u[i] = p1[(size_t)(r + i * kBnColFinRows) * g.L];
                    v[i] = p2[(size_t)(r + i * kBnColFinRows) * g.L];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    a += (double)u[i];
                    b += (double)v[i];
                }
            }
            for (; r < g.rb; r += kBnColFinRows) {
                a += (double)p1[(size_t)r * g.L];
                b += (double)p2[(size_t)r * g.L];
            }
        }
        red[0][rf][lane] = a;
        red[1][rf][lane] = b;
        __syncthreads();
        if (rf == 0 && col < ncol) {
            for (int r = 1; r < kBnColFinRows; ++r) {
                a += red[0][r][lane];
                b += red[1][r][lane];
            }
            red[0][0][lane] = a;
            red[1][0][lane] = b;
        }
        __syncthreads();
        if (t < kc) {
            const int h0 = t * g.HW > cb ? t * g.HW : cb;
            const int h1 = (t + 1) * g.HW < cb + kBnColLanes ? (t + 1) * g.HW : cb + kBnColLanes;
            for (int h = h0; h < h1; ++h) {
                s1 += red[0][0][h - cb];
                s2 += red[1][0][h - cb];
            }
        }
        __syncthreads();
    }
    c = c0 + t;
    return t < kc;
}

template <typename T, int RF>
__global__ void __launch_bounds__(RF == 0 ? kBnThreads : kBnColLanes * RF)
bn_col_fwd_finalize(const float *__restrict__ partials, const T *__restrict__ x, BnColGeom g,
                    const float *__restrict__ gamma, float *__restrict__ running_mean,
                    float *__restrict__ running_var, float momentum, float eps, float *__restrict__ stats)
{
    int c;
    double S1, S2;
    if constexpr (RF == 0) {
        if (!bn_col_wave_sums(partials, g, c, S1, S2)) return;
    } else {
        if (!bn_col_channel_sums<RF>(partials, g, c, S1, S2)) return;
    }
    float mean, scale;
    fwd_finalize_channel(S1, S2, to_f32(x[(size_t)c * g.HW]), g.C, c, (int64_t)g.N * g.HW, gamma,
                         running_mean, running_var, momentum, eps, true, stats, mean, scale);
}

// Per-column constants of the elementwise passes.
template <int V>
__device__ __forceinline__ void bn_col_channels(const BnColGeom &g, int j0, int (&ch)[V])
{
#pragma unroll
    for (int e = 0; e < V; ++e) ch[e] = (int)g.div_hw.div((uint32_t)(j0 + e));
}

template <typename T, int V, int SRC, int NT, int ACT>
__global__ void __launch_bounds__(kBnThreads)
bn_col_apply_kernel(const T *__restrict__ x, T *__restrict__ y, const float *__restrict__ stats,
                    const float *__restrict__ beta, BnColGeom g, FwdFinalizeArgs f, float slope)
{
    constexpr int U = bn_col_unroll<V>();
    const BnColLane c = bn_col_lane(g);
    const int RL = g.rl;
    if (c.grp >= g.L / V) return;
    const int j0 = c.grp * V;
    int ch[V];
    bn_col_channels<V>(g, j0, ch);
    float mean[V], scale[V], b[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        const int cc = ch[e];
        if constexpr (SRC == kApplyRunning) {
            // as bn_apply_kernel: inv_std in fp64, scale rounded once to fp32
            mean[e] = f.running_mean[cc];
            const double inv_std = 1.0 / sqrt((double)f.running_var[cc] + (double)f.eps);
            scale[e] = (float)((f.gamma ? (double)f.gamma[cc] : 1.0) * inv_std);
        } else {
            mean[e] = stats[cc];
            scale[e] = stats[3 * g.C + cc];
        }
        b[e] = beta ? beta[cc] : 0.f;
    }
    auto out = [&](int64_t r, const float (&v)[V]) {
        float o[V];
#pragma unroll
        for (int e = 0; e < V; ++e) o[e] = act_fwd<ACT>(fmaf(v[e] - mean[e], scale[e], b[e]), slope);
        st<(NT & kNtStores) != 0, T, V>(y + (size_t)r * g.L + j0, o);
    };
    int64_t r = c.r0 + c.rl;
    for (; r + (U - 1) * RL < c.r1; r += U * RL) {
        float v[U][V];
#pragma unroll
        for (int k = 0; k < U; ++k)
            ld<(NT & kNtEwLoads) != 0, T, V>(x + (size_t)(r + k * RL) * g.L + j0, v[k]);
#pragma unroll
        for (int k = 0; k < U; ++k) out(r + k * RL, v[k]);
    }
    for (; r < c.r1; r += RL) {
        float v[V];
        ld<(NT & kNtEwLoads) != 0, T, V>(x + (size_t)r * g.L + j0, v);
        out(r, v);
    }
}

template <typename T, int V, int NT, int ACT>
__global__ void __launch_bounds__(kBnThreads)
bn_col_grad_sums_kernel(const T *__restrict__ dy, const T *__restrict__ x, const float *__restrict__ stats,
                        const float *__restrict__ beta, float slope, BnColGeom g, float *__restrict__ partials)
{
    constexpr int U = bn_col_unroll<V>();
    const BnColLane c = bn_col_lane(g);
    const int RL = g.rl;
    const bool ok = c.grp < g.L / V;
    const int j0 = ok ? c.grp * V : 0;
    int ch[V];
    bn_col_channels<V>(g, j0, ch);
    float mean[V], scale[V], bz[V], s1[V], s2[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        mean[e] = stats[ch[e]];
        scale[e] = ACT != 0 ? stats[3 * g.C + ch[e]] : 0.f;
        bz[e] = (ACT != 0 && beta) ? beta[ch[e]] : 0.f;
        s1[e] = 0.f;
        s2[e] = 0.f;
    }
    auto add = [&](const float (&vx)[V], const float (&vd)[V]) {
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const float xc = vx[e] - mean[e];
            const float dz = act_bwd<ACT>(vd[e], fmaf(xc, scale[e], bz[e]), slope);
            s1[e] += dz;
            s2[e] = fmaf(dz, xc, s2[e]);
        }
    };
    if (ok) {
        int64_t r = c.r0 + c.rl;
        for (; r + (U - 1) * RL < c.r1; r += U * RL) {
            float vx[U][V], vd[U][V];
#pragma unroll
            for (int k = 0; k < U; ++k) {
                const size_t off = (size_t)(r + k * RL) * g.L + j0;
                ld<(NT & kNtReduceLoads) != 0, T, V>(x + off, vx[k]);
                ld<(NT & kNtReduceLoads) != 0, T, V>(dy + off, vd[k]);
            }
#pragma unroll
            for (int k = 0; k < U; ++k) add(vx[k], vd[k]);
        }
        for (; r < c.r1; r += RL) {
            float vx[V], vd[V];
            ld<(NT & kNtReduceLoads) != 0, T, V>(x + (size_t)r * g.L + j0, vx);
            ld<(NT & kNtReduceLoads) != 0, T, V>(dy + (size_t)r * g.L + j0, vd);
            add(vx, vd);
        }
    }
    bn_col_write_partials<V>(s1, s2, c, ok, j0, g, partials);
}

template <int RF>
__global__ void __launch_bounds__(RF == 0 ? kBnThreads : kBnColLanes * RF)
bn_col_bwd_finalize(const float *__restrict__ partials, BnColGeom g, const float *__restrict__ stats,
                    float *__restrict__ grads)
{
    int c;
    double Sdy, Sdyxc;
    if constexpr (RF == 0) {
        if (!bn_col_wave_sums(partials, g, c, Sdy, Sdyxc)) return;
    } else {
        if (!bn_col_channel_sums<RF>(partials, g, c, Sdy, Sdyxc)) return;
    }
    float k1, k2;
    bwd_finalize_channel(Sdy, Sdyxc, g.C, c, (int64_t)g.N * g.HW, stats, true, grads, k1, k2);
}

template <typename T, int V, int NT, int ACT>
__global__ void __launch_bounds__(kBnThreads)
bn_col_dx_kernel(const T *__restrict__ dy, const T *__restrict__ x, T *__restrict__ dx,
                 const float *__restrict__ stats, const float *__restrict__ grads,
                 const float *__restrict__ beta, float slope, BnColGeom g)
{
    constexpr int U = bn_col_unroll<V>();
    const BnColLane c = bn_col_lane(g);
    const int RL = g.rl;
    if (c.grp >= g.L / V) return;
    const int j0 = c.grp * V;
    int ch[V];
    bn_col_channels<V>(g, j0, ch);
    float mean[V], scale[V], b[V], k1[V], k2[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        const int cc = ch[e];
        mean[e] = stats[cc];
        scale[e] = stats[3 * g.C + cc];
        b[e] = (ACT != 0 && beta) ? beta[cc] : 0.f;
        k1[e] = grads[2 * g.C + cc];
        k2[e] = grads[3 * g.C + cc];
    }
    auto out = [&](int64_t r, const float (&vx)[V], const float (&vd)[V]) {
        float o[V];
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const float xc = vx[e] - mean[e];
            const float dz = act_bwd<ACT>(vd[e], fmaf(xc, scale[e], b[e]), slope);
            o[e] = fmaf(dz, scale[e], fmaf(xc, k1[e], k2[e]));
        }
        st<(NT & kNtStores) != 0, T, V>(dx + (size_t)r * g.L + j0, o);
    };
    int64_t r = c.r0 + c.rl;
    for (; r + (U - 1) * RL < c.r1; r += U * RL) {
        float vx[U][V], vd[U][V];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const size_t off = (size_t)(r + k * RL) * g.L + j0;
            ld<(NT & kNtEwLoads) != 0, T, V>(x + off, vx[k]);
            ld<(NT & kNtEwLoads) != 0, T, V>(dy + off, vd[k]);
        }
#pragma unroll
        for (int k = 0; k < U; ++k) out(r + k * RL, vx[k], vd[k]);
    }
    for (; r < c.r1; r += RL) {
        float vx[V], vd[V];
        ld<(NT & kNtEwLoads) != 0, T, V>(x + (size_t)r * g.L + j0, vx);
        ld<(NT & kNtEwLoads) != 0, T, V>(dy + (size_t)r * g.L + j0, vd);
        out(r, vx, vd);
    }
}

template <typename T, int V, int ACT>
static hipError_t bn_col_forward_t(const BnCall &a, hipStream_t s)
{
    const BnColGeom &g = a.colg;
    const T *x = static_cast<const T *>(a.x);
    const dim3 grid((unsigned)(g.strips * g.rb)), block(kBnThreads);
    FwdFinalizeArgs f{a.partials, 1, a.gamma, a.running_mean, a.running_var, a.momentum, a.eps,
                      (int64_t)a.N * a.HW};
    if (a.inference)
        return launch(NH_K_BN_INFER, bn_col_apply_kernel<T, V, kApplyRunning, kBnNtPolicy, ACT>, grid, block, 0,
                      s, x, static_cast<T *>(a.out), a.stats, a.beta, g, f, a.slope);
    hipError_t e = hipSuccess;
    if (a.stage != 2) {
        e = launch(NH_K_BN_STATS, bn_col_stats_kernel<T, V, kBnNtPolicy>, grid, block, 0, s, x, g, a.partials);
        if (e != hipSuccess || a.stage == 1) return e;
    }
    const dim3 fgrid((unsigned)ceil_div(a.C, bn_col_fin_channels(g)));
    if (g.HW >= kBnColWaveFinalizeHW)
        e = launch(NH_K_BN_FWD_FINALIZE, bn_col_fwd_finalize<T, 0>, dim3((unsigned)ceil_div(a.C, kBnThreads / kWave)),
                   block, 0, s, (const float *)a.partials, x, g, a.gamma, a.running_mean, a.running_var, a.momentum,
                   a.eps, a.stats);
    else if (g.rb >= kBnColFinManyChunks)
        e = launch(NH_K_BN_FWD_FINALIZE, bn_col_fwd_finalize<T, 16>, fgrid, dim3(kBnColLanes * 16), 0, s,
                   (const float *)a.partials, x, g, a.gamma, a.running_mean, a.running_var, a.momentum, a.eps,
                   a.stats);
    else
        e = launch(NH_K_BN_FWD_FINALIZE, bn_col_fwd_finalize<T, 4>, fgrid, dim3(kBnColLanes * 4), 0, s,
                   (const float *)a.partials, x, g, a.gamma, a.running_mean, a.running_var, a.momentum, a.eps,
                   a.stats);
    if (e != hipSuccess) return e;
    return launch(NH_K_BN_APPLY, bn_col_apply_kernel<T, V, kApplyStats, kBnNtPolicy, ACT>, grid, block, 0, s, x,
                  static_cast<T *>(a.out), a.stats, a.beta, g, f, a.slope);
}

template <typename T, int V, int ACT>
static hipError_t bn_col_backward_t(const BnCall &a, hipStream_t s)
{
    const BnColGeom &g = a.colg;
    const T *x = static_cast<const T *>(a.x);
    const T *dy = static_cast<const T *>(a.dy);
    const dim3 grid((unsigned)(g.strips * g.rb)), block(kBnThreads);
    hipError_t e = hipSuccess;
    if (a.stage != 2) {
        e = launch(NH_K_BN_GRAD_SUMS, bn_col_grad_sums_kernel<T, V, kBnNtPolicy, ACT>, grid, block, 0, s, dy, x,
                   a.stats, a.beta, a.slope, g, a.partials);
        if (e != hipSuccess || a.stage == 1) return e;
    }
    const dim3 fgrid((unsigned)ceil_div(a.C, bn_col_fin_channels(g)));
    if (g.HW >= kBnColWaveFinalizeHW)
        e = launch(NH_K_BN_BWD_FINALIZE, bn_col_bwd_finalize<0>, dim3((unsigned)ceil_div(a.C, kBnThreads / kWave)),
                   block, 0, s, (const float *)a.partials, g, a.stats, a.grads);
    else if (g.rb >= kBnColFinManyChunks)
        e = launch(NH_K_BN_BWD_FINALIZE, bn_col_bwd_finalize<16>, fgrid, dim3(kBnColLanes * 16), 0, s,
                   (const float *)a.partials, g, a.stats, a.grads);
    else
        e = launch(NH_K_BN_BWD_FINALIZE, bn_col_bwd_finalize<4>, fgrid, dim3(kBnColLanes * 4), 0, s,
                   (const float *)a.partials, g, a.stats, a.grads);
    if (e != hipSuccess || a.out == nullptr) return e;
    return launch(NH_K_BN_DX, bn_col_dx_kernel<T, V, kBnNtPolicy, ACT>, grid, block, 0, s, dy, x,
                  static_cast<T *>(a.out), a.stats, a.grads, a.beta, a.slope, g);
}

// ---- host launchers -----------------------------------------------------------
// The reductions run on a.grid_y blocks per channel, the elementwise passes on
// a.ew_grid_y: the elementwise prologue reads the reduction's partial slots,
// whatever its own split.
template <typename T, int V, int ACT>
static hipError_t bn_forward_t(const BnCall &a, hipStream_t s)
{
    const BnGeom gr = make_bn_geom(a.N, a.C, a.HW, a.vec, a.grid_y, a.chan_fast, a.ilv);
    const BnGeom ge = make_bn_geom(a.N, a.C, a.HW, a.vec, a.ew_grid_y, a.chan_fast, a.ilv);
    const T *x = static_cast<const T *>(a.x);
    const dim3 rgrid((unsigned)(a.C * a.grid_y)), egrid((unsigned)(a.C * a.ew_grid_y)), block(kBnThreads);
    const int64_t M = (int64_t)a.N * a.HW;
    FwdFinalizeArgs f{a.partials, a.grid_y, a.gamma, a.running_mean, a.running_var, a.momentum, a.eps, M};
    if (a.inference)
        return launch(NH_K_BN_INFER, bn_apply_kernel<T, V, kApplyRunning, kBnNtPolicy, ACT>, egrid, block,
                      0, s, x, static_cast<T *>(a.out), a.stats, a.beta, ge, f, a.slope);
    if (a.channel_fused) {
        // one kernel per direction: it runs as the second stage
        if (a.stage == 1) return hipSuccess;
        const BnGeom g1 = make_bn_geom(a.N, a.C, a.HW, a.vec, 1, 0, 0);
        if (a.channel_threads == kBnChannelBigBlock)
            return launch(NH_K_BN_FWD_CHANNEL, bn_fwd_channel_kernel<T, V, kBnNtPolicy, ACT, kBnChannelBigBlock>,
                          dim3((unsigned)a.C), dim3(kBnChannelBigBlock), 0, s, x, static_cast<T *>(a.out),
                          a.stats, a.beta, g1, f, a.slope);
        return launch(NH_K_BN_FWD_CHANNEL, bn_fwd_channel_kernel<T, V, kBnNtPolicy, ACT, kBnThreads>,
                      dim3((unsigned)a.C), block, 0, s, x, static_cast<T *>(a.out), a.stats, a.beta, g1, f,
                      a.slope);
    }
    hipError_t e = hipSuccess;
    if (a.stage != 2) {
        e = launch(NH_K_BN_STATS, bn_stats_kernel<T, V, kBnNtPolicy>, rgrid, block, 0, s, x, gr, a.partials);
        if (e != hipSuccess || a.stage == 1) return e;
    }
    if (a.separate_finalize) {
        const dim3 fgrid((unsigned)ceil_div(a.C, kBnThreads / kWave));
        e = launch(NH_K_BN_FWD_FINALIZE, bn_fwd_finalize, fgrid, block, 0, s, a.partials,
                   a.grid_y, a.C, M, a.gamma, a.running_mean, a.running_var, a.momentum,
                   a.eps, a.stats);
        if (e != hipSuccess) return e;
        return launch(NH_K_BN_APPLY, bn_apply_kernel<T, V, kApplyStats, kBnNtPolicy, ACT>, egrid, block, 0,
                      s, x, static_cast<T *>(a.out), a.stats, a.beta, ge, f, a.slope);
    }
    return launch(NH_K_BN_APPLY, bn_apply_kernel<T, V, kApplyFinalize, kBnNtPolicy, ACT>, egrid, block, 0,
                  s, x, static_cast<T *>(a.out), a.stats, a.beta, ge, f, a.slope);
}

template <typename T, int V, int ACT>
static hipError_t bn_backward_t(const BnCall &a, hipStream_t s)
{
    const BnGeom gr = make_bn_geom(a.N, a.C, a.HW, a.vec, a.grid_y, a.chan_fast, a.ilv);
    const BnGeom ge = make_bn_geom(a.N, a.C, a.HW, a.vec, a.ew_grid_y, a.chan_fast, a.ilv);
    const T *x = static_cast<const T *>(a.x);
    const T *dy = static_cast<const T *>(a.dy);
    const dim3 rgrid((unsigned)(a.C * a.grid_y)), egrid((unsigned)(a.C * a.ew_grid_y)), block(kBnThreads);
    const int64_t M = (int64_t)a.N * a.HW;
    if (a.channel_fused) {
        if (a.stage == 1) return hipSuccess;
        const BnGeom g1 = make_bn_geom(a.N, a.C, a.HW, a.vec, 1, 0, 0);
        if (a.channel_threads == kBnChannelBigBlock)
            return launch(NH_K_BN_BWD_CHANNEL, bn_bwd_channel_kernel<T, V, kBnNtPolicy, ACT, kBnChannelBigBlock>,
                          dim3((unsigned)a.C), dim3(kBnChannelBigBlock), 0, s, dy, x, static_cast<T *>(a.out),
                          a.stats, a.grads, a.beta, a.slope, g1, M);
        return launch(NH_K_BN_BWD_CHANNEL, bn_bwd_channel_kernel<T, V, kBnNtPolicy, ACT, kBnThreads>,
                      dim3((unsigned)a.C), block, 0, s, dy, x, static_cast<T *>(a.out), a.stats, a.grads, a.beta,
                      a.slope, g1, M);
    }
    hipError_t e = hipSuccess;
    if (a.stage != 2) {
        e = launch(NH_K_BN_GRAD_SUMS, bn_grad_sums_kernel<T, V, kBnNtPolicy, ACT>, rgrid, block, 0, s, dy, x,
                   a.stats, a.beta, a.slope, gr, a.partials);
        if (e != hipSuccess || a.stage == 1) return e;
    }
    if (a.separate_finalize || a.out == nullptr) {
        const dim3 fgrid((unsigned)ceil_div(a.C, kBnThreads / kWave));
        e = launch(NH_K_BN_BWD_FINALIZE, bn_bwd_finalize, fgrid, block, 0, s, a.partials, a.grid_y,
                   a.C, M, a.stats, a.grads);
        if (e != hipSuccess || a.out == nullptr) return e;
        return launch(NH_K_BN_DX, bn_dx_kernel<T, V, false, kBnNtPolicy, ACT>, egrid, block, 0, s, dy, x,
                      static_cast<T *>(a.out), a.stats, a.grads, ge, a.partials, a.grid_y, M, a.beta,
                      a.slope);
    }
    return launch(NH_K_BN_DX, bn_dx_kernel<T, V, true, kBnNtPolicy, ACT>, egrid, block, 0, s, dy, x,
                  static_cast<T *>(a.out), a.stats, a.grads, ge, a.partials, a.grid_y, M, a.beta, a.slope);
}

// Unit widths: fp32 4 or 1 elements; bf16 8, 4 (8-byte units for planes of
// 4k elements) or 1.
template <int ACT>
static hipError_t bn_forward_act(const BnCall &a, hipStream_t s)
{
    if (a.col) {
        if (a.io == 0) return a.vec == 4 ? bn_col_forward_t<float, 4, ACT>(a, s) : bn_col_forward_t<float, 1, ACT>(a, s);
        if (a.vec == 8) return bn_col_forward_t<uint16_t, 8, ACT>(a, s);
        if (a.vec == 4) return bn_col_forward_t<uint16_t, 4, ACT>(a, s);
        return bn_col_forward_t<uint16_t, 1, ACT>(a, s);
    }
    if (a.io == 0) return a.vec == 4 ? bn_forward_t<float, 4, ACT>(a, s) : bn_forward_t<float, 1, ACT>(a, s);
    if (a.vec == 8) return bn_forward_t<uint16_t, 8, ACT>(a, s);
    if (a.vec == 4) return bn_forward_t<uint16_t, 4, ACT>(a, s);
    return bn_forward_t<uint16_t, 1, ACT>(a, s);
}

template <int ACT>
static hipError_t bn_backward_act(const BnCall &a, hipStream_t s)
{
    if (a.col) {
        if (a.io == 0) return a.vec == 4 ? bn_col_backward_t<float, 4, ACT>(a, s) : bn_col_backward_t<float, 1, ACT>(a, s);
        if (a.vec == 8) return bn_col_backward_t<uint16_t, 8, ACT>(a, s);
        if (a.vec == 4) return bn_col_backward_t<uint16_t, 4, ACT>(a, s);
        return bn_col_backward_t<uint16_t, 1, ACT>(a, s);
    }
    if (a.io == 0) return a.vec == 4 ? bn_backward_t<float, 4, ACT>(a, s) : bn_backward_t<float, 1, ACT>(a, s);
    if (a.vec == 8) return bn_backward_t<uint16_t, 8, ACT>(a, s);
    if (a.vec == 4) return bn_backward_t<uint16_t, 4, ACT>(a, s);
    return bn_backward_t<uint16_t, 1, ACT>(a, s);
}

hipError_t bn_forward_launch(const BnCall &a, hipStream_t s)
{
    switch (a.act) {
    case 0: return bn_forward_act<0>(a, s);
    case 1: return bn_forward_act<1>(a, s);
    case 2: return bn_forward_act<2>(a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t bn_backward_launch(const BnCall &a, hipStream_t s)
{
    switch (a.act) {
    case 0: return bn_backward_act<0>(a, s);
    case 1: return bn_backward_act<1>(a, s);
    case 2: return bn_backward_act<2>(a, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace nh
