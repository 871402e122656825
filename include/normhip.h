/*
 * normhip: training-mode normalization forward/backward for AMD Instinct
 * MI355X (gfx950), as a C ABI over hand-written HIP kernels.
 *
 * Operations (and the pages that define them):
 *   bn_forward_train    BatchNorm2d training forward.  Aether-ML PR #18,
 *                       "perf(batchnorm): device-sized grid, one-pass
 *                       statistics, finalize kernels": "One-pass statistics"
 *                       section and the stats / bn_forward_finalize /
 *                       _bn_apply_ew commit.
 *   bn_backward         BatchNorm2d training backward.  Same PR, "Backward
 *                       finalize" section and the bn_backward_finalize commit.
 *   bn_act_forward_train, bn_act_backward, bn_forward_infer
 *                       BatchNorm2d fused with ReLU/LeakyReLU (the same PR's
 *                       "Follow-ups") and inference through the shared apply
 *                       (its _bn_apply_ew commit).
 *   layernorm_backward  LayerNorm backward over the last dimension with saved
 *                       mean/rstd.  NVIDIA/Fuser issue #1473, "Why is
 *                       LayerNorm Backward Segmenting?", the layer_norm
 *                       backward definition (nvfuser_fusion_id14).
 *   bda_layernorm_backward
 *                       Backward of bias + dropout + add + LayerNorm.  Same
 *                       issue, its one-kernel fusion example
 *                       (nvfuser_fusion_id9).
 *   rmsnorm_backward    RMSNorm backward over the last dimension.
 *                       NVIDIA/Fuser issue #3629, "Performance gap between
 *                       manual nvfuser definition and thunder.jit for
 *                       rmsnorm": rmsnorm_prims and rmsnorm_bwd_fusion.
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers to contiguous row-major buffers on
 *     the current HIP device (hipGetDevice at call time).  `stream` is a
 *     hipStream_t of that device passed as void* (NULL = the null stream).
 *   - The caller owns every buffer, including the workspace: query its size
 *     with the matching *_workspace function, allocate it, pass it in.  The
 *     library never allocates, frees or synchronizes device memory in these
 *     calls.  Workspace needs no initialisation: every slot is written before
 *     it is read.
 *   - Calls are asynchronous on `stream`.  Results are bit-identical across
 *     runs for the same inputs, shape, device and build (no atomics; every
 *     reduction has a fixed order).
 *   - In-place is allowed for y == x (forward) and dx == dy (backward); any
 *     other overlap between outputs and inputs is undefined.
 *   - Validation happens before any launch.  On an error nothing is written
 *     and the running statistics are untouched.  Order of checks: dtype,
 *     shape, empty (a tensor with zero elements returns NH_OK and launches
 *     nothing; its pointers may be NULL), pointers, argument values,
 *     workspace.
 *   - Element counts must be below 2^31 (32-bit index arithmetic on device).
 *   - Misaligned pointers (not 16-byte aligned) and sizes that are not a
 *     multiple of the vector width are accepted; they take a scalar path.
 *   - Arithmetic: inputs are widened to fp32 at load, every reduction
 *     accumulates in fp32 per thread and combines block partials in fp64,
 *     outputs are rounded to their storage type at store (bf16: round to
 *     nearest even).
 */
#ifndef NORMHIP_H
#define NORMHIP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums a caller passes in carry two range markers that are not valid
 * values: they make every int value representable in the enum type, so an
 * out-of-range value reaches the library's validation as a well-defined
 * value and is rejected there (C++ gives an enum without them only the
 * range of its enumerators' bits). */
typedef enum {
    NH_F32 = 0,  /* IEEE binary32 */
    NH_BF16 = 1, /* bfloat16, stored as uint16 bit patterns */
    NH_DTYPE_RANGE_MIN_ = -0x7fffffff - 1, /* range markers, not dtypes */
    NH_DTYPE_RANGE_MAX_ = 0x7fffffff
} nh_dtype;

typedef enum {
    NH_OK = 0,
    NH_ERR_NULL = 1,      /* a required pointer is NULL */
    NH_ERR_SHAPE = 2,     /* negative size, element count >= 2^31, or one element
                             per channel with running statistics requested */
    NH_ERR_DTYPE = 3,     /* dtype value not in nh_dtype, or an unsupported mix */
    NH_ERR_WORKSPACE = 4, /* workspace NULL or smaller than the queried size */
    NH_ERR_HIP = 5,       /* HIP runtime error (no device, launch failure) */
    NH_ERR_ARG = 6        /* invalid scalar argument (eps < 0 or NaN, bad id) */
} nh_status;

/* Static string naming a status code ("NH_OK", ...); never NULL. */
const char *nh_status_string(int status);

/* Detail message of the last failing call on this host thread ("" if none). */
const char *nh_last_error(void);

/* ------------------------------------------------------------------------
 * BatchNorm2d, NCHW, statistics per channel over (N, H, W); HW = H*W,
 * M = N*HW elements per channel.  A channels-last (NHWC) tensor, and
 * BatchNorm over [N, C], is the case HW = 1 with N*H*W (or N) rows of C
 * channels: pass it as N' = N*H*W, C, HW = 1.
 * ---------------------------------------------------------------------- */

/* Workspace bytes needed by bn_forward_train / bn_backward for this shape on
 * the current device (the same size serves both calls and both dtypes). */
nh_status bn_forward_train_workspace(int64_t N, int64_t C, int64_t HW, size_t *ws_bytes);
nh_status bn_backward_workspace(int64_t N, int64_t C, int64_t HW, size_t *ws_bytes);

/*
 * Training forward.  Aether-ML PR #18, "One-pass statistics": per channel c
 * the shifted sums of d = x - x[0,c,0,0] and d^2 give
 *   mean = x[0,c,0,0] + sum d / M,  var = sum d^2 / M - (sum d / M)^2 (biased,
 *   clamped at 0),  inv_std = 1/sqrt(var + eps),  scale = gamma*inv_std,
 * and y = (x - mean)*scale + beta (the centred apply of that PR).
 *
 *   x, y          [N, C, HW] of dtype io (y may equal x)
 *   gamma, beta   fp32 [C]; NULL means gamma = 1 / beta = 0 (affine off)
 *   running_mean, running_var
 *                 fp32 [C], updated in place when non-NULL:
 *                 rm = (1-momentum)*rm + momentum*mean,
 *                 rv = (1-momentum)*rv + momentum*var*M/(M-1)
 *                 (PyTorch's rule; M must then be > 1, else NH_ERR_SHAPE)
 *   stats         fp32 [4, C] out: rows (mean, var, inv_std, scale)
 *   ws, ws_bytes  workspace from bn_forward_train_workspace
 */
nh_status bn_forward_train(const void *x, void *y, nh_dtype io,
                           int64_t N, int64_t C, int64_t HW,
                           const float *gamma, const float *beta,
                           float *running_mean, float *running_var,
                           float momentum, float eps,
                           float *stats, void *ws, size_t ws_bytes, void *stream);

/*
 * Training backward.  Aether-ML PR #18, "Backward finalize": per channel the
 * sums sum dy and sum dy*(x - mean) give
 *   dbeta = sum dy,  dgamma = inv_std * sum dy*(x - mean),
 *   k1 = -scale*inv_std^2 * sum dy*(x - mean) / M,  k2 = -scale*dbeta / M,
 * and dx = dy*scale + (x - mean)*k1 + k2.
 *
 *   dy, x         [N, C, HW] of dtype io
 *   stats         fp32 [4, C] as written by bn_forward_train (mean, var,
 *                 inv_std, scale); var is not read
 *   dx            [N, C, HW] of dtype io, or NULL to skip the input gradient
 *                 (dx may equal dy)
 *   grads         fp32 [4, C] out: rows (dgamma, dbeta, k1, k2)
 */
nh_status bn_backward(const void *dy, const void *x, nh_dtype io,
                      int64_t N, int64_t C, int64_t HW,
                      const float *stats, void *dx, float *grads,
                      void *ws, size_t ws_bytes, void *stream);

/*
 * Allocation-free training forward, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): bn_forward_train without the workspace arguments.  Its
 * workspace is a library-owned device array of 16 MiB (16777216 bytes) per GPU,
 * held until the process ends; its address on each device is looked up once,
 * on the first call on that device.  The call allocates nothing.
 *   arguments     as bn_forward_train, minus ws and ws_bytes
 *   errors        as bn_forward_train; NH_ERR_WORKSPACE (nothing launched)
 *                 when the shape's workspace, bn_forward_train_workspace,
 *                 exceeds 16 MiB
 * Every call on one GPU uses that GPU's one array (nothing in it carries over
 * from call to call): calls that overlap on one GPU -- on two streams, or from
 * two threads -- race and give undefined results.  Results equal
 * bn_forward_train's bit for bit.
 */
nh_status bn_forward_train_noalloc(const void *x, void *y, nh_dtype io,
                                   int64_t N, int64_t C, int64_t HW,
                                   const float *gamma, const float *beta,
                                   float *running_mean, float *running_var,
                                   float momentum, float eps, float *stats, void *stream);

/*
 * The two stages of each BatchNorm call, as the Aether-ML PR #18 kernels split
 * it: the forward's statistics pass (stats kernel: shifted sums into
 * per-block partials) and then its finalize + apply; the backward's grad_sums
 * pass and then its finalize + dx.  The stage-1 results stay in the
 * workspace, so a host can start the reduction early and the rest later, or
 * run the reduction alone (a data-parallel BatchNorm exchanges the per-block
 * sums between the two stages).
 *
 *   stage         1: the reduction pass only -- writes the workspace, nothing
 *                    else (stats, grads, y, dx and the running statistics are
 *                    untouched);
 *                 2: everything after it, from the workspace stage 1 wrote.
 *                 Any other value: NH_ERR_ARG.
 *   other arguments   exactly those of bn_forward_train / bn_backward, and the
 *                 SAME values for both stages (the launch plan depends on the
 *                 shape and on the pointers' alignment, y's and dx's included).
 * Stage 1 then stage 2 on the same stream, with the same arguments and no
 * other use of the workspace in between, gives bit for bit the results of the
 * one-call form.  Shapes whose whole direction runs as one kernel (channels
 * of a few thousand elements) launch nothing in stage 1 and that kernel in
 * stage 2.
 */
nh_status bn_forward_train_stage(int stage, const void *x, void *y, nh_dtype io,
                                 int64_t N, int64_t C, int64_t HW,
                                 const float *gamma, const float *beta,
                                 float *running_mean, float *running_var,
                                 float momentum, float eps,
                                 float *stats, void *ws, size_t ws_bytes, void *stream);
nh_status bn_backward_stage(int stage, const void *dy, const void *x, nh_dtype io,
                            int64_t N, int64_t C, int64_t HW,
                            const float *stats, void *dx, float *grads,
                            void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * BatchNorm2d + activation, and BatchNorm2d inference.
 *
 * The Aether-ML PR #18 description lists fusing ReLU/LeakyReLU into
 * BatchNorm as its follow-up ("Follow-ups"), and its _bn_apply_ew commit
 * shares the centred apply between training and inference.  With
 * z = (x - mean)*scale + beta (the training forward above):
 *   act NH_ACT_NONE        y = z
 *   act NH_ACT_RELU        y = z > 0 ? z : 0
 *   act NH_ACT_LEAKY_RELU  y = z > 0 ? z : slope*z
 * and the backward is bn_backward applied to dz = dy * act'(z), with act'(z)
 * = 1 for z > 0, else 0 (ReLU) or slope (LeakyReLU): the derivative at 0 is
 * taken from the left.  The backward recomputes z from x, stats and beta
 * (no read of y), in the same fp32 steps as the forward, so with the forward's
 * stats it sees exactly the forward's signs of z.
 * ---------------------------------------------------------------------- */

typedef enum {
    NH_ACT_NONE = 0,
    NH_ACT_RELU = 1,
    NH_ACT_LEAKY_RELU = 2,
    NH_ACT_RANGE_MIN_ = -0x7fffffff - 1, /* range markers, not activations */
    NH_ACT_RANGE_MAX_ = 0x7fffffff
} nh_act;

/*
 * Training forward with activation: bn_forward_train, then y = act(z) in the
 * same elementwise pass.  Arguments as bn_forward_train, plus
 *   act           an nh_act value (else NH_ERR_ARG)
 *   slope         LeakyReLU negative slope, finite (read for
 *                 NH_ACT_LEAKY_RELU only)
 * The workspace is bn_forward_train_workspace's.  stats hold the statistics
 * of x (z's, not y's).
 */
nh_status bn_act_forward_train(const void *x, void *y, nh_dtype io,
                               int64_t N, int64_t C, int64_t HW,
                               const float *gamma, const float *beta,
                               float *running_mean, float *running_var,
                               float momentum, float eps, nh_act act, float slope,
                               float *stats, void *ws, size_t ws_bytes, void *stream);

/*
 * Training backward through the activation: dz = dy*act'(z) inside both
 * passes, then bn_backward's (dgamma, dbeta, k1, k2) and dx for dz.
 *   dy, x, stats, dx, grads, ws   as bn_backward (x must be the forward's
 *                 input, not its output: an in-place forward's x is gone)
 *   beta          fp32 [C] as given to the forward, or NULL (beta = 0)
 *   act, slope    as given to the forward
 * grads row 1 (dbeta) is sum dz; row 0 (dgamma) is inv_std * sum dz*(x - mean).
 */
nh_status bn_act_backward(const void *dy, const void *x, nh_dtype io,
                          int64_t N, int64_t C, int64_t HW,
                          const float *stats, const float *beta, nh_act act, float slope,
                          void *dx, float *grads, void *ws, size_t ws_bytes, void *stream);

/*
 * Inference (evaluation mode): the training apply with the running statistics
 * in place of the batch statistics,
 *   y = act((x - running_mean) * gamma/sqrt(running_var + eps) + beta),
 * one elementwise pass, no workspace, nothing but y written.
 *   x, y          [N, C, HW] of dtype io (y may equal x)
 *   gamma, beta   fp32 [C], or NULL (1 / 0)
 *   running_mean, running_var   fp32 [C], required
 *   eps           finite, >= 0; act, slope as bn_act_forward_train
 */
nh_status bn_forward_infer(const void *x, void *y, nh_dtype io,
                           int64_t N, int64_t C, int64_t HW,
                           const float *gamma, const float *beta,
                           const float *running_mean, const float *running_var,
                           float eps, nh_act act, float slope, void *stream);

/* ------------------------------------------------------------------------
 * LayerNorm / RMSNorm backward over the last dimension of [rows, cols].
 * dweight/dbias are split over rows into per-block partials in the
 * workspace and summed by a finalize kernel in a fixed order.  Rows wider
 * than 64 columns that the register-resident kernels do not take (wider
 * than they hold, odd widths, misaligned tensors) also keep two fp32
 * coefficients per row in the workspace.
 * ---------------------------------------------------------------------- */

nh_status layernorm_backward_workspace(int64_t rows, int64_t cols, size_t *ws_bytes);

/*
 * NVIDIA/Fuser issue #1473, layer_norm backward definition: with
 * xhat = (x - mean)*rstd and g = dy*weight,
 *   dx = rstd*(g - sum_j g / H - xhat * sum_j g*xhat / H)
 *   dweight_j = sum_rows dy*xhat,  dbias_j = sum_rows dy.
 *
 *   dy            [rows, cols] of dy_t;   x [rows, cols] of x_t
 *   mean, rstd    fp32 [rows], the forward's saved statistics
 *   weight        [cols] of w_t, or NULL (weight = 1)
 *   dx            [rows, cols] of dx_t, or NULL (skip)
 *   dweight, dbias [cols] of w_t, each may be NULL (skip)
 * Every dtype is NH_F32 or NH_BF16, in any combination.
 */
nh_status layernorm_backward(const void *dy, nh_dtype dy_t,
                             const void *x, nh_dtype x_t,
                             const float *mean, const float *rstd,
                             const void *weight, nh_dtype w_t,
                             int64_t rows, int64_t cols,
                             void *dx, nh_dtype dx_t,
                             void *dweight, void *dbias,
                             void *ws, size_t ws_bytes, void *stream);

nh_status rmsnorm_backward_workspace(int64_t rows, int64_t cols, size_t *ws_bytes);

/*
 * NVIDIA/Fuser issue #3629, rmsnorm_bwd_fusion: with rinv = 1/rms_r and
 * g = dy*weight,
 *   dx = g*rinv - x * rinv^3 * sum_j g*x / H,   dweight_j = sum_rows dy*x*rinv.
 *
 *   dy, x, dx     [rows, cols] of dtype t (dx may equal dy; dx NULL = skip)
 *   rms           fp32 [rows] saved rms = sqrt(mean(x^2) + eps), or NULL to
 *                 recompute it from x with eps
 *   weight        [cols] of dtype t, or NULL (weight = 1)
 *   dweight       [cols] of dtype t, or NULL (skip)
 */
nh_status rmsnorm_backward(const void *dy, const void *x, nh_dtype t,
                           const float *rms, float eps,
                           const void *weight,
                           int64_t rows, int64_t cols,
                           void *dx, void *dweight,
                           void *ws, size_t ws_bytes, void *stream);

nh_status bda_layernorm_backward_workspace(int64_t rows, int64_t cols, size_t *ws_bytes);

/*
 * Backward of bias + dropout + add + LayerNorm.  NVIDIA/Fuser issue #1473,
 * the one-kernel fusion of its first example (nvfuser_fusion_id9).  The
 * forward is h = residual + dropout(a + bias), y = LayerNorm(h), dropout
 * being a multiply by a 0/1 keep-mask and by `scale`.  With dx_ln the
 * layernorm_backward input gradient for (dy, h, mean, rstd, weight):
 *   dh        = dresidual + dx_ln    (the gradient of residual, and of h)
 *   da        = dh * scale * mask    (the gradient of a)
 *   dbias_in  = sum over rows of da  (the gradient of bias)
 *   dweight, dbias                    as layernorm_backward.
 *
 *   dy            [rows, cols] of dy_t;   x [rows, cols] of x_t: h
 *   mean, rstd    fp32 [rows], saved by the forward for h
 *   weight        [cols] of w_t, or NULL (weight = 1)
 *   dresidual     fp32 [rows, cols], the gradient reaching h from its other
 *                 consumers, or NULL (zero)
 *   mask          [rows, cols] bytes, nonzero = kept, or NULL (all kept)
 *   scale         dropout scale, finite (typically 1/(1 - p))
 *   dh            fp32 [rows, cols] out, or NULL (skip)
 *   da            [rows, cols] of dy_t out, or NULL (skip)
 *   dweight, dbias, dbias_in   [cols] of w_t out, each may be NULL (skip)
 * dy_t, x_t, w_t are NH_F32 or NH_BF16 in any combination.  dh and da may
 * not alias any input.
 */
nh_status bda_layernorm_backward(const void *dy, nh_dtype dy_t,
                                 const void *x, nh_dtype x_t,
                                 const float *mean, const float *rstd,
                                 const void *weight, nh_dtype w_t,
                                 const float *dresidual, const uint8_t *mask, float scale,
                                 int64_t rows, int64_t cols,
                                 float *dh, void *da,
                                 void *dweight, void *dbias, void *dbias_in,
                                 void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * LayerNorm / RMSNorm training forward over the last dimension of
 * [rows, cols]: the forwards whose saved statistics the backwards above take.
 * No workspace.
 * ---------------------------------------------------------------------- */

/*
 * LayerNorm forward.  NVIDIA/Fuser issue #1473's layer_norm backward takes
 * the per-row mean and rstd of this forward as inputs.  The variance comes
 * from the one-pass shifted sums of Aether-ML PR #18 ("One-pass statistics")
 * applied per row, with K = the row's first element, d = x - K, md = sum d / H:
 *   var = sum d^2 / H - md^2 (clamped at 0),  rstd = 1/sqrt(var + eps),
 *   y = ((x - K) - md)*rstd*weight + bias,
 * and the stored mean is K + md or sum x / H, whichever sums the smaller
 * terms (|md| < |sum x / H| picks K + md): both equal the row mean up to
 * rounding.
 *
 *   x             [rows, cols] of x_t;   y [rows, cols] of y_t (y may equal x)
 *   weight, bias  [cols] of w_t, each may be NULL (weight = 1, bias = 0)
 *   mean          fp32 [rows] out (required); rstd fp32 [rows] out, or NULL
 */
nh_status layernorm_forward(const void *x, nh_dtype x_t, const void *weight, const void *bias,
                            nh_dtype w_t, int64_t rows, int64_t cols, float eps,
                            void *y, nh_dtype y_t, float *mean, float *rstd, void *stream);

/*
 * RMSNorm forward, NVIDIA/Fuser issue #3629's rmsnorm_prims:
 *   rms = sqrt(sum_j x^2 / H + eps),  y = weight * (x / rms).
 *
 *   x, y          [rows, cols] of dtype t (y may equal x)
 *   weight        [cols] of dtype t, or NULL (weight = 1)
 *   rms           fp32 [rows] out (the saved input of rmsnorm_backward), or NULL
 */
nh_status rmsnorm_forward(const void *x, nh_dtype t, const void *weight,
                          int64_t rows, int64_t cols, float eps, void *y, float *rms,
                          void *stream);

/* ------------------------------------------------------------------------
 * Measurement support.
 * ---------------------------------------------------------------------- */

/* Kernel ids for per-kernel timing. */
typedef enum {
    NH_K_BN_STATS = 0,        /* shifted sums -> partials[C, 2, grid_y] */
    NH_K_BN_FWD_FINALIZE = 1, /* partials -> stats[4, C], running stats */
    NH_K_BN_APPLY = 2,        /* y = (x - mean)*scale + beta */
    NH_K_BN_GRAD_SUMS = 3,    /* sum dy, sum dy*(x - mean) -> partials */
    NH_K_BN_BWD_FINALIZE = 4, /* partials -> grads[4, C] */
    NH_K_BN_DX = 5,           /* dx = dy*scale + (x - mean)*k1 + k2 */
    NH_K_LN_ROWS = 6,         /* LayerNorm row pass: dx + column partials */
    NH_K_LN_COLSUM = 7,       /* LayerNorm dweight/dbias finalize */
    NH_K_RMS_ROWS = 8,        /* RMSNorm row pass: dx + column partials */
    NH_K_RMS_COLSUM = 9,      /* RMSNorm dweight finalize */
    NH_K_CALIB = 10,          /* calibration kernels below */
    NH_K_LN_FWD = 11,         /* LayerNorm forward row pass */
    NH_K_RMS_FWD = 12,        /* RMSNorm forward row pass */
    NH_K_BN_INFER = 13,       /* BatchNorm inference apply */
    NH_K_BDA_ROWS = 14,       /* bias+dropout+add+LayerNorm backward row pass */
    NH_K_BDA_COLSUM = 15,     /* its dweight/dbias/dbias_in finalize */
    NH_K_ROWS_COEF = 16,      /* per-row gradient coefficients (wide or misaligned rows) */
    NH_K_BN_FWD_CHANNEL = 17, /* BatchNorm forward, one block per small channel */
    NH_K_BN_BWD_CHANNEL = 18, /* BatchNorm backward, one block per small channel */
    NH_K_COUNT = 19,
    NH_K_RANGE_MIN_ = -0x7fffffff - 1, /* range markers, not kernel ids */
    NH_K_RANGE_MAX_ = 0x7fffffff
} nh_kernel;

/* Static name of a kernel id; "" for an unknown id. */
const char *nh_kernel_name(int kernel);

/*
 * Per-kernel timing.  nh_timing_enable(1) clears earlier records and from
 * then on launches every kernel with hipExtLaunchKernel start/stop events,
 * which time the dispatch itself (no extra packets between kernels).
 * nh_timing_enable(0) stops recording and keeps the records.
 * nh_timing_read waits for the recorded events of one kernel id and returns
 * the sum of their durations in milliseconds and the number of launches.
 * Records are process-wide; do not enable timing while another thread
 * launches normhip kernels that should not be counted.
 */
nh_status nh_timing_enable(int on);
/* Pre-creates events for `launches` timed launches so that event creation
 * does not fall inside a timed region. */
nh_status nh_timing_reserve(int64_t launches);
nh_status nh_timing_read(int kernel, double *total_ms, int64_t *launches);

/*
 * Calibration streams for bandwidth floors (the PR #18 comparison of the
 * backward elementwise pass against a plain add with the same traffic):
 *   nh_calib_copy: dst[i] = src[i] for `bytes` bytes (16-byte multiples take
 *                  the vector path);
 *   nh_calib_read: reads n fp32 elements (n a multiple of 4, a 16-byte
 *                  aligned) with the BatchNorm stats pass's shape: one
 *                  contiguous chunk per block, cacheable 16-byte loads, one
 *                  block sum written to block_sums[b] per block b; at most
 *                  max_blocks blocks (block_sums holds max_blocks floats);
 *   nh_calib_add:  out[i] = a[i] + b[i] over n fp32 elements (two reads, one
 *                  write).
 * Both are timed under NH_K_CALIB.
 */
nh_status nh_calib_copy(const void *src, void *dst, size_t bytes, void *stream);
nh_status nh_calib_add(const float *a, const float *b, float *out, int64_t n, void *stream);
nh_status nh_calib_read(const float *a, int64_t n, float *block_sums, int64_t max_blocks, void *stream);

/*
 * Launch plan of the BatchNorm reductions on the current device: the number
 * of blocks per channel (grid_y) that the stats and grad_sums passes of
 * bn_forward_train / bn_backward use for this shape and dtype.  Tests use it to cover single- and multi-block
 * channels.
 */
nh_status nh_bn_plan(int64_t N, int64_t C, int64_t HW, nh_dtype io, int *grid_y);

/* Row-kernel plan: the largest number of blocks G (column-partial rows) a
 * [rows, cols] LayerNorm or RMSNorm backward uses on the current device
 * (the workspace is sized for it; the dtypes and alignment decide the
 * actual G). */
nh_status nh_rows_plan(int64_t rows, int64_t cols, int *blocks);

/*
 * Plan overrides for tests and tuning sweeps: key "bn_grid_y" forces the
 * BatchNorm blocks per channel (reductions, and the elementwise passes unless
 * "bn_ew_grid_y" forces those separately), key "rows_blocks" forces the row-kernel
 * block count (at most 2048 and at most one per row; both keys also size
 * the workspace queried afterwards), key
 * "bn_finalize_kernels" = 1 runs the BatchNorm finalize steps as separate
 * kernels instead of inside the elementwise kernels (same results), key
 * "rows_depth" = 1..4 forces the number of rows a row-kernel team keeps in
 * flight (its software-pipeline depth; same results), key "colsum_cols" =
 * 8, 16, 32 or 64 sets the columns per block of the column finalize (same
 * results), key "bn_layout" = 1 or 2 forces the BatchNorm channel layout or
 * the row layout (the tensor as [N, C*HW] rows, used automatically for planes
 * of at most 128 bytes), key "bn_channel" = 1 or 2 turns the one-block-per-channel
 * fused BatchNorm kernels (used automatically for small channels) off or
 * on, key "bn_channel_threads" = 256 or 1024 sets their block size, key "rows_narrow" = 1 keeps aligned rows of at most 64 vector groups
 * on the 256-thread team kernels instead of the lane-subgroup kernels, key
 * "rows_teams" = 1 or 2 forces the row teams per block of the
 * LayerNorm and RMSNorm backwards' vector kernels (same results up to the
 * order of the column sums), key "bn_block_order" = 1 or 2 numbers the split
 * BatchNorm passes' blocks channel-major or channel-fastest (same results),
 * key "bn_unit_order" = 1 gives each block of a channel one contiguous range
 * of its units, on a grid of at most one round of resident blocks, instead
 * of the automatic plan (2 forces that plan): every grid_y-th sweep of 1024
 * units to one block, where each block gets a whole sweep, on up to two
 * rounds (results equal up to the rounding of the per-block sums; a
 * workspace queried under 1 may be too small for the automatic plan).
 * value 0 restores the automatic plan.  Process-wide; not for concurrent use with
 * other calls.
 */
nh_status nh_plan_override(const char *key, int64_t value);

/* Host-side self test of the library's integer helpers (fast division,
 * planner invariants).  Needs no GPU.  Returns NH_OK or NH_ERR_ARG with a
 * message in nh_last_error(). */
nh_status nh_selftest_host(void);

#ifdef __cplusplus
}
#endif

#endif /* NORMHIP_H */
