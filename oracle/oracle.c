/*
 * CPU fp64 oracle for training-mode normalization forward/backward.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain definition that the
 * HIP library is checked against.  Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg load it; the library never does, and the
 * two share no source, header, table or helper.
 *
 * Every quantity is computed in double precision, straight from its
 * definition: means and variances by two passes over the data, sums with
 * Neumaier-compensated accumulation, no one-pass shifted sums, no partials,
 * no coefficient-form shortcuts.  Loops run sequentially by default;
 * oracle_set_threads(n) spreads independent channels (BatchNorm) or rows
 * (LayerNorm/RMSNorm) over n OpenMP threads, and column sums over disjoint
 * blocks of columns.  Every sum still adds its terms in the same order, so
 * the results are bit-identical at any thread count.  (This is for timing
 * the oracle on a host's cores; the arithmetic is the sequential one.)
 *
 * Layouts: BatchNorm tensors are NCHW, contiguous, element (n,c,j) at
 * (n*C + c)*HW + j with HW = H*W.  LayerNorm/RMSNorm tensors are
 * [rows, cols] row-major, reduced over cols.
 *
 * Sources (the pages these definitions are read from):
 *  [AE]  Aether-ML PR #18, "perf(batchnorm): device-sized grid, one-pass
 *        statistics, finalize kernels": commit messages and the PR body's
 *        "One-pass statistics", "Backward finalize", "Behavior changes" and
 *        "Testing" sections.
 *  [TH]  lightning-thunder PR #182, "Improve batch_norm backward performance
 *        for automatically generated backward" (batch_norm decomposition,
 *        running_var accuracy fix).
 *  [LN]  NVIDIA/Fuser issue #1473, "Why is LayerNorm Backward Segmenting?",
 *        the 3-kernel layer_norm backward repro (nvfuser_fusion_id14).
 *  [RM]  NVIDIA/Fuser issue #3629, "Performance gap between manual nvfuser
 *        definition and thunder.jit for rmsnorm": rmsnorm_prims and the
 *        pre-generated rmsnorm_bwd_fusion definition.
 *
 * Parity pins (tests/test_oracle_*.py): PyTorch CPU fp64 autograd of
 * F.batch_norm / F.layer_norm / F.rms_norm, central finite differences of
 * each forward, exact rational arithmetic on tiny inputs, the shift and
 * scale invariants with their eps closed forms, and the large-offset
 * variance case.  No function here is "parity unpinned".
 *
 * Return value of every entry point: 0 on success, -1 on a bad argument.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

/* ---- threads for the independent loops (1 = sequential) ------------------ */
static int g_threads = 1;

int oracle_set_threads(int n)
{
    if (n < 1) return -1;
    g_threads = n;
    return 0;
}

/* Columns per block of the threaded column sums: each block's columns are
 * summed by one thread in row order. */
#define COL_BLOCK 64

/* ---- compensated summation (Neumaier's improvement of Kahan's method) ---- */
typedef struct {
    double s; /* running sum */
    double c; /* running compensation: the low-order bits lost from s */
} ksum_t;

static void ks_init(ksum_t *k) { k->s = 0.0; k->c = 0.0; }

static void ks_add(ksum_t *k, double v)
{
    double t = k->s + v;
    if (fabs(k->s) >= fabs(v))
        k->c += (k->s - t) + v;
    else
        k->c += (v - t) + k->s;
    k->s = t;
}

static double ks_value(const ksum_t *k) { return k->s + k->c; }

static size_t bn_index(int64_t n, int64_t c, int64_t j, int64_t C, int64_t HW)
{
    return (size_t)((n * C + c) * HW + j);
}

/* Per-channel batch statistics of an NCHW tensor: the mean over (N,H,W) and
 * the biased variance (divide by M = N*H*W), two passes.  [AE] checks
 * batch_var against "the float64 variance of the same data" ("Testing"); its
 * k1 coefficient uses inv_std^2 with that same variance, which only holds for
 * the biased estimator. */
static void bn_channel_moments(const double *x, int64_t N, int64_t C, int64_t HW,
                               int64_t c, double *mean, double *var)
{
    const double M = (double)(N * HW);
    ksum_t s;
    ks_init(&s);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < HW; ++j)
            ks_add(&s, x[bn_index(n, c, j, C, HW)]);
    double mu = ks_value(&s) / M;
    ksum_t q;
    ks_init(&q);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < HW; ++j) {
            double d = x[bn_index(n, c, j, C, HW)] - mu;
            ks_add(&q, d * d);
        }
    *mean = mu;
    *var = ks_value(&q) / M;
}

/*
 * BatchNorm2d training forward.  [AE] commit "one-pass statistics": the
 * forward produces stats[4,C] = (mean, var, inv_std, gamma*inv_std), the
 * output y = (x - mean)*scale + beta in its centred form, and updates the
 * running statistics in place.
 *
 * Running-statistics update (the pages name it but give no formula; [TH]
 * decomposes PyTorch's batch_norm, whose rule is taken):
 *   running_mean <- (1 - momentum)*running_mean + momentum*mean
 *   running_var  <- (1 - momentum)*running_var  + momentum*var*M/(M-1)
 * i.e. the running variance uses the unbiased estimator.  running_mean and
 * running_var may be NULL (no update); with them given, M must exceed 1.
 *
 * Inputs: x[N*C*HW], gamma[C], beta[C].  Outputs: y[N*C*HW], stats[4*C]
 * (row-major: stats[0*C + c] = mean, [1*C + c] = var, [2*C + c] = inv_std,
 * [3*C + c] = scale).
 */
int oracle_bn_forward_train(int64_t N, int64_t C, int64_t HW,
                            const double *x, const double *gamma, const double *beta,
                            double momentum, double eps,
                            double *running_mean, double *running_var,
                            double *y, double *stats)
{
    if (N < 0 || C < 0 || HW < 0) return -1;
    const int64_t M = N * HW;
    if (M == 0) return -1;
    if ((running_mean || running_var) && M < 2) return -1;
#pragma omp parallel for num_threads(g_threads) schedule(dynamic, 1) if (g_threads > 1)
    for (int64_t c = 0; c < C; ++c) {
        double mean, var;
        bn_channel_moments(x, N, C, HW, c, &mean, &var);
        double inv_std = 1.0 / sqrt(var + eps);
        double scale = gamma[c] * inv_std;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t j = 0; j < HW; ++j) {
                size_t i = bn_index(n, c, j, C, HW);
                double xhat = (x[i] - mean) * inv_std;
                y[i] = gamma[c] * xhat + beta[c];
            }
        stats[0 * C + c] = mean;
        stats[1 * C + c] = var;
        stats[2 * C + c] = inv_std;
        stats[3 * C + c] = scale;
        if (running_mean)
            running_mean[c] = (1.0 - momentum) * running_mean[c] + momentum * mean;
        if (running_var)
            running_var[c] = (1.0 - momentum) * running_var[c]
                           + momentum * var * (double)M / (double)(M - 1);
    }
    return 0;
}

/*
 * BatchNorm2d training backward: the gradient of the training forward above
 * with respect to x, gamma and beta, for an incoming gradient dy.  The batch
 * statistics are recomputed from x (two passes), so nothing saved by a
 * forward run enters.
 *
 * Textbook form, per channel with xhat = (x - mean)*inv_std:
 *   dbeta  = sum dy
 *   dgamma = sum dy*xhat
 *   dx     = gamma*inv_std/M * (M*dy - dbeta - xhat*dgamma)
 * (deliberately not the coefficient form the pages' kernel uses).
 *
 * grads[4*C] = (dgamma, dbeta, k1, k2) as [AE]'s backward-finalize commit
 * defines them:
 *   k1 = -scale*inv_std^2 * sum(dy*(x - mean)) / M
 *   k2 = -scale*dbeta / M
 * with scale = gamma*inv_std.
 */
int oracle_bn_backward(int64_t N, int64_t C, int64_t HW,
                       const double *x, const double *dy, const double *gamma,
                       double eps, double *dx, double *grads)
{
    if (N < 0 || C < 0 || HW < 0) return -1;
    const int64_t Mi = N * HW;
    if (Mi == 0) return -1;
    const double M = (double)Mi;
#pragma omp parallel for num_threads(g_threads) schedule(dynamic, 1) if (g_threads > 1)
    for (int64_t c = 0; c < C; ++c) {
        double mean, var;
        bn_channel_moments(x, N, C, HW, c, &mean, &var);
        double inv_std = 1.0 / sqrt(var + eps);
        double scale = gamma[c] * inv_std;
        ksum_t sdy, sdyxhat, sdyxc;
        ks_init(&sdy);
        ks_init(&sdyxhat);
        ks_init(&sdyxc);
        for (int64_t n = 0; n < N; ++n)
            for (int64_t j = 0; j < HW; ++j) {
                size_t i = bn_index(n, c, j, C, HW);
                double xc = x[i] - mean;
                ks_add(&sdy, dy[i]);
                ks_add(&sdyxhat, dy[i] * xc * inv_std);
                ks_add(&sdyxc, dy[i] * xc);
            }
        double dbeta = ks_value(&sdy);
        double dgamma = ks_value(&sdyxhat);
        for (int64_t n = 0; n < N; ++n)
            for (int64_t j = 0; j < HW; ++j) {
                size_t i = bn_index(n, c, j, C, HW);
                double xhat = (x[i] - mean) * inv_std;
                dx[i] = gamma[c] * inv_std / M * (M * dy[i] - dbeta - xhat * dgamma);
            }
        grads[0 * C + c] = dgamma;
        grads[1 * C + c] = dbeta;
        grads[2 * C + c] = -scale * inv_std * inv_std * ks_value(&sdyxc) / M;
        grads[3 * C + c] = -scale * dbeta / M;
    }
    return 0;
}

/*
 * BatchNorm2d followed by an activation, the fusion [AE] names as its next
 * step ("Follow-ups": ReLU/LeakyReLU fused into BatchNorm).  z = the
 * BatchNorm training forward output above, y = act(z) with
 *   act = none (act 0), ReLU max(z, 0) (act 1), LeakyReLU z > 0 ? z : slope*z (act 2).
 * Backward: dz = dy * act'(z) with act'(z) = 1 for z > 0, else 0 (ReLU) or
 * slope (LeakyReLU) -- the derivative at z = 0 taken from the left, as
 * PyTorch does -- then the BatchNorm backward of dz.
 */
static double act_value(int act, double slope, double z)
{
    if (act == 1) return z > 0.0 ? z : 0.0;
    if (act == 2) return z > 0.0 ? z : slope * z;
    return z;
}

static double act_slope(int act, double slope, double z)
{
    if (act == 0 || z > 0.0) return 1.0;
    return act == 1 ? 0.0 : slope;
}

int oracle_bn_act_forward_train(int64_t N, int64_t C, int64_t HW, const double *x,
                                const double *gamma, const double *beta, double momentum,
                                double eps, int act, double slope, double *running_mean,
                                double *running_var, double *y, double *stats)
{
    if (act < 0 || act > 2) return -1;
    int rc = oracle_bn_forward_train(N, C, HW, x, gamma, beta, momentum, eps, running_mean,
                                     running_var, y, stats);
    if (rc != 0) return rc;
    const size_t n = (size_t)(N * C * HW);
    for (size_t i = 0; i < n; ++i) y[i] = act_value(act, slope, y[i]);
    return 0;
}

int oracle_bn_act_backward(int64_t N, int64_t C, int64_t HW, const double *x, const double *dy,
                           const double *gamma, const double *beta, double eps, int act,
                           double slope, double *dx, double *grads)
{
    if (N < 0 || C < 0 || HW < 0 || act < 0 || act > 2) return -1;
    const size_t n = (size_t)(N * C * HW);
    if (n == 0) return -1;
    double *z = (double *)malloc(n * sizeof(double));
    double *dz = (double *)malloc(n * sizeof(double));
    double *stats = (double *)malloc((size_t)(4 * C) * sizeof(double));
    if (!z || !dz || !stats) { free(z); free(dz); free(stats); return -1; }
    int rc = oracle_bn_forward_train(N, C, HW, x, gamma, beta, 0.0, eps, NULL, NULL, z, stats);
    if (rc == 0) {
        for (size_t i = 0; i < n; ++i) dz[i] = dy[i] * act_slope(act, slope, z[i]);
        rc = oracle_bn_backward(N, C, HW, x, dz, gamma, eps, dx, grads);
    }
    free(z);
    free(dz);
    free(stats);
    return rc;
}

/*
 * BatchNorm2d inference (evaluation mode) with the same optional activation:
 * the running statistics stand in for the batch statistics,
 *   y = act(gamma * (x - running_mean) / sqrt(running_var + eps) + beta).
 * The Aether-ML BatchNorm PR applies inference with the same centred
 * elementwise step as training (its _bn_apply_ew commit).
 */
int oracle_bn_infer(int64_t N, int64_t C, int64_t HW, const double *x, const double *gamma,
                    const double *beta, const double *running_mean, const double *running_var,
                    double eps, int act, double slope, double *y)
{
    if (N < 0 || C < 0 || HW < 0 || act < 0 || act > 2 || !running_mean || !running_var) return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t c = 0; c < C; ++c) {
            const double g = gamma ? gamma[c] : 1.0, b = beta ? beta[c] : 0.0;
            const double sd = sqrt(running_var[c] + eps);
            for (int64_t j = 0; j < HW; ++j) {
                const size_t i = bn_index(n, c, j, C, HW);
                y[i] = act_value(act, slope, g * (x[i] - running_mean[c]) / sd + b);
            }
        }
    return 0;
}

/*
 * LayerNorm forward statistics over the last dimension, used to make the
 * saved mean/rstd that the backward consumes: mean = sum x / H,
 * var = sum (x - mean)^2 / H (biased), rstd = 1/sqrt(var + eps).
 */
int oracle_layernorm_stats(int64_t rows, int64_t cols, const double *x, double eps,
                           double *mean, double *rstd)
{
    if (rows < 0 || cols <= 0) return -1;
#pragma omp parallel for num_threads(g_threads) schedule(static) if (g_threads > 1)
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + (size_t)r * (size_t)cols;
        ksum_t s;
        ks_init(&s);
        for (int64_t j = 0; j < cols; ++j) ks_add(&s, xr[j]);
        double mu = ks_value(&s) / (double)cols;
        ksum_t q;
        ks_init(&q);
        for (int64_t j = 0; j < cols; ++j) {
            double d = xr[j] - mu;
            ks_add(&q, d * d);
        }
        mean[r] = mu;
        rstd[r] = 1.0 / sqrt(ks_value(&q) / (double)cols + eps);
    }
    return 0;
}

/*
 * LayerNorm training forward over the last dimension (the forward whose saved
 * statistics [LN]'s backward consumes as its mean and rstd inputs):
 *   mean_r = sum_j x / H,  var_r = sum_j (x - mean)^2 / H  (two passes),
 *   rstd_r = 1/sqrt(var_r + eps),  y = (x - mean)*rstd*w + b.
 * w may be NULL (1), b may be NULL (0); mean/rstd may be NULL (not returned).
 */
int oracle_layernorm_forward(int64_t rows, int64_t cols, const double *x,
                             const double *w, const double *b, double eps,
                             double *y, double *mean, double *rstd)
{
    if (rows < 0 || cols <= 0) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + (size_t)r * (size_t)cols;
        double *yr = y + (size_t)r * (size_t)cols;
        double mu, rs;
        oracle_layernorm_stats(1, cols, xr, eps, &mu, &rs);
        for (int64_t j = 0; j < cols; ++j)
            yr[j] = (xr[j] - mu) * rs * (w ? w[j] : 1.0) + (b ? b[j] : 0.0);
        if (mean) mean[r] = mu;
        if (rstd) rstd[r] = rs;
    }
    return 0;
}

/*
 * LayerNorm backward over the last dimension with saved per-row mean and rstd,
 * as [LN]'s layer_norm backward definition computes it (tensor names of that
 * definition in brackets):
 *   g      = dy * w                                   [T18]
 *   dvar_r = -1/2 * rstd^3 * sum_j g*(x - mean)       [T24, T38, T40, T41]
 *   dmean_r = -sum_j g*rstd                           [T22, T30, T31]
 *   dx     = g*rstd + 2*dvar*(x - mean)/H + dmean/H   [T55..T74]
 *   dweight_j = sum_rows dy*(x - mean)*rstd           [T13, T19, T20]
 *   dbias_j   = sum_rows dy                           [T16]
 * The definition's incoming-gradient add (its T2) is not part of this
 * backward.  weight may be NULL (weight = 1).  dweight/dbias may be NULL.
 */
int oracle_layernorm_backward(int64_t rows, int64_t cols,
                              const double *x, const double *dy,
                              const double *mean, const double *rstd,
                              const double *w,
                              double *dx, double *dweight, double *dbias)
{
    if (rows < 0 || cols <= 0) return -1;
    const double H = (double)cols;
#pragma omp parallel for num_threads(g_threads) schedule(static) if (g_threads > 1)
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + (size_t)r * (size_t)cols;
        const double *dyr = dy + (size_t)r * (size_t)cols;
        double *dxr = dx + (size_t)r * (size_t)cols;
        const double mu = mean[r], rs = rstd[r];
        ksum_t sgx, sg;
        ks_init(&sgx);
        ks_init(&sg);
        for (int64_t j = 0; j < cols; ++j) {
            double g = dyr[j] * (w ? w[j] : 1.0);
            ks_add(&sgx, g * (xr[j] - mu));
            ks_add(&sg, g * rs);
        }
        double dvar = -0.5 * rs * rs * rs * ks_value(&sgx);
        double dmean = -ks_value(&sg);
        for (int64_t j = 0; j < cols; ++j) {
            double g = dyr[j] * (w ? w[j] : 1.0);
            dxr[j] = g * rs + 2.0 * dvar * (xr[j] - mu) / H + dmean / H;
        }
    }
    /* Column sums over rows, each column accumulated in row order. */
    ksum_t *sw = (ksum_t *)malloc((size_t)cols * sizeof(ksum_t));
    ksum_t *sb = (ksum_t *)malloc((size_t)cols * sizeof(ksum_t));
    if (!sw || !sb) { free(sw); free(sb); return -1; }
    for (int64_t j = 0; j < cols; ++j) { ks_init(&sw[j]); ks_init(&sb[j]); }
#pragma omp parallel for num_threads(g_threads) schedule(static) if (g_threads > 1)
    for (int64_t jb = 0; jb < cols; jb += COL_BLOCK) {
        const int64_t je = jb + COL_BLOCK < cols ? jb + COL_BLOCK : cols;
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t j = jb; j < je; ++j) {
                size_t i = (size_t)r * (size_t)cols + (size_t)j;
                ks_add(&sw[j], dy[i] * (x[i] - mean[r]) * rstd[r]);
                ks_add(&sb[j], dy[i]);
            }
    }
    for (int64_t j = 0; j < cols; ++j) {
        if (dweight) dweight[j] = ks_value(&sw[j]);
        if (dbias) dbias[j] = ks_value(&sb[j]);
    }
    free(sw);
    free(sb);
    return 0;
}

/*
 * Backward of bias + dropout + add + LayerNorm: NVIDIA/Fuser issue #1473,
 * the one-kernel fusion of its first example (nvfuser_fusion_id9).  The
 * forward it differentiates is h = residual + dropout(a + bias), y =
 * LayerNorm(h) with the saved mean/rstd of h; dropout multiplies by a 0/1
 * mask and by `scale` (the fusion's scalar input).  With dx_ln the LayerNorm
 * backward above (the same steps: g = dy*w, dvar, dmean, the three-term
 * input gradient):
 *   dh        = dresidual + dx_ln        (gradient at h; dresidual is the
 *                                         gradient reaching h from its other
 *                                         consumers, NULL = 0)
 *   da        = dh * scale * mask         (gradient of a, and of bias per row)
 *   dbias_in  = sum over rows of da
 *   dweight, dbias = the LayerNorm parameter gradients.
 * mask holds 0/1 bytes (NULL = all ones).
 */
int oracle_bda_layernorm_backward(int64_t rows, int64_t cols, const double *x, const double *dy,
                                  const double *mean, const double *rstd, const double *w,
                                  const double *dresidual, const uint8_t *mask, double scale,
                                  double *dh, double *da, double *dweight, double *dbias,
                                  double *dbias_in)
{
    if (rows < 0 || cols <= 0) return -1;
    const size_t n = (size_t)rows * (size_t)cols;
    double *dx = (double *)malloc((n ? n : 1) * sizeof(double));
    ksum_t *sa = (ksum_t *)malloc((size_t)cols * sizeof(ksum_t));
    if (!dx || !sa) { free(dx); free(sa); return -1; }
    int rc = oracle_layernorm_backward(rows, cols, x, dy, mean, rstd, w, dx, dweight, dbias);
    if (rc == 0) {
        for (int64_t j = 0; j < cols; ++j) ks_init(&sa[j]);
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t j = 0; j < cols; ++j) {
                const size_t i = (size_t)r * (size_t)cols + (size_t)j;
                const double h = (dresidual ? dresidual[i] : 0.0) + dx[i];
                const double m = mask ? (mask[i] ? 1.0 : 0.0) : 1.0;
                const double a = h * scale * m;
                if (dh) dh[i] = h;
                if (da) da[i] = a;
                ks_add(&sa[j], a);
            }
        if (dbias_in)
            for (int64_t j = 0; j < cols; ++j) dbias_in[j] = ks_value(&sa[j]);
    }
    free(dx);
    free(sa);
    return rc;
}

/*
 * RMSNorm forward statistic, [RM] rmsnorm_prims:
 *   rms_r = sqrt(sum_j x^2 / H + eps)
 */
int oracle_rmsnorm_rms(int64_t rows, int64_t cols, const double *x, double eps,
                       double *rms)
{
    if (rows < 0 || cols <= 0) return -1;
#pragma omp parallel for num_threads(g_threads) schedule(static) if (g_threads > 1)
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + (size_t)r * (size_t)cols;
        ksum_t s;
        ks_init(&s);
        for (int64_t j = 0; j < cols; ++j) ks_add(&s, xr[j] * xr[j]);
        rms[r] = sqrt(ks_value(&s) / (double)cols + eps);
    }
    return 0;
}

/*
 * RMSNorm forward, [RM] rmsnorm_prims:  y = w * (x / rms),
 * rms = sqrt(sum_j x^2 / H + eps).  w may be NULL (1); rms may be NULL.
 */
int oracle_rmsnorm_forward(int64_t rows, int64_t cols, const double *x, const double *w,
                           double eps, double *y, double *rms_out)
{
    if (rows < 0 || cols <= 0) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + (size_t)r * (size_t)cols;
        double *yr = y + (size_t)r * (size_t)cols;
        double rms;
        oracle_rmsnorm_rms(1, cols, xr, eps, &rms);
        for (int64_t j = 0; j < cols; ++j) yr[j] = (w ? w[j] : 1.0) * (xr[j] / rms);
        if (rms_out) rms_out[r] = rms;
    }
    return 0;
}

/*
 * RMSNorm backward, following [RM]'s pre-generated rmsnorm_bwd_fusion step by
 * step (tensor names of that definition in brackets), with the saved rms:
 *   rinv = 1/rms                                  [T15]
 *   g    = dy * w                                 [T24]
 *   s_r  = sum_j (-g * x / rms^2)                 [T29, T30, T32..T35]
 *   t_r  = s_r / (2*rms) / H                      [T43..T49]
 *   dx   = g*rinv + 2*t_r*x                       [T28, T59, T62, T63]
 *   dweight_j = sum_rows dy * x * rinv            [T16, T23, T25]
 * which is dx = g/rms - x*sum(g*x)/(H*rms^3).
 * rms may be NULL: it is then recomputed from x with eps (oracle_rmsnorm_rms).
 * w may be NULL (weight = 1).  dweight may be NULL.
 */
int oracle_rmsnorm_backward(int64_t rows, int64_t cols,
                            const double *x, const double *dy, const double *w,
                            const double *rms_saved, double eps,
                            double *dx, double *dweight)
{
    if (rows < 0 || cols <= 0) return -1;
    const double H = (double)cols;
    double *rms = (double *)malloc((size_t)(rows > 0 ? rows : 1) * sizeof(double));
    ksum_t *sw = (ksum_t *)malloc((size_t)cols * sizeof(ksum_t));
    if (!rms || !sw) { free(rms); free(sw); return -1; }
    if (rms_saved) {
        for (int64_t r = 0; r < rows; ++r) rms[r] = rms_saved[r];
    } else {
        oracle_rmsnorm_rms(rows, cols, x, eps, rms);
    }
    for (int64_t j = 0; j < cols; ++j) ks_init(&sw[j]);
#pragma omp parallel for num_threads(g_threads) schedule(static) if (g_threads > 1)
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + (size_t)r * (size_t)cols;
        const double *dyr = dy + (size_t)r * (size_t)cols;
        double *dxr = dx + (size_t)r * (size_t)cols;
        const double rinv = 1.0 / rms[r];
        ksum_t s;
        ks_init(&s);
        for (int64_t j = 0; j < cols; ++j) {
            double g = dyr[j] * (w ? w[j] : 1.0);
            ks_add(&s, -g * xr[j] / (rms[r] * rms[r]));
        }
        double t = ks_value(&s) / (2.0 * rms[r]) / H;
        for (int64_t j = 0; j < cols; ++j) {
            double g = dyr[j] * (w ? w[j] : 1.0);
            dxr[j] = g * rinv + 2.0 * t * xr[j];
        }
    }
    /* dweight: each column summed over the rows in row order. */
#pragma omp parallel for num_threads(g_threads) schedule(static) if (g_threads > 1)
    for (int64_t jb = 0; jb < cols; jb += COL_BLOCK) {
        const int64_t je = jb + COL_BLOCK < cols ? jb + COL_BLOCK : cols;
        for (int64_t r = 0; r < rows; ++r) {
            const double *xr = x + (size_t)r * (size_t)cols;
            const double *dyr = dy + (size_t)r * (size_t)cols;
            const double rinv = 1.0 / rms[r];
            for (int64_t j = jb; j < je; ++j) ks_add(&sw[j], dyr[j] * xr[j] * rinv);
        }
    }
    if (dweight)
        for (int64_t j = 0; j < cols; ++j) dweight[j] = ks_value(&sw[j]);
    free(rms);
    free(sw);
    return 0;
}
