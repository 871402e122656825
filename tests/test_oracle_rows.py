"""Pins for the oracle's LayerNorm and RMSNorm backward (CPU only).

Pins: PyTorch's fp64 CPU F.layer_norm / F.rms_norm with autograd, central
finite differences of the forwards written out here, the shift/scale
invariants with their eps closed forms, exact rational arithmetic on tiny
rows, and special cases.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from bwd_bn_stats_amd import workloads as wl


def _rel(a, b, floor=1e-300):
    """Normwise relative difference; floor bounds the denominator below (for
    outputs that are exactly zero by construction, e.g. a one-column row)."""
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), floor))


def _dsqrt(q: Fraction) -> Fraction:
    getcontext().prec = 60
    return Fraction((Decimal(q.numerator) / Decimal(q.denominator)).sqrt())


# ---------------------------------------------------------------- LayerNorm

@pytest.mark.parametrize("rows,cols,seed", [(3, 7, 1), (16, 1600, 1003), (5, 1, 2), (9, 33, 4)])
def test_ln_matches_torch_fp64(oracle_mod, rows, cols, seed):
    c = wl.rows_case(rows, cols, x_t=wl.F32, dy_t=wl.BF16, w_t=wl.BF16, seed=seed, with_bias=True)
    x, dy, w, b = c.x.value, c.dy.value, c.w.value, c.b.value
    mean, rstd = oracle_mod.layernorm_stats(x, eps=c.eps)
    tv, tm = torch.var_mean(torch.tensor(x), dim=1, unbiased=False)
    assert _rel(mean, tm.numpy()) < 1e-13
    assert _rel(rstd, 1.0 / np.sqrt(tv.numpy() + c.eps)) < 1e-12
    dx, dw, db = oracle_mod.layernorm_backward(x, dy, mean, rstd, w)
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    bt = torch.tensor(b, requires_grad=True)
    y = F.layer_norm(xt, (cols,), wt, bt, eps=c.eps)
    y.backward(torch.tensor(dy))
    assert _rel(dx, xt.grad.numpy(), 1.0) < 1e-11
    assert _rel(dw, wt.grad.numpy(), 1.0) < 1e-12
    assert _rel(db, bt.grad.numpy()) < 1e-13


def test_ln_weight_none_means_one(oracle_mod):
    c = wl.rows_case(4, 19, x_t=wl.F32, dy_t=wl.F32, w_t=wl.F32, seed=8)
    x, dy = c.x.value, c.dy.value
    mean, rstd = oracle_mod.layernorm_stats(x)
    a = oracle_mod.layernorm_backward(x, dy, mean, rstd, None)
    b = oracle_mod.layernorm_backward(x, dy, mean, rstd, np.ones(19))
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_ln_finite_differences(oracle_mod):
    rng = np.random.default_rng(21)
    R, H, eps = 3, 7, 1e-5
    x = rng.normal(0.5, 1.5, size=(R, H))
    dy = rng.normal(size=(R, H))
    w = rng.uniform(0.5, 1.5, H)
    b = rng.normal(size=H)

    def fwd(xx, ww, bb):  # y = (x - mean) / sqrt(var + eps) * w + b
        mu = xx.mean(axis=1, keepdims=True)
        var = ((xx - mu) ** 2).mean(axis=1, keepdims=True)
        return (xx - mu) / np.sqrt(var + eps) * ww + bb

    def loss(xx, ww, bb):
        return float(np.sum(dy * fwd(xx, ww, bb)))

    mean, rstd = oracle_mod.layernorm_stats(x, eps=eps)
    dx, dw, db = oracle_mod.layernorm_backward(x, dy, mean, rstd, w)
    fd = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        h = 1e-6 * (1 + abs(x[idx]))
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        fd[idx] = (loss(xp, w, b) - loss(xm, w, b)) / (2 * h)
    assert _rel(dx, fd) < 1e-7
    fdw, fdb = np.zeros(H), np.zeros(H)
    for j in range(H):
        e = np.zeros(H)
        e[j] = 1e-6
        fdw[j] = (loss(x, w + e, b) - loss(x, w - e, b)) / 2e-6
        fdb[j] = (loss(x, w, b + e) - loss(x, w, b - e)) / 2e-6
    assert _rel(dw, fdw) < 1e-7
    assert _rel(db, fdb) < 1e-7


def test_ln_invariants(oracle_mod):
    c = wl.ln_bwd(rows=64)
    x, dy, w = c.x.value, c.dy.value, c.w.value
    mean, rstd = oracle_mod.layernorm_stats(x, eps=c.eps)
    dx, dw, db = oracle_mod.layernorm_backward(x, dy, mean, rstd, w)
    xhat = (x - mean[:, None]) * rstd[:, None]
    g = dy * w
    mag = np.abs(dx).max(axis=1) * x.shape[1]
    assert np.all(np.abs(dx.sum(axis=1)) < 1e-13 * mag)
    lhs = (dx * xhat).sum(axis=1)
    rhs = c.eps * rstd ** 3 * (g * xhat).sum(axis=1)
    assert np.all(np.abs(lhs - rhs) < 1e-12 * mag)
    # closed forms of the parameter gradients
    assert _rel(db, dy.sum(axis=0)) < 1e-13
    assert _rel(dw, (dy * xhat).sum(axis=0)) < 1e-12


def test_ln_exact_rational_given_stats(oracle_mod):
    """Saved mean/rstd that are not the row's own statistics (the backward
    takes them as inputs): the oracle equals the definition's formula
    evaluated exactly."""
    rng = np.random.default_rng(9)
    R, H = 2, 5
    x = np.round(rng.normal(size=(R, H)), 3)
    dy = np.round(rng.normal(size=(R, H)), 3)
    w = np.round(rng.uniform(0.5, 1.5, H), 3)
    mean = np.array([0.125, -0.25])
    rstd = np.array([1.5, 0.75])
    dx, dw, db = oracle_mod.layernorm_backward(x, dy, mean, rstd, w)
    for r in range(R):
        X = [Fraction(float(v)) for v in x[r]]
        D = [Fraction(float(v)) for v in dy[r]]
        Wf = [Fraction(float(v)) for v in w]
        mu, rs = Fraction(float(mean[r])), Fraction(float(rstd[r]))
        g = [d * ww for d, ww in zip(D, Wf)]
        xhat = [(v - mu) * rs for v in X]
        A = sum(g) / H
        B = sum(gg * xh for gg, xh in zip(g, xhat)) / H
        want = [rs * (gg - A - xh * B) for gg, xh in zip(g, xhat)]
        assert max(abs(float(a) - b) for a, b in zip(want, dx[r])) < 1e-14
    for j in range(H):
        want_w = sum(Fraction(float(dy[r, j])) * (Fraction(float(x[r, j])) - Fraction(float(mean[r])))
                     * Fraction(float(rstd[r])) for r in range(R))
        assert abs(float(want_w) - dw[j]) < 1e-15
        assert abs(float(sum(Fraction(float(dy[r, j])) for r in range(R))) - db[j]) < 1e-15


# ------------------------------------------------------------------ RMSNorm

@pytest.mark.parametrize("rows,cols,seed,dt", [(3, 7, 1, wl.F32), (8, 8192, 1004, wl.BF16),
                                              (6, 1, 5, wl.F32), (7, 100, 6, wl.BF16)])
def test_rms_matches_torch_fp64(oracle_mod, rows, cols, seed, dt):
    c = wl.rows_case(rows, cols, x_t=dt, dy_t=dt, w_t=dt, seed=seed)
    x, dy, w = c.x.value, c.dy.value, c.w.value
    rms = oracle_mod.rmsnorm_rms(x, eps=c.eps)
    assert _rel(rms, np.sqrt((x * x).mean(axis=1) + c.eps)) < 1e-14
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    y = F.rms_norm(xt, (cols,), wt, eps=c.eps)
    y.backward(torch.tensor(dy))
    for saved in (rms, None):
        dx, dw = oracle_mod.rmsnorm_backward(x, dy, w, saved, eps=c.eps)
        assert _rel(dx, xt.grad.numpy(), 1.0) < 1e-11
        assert _rel(dw, wt.grad.numpy(), 1.0) < 1e-12


def test_rms_matches_prims_definition(oracle_mod):
    """rmsnorm_prims of the nvFuser RMSNorm issue: w * (x / sqrt(mean(x^2) + 1e-5)),
    differentiated by torch autograd."""
    rng = np.random.default_rng(33)
    x = rng.normal(size=(4, 64))
    dy = rng.normal(size=(4, 64))
    w = rng.uniform(0.5, 1.5, 64)
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    out = wt * (xt / torch.sqrt((xt ** 2).mean(1, keepdim=True) + 1e-5))
    out.backward(torch.tensor(dy))
    dx, dw = oracle_mod.rmsnorm_backward(x, dy, w, None, eps=1e-5)
    assert _rel(dx, xt.grad.numpy()) < 1e-12
    assert _rel(dw, wt.grad.numpy()) < 1e-12


def test_rms_finite_differences(oracle_mod):
    rng = np.random.default_rng(23)
    R, H, eps = 3, 7, 1e-5
    x = rng.normal(size=(R, H))
    dy = rng.normal(size=(R, H))
    w = rng.uniform(0.5, 1.5, H)

    def loss(xx, ww):
        rms = np.sqrt((xx * xx).mean(axis=1, keepdims=True) + eps)
        return float(np.sum(dy * ww * xx / rms))

    dx, dw = oracle_mod.rmsnorm_backward(x, dy, w, None, eps=eps)
    fd = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        h = 1e-6 * (1 + abs(x[idx]))
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        fd[idx] = (loss(xp, w) - loss(xm, w)) / (2 * h)
    assert _rel(dx, fd) < 1e-7
    fdw = np.zeros(H)
    for j in range(H):
        e = np.zeros(H)
        e[j] = 1e-6
        fdw[j] = (loss(x, w + e) - loss(x, w - e)) / 2e-6
    assert _rel(dw, fdw) < 1e-7


def test_rms_invariant_and_special_cases(oracle_mod):
    c = wl.rms_bwd(wl.F32, rows=32, cols=512)
    x, dy, w = c.x.value, c.dy.value, c.w.value
    rms = oracle_mod.rmsnorm_rms(x, eps=c.eps)
    dx, _ = oracle_mod.rmsnorm_backward(x, dy, w, rms, eps=c.eps)
    rinv = 1.0 / rms
    lhs = (dx * x).sum(axis=1)
    rhs = c.eps * rinv ** 3 * (dy * w * x).sum(axis=1)
    mag = np.abs(dx * x).sum(axis=1)
    assert np.all(np.abs(lhs - rhs) < 1e-12 * mag)
    assert np.all(np.abs(rhs) > 1e-9 * mag)  # the eps term is present
    # constant row a: rms = sqrt(a^2 + eps)
    r = oracle_mod.rmsnorm_rms(np.full((1, 10), -3.0), eps=0.5)
    assert abs(r[0] - np.sqrt(9.5)) < 1e-15
    # eps = 0: dx is orthogonal to x, and scaling x leaves dx*x unchanged in shape
    dx0, _ = oracle_mod.rmsnorm_backward(x, dy, w, None, eps=0.0)
    assert np.all(np.abs((dx0 * x).sum(axis=1)) < 1e-12 * np.abs(dx0 * x).sum(axis=1))
    dx2, _ = oracle_mod.rmsnorm_backward(2.0 * x, dy, w, None, eps=0.0)
    assert _rel(2.0 * dx2, dx0) < 1e-13


def test_rms_exact_rational(oracle_mod):
    rng = np.random.default_rng(19)
    R, H, eps = 2, 6, 1e-5
    x = np.round(rng.normal(size=(R, H)), 3)
    dy = np.round(rng.normal(size=(R, H)), 3)
    w = np.round(rng.uniform(0.5, 1.5, H), 3)
    dx, dw = oracle_mod.rmsnorm_backward(x, dy, w, None, eps=eps)
    want_w = [Fraction(0)] * H
    for r in range(R):
        X = [Fraction(float(v)) for v in x[r]]
        D = [Fraction(float(v)) for v in dy[r]]
        Wf = [Fraction(float(v)) for v in w]
        rms = _dsqrt(sum(v * v for v in X) / H + Fraction(eps))
        g = [d * ww for d, ww in zip(D, Wf)]
        S = sum(gg * v for gg, v in zip(g, X))
        want = [gg / rms - v * S / (H * rms ** 3) for gg, v in zip(g, X)]
        assert max(abs(float(a) - b) for a, b in zip(want, dx[r])) < 1e-14
        for j in range(H):
            want_w[j] += D[j] * X[j] / rms
    assert max(abs(float(a) - b) for a, b in zip(want_w, dw)) < 1e-14


# ---------------------------------------------------------- forwards (next)

@pytest.mark.parametrize("rows,cols,seed", [(3, 7, 1), (16, 1600, 1003), (5, 1, 2)])
def test_ln_forward_matches_torch(oracle_mod, rows, cols, seed):
    c = wl.rows_case(rows, cols, x_t=wl.F32, dy_t=wl.BF16, w_t=wl.BF16, seed=seed, with_bias=True)
    x, w, b = c.x.value, c.w.value, c.b.value
    y, mean, rstd = oracle_mod.layernorm_forward(x, w, b, eps=c.eps)
    ty = F.layer_norm(torch.tensor(x), (cols,), torch.tensor(w), torch.tensor(b), eps=c.eps).numpy()
    assert _rel(y, ty, 1.0) < 1e-13
    m2, r2 = oracle_mod.layernorm_stats(x, eps=c.eps)
    assert np.array_equal(mean, m2) and np.array_equal(rstd, r2)
    # no affine parameters: every row of y has mean 0 and variance var/(var+eps)
    y0, _, _ = oracle_mod.layernorm_forward(x, None, None, eps=c.eps)
    if cols > 1:
        assert np.all(np.abs(y0.mean(axis=1)) < 1e-14 * np.abs(y0).max())
        var = 1.0 / rstd ** 2 - c.eps
        assert _rel(y0.var(axis=1), var / (var + c.eps)) < 1e-12


@pytest.mark.parametrize("rows,cols,seed", [(3, 7, 1), (8, 8192, 1004), (6, 1, 5)])
def test_rms_forward_matches_torch(oracle_mod, rows, cols, seed):
    c = wl.rows_case(rows, cols, x_t=wl.BF16, dy_t=wl.BF16, w_t=wl.BF16, seed=seed)
    x, w = c.x.value, c.w.value
    y, rms = oracle_mod.rmsnorm_forward(x, w, eps=c.eps)
    ty = F.rms_norm(torch.tensor(x), (cols,), torch.tensor(w), eps=c.eps).numpy()
    assert _rel(y, ty) < 1e-13
    assert np.array_equal(rms, oracle_mod.rmsnorm_rms(x, eps=c.eps))
    # rmsnorm_prims of the RMSNorm issue
    xt = torch.tensor(x)
    prims = (torch.tensor(w) * (xt / torch.sqrt((xt ** 2).mean(1, keepdim=True) + 1e-5))).numpy()
    assert _rel(y, prims) < 1e-13
    # w = 1: mean(y^2) = ms / (ms + eps)
    y1, _ = oracle_mod.rmsnorm_forward(x, None, eps=c.eps)
    ms = (x * x).mean(axis=1)
    assert _rel((y1 * y1).mean(axis=1), ms / (ms + c.eps)) < 1e-13


def test_forwards_exact_rational(oracle_mod):
    rng = np.random.default_rng(77)
    x = np.round(rng.normal(size=(2, 5)), 3)
    w = np.round(rng.uniform(0.5, 1.5, 5), 3)
    b = np.round(rng.normal(size=5), 3)
    eps = 1e-5
    y, mean, rstd = oracle_mod.layernorm_forward(x, w, b, eps=eps)
    yr, rms = oracle_mod.rmsnorm_forward(x, w, eps=eps)
    for r in range(2):
        X = [Fraction(float(v)) for v in x[r]]
        mu = sum(X) / 5
        var = sum((v - mu) ** 2 for v in X) / 5
        rs = 1 / _dsqrt(var + Fraction(eps))
        want = [(v - mu) * rs * Fraction(float(ww)) + Fraction(float(bb)) for v, ww, bb in zip(X, w, b)]
        assert max(abs(float(a) - c) for a, c in zip(want, y[r])) < 1e-14
        ms = _dsqrt(sum(v * v for v in X) / 5 + Fraction(eps))
        want_r = [Fraction(float(ww)) * (v / ms) for v, ww in zip(X, w)]
        assert max(abs(float(a) - c) for a, c in zip(want_r, yr[r])) < 1e-14
        assert abs(float(ms) - rms[r]) < 1e-15 * float(ms)


# ------------------------------------- bias + dropout + add + LayerNorm backward

def _torch_bda(x0, a0, bias0, w0, b0, mask, scale, dy, dres, eps):
    """The forward written out in torch fp64 with autograd: h = residual +
    (a + bias)*mask*scale (residual = x0 - that term, so h equals x0), y =
    layer_norm(h); the loss sum(y*dy) + sum(h*dres) makes dres the gradient
    reaching h from elsewhere."""
    t = lambda v, g=True: torch.tensor(v, dtype=torch.float64, requires_grad=g)
    a, bias, w, b = t(a0), t(bias0), t(w0), t(b0)
    mk = torch.tensor(mask, dtype=torch.float64)
    drop = (a + bias) * mk * scale
    resid = t(x0 - drop.detach().numpy())
    h = resid + drop
    y = F.layer_norm(h, (x0.shape[1],), w, b, eps=eps)
    loss = (y * torch.tensor(dy)).sum() + (h * torch.tensor(dres)).sum()
    loss.backward()
    return h.detach().numpy(), resid.grad.numpy(), a.grad.numpy(), w.grad.numpy(), b.grad.numpy(), \
        bias.grad.numpy()


@pytest.mark.parametrize("rows,cols,p_drop,seed", [(6, 10, 0.3, 71), (4, 33, 0.0, 72), (3, 7, 0.9, 73)])
def test_bda_matches_torch(oracle_mod, rows, cols, p_drop, seed):
    c = wl.bda_case(rows, cols, x_t=wl.F32, dy_t=wl.F32, w_t=wl.F32, seed=seed, p_drop=p_drop)
    rng = np.random.default_rng(seed)
    a0 = rng.normal(size=(rows, cols))
    bias0 = rng.normal(size=cols)
    b0 = rng.normal(size=cols)
    x0 = c.ln.x.value
    h, dres_t, da_t, dw_t, db_t, dbias_t = _torch_bda(x0, a0, bias0, c.ln.w.value, b0, c.mask, c.scale,
                                                      c.ln.dy.value, c.dresidual.astype(np.float64),
                                                      c.ln.eps)
    mean, rstd = oracle_mod.layernorm_stats(h, eps=c.ln.eps)
    dh, da, dw, db, dbi = oracle_mod.bda_layernorm_backward(h, c.ln.dy.value, mean, rstd, c.ln.w.value,
                                                            c.dresidual, c.mask, c.scale)
    assert _rel(dh, dres_t) < 1e-12
    assert _rel(da, da_t) < 1e-12
    assert _rel(dw, dw_t) < 1e-12
    assert _rel(db, db_t) < 1e-12
    assert _rel(dbi, dbias_t) < 1e-12


def test_bda_special_cases(oracle_mod):
    """No dropout (mask all ones, scale 1) and no incoming gradient: dh = da =
    the LayerNorm input gradient, dbias_in = its column sums; every row of dh
    - dresidual sums to 0; a zero mask zeroes da and dbias_in exactly."""
    c = wl.bda_case(9, 24, x_t=wl.F32, dy_t=wl.F32, w_t=wl.F32, seed=74)
    x, dy, w = c.ln.x.value, c.ln.dy.value, c.ln.w.value
    mean, rstd = oracle_mod.layernorm_stats(x, eps=c.ln.eps)
    dx, dw0, db0 = oracle_mod.layernorm_backward(x, dy, mean, rstd, w)
    dh, da, dw, db, dbi = oracle_mod.bda_layernorm_backward(x, dy, mean, rstd, w, None, None, 1.0)
    assert np.array_equal(dh, dx) and np.array_equal(da, dx)
    assert np.array_equal(dw, dw0) and np.array_equal(db, db0)
    assert _rel(dbi, dx.sum(axis=0), floor=1.0) < 1e-13
    dh, da, _, _, dbi = oracle_mod.bda_layernorm_backward(x, dy, mean, rstd, w, c.dresidual, c.mask,
                                                          c.scale)
    rows_sum = (dh - c.dresidual).sum(axis=1)
    assert np.max(np.abs(rows_sum)) < 1e-12 * np.max(np.abs(dh)) * x.shape[1]
    # dropped elements are exactly zero, kept ones are dh*scale
    assert np.all(da[c.mask == 0] == 0.0)
    assert _rel(da[c.mask == 1], dh[c.mask == 1] * c.scale) < 1e-15
    _, da0, _, _, dbi0 = oracle_mod.bda_layernorm_backward(x, dy, mean, rstd, w, c.dresidual,
                                                           np.zeros_like(c.mask), c.scale)
    assert np.all(da0 == 0.0) and np.all(dbi0 == 0.0)


def test_bda_exact_rational(oracle_mod):
    """Tiny case in exact rational arithmetic given the saved statistics."""
    rng = np.random.default_rng(75)
    rows, cols = 3, 5
    x = np.round(rng.normal(size=(rows, cols)), 3)
    dy = np.round(rng.normal(size=(rows, cols)), 3)
    w = np.round(rng.uniform(0.5, 1.5, size=cols), 3)
    dres = np.round(rng.normal(size=(rows, cols)), 3)
    mask = (rng.random(size=(rows, cols)) > 0.4).astype(np.uint8)
    scale = 1.25
    mean = np.round(x.mean(axis=1), 3)
    rstd = np.array([0.875, 1.125, 1.5])
    dh, da, _, _, dbi = oracle_mod.bda_layernorm_backward(x, dy, mean, rstd, w, dres, mask, scale)
    F_ = lambda v: Fraction(float(v))
    H = Fraction(cols)
    for r in range(rows):
        mu, rs = F_(mean[r]), F_(rstd[r])
        g = [F_(dy[r, j]) * F_(w[j]) for j in range(cols)]
        xc = [F_(x[r, j]) - mu for j in range(cols)]
        dvar = Fraction(-1, 2) * rs ** 3 * sum(gj * xj for gj, xj in zip(g, xc))
        dmean = -rs * sum(g)
        for j in range(cols):
            want_h = F_(dres[r, j]) + g[j] * rs + 2 * dvar * xc[j] / H + dmean / H
            want_a = want_h * Fraction(scale) * int(mask[r, j])
            assert abs(float(want_h) - dh[r, j]) < 1e-14
            assert abs(float(want_a) - da[r, j]) < 1e-14
    for j in range(cols):
        assert abs(sum(da[:, j]) - dbi[j]) < 1e-14
