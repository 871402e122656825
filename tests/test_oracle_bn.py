"""Pins for the oracle's BatchNorm2d training forward/backward (CPU only).

Each pin is something other than the oracle itself: PyTorch's fp64 CPU
batch_norm with autograd (an independent library implementation), central
finite differences of the forward, exact rational arithmetic, invariants
with their closed forms, and the large-offset variance case of the Aether-ML
BatchNorm PR ("Testing" and "Behavior changes" sections).
"""
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from bwd_bn_stats_amd import workloads as wl


def _torch_bn(x, gamma, beta, dy, eps, momentum, rm, rv):
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    g = torch.tensor(gamma, dtype=torch.float64, requires_grad=True)
    b = torch.tensor(beta, dtype=torch.float64, requires_grad=True)
    rmt = torch.tensor(rm, dtype=torch.float64)
    rvt = torch.tensor(rv, dtype=torch.float64)
    y = F.batch_norm(xt, rmt, rvt, g, b, training=True, momentum=momentum, eps=eps)
    y.backward(torch.tensor(dy, dtype=torch.float64))
    return (y.detach().numpy(), xt.grad.numpy(), g.grad.numpy(), b.grad.numpy(),
            rmt.numpy(), rvt.numpy())


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("shape,seed,xm,xs", [
    ((2, 3, 2, 3), 11, 0.0, 1.0),
    ((3, 37, 41, 40), 1001, 5.0, 0.5),
    ((5, 4, 1, 7), 12, -2.0, 3.0),
    ((1, 6, 3, 3), 13, 0.0, 1.0),
])
def test_bn_matches_torch_fp64(oracle_mod, shape, seed, xm, xs):
    c = wl.bn_case(*shape, seed=seed, x_mean=xm, x_std=xs, beta_std=1.0)
    x, dy = c.x.value, c.dy.value
    rm0 = np.linspace(-0.5, 0.5, c.C)
    rv0 = np.linspace(0.5, 2.0, c.C)
    y, stats, rm, rv = oracle_mod.bn_forward_train(
        x, c.gamma, c.beta, eps=c.eps, momentum=c.momentum,
        running_mean=rm0, running_var=rv0)
    dx, grads = oracle_mod.bn_backward(x, dy, c.gamma, eps=c.eps)
    ty, tdx, tdg, tdb, trm, trv = _torch_bn(x, c.gamma.astype(np.float64),
                                            c.beta.astype(np.float64), dy,
                                            c.eps, c.momentum, rm0, rv0)
    assert _rel(y, ty) < 1e-13
    assert _rel(dx, tdx) < 1e-12
    assert _rel(grads[0], tdg) < 1e-12
    assert _rel(grads[1], tdb) < 1e-12
    # running statistics: momentum rule and the unbiased running variance
    assert _rel(rm, trm) < 1e-14
    assert _rel(rv, trv) < 1e-14
    # stats rows against torch's own var_mean (biased)
    tv, tm = torch.var_mean(torch.tensor(x), dim=(0, 2, 3), unbiased=False)
    assert _rel(stats[0], tm.numpy()) < 1e-13
    assert _rel(stats[1], tv.numpy()) < 1e-12
    assert _rel(stats[2], 1.0 / np.sqrt(tv.numpy() + c.eps)) < 1e-12
    assert _rel(stats[3], c.gamma / np.sqrt(tv.numpy() + c.eps)) < 1e-12


def test_bn_finite_differences(oracle_mod):
    rng = np.random.default_rng(5)
    N, C, H, W = 2, 3, 2, 3
    x = rng.normal(0.3, 1.2, size=(N, C, H, W))
    dy = rng.normal(size=x.shape)
    gamma = rng.uniform(0.5, 1.5, size=C)
    beta = rng.normal(size=C)
    eps = 1e-5

    def loss(xx, gg, bb):
        y, _, _, _ = oracle_mod.bn_forward_train(xx, gg, bb, eps=eps)
        return float(np.sum(dy * y))

    dx, grads = oracle_mod.bn_backward(x, dy, gamma, eps=eps)
    fd = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        h = 1e-6 * (1 + abs(x[idx]))
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        fd[idx] = (loss(xp, gamma, beta) - loss(xm, gamma, beta)) / (2 * h)
    assert _rel(dx, fd) < 1e-7
    fdg, fdb = np.zeros(C), np.zeros(C)
    for c in range(C):
        e = np.zeros(C)
        e[c] = 1e-6
        fdg[c] = (loss(x, gamma + e, beta) - loss(x, gamma - e, beta)) / 2e-6
        fdb[c] = (loss(x, gamma, beta + e) - loss(x, gamma, beta - e)) / 2e-6
    assert _rel(grads[0], fdg) < 1e-7
    assert _rel(grads[1], fdb) < 1e-7


def _dsqrt(q: Fraction) -> Fraction:
    getcontext().prec = 60
    d = (Decimal(q.numerator) / Decimal(q.denominator)).sqrt()
    return Fraction(d)


def test_bn_exact_rational(oracle_mod):
    """Tiny NCHW input, every sum and product exact (Fraction); square root to
    60 digits.  The oracle must agree to fp64 rounding."""
    rng = np.random.default_rng(7)
    N, C, HW = 2, 2, 5
    x = np.round(rng.normal(1.0, 2.0, size=(N, C, HW)), 3)
    dy = np.round(rng.normal(size=(N, C, HW)), 3)
    gamma = np.array([0.75, 1.25])
    beta = np.array([0.5, -1.0])
    eps = 1e-5
    y, stats, rm, rv = oracle_mod.bn_forward_train(x, gamma, beta, eps=eps, momentum=0.1,
                                                   running_mean=np.zeros(C),
                                                   running_var=np.ones(C))
    dx, grads = oracle_mod.bn_backward(x, dy, gamma, eps=eps)
    E = Fraction(eps)
    M = N * HW
    for c in range(C):
        xs = [Fraction(float(x[n, c, j])) for n in range(N) for j in range(HW)]
        ds = [Fraction(float(dy[n, c, j])) for n in range(N) for j in range(HW)]
        mu = sum(xs) / M
        var = sum((v - mu) ** 2 for v in xs) / M
        inv = 1 / _dsqrt(var + E)
        g, b = Fraction(float(gamma[c])), Fraction(float(beta[c]))
        ys = [g * (v - mu) * inv + b for v in xs]
        xh = [(v - mu) * inv for v in xs]
        dbeta = sum(ds)
        dgamma = sum(d * h for d, h in zip(ds, xh))
        dxs = [g * inv / M * (M * d - dbeta - h * dgamma) for d, h in zip(ds, xh)]
        k1 = -g * inv * inv * inv * sum(d * (v - mu) for d, v in zip(ds, xs)) / M
        k2 = -g * inv * dbeta / M
        got_y = [y[n, c, j] for n in range(N) for j in range(HW)]
        got_dx = [dx[n, c, j] for n in range(N) for j in range(HW)]
        assert max(abs(float(a) - b_) for a, b_ in zip(ys, got_y)) < 1e-14 * 10
        assert max(abs(float(a) - b_) for a, b_ in zip(dxs, got_dx)) < 1e-13
        assert abs(float(mu) - stats[0, c]) <= 1e-15 * abs(float(mu)) + 1e-300
        assert abs(float(var) - stats[1, c]) <= 4e-16 * float(var)
        assert abs(float(dbeta) - grads[1, c]) < 1e-14
        assert abs(float(dgamma) - grads[0, c]) < 1e-13
        assert abs(float(k1) - grads[2, c]) < 1e-13
        assert abs(float(k2) - grads[3, c]) < 1e-13
        assert abs(float(Fraction(1, 10) * mu) - rm[c]) < 1e-15
        assert abs(float(Fraction(9, 10) + Fraction(1, 10) * var * M / (M - 1)) - rv[c]) < 1e-15


def test_bn_invariants_and_coefficient_form(oracle_mod):
    """Per channel: sum dx = 0 (shift invariance); sum dx*xhat =
    scale*dgamma*eps*inv_std^2 (the eps closed form of scale invariance); the
    coefficient identity dx = dy*scale + (x - mean)*k1 + k2 of the pages'
    backward-finalize commit holds for the textbook dx."""
    c = wl.bn_ragged()
    x, dy = c.x.value, c.dy.value
    _, stats, _, _ = oracle_mod.bn_forward_train(x, c.gamma, c.beta, eps=c.eps)
    dx, grads = oracle_mod.bn_backward(x, dy, c.gamma, eps=c.eps)
    mean, var, inv, scale = stats
    dgamma, dbeta, k1, k2 = grads
    xs = x.transpose(1, 0, 2, 3).reshape(c.C, -1)
    dxs = dx.transpose(1, 0, 2, 3).reshape(c.C, -1)
    dys = dy.transpose(1, 0, 2, 3).reshape(c.C, -1)
    xhat = (xs - mean[:, None]) * inv[:, None]
    scale_dx = np.max(np.abs(dxs), axis=1) * xs.shape[1]
    assert np.all(np.abs(dxs.sum(axis=1)) < 1e-13 * scale_dx)
    lhs = (dxs * xhat).sum(axis=1)
    rhs = scale * dgamma * c.eps * inv ** 2
    assert np.all(np.abs(lhs - rhs) < 1e-12 * scale_dx)
    # at var ~ 0.25 the eps term is ~4e-5 relative: not negligible
    assert np.all(np.abs(rhs) > 1e-6 * np.abs(scale * dgamma))
    coef = dys * scale[:, None] + (xs - mean[:, None]) * k1[:, None] + k2[:, None]
    assert _rel(coef, dxs) < 1e-12


def test_bn_scale_invariance_exact_at_eps0(oracle_mod):
    rng = np.random.default_rng(3)
    x = rng.normal(2.0, 0.7, size=(4, 3, 5, 5))
    dy = rng.normal(size=x.shape)
    gamma = rng.uniform(0.5, 1.5, 3)
    dx, grads = oracle_mod.bn_backward(x, dy, gamma, eps=0.0)
    _, stats, _, _ = oracle_mod.bn_forward_train(x, gamma, np.zeros(3), eps=0.0)
    xhat = (x - stats[0][None, :, None, None]) * stats[2][None, :, None, None]
    s = (dx * xhat).sum(axis=(0, 2, 3))
    assert np.all(np.abs(s) < 1e-12 * np.abs(dx).sum(axis=(0, 2, 3)))
    # dx is unchanged when x is scaled by a positive factor (eps = 0)
    dx2, _ = oracle_mod.bn_backward(3.0 * x, dy, gamma, eps=0.0)
    assert _rel(3.0 * dx2, dx) < 1e-12


def test_bn_large_offset_variance(oracle_mod):
    """mean 1e4, std 0.01: the oracle's two-pass variance matches the exact
    variance of the fp32 data; the naive E[x^2]-E[x]^2 visibly fails (in fp32
    it collapses, in fp64 it is off by far more than the fp32 tolerance)."""
    c = wl.bn_case(3, 2, 41, 40, wl.F32, seed=2024, x_mean=1e4, x_std=0.01)
    x32 = c.x.store
    x = c.x.value
    _, stats, _, _ = oracle_mod.bn_forward_train(x, c.gamma, c.beta, eps=c.eps)
    for ch in range(c.C):
        v = x[:, ch].ravel()
        fr = [Fraction(float(t)) for t in v]
        mu = sum(fr) / len(fr)
        var = sum((t - mu) ** 2 for t in fr) / len(fr)
        assert abs(stats[1, ch] - float(var)) <= 1e-12 * float(var)
        naive64 = float(np.mean(v * v) - np.mean(v) ** 2)
        assert abs(naive64 - float(var)) > 2e-5 * float(var)
        v32 = x32[:, ch].ravel()
        naive32 = float(np.mean(v32 * v32, dtype=np.float32) - np.mean(v32, dtype=np.float32) ** 2)
        assert abs(naive32 - float(var)) > 0.5 * float(var)


def test_bn_special_cases(oracle_mod):
    # constant channel: var = 0, y = beta, dx = gamma/sqrt(eps)*(dy - mean dy)
    x = np.full((2, 1, 3, 3), 4.25)
    dy = np.arange(18, dtype=np.float64).reshape(2, 1, 3, 3) / 7.0
    y, stats, _, _ = oracle_mod.bn_forward_train(x, [1.5], [0.25], eps=1e-5)
    assert stats[1, 0] == 0.0 and stats[0, 0] == 4.25
    assert np.all(y == 0.25)
    dx, grads = oracle_mod.bn_backward(x, dy, [1.5], eps=1e-5)
    want = 1.5 / math.sqrt(1e-5) * (dy - dy.mean())
    assert _rel(dx, want) < 1e-14
    assert grads[0, 0] == 0.0
    # momentum 0 keeps the running statistics; momentum 1 replaces them
    rng = np.random.default_rng(1)
    x = rng.normal(size=(3, 2, 2, 2))
    _, st, rm, rv = oracle_mod.bn_forward_train(x, [1, 1], [0, 0], momentum=0.0,
                                                running_mean=[7.0, 8.0], running_var=[2.0, 3.0])
    assert list(rm) == [7.0, 8.0] and list(rv) == [2.0, 3.0]
    _, st, rm, rv = oracle_mod.bn_forward_train(x, [1, 1], [0, 0], momentum=1.0,
                                                running_mean=[7.0, 8.0], running_var=[2.0, 3.0])
    assert _rel(rm, st[0]) < 1e-15
    assert _rel(rv, st[1] * 12 / 11) < 1e-15
    # a single element per channel cannot give an unbiased running variance
    with pytest.raises(ValueError):
        oracle_mod.bn_forward_train(np.ones((1, 2, 1, 1)), [1, 1], [0, 0],
                                    running_mean=np.zeros(2), running_var=np.ones(2))


# ------------------------------------------- BatchNorm + activation (next step)

@pytest.mark.parametrize("act,slope", [("relu", 0.0), ("leaky_relu", 0.01), ("leaky_relu", 0.2),
                                       ("none", 0.0)])
def test_bn_act_matches_torch(oracle_mod, act, slope):
    c = wl.bn_case(3, 5, 6, 7, wl.F32, seed=91, x_mean=0.3, x_std=1.3, beta_std=0.5)
    x, dy = c.x.value, c.dy.value
    g, b = c.gamma.astype(np.float64), c.beta.astype(np.float64)
    y, stats, rm, rv = oracle_mod.bn_act_forward_train(x, g, b, act, slope, eps=c.eps,
                                                       running_mean=np.zeros(5), running_var=np.ones(5))
    dx, grads = oracle_mod.bn_act_backward(x, dy, g, b, act, slope, eps=c.eps)
    xt = torch.tensor(x, requires_grad=True)
    gt = torch.tensor(g, requires_grad=True)
    bt = torch.tensor(b, requires_grad=True)
    rmt, rvt = torch.zeros(5, dtype=torch.float64), torch.ones(5, dtype=torch.float64)
    z = F.batch_norm(xt, rmt, rvt, gt, bt, training=True, momentum=0.1, eps=c.eps)
    yt = F.relu(z) if act == "relu" else (F.leaky_relu(z, slope) if act == "leaky_relu" else z)
    yt.backward(torch.tensor(dy))
    assert _rel(y, yt.detach().numpy()) < 1e-13
    assert _rel(dx, xt.grad.numpy()) < 1e-12
    assert _rel(grads[0], gt.grad.numpy()) < 1e-12
    assert _rel(grads[1], bt.grad.numpy()) < 1e-12
    assert _rel(rm, rmt.numpy()) < 1e-14 and _rel(rv, rvt.numpy()) < 1e-14
    # act = none reduces to the plain BatchNorm functions
    if act == "none":
        y0, _, _, _ = oracle_mod.bn_forward_train(x, g, b, eps=c.eps)
        dx0, gr0 = oracle_mod.bn_backward(x, dy, g, eps=c.eps)
        assert np.array_equal(y, y0) and np.array_equal(dx, dx0) and np.array_equal(grads, gr0)


def test_bn_act_finite_differences(oracle_mod):
    """Away from the kink (every |z| > 0.05), the backward is the derivative of
    the forward."""
    rng = np.random.default_rng(92)
    N, C, H, W = 2, 2, 3, 3
    for _ in range(100):
        x = rng.normal(0.0, 1.0, size=(N, C, H, W))
        g = rng.uniform(0.5, 1.5, size=C)
        b = rng.normal(0.0, 0.3, size=C)
        z, _, _, _ = oracle_mod.bn_forward_train(x, g, b, eps=1e-5)
        if np.min(np.abs(z)) > 0.05:
            break
    dy = rng.normal(size=x.shape)
    for act, slope in (("relu", 0.0), ("leaky_relu", 0.1)):
        def loss(xx):
            y, _, _, _ = oracle_mod.bn_act_forward_train(xx, g, b, act, slope, eps=1e-5)
            return float(np.sum(dy * y))
        dx, _ = oracle_mod.bn_act_backward(x, dy, g, b, act, slope, eps=1e-5)
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            h = 1e-7
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            fd[idx] = (loss(xp) - loss(xm)) / (2 * h)
        assert _rel(dx, fd) < 1e-6


@pytest.mark.parametrize("act,slope", [("none", 0.0), ("relu", 0.0), ("leaky_relu", 0.1)])
def test_bn_infer_matches_torch(oracle_mod, act, slope):
    c = wl.bn_case(4, 6, 5, 3, wl.F32, seed=93, x_mean=1.0, x_std=2.0, beta_std=0.5)
    rng = np.random.default_rng(94)
    rm = rng.normal(1.0, 0.5, size=6)
    rv = rng.uniform(0.5, 4.0, size=6)
    g, b = c.gamma.astype(np.float64), c.beta.astype(np.float64)
    y = oracle_mod.bn_infer(c.x.value, g, b, rm, rv, act, slope, eps=c.eps)
    z = F.batch_norm(torch.tensor(c.x.value), torch.tensor(rm), torch.tensor(rv), torch.tensor(g),
                     torch.tensor(b), training=False, eps=c.eps)
    yt = F.relu(z) if act == "relu" else (F.leaky_relu(z, slope) if act == "leaky_relu" else z)
    assert _rel(y, yt.numpy()) < 1e-14
    # affine off
    y0 = oracle_mod.bn_infer(c.x.value, None, None, rm, rv, act, slope, eps=c.eps)
    z0 = F.batch_norm(torch.tensor(c.x.value), torch.tensor(rm), torch.tensor(rv), training=False,
                      eps=c.eps)
    y0t = F.relu(z0) if act == "relu" else (F.leaky_relu(z0, slope) if act == "leaky_relu" else z0)
    assert _rel(y0, y0t.numpy()) < 1e-14


def test_bn_infer_with_batch_statistics_is_training_forward(oracle_mod):
    """Evaluation with running statistics equal to the batch's own (mean,
    biased var) reproduces the training forward output."""
    c = wl.bn_case(3, 5, 4, 4, wl.F32, seed=95, x_mean=-2.0, x_std=0.7, beta_std=1.0)
    for act, slope in (("none", 0.0), ("relu", 0.0), ("leaky_relu", 0.3)):
        yt, stats, _, _ = oracle_mod.bn_act_forward_train(c.x.value, c.gamma, c.beta, act, slope,
                                                          eps=c.eps)
        yi = oracle_mod.bn_infer(c.x.value, c.gamma, c.beta, stats[0], stats[1], act, slope,
                                 eps=c.eps)
        assert _rel(yi, yt) < 1e-14
