"""GPU parity of layernorm_forward / rmsnorm_forward against the CPU fp64
oracle (normwise relative error <= 2e-5 fp32, <= 8e-3 bf16), and the
forward -> backward chain on the GPU against the oracle's chain."""
import itertools

import numpy as np
import pytest

from bwd_bn_stats_amd import workloads as wl

from helpers import check, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def nh():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bwd_bn_stats_amd import normhip
    return normhip


def _td(t):
    return torch.float32 if t == wl.F32 else torch.bfloat16


def _ln_fwd_case(nh, oracle_mod, c, y_t, *, weight=True, bias=True, need_rstd=True, in_place=False):
    w = c.w.value if weight else None
    b = c.b.value if bias else None
    want_y, want_m, want_r = oracle_mod.layernorm_forward(c.x.value, w, b, eps=c.eps)
    print(f"[ln fwd parity] {c.rows}x{c.cols} x={c.x.dtype} w={c.w.dtype} y={y_t} "
          f"weight={weight} bias={bias} in_place={in_place}", flush=True)
    x = dev(c.x)
    y = x if in_place else None
    gy, gm, gr = nh.layernorm_forward(x, dev(c.w) if weight else None, dev(c.b) if bias else None,
                                      c.eps, y_dtype=_td(y_t), w_dtype=_td(c.w.dtype), y=y,
                                      need_rstd=need_rstd)
    torch.cuda.synchronize()
    check("y", host(gy), want_y, y_t)
    check("mean", host(gm), want_m, wl.F32)
    if need_rstd:
        check("rstd", host(gr), want_r, wl.F32)
    return gy, gm, gr


def test_ln_forward_full_config(nh, oracle_mod):
    c = wl.ln_bwd()
    _ln_fwd_case(nh, oracle_mod, c, wl.F32)


@pytest.mark.parametrize("xt,wt,yt", list(itertools.product((wl.F32, wl.BF16), repeat=3)))
def test_ln_forward_dtypes(nh, oracle_mod, xt, wt, yt):
    c = wl.rows_case(300, 1600, x_t=xt, dy_t=wl.BF16, w_t=wt, seed=71, with_bias=True)
    _ln_fwd_case(nh, oracle_mod, c, yt)


@pytest.mark.parametrize("rows,cols,xt", [(1, 1600, wl.F32), (7, 4, wl.F32), (513, 4096, wl.BF16),
                                          (100, 8192, wl.F32), (77, 8196, wl.F32), (64, 1001, wl.F32),
                                          (33, 16384, wl.BF16), (2000, 64, wl.BF16)])
def test_ln_forward_shapes(nh, oracle_mod, rows, cols, xt):
    c = wl.rows_case(rows, cols, x_t=xt, dy_t=wl.BF16, w_t=wl.BF16, seed=rows + 3 * cols, with_bias=True)
    _ln_fwd_case(nh, oracle_mod, c, xt)


def test_ln_forward_options(nh, oracle_mod):
    c = wl.rows_case(129, 1600, x_t=wl.F32, dy_t=wl.BF16, w_t=wl.F32, seed=72, with_bias=True)
    _ln_fwd_case(nh, oracle_mod, c, wl.F32, weight=False, bias=False)
    _ln_fwd_case(nh, oracle_mod, c, wl.F32, bias=False, need_rstd=False)
    _ln_fwd_case(nh, oracle_mod, c, wl.F32, in_place=True)


def _mean_ulps(got, want):
    """Largest |got - want| per row in units of the fp32 spacing at want."""
    u = np.spacing(np.abs(np.asarray(want)).astype(np.float32)).astype(np.float64)
    return float(np.max(np.abs(np.asarray(got, np.float64) - want) / u))


def test_ln_forward_large_offset(nh, oracle_mod):
    """Rows with |mean| >> std: the shifted one-pass variance keeps rstd
    accurate, and the stored mean is the shifted K + md (the sum of the
    smaller terms), within 0.6 ulp of the exact mean: one rounding of it
    plus the shifted sum's error.  (The plain sum x / H errs by up to 0.9
    ulp on these rows.)"""
    rng = np.random.Generator(np.random.PCG64(73))
    x = (1e4 + 0.01 * rng.normal(size=(64, 1600))).astype(np.float32)
    want_y, want_m, want_r = oracle_mod.layernorm_forward(x.astype(np.float64), eps=1e-5)
    gy, gm, gr = nh.layernorm_forward(torch.from_numpy(x).cuda(), None, None, 1e-5)
    torch.cuda.synchronize()
    check("rstd", host(gr), want_r, wl.F32)
    check("mean", host(gm), want_m, wl.F32)
    assert _mean_ulps(host(gm), want_m) <= 0.6


# Rows whose outputs are ill-conditioned in fp32, found by a seeded random
# sweep: wide rows whose mean is far smaller than their elements (the stored
# mean), and 2-column rows whose two values nearly coincide (rstd near
# 1/sqrt(eps) amplifies any rounding of x - mean).  Summed as K + sum(x - K)
# (K the first element) and applied as x - mean, they missed the fp32 bound
# by up to 1.7x; the plain sum for the mean and (x - K) - sum(x - K)/H for the
# output keep them within it.
@pytest.mark.parametrize("rows,cols,xt,wt,yt,bias,in_place,seed", [
    (195, 39921, wl.BF16, wl.F32, wl.F32, False, False, 20002),
    (208, 32768, wl.BF16, wl.BF16, wl.BF16, True, True, 20016),
    (86, 36335, wl.F32, wl.F32, wl.F32, True, False, 20026),
    (65536, 2, wl.F32, wl.BF16, wl.F32, True, False, 20029)])
def test_ln_forward_ill_conditioned_rows(nh, oracle_mod, rows, cols, xt, wt, yt, bias, in_place, seed):
    c = wl.rows_case(rows, cols, x_t=xt, dy_t=xt, w_t=wt, seed=seed, with_bias=True)
    _ln_fwd_case(nh, oracle_mod, c, yt, bias=bias, in_place=in_place)


def test_ln_forward_nearly_constant_rows(nh, oracle_mod):
    """Rows of 2-5 elements around 2.5 with a spread of 1e-3 (variance far
    below eps): the output is (x - mean) * rstd with rstd near 1/sqrt(eps),
    and the stored mean stays within 0.6 ulp (the plain sum errs by up to
    1.6 ulp on these rows)."""
    rng = np.random.Generator(np.random.PCG64(74))
    for cols in (2, 3, 5):
        x = (2.5 + 1e-3 * rng.normal(size=(8192, cols))).astype(np.float32)
        w = (0.5 + rng.random(cols)).astype(np.float32)
        b = (0.1 * rng.normal(size=cols)).astype(np.float32)
        want_y, want_m, want_r = oracle_mod.layernorm_forward(x.astype(np.float64), w.astype(np.float64),
                                                              b.astype(np.float64), eps=1e-5)
        print(f"[ln fwd parity] nearly constant rows 8192x{cols}", flush=True)
        gy, gm, gr = nh.layernorm_forward(torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda(),
                                          torch.from_numpy(b).cuda(), 1e-5)
        torch.cuda.synchronize()
        check("y", host(gy), want_y, wl.F32)
        check("mean", host(gm), want_m, wl.F32)
        check("rstd", host(gr), want_r, wl.F32)
        assert _mean_ulps(host(gm), want_m) <= 0.6


def _rms_fwd_case(nh, oracle_mod, c, *, weight=True, need_rms=True, in_place=False):
    want_y, want_rms = oracle_mod.rmsnorm_forward(c.x.value, c.w.value if weight else None, eps=c.eps)
    print(f"[rms fwd parity] {c.rows}x{c.cols} t={c.x.dtype} weight={weight} in_place={in_place}",
          flush=True)
    x = dev(c.x)
    gy, grms = nh.rmsnorm_forward(x, dev(c.w) if weight else None, c.eps, y=x if in_place else None,
                                  need_rms=need_rms)
    torch.cuda.synchronize()
    check("y", host(gy), want_y, c.x.dtype)
    if need_rms:
        check("rms", host(grms), want_rms, wl.F32)
    return gy, grms


@pytest.mark.parametrize("dt", [wl.BF16, wl.F32])
def test_rms_forward_full_config(nh, oracle_mod, dt):
    _rms_fwd_case(nh, oracle_mod, wl.rms_bwd(dt))


@pytest.mark.parametrize("rows,cols,dt", [(1, 8192, wl.BF16), (3, 8, wl.BF16), (257, 1024, wl.F32),
                                          (40, 16384, wl.BF16), (20, 12288, wl.F32), (31, 999, wl.F32)])
def test_rms_forward_shapes(nh, oracle_mod, rows, cols, dt):
    c = wl.rows_case(rows, cols, x_t=dt, dy_t=dt, w_t=dt, seed=rows * 11 + cols)
    _rms_fwd_case(nh, oracle_mod, c)


def test_rms_forward_options(nh, oracle_mod):
    c = wl.rows_case(64, 4096, x_t=wl.BF16, dy_t=wl.BF16, w_t=wl.BF16, seed=74)
    _rms_fwd_case(nh, oracle_mod, c, weight=False)
    _rms_fwd_case(nh, oracle_mod, c, need_rms=False)
    _rms_fwd_case(nh, oracle_mod, c, in_place=True)


def test_ln_chain_forward_to_backward(nh, oracle_mod):
    """GPU forward statistics feed the GPU backward; compared with the
    oracle's forward -> backward on the same inputs."""
    c = wl.ln_bwd()
    _, m, r = oracle_mod.layernorm_forward(c.x.value, c.w.value, c.b.value, eps=c.eps)
    want_dx, want_dw, want_db = oracle_mod.layernorm_backward(c.x.value, c.dy.value, m, r, c.w.value)
    x = dev(c.x)
    _, gm, gr = nh.layernorm_forward(x, dev(c.w), dev(c.b), c.eps)
    dx, dw, db = nh.layernorm_backward(dev(c.dy), x, gm, gr, dev(c.w), dx_dtype=torch.float32)
    torch.cuda.synchronize()
    check("dx", host(dx), want_dx, wl.F32)
    check("dweight", host(dw), want_dw, wl.BF16)
    check("dbias", host(db), want_db, wl.BF16)


@pytest.mark.parametrize("dt", [wl.BF16, wl.F32])
def test_rms_chain_forward_to_backward(nh, oracle_mod, dt):
    c = wl.rms_bwd(dt)
    want_dx, want_dw = oracle_mod.rmsnorm_backward(c.x.value, c.dy.value, c.w.value, None, eps=c.eps)
    x = dev(c.x)
    _, grms = nh.rmsnorm_forward(x, dev(c.w), c.eps)
    dx, dw = nh.rmsnorm_backward(dev(c.dy), x, grms, dev(c.w), c.eps)
    torch.cuda.synchronize()
    check("dx", host(dx), want_dx, dt)
    check("dweight", host(dw), want_dw, dt)


def test_forwards_bit_identical_runs(nh):
    c = wl.ln_bwd()
    x, w, b = dev(c.x), dev(c.w), dev(c.b)
    a = nh.layernorm_forward(x, w, b, 1e-5)
    bb = nh.layernorm_forward(x, w, b, 1e-5)
    r = wl.rms_bwd(wl.BF16)
    xr, wr = dev(r.x), dev(r.w)
    ra = nh.rmsnorm_forward(xr, wr, 1e-5)
    rb = nh.rmsnorm_forward(xr, wr, 1e-5)
    torch.cuda.synchronize()
    for u, v in list(zip(a, bb)) + list(zip(ra, rb)):
        iv = torch.int16 if u.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(u.view(iv), v.view(iv))


@pytest.mark.parametrize("depth", [1, 2, 3, 4])
def test_forward_pipeline_depths(nh, oracle_mod, depth):
    nh.plan_override("rows_depth", depth)
    try:
        c = wl.rows_case(1037, 1600, x_t=wl.F32, dy_t=wl.BF16, w_t=wl.BF16, seed=75, with_bias=True)
        _ln_fwd_case(nh, oracle_mod, c, wl.F32)
        _rms_fwd_case(nh, oracle_mod, wl.rows_case(333, 4096, x_t=wl.BF16, dy_t=wl.BF16, w_t=wl.BF16,
                                                    seed=76))
    finally:
        nh.plan_override("rows_depth", 0)


@pytest.mark.parametrize("rows,cols,dt", [(64, 16384, wl.F32), (80, 12288, wl.BF16), (9, 32768, wl.BF16)])
def test_forward_wide_rows(nh, oracle_mod, rows, cols, dt):
    c = wl.rows_case(rows, cols, x_t=dt, dy_t=dt, w_t=wl.BF16, seed=rows + 7 * cols, with_bias=True)
    _ln_fwd_case(nh, oracle_mod, c, dt)
    r = wl.rows_case(rows, cols, x_t=dt, dy_t=dt, w_t=dt, seed=rows + 9 * cols)
    _rms_fwd_case(nh, oracle_mod, r)
