"""The BatchNorm row layout (the tensor as [N, C*HW] rows, bn_col_* kernels),
taken for small planes that the channel layout would read with scalar units
or on its split path -- BatchNorm over [N, C] (1x1 planes), odd planes of a
few elements -- against the oracle: training forward and
backward with and without an activation, inference, in place, grads only,
misaligned tensors, both layouts forced on one shape, repeat runs."""
import dataclasses

import numpy as np
import pytest

from bwd_bn_stats_amd import workloads as wl

from helpers import check, clear_of_kink, dev, host, place

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

F32, BF16 = wl.F32, wl.BF16


@pytest.fixture(scope="module")
def nh():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bwd_bn_stats_amd import normhip
    return normhip


def _gpu(nh, c, act, slope, offset=0, in_place=False, need_dx=True):
    x, dy = place(c.x, offset), place(c.dy, offset)
    g, b = dev(c.gamma), dev(c.beta)
    rm, rv = dev(c.running_mean), dev(c.running_var)
    xk = x.clone() if in_place else x
    y, stats = nh.bn_forward_train(xk, g, b, rm, rv, c.momentum, c.eps, act=act, slope=slope,
                                   y=xk if in_place else None)
    dyk = dy.clone() if in_place else dy
    dx, grads = nh.bn_backward(dyk, x, stats, beta=b, act=act, slope=slope, need_dx=need_dx,
                               dx=dyk if in_place else None)
    torch.cuda.synchronize()
    out = dict(y=host(y), stats=host(stats), grads=host(grads), rm=host(rm), rv=host(rv))
    if need_dx:
        out["dx"] = host(dx)
    return out


def _check_oracle(oracle_mod, c, got, act, slope):
    wy, wstats, wrm, wrv = oracle_mod.bn_act_forward_train(
        c.x.value, c.gamma, c.beta, act, slope, eps=c.eps, momentum=c.momentum,
        running_mean=c.running_mean, running_var=c.running_var)
    wdx, wgrads = oracle_mod.bn_act_backward(c.x.value, c.dy.value, c.gamma, c.beta, act, slope, eps=c.eps)
    check("y", got["y"], wy, c.io)
    if "dx" in got:
        check("dx", got["dx"], wdx, c.io)
    for k in range(4):
        check(f"stats[{k}]", got["stats"][k], wstats[k], F32)
        check(f"grads[{k}]", got["grads"][k], wgrads[k], F32)
    check("running_mean", got["rm"], wrm, F32)
    check("running_var", got["rv"], wrv, F32)


SHAPES = [((4096, 1024, 1, 1), F32, "none"),      # BatchNorm over [N, C]
          ((256, 4096, 1, 1), BF16, "relu"),
          ((1000, 37, 1, 3), F32, "leaky_relu"),   # 1x3 planes, a row of 111
          ((333, 64, 3, 3), BF16, "none"),         # 3x3 planes
          ((64, 100, 7, 7), BF16, "relu"),         # 7x7 bf16 planes (98 bytes)
          ((17, 5, 1, 1), F32, "none"),            # one partial chunk, one strip
          ((5000, 3, 1, 1), BF16, "leaky_relu"),   # rows shorter than a group
          ((40000, 64, 1, 1), F32, "none"),        # 16 column lanes, 2000 chunks, a block per channel finalizes
          ((30000, 256, 1, 1), BF16, "relu"),      # 32 column lanes, 1875 chunks
          ((3000, 8, 1, 1), BF16, "none"),         # one column lane, 256 row lanes
          ((2000, 2, 3, 1), F32, "none"),          # scalar units, 8 column lanes
          ((20000, 4, 2, 2), F32, "leaky_relu")]   # 2x2 planes, a block finalizes HW * rb sums


@pytest.mark.parametrize("shape,io,act", SHAPES, ids=lambda v: str(v))
def test_row_layout_matches_oracle(nh, oracle_mod, shape, io, act):
    N, C, H, W = shape
    c = wl.bn_case(N, C, H, W, io, seed=N + 7 * C + H, x_mean=1.5, x_std=0.7, beta_std=0.5)
    if act != "none":
        c = dataclasses.replace(c, x=clear_of_kink(oracle_mod, c.x, c.gamma, c.beta, c.eps,
                                                   1e-3 if io == F32 else 1e-2))
    print(f"[bn row layout] {shape} {io} act={act}", flush=True)
    nh.timing_enable(True)
    try:
        got = _gpu(nh, c, act, 0.1)
        _, n_stats = nh.timing_read("bn_stats")
        _, n_fin = nh.timing_read("bn_fwd_finalize")
    finally:
        nh.timing_enable(False)
    assert n_stats == 1 and n_fin == 1, "expected the row layout (reduction, finalize, apply)"
    _check_oracle(oracle_mod, c, got, act, 0.1)


def test_row_layout_options(nh, oracle_mod):
    """In place, grads only, misaligned (scalar units) and repeat runs."""
    c = wl.bn_case(512, 96, 1, 2, F32, seed=91, x_mean=-2.0)
    ref = _gpu(nh, c, "none", 0.0)
    _check_oracle(oracle_mod, c, ref, "none", 0.0)
    again = _gpu(nh, c, "none", 0.0)
    for k in ref:
        assert np.array_equal(ref[k].view(np.uint64), again[k].view(np.uint64)), f"repeat: {k}"
    inp = _gpu(nh, c, "none", 0.0, in_place=True)
    for k in ref:
        assert np.array_equal(ref[k].view(np.uint64), inp[k].view(np.uint64)), f"in place: {k}"
    go = _gpu(nh, c, "none", 0.0, need_dx=False)
    for k in ("stats", "grads", "rm", "rv"):
        assert np.array_equal(ref[k].view(np.uint64), go[k].view(np.uint64)), f"grads only: {k}"
    mis = _gpu(nh, c, "none", 0.0, offset=1)
    _check_oracle(oracle_mod, c, mis, "none", 0.0)


@pytest.mark.parametrize("layout", [1, 2])
def test_both_layouts_forced(nh, oracle_mod, layout):
    """One small-plane shape through either layout: the oracle's results."""
    c = wl.bn_case(300, 40, 4, 4, BF16, seed=92, x_mean=3.0)
    c = dataclasses.replace(c, x=clear_of_kink(oracle_mod, c.x, c.gamma, c.beta, c.eps, 1e-2))
    nh.plan_override("bn_layout", layout)
    try:
        got = _gpu(nh, c, "leaky_relu", 0.05)
    finally:
        nh.plan_override("bn_layout", 0)
    _check_oracle(oracle_mod, c, got, "leaky_relu", 0.05)


@pytest.mark.parametrize("shape,io", [((4096, 256, 1, 1), F32), ((100, 64, 3, 3), BF16)])
def test_row_layout_inference(nh, oracle_mod, shape, io):
    N, C, H, W = shape
    c = wl.bn_case(N, C, H, W, io, seed=93 + C, x_mean=0.5)
    rng = np.random.Generator(np.random.PCG64(94))
    rm = rng.normal(0.5, 0.2, C).astype(np.float32)
    rv = rng.uniform(0.5, 2.0, C).astype(np.float32)
    want = oracle_mod.bn_infer(c.x.value, c.gamma, c.beta, rm, rv, "relu", 0.0, eps=c.eps)
    y = nh.bn_forward_infer(dev(c.x), dev(rm), dev(rv), dev(c.gamma), dev(c.beta), c.eps, act="relu")
    torch.cuda.synchronize()
    check("y", host(y), want, io)
