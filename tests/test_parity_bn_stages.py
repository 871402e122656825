"""bn_forward_train_stage / bn_backward_stage: the two stages of each
BatchNorm call (Aether-ML PR #18's reduction kernel, then its finalize and
elementwise kernel), run one after the other with the same arguments, give
bit for bit the outputs of the one-call form, on every launch plan (split
channel layout, one block per small channel, the row layout for small
planes, separate finalize kernels) and with dx skipped.  The one-call form
is itself checked against the oracle in test_parity_bn.py; one case here also
checks the staged outputs against the oracle directly."""
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


CASES = {
    "cifar_256x32x32x32_f32": lambda: wl.bn_cifar(wl.F32),
    "cifar_256x32x32x32_bf16": lambda: wl.bn_cifar(wl.BF16),
    "resnet_64x256x56x56_bf16": lambda: wl.bn_resnet(),
    # one block per small channel: stage 1 launches nothing
    "ragged_3x37x41x40_f32": lambda: wl.bn_ragged(),
    # the row layout (planes of at most 128 bytes)
    "rows_4096x64x1x1_f32": lambda: wl.bn_case(4096, 64, 1, 1, wl.F32, seed=61, x_mean=2.0),
    "rows_64x512x7x7_bf16": lambda: wl.bn_case(64, 512, 7, 7, wl.BF16, seed=62, x_mean=-1.0),
    # scalar units, several blocks per channel, ragged block tails
    "odd_plane_64x3x33x31_f32": lambda: wl.bn_case(64, 3, 33, 31, wl.F32, seed=63, x_mean=0.5, x_std=3.0),
}


def _run(nh, c, staged, need_dx=True):
    x, dy = dev(c.x), dev(c.dy)
    g, b = dev(c.gamma), dev(c.beta)
    rm, rv = dev(c.running_mean), dev(c.running_var)
    y = torch.empty_like(x)
    dx = torch.empty_like(x) if need_dx else None
    stats = torch.empty(4, c.C, device=x.device)
    grads = torch.empty(4, c.C, device=x.device)
    ws = torch.empty(max(16, nh.bn_forward_train_workspace(c.N, c.C, c.hw)), dtype=torch.uint8, device=x.device)
    if staged:
        nh.bn_forward_train_stage(1, x, y, stats, ws, g, b, rm, rv, c.momentum, c.eps)
        nh.bn_forward_train_stage(2, x, y, stats, ws, g, b, rm, rv, c.momentum, c.eps)
        nh.bn_backward_stage(1, dy, x, stats, dx, grads, ws)
        nh.bn_backward_stage(2, dy, x, stats, dx, grads, ws)
    else:
        nh.bn_forward_train(x, g, b, rm, rv, c.momentum, c.eps, y=y, stats=stats, workspace=ws)
        nh.bn_backward(dy, x, stats, dx=dx, grads=grads, need_dx=need_dx, workspace=ws)
    torch.cuda.synchronize()
    out = dict(y=host(y), stats=host(stats), rm=host(rm), rv=host(rv), grads=host(grads))
    if need_dx:
        out["dx"] = host(dx)
    return out


def _same_bits(a, b):
    for k in a:
        assert np.array_equal(np.asarray(a[k]).view(np.uint8), np.asarray(b[k]).view(np.uint8)), k


@pytest.mark.parametrize("name", list(CASES))
def test_stages_equal_one_call(nh, name):
    c = CASES[name]()
    print(f"[stages] {name}", flush=True)
    _same_bits(_run(nh, c, True), _run(nh, c, False))


def test_stages_without_dx(nh):
    c = wl.bn_cifar(wl.F32)
    _same_bits(_run(nh, c, True, need_dx=False), _run(nh, c, False, need_dx=False))


def test_stages_with_separate_finalize_kernels(nh):
    c = wl.bn_cifar(wl.BF16)
    nh.plan_override("bn_finalize_kernels", 1)
    try:
        _same_bits(_run(nh, c, True), _run(nh, c, False))
    finally:
        nh.plan_override("bn_finalize_kernels", 0)


def test_stages_against_oracle(nh, oracle_mod):
    c = wl.bn_cifar(wl.F32)
    got = _run(nh, c, True)
    y, stats, rm, rv = oracle_mod.bn_forward_train(c.x.value, c.gamma.astype(np.float64),
                                                   c.beta.astype(np.float64), eps=c.eps, momentum=c.momentum,
                                                   running_mean=c.running_mean, running_var=c.running_var)
    dx, grads = oracle_mod.bn_backward(c.x.value, c.dy.value, c.gamma.astype(np.float64), eps=c.eps)
    check("y", got["y"], y, c.io)
    check("dx", got["dx"], dx, c.io)
    check("running_mean", got["rm"], rm, wl.F32)
    check("running_var", got["rv"], rv, wl.F32)
    for i in range(4):
        check(f"stats[{i}]", got["stats"][i], stats[i], wl.F32)
        check(f"grads[{i}]", got["grads"][i], grads[i], wl.F32)


def test_stage_1_writes_only_the_workspace(nh):
    c = wl.bn_cifar(wl.F32)
    x = dev(c.x)
    y = torch.full_like(x, 7.0)
    stats = torch.full((4, c.C), 3.0, device=x.device)
    rm, rv = dev(c.running_mean), dev(c.running_var)
    ws = torch.empty(nh.bn_forward_train_workspace(c.N, c.C, c.hw), dtype=torch.uint8, device=x.device)
    nh.bn_forward_train_stage(1, x, y, stats, ws, dev(c.gamma), dev(c.beta), rm, rv, c.momentum, c.eps)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()) and bool((stats == 3.0).all())
    assert np.array_equal(host(rm), c.running_mean) and np.array_equal(host(rv), c.running_var)
