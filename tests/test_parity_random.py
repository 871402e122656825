"""Randomized shapes and layouts against the oracle (GPU).

A fixed, seeded list of small cases per operation: random N, C, H, W (or
rows, cols), dtypes, activation, affine on/off, and tensors placed at an
element offset inside a larger buffer (so pointers are misaligned and the
scalar paths run).  Odd-numbered BatchNorm cases force the split path
(reduction, then elementwise kernel) where the small random shapes would
otherwise take the one-block-per-channel kernels; a second set of row cases
covers short aligned rows (the lane-subgroup kernels with vector groups).
A third set draws LayerNorm and RMSNorm forward rows (1 to 40000 columns,
every dtype mix, in place), bias+dropout+add backward rows and BatchNorm
inference shapes, the paths a wider seeded sweep covered.
Every output is compared with the oracle at the parity tolerances.  The cases
are the same on every run."""
import numpy as np
import pytest

from bwd_bn_stats_amd import workloads as wl

from helpers import check, host, place as _place

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def nh():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bwd_bn_stats_amd import normhip
    return normhip


def _bn_cases():
    rng = np.random.Generator(np.random.PCG64(4242))
    cases = []
    for i in range(24):
        N = int(rng.integers(1, 9))
        C = int(rng.integers(1, 70))
        H = int(rng.integers(1, 40))
        W = int(rng.integers(1, 40))
        if N * H * W < 2:
            W += 1
        io = wl.F32 if rng.random() < 0.5 else wl.BF16
        act = ["none", "relu", "leaky_relu"][int(rng.integers(0, 3))]
        offset = int(rng.integers(0, 3))
        affine = rng.random() < 0.8
        cases.append((i, N, C, H, W, io, act, offset, affine, float(rng.normal(0, 3))))
    return cases


@pytest.mark.parametrize("case", _bn_cases(), ids=lambda c: f"bn{c[0]}")
def test_bn_random(nh, oracle_mod, case):
    from helpers import clear_of_kink
    i, N, C, H, W, io, act, offset, affine, xm = case
    c = wl.bn_case(N, C, H, W, io, seed=5000 + i, x_mean=xm, x_std=1.5, beta_std=0.5)
    gamma = c.gamma if affine else np.ones(C)
    beta = c.beta if affine else np.zeros(C)
    x_t = clear_of_kink(oracle_mod, c.x, gamma, beta, c.eps, 1e-3 if io == wl.F32 else 1e-2) \
        if act != "none" else c.x
    split = i % 2 == 1  # odd cases: the split path even where one block per channel would be taken
    print(f"[bn random {i}] N={N} C={C} H={H} W={W} io={io} act={act} offset={offset} "
          f"affine={affine} split={split}", flush=True)
    wy, wstats, wrm, wrv = oracle_mod.bn_act_forward_train(
        x_t.value, gamma, beta, act, 0.1, eps=c.eps, momentum=c.momentum,
        running_mean=c.running_mean, running_var=c.running_var)
    wdx, wgrads = oracle_mod.bn_act_backward(x_t.value, c.dy.value, gamma, beta, act, 0.1, eps=c.eps)
    x, dy = _place(x_t, offset), _place(c.dy, offset)
    g = torch.from_numpy(c.gamma).cuda() if affine else None
    b = torch.from_numpy(c.beta).cuda() if affine else None
    rm, rv = torch.from_numpy(c.running_mean).cuda(), torch.from_numpy(c.running_var).cuda()
    if split:
        nh.plan_override("bn_channel", 1)
    try:
        y, stats = nh.bn_forward_train(x, g, b, rm, rv, c.momentum, c.eps, act=act, slope=0.1)
        dx, grads = nh.bn_backward(dy, x, stats, beta=b, act=act, slope=0.1)
        torch.cuda.synchronize()
    finally:
        nh.plan_override("bn_channel", 0)
    check("y", host(y), wy, io)
    check("dx", host(dx), wdx, io)
    for k in range(4):
        check(f"stats[{k}]", host(stats)[k], wstats[k], wl.F32)
        check(f"grads[{k}]", host(grads)[k], wgrads[k], wl.F32)
    check("running_mean", host(rm), wrm, wl.F32)
    check("running_var", host(rv), wrv, wl.F32)


def _rows_cases():
    rng = np.random.Generator(np.random.PCG64(4343))
    cases = []
    for i in range(24):
        rows = int(rng.integers(1, 300))
        cols = int(rng.choice([1, 3, 8, 64, 100, 257, 512, 1024, 1600, 2048, 3000, 4096]))
        xt = wl.F32 if rng.random() < 0.5 else wl.BF16
        dyt = wl.F32 if rng.random() < 0.5 else wl.BF16
        wt = wl.F32 if rng.random() < 0.5 else wl.BF16
        offset = int(rng.integers(0, 3))
        cases.append((i, rows, cols, xt, dyt, wt, offset))
    # short aligned rows (lane-subgroup kernels with vector groups), more rows
    rng = np.random.Generator(np.random.PCG64(4344))
    for i in range(24, 36):
        rows = int(rng.integers(100, 3000))
        cols = int(rng.choice([8, 16, 24, 32, 96, 128, 200, 256, 384, 512]))
        xt = wl.F32 if rng.random() < 0.5 else wl.BF16
        dyt = wl.F32 if rng.random() < 0.5 else wl.BF16
        wt = wl.F32 if rng.random() < 0.5 else wl.BF16
        offset = 0
        cases.append((i, rows, cols, xt, dyt, wt, offset))
    return cases


@pytest.mark.parametrize("case", _rows_cases(), ids=lambda c: f"rows{c[0]}")
def test_rows_random(nh, oracle_mod, case):
    """LayerNorm forward -> backward, RMSNorm forward -> backward and the
    bias+dropout+add backward on one random shape and layout."""
    i, rows, cols, xt, dyt, wt, offset = case
    print(f"[rows random {i}] rows={rows} cols={cols} x={xt} dy={dyt} w={wt} offset={offset}",
          flush=True)
    c = wl.bda_case(rows, cols, x_t=xt, dy_t=dyt, w_t=wt, seed=6000 + i, p_drop=0.3)
    ln = c.ln
    x, dy, w = _place(ln.x, offset), _place(ln.dy, offset), _place(ln.w, offset)
    wdt = torch.float32 if wt == wl.F32 else torch.bfloat16
    # LayerNorm forward, then backward from the GPU statistics
    wy, wmean, wrstd = oracle_mod.layernorm_forward(ln.x.value, ln.w.value, eps=ln.eps)
    y, mean, rstd = nh.layernorm_forward(x, w, None, ln.eps, y_dtype=x.dtype)
    torch.cuda.synchronize()
    check("ln y", host(y), wy, xt)
    check("ln mean", host(mean), wmean, wl.F32)
    check("ln rstd", host(rstd), wrstd, wl.F32)
    m32, r32 = host(mean), host(rstd)
    wdx, wdw, wdb = oracle_mod.layernorm_backward(ln.x.value, ln.dy.value, m32, r32, ln.w.value)
    dx, dw, db = nh.layernorm_backward(dy, x, mean, rstd, w, dx_dtype=torch.float32)
    torch.cuda.synchronize()
    check("ln dx", host(dx), wdx, wl.F32)
    check("ln dweight", host(dw), wdw, wt)
    check("ln dbias", host(db), wdb, wt)
    # bias+dropout+add backward on the same statistics
    mask = torch.from_numpy(c.mask).cuda()
    dres = torch.from_numpy(c.dresidual).cuda()
    want = oracle_mod.bda_layernorm_backward(ln.x.value, ln.dy.value, m32, r32, ln.w.value,
                                             c.dresidual, c.mask, c.scale)
    got = nh.bda_layernorm_backward(dy, x, mean, rstd, w, dres, mask, c.scale)
    torch.cuda.synchronize()
    for name, g, wv, dt in zip(("dh", "da", "dweight", "dbias", "dbias_in"), got, want,
                               (wl.F32, dyt, wt, wt, wt)):
        check(f"bda {name}", host(g), wv, dt)
    # RMSNorm forward -> backward (one dtype for x, dy, w: x's)
    r = wl.rows_case(rows, cols, x_t=xt, dy_t=xt, w_t=xt, seed=7000 + i)
    rx, rdy, rw = _place(r.x, offset), _place(r.dy, offset), _place(r.w, offset)
    wy, wrms = oracle_mod.rmsnorm_forward(r.x.value, r.w.value, eps=r.eps)
    y, rms = nh.rmsnorm_forward(rx, rw, r.eps)
    torch.cuda.synchronize()
    check("rms y", host(y), wy, xt)
    check("rms rms", host(rms), wrms, wl.F32)
    wdx, wdw = oracle_mod.rmsnorm_backward(r.x.value, r.dy.value, r.w.value, host(rms), eps=r.eps)
    dx, dw = nh.rmsnorm_backward(rdy, rx, rms, rw, r.eps)
    torch.cuda.synchronize()
    check("rms dx", host(dx), wdx, xt)
    check("rms dweight", host(dw), wdw, xt)


# ---- forward rows, bias+dropout+add backward, BatchNorm inference ---------------
_FWD_COLS = [1, 2, 3, 5, 17, 31, 64, 100, 513, 1600, 3000, 4096, 8192, 12288, 20000, 32768, 39921]


def _fwd_cases():
    rng = np.random.Generator(np.random.PCG64(4343))
    dts = (wl.F32, wl.BF16)
    cases = []
    for i in range(28):
        cols = int(rng.choice(_FWD_COLS)) if rng.random() < 0.7 else int(rng.integers(1, 40000))
        rows = int(max(1, min(65536, int(rng.integers(1, 2_000_000)) // cols)))
        xt, wt, yt = (dts[int(rng.integers(2))] for _ in range(3))
        cases.append((i, "ln" if i % 2 == 0 else "rms", rows, cols, xt, wt, yt, bool(rng.random() < 0.8),
                      bool(rng.random() < 0.7), bool(rng.random() < 0.2)))
    return cases


@pytest.mark.parametrize("case", _fwd_cases(), ids=lambda c: f"fwd{c[0]}")
def test_forward_random(nh, oracle_mod, case):
    import test_parity_fwd as TF
    i, kind, rows, cols, xt, wt, yt, weight, bias, in_place = case
    if kind == "ln":
        c = wl.rows_case(rows, cols, x_t=xt, dy_t=xt, w_t=wt, seed=6000 + i, with_bias=True)
        TF._ln_fwd_case(nh, oracle_mod, c, yt, weight=weight, bias=bias, in_place=in_place and yt == xt)
    else:
        c = wl.rows_case(rows, cols, x_t=xt, dy_t=xt, w_t=xt, seed=6000 + i)
        TF._rms_fwd_case(nh, oracle_mod, c, weight=weight, in_place=in_place)


def _bda_cases():
    rng = np.random.Generator(np.random.PCG64(4444))
    dts = (wl.F32, wl.BF16)
    cases = []
    for i in range(10):
        cols = int(rng.choice(_FWD_COLS[4:])) if rng.random() < 0.7 else int(rng.integers(1, 20000))
        rows = int(max(1, min(65536, int(rng.integers(1, 1_000_000)) // cols)))
        xt, dyt, wt = (dts[int(rng.integers(2))] for _ in range(3))
        flags = tuple(bool(rng.random() < 0.8) for _ in range(3))
        need = tuple(bool(rng.random() < 0.85) for _ in range(5))
        cases.append((i, rows, cols, xt, dyt, wt, float(rng.uniform(0.0, 0.5)), flags, need))
    return cases


@pytest.mark.parametrize("case", _bda_cases(), ids=lambda c: f"bda{c[0]}")
def test_bda_random(nh, oracle_mod, case):
    import test_parity_bda as TB
    i, rows, cols, xt, dyt, wt, p_drop, (weight, dres, mask), need = case
    c = wl.bda_case(rows, cols, x_t=xt, dy_t=dyt, w_t=wt, seed=6100 + i, p_drop=p_drop)
    TB._bda_case(nh, oracle_mod, c, weight=weight, dres=dres, mask=mask, need=need)


def _infer_cases():
    rng = np.random.Generator(np.random.PCG64(4545))
    cases = []
    for i in range(8):
        C = int(rng.choice([1, 3, 16, 64, 256, 1024]))
        HW = int(rng.choice([1, 2, 3, 7, 49, 196, 784, 1000, 3136]))
        N = int(max(1, min(4096, int(rng.integers(1, 4_000_000)) // (C * HW))))
        cases.append((i, N, C, HW, wl.F32 if rng.random() < 0.5 else wl.BF16,
                      ["none", "relu", "leaky_relu"][int(rng.integers(0, 3))], bool(rng.random() < 0.8)))
    return cases


@pytest.mark.parametrize("case", _infer_cases(), ids=lambda c: f"infer{c[0]}")
def test_bn_infer_random(nh, oracle_mod, case):
    from helpers import dev
    i, N, C, HW, io, act, affine = case
    c = wl.bn_case(N, C, HW, 1, io, seed=6200 + i, x_mean=1.0, x_std=1.0, beta_std=0.5)
    rng = np.random.Generator(np.random.PCG64(6300 + i))
    rm = wl.round_f32(rng.normal(0.0, 1.0, size=C))
    rv = wl.round_f32(rng.uniform(0.2, 4.0, size=C))
    g, b = (c.gamma, c.beta) if affine else (None, None)
    print(f"[bn infer random {i}] N={N} C={C} HW={HW} io={io} act={act} affine={affine}", flush=True)
    want = oracle_mod.bn_infer(c.x.value, g, b, rm, rv, act, 0.1, eps=c.eps)
    y = nh.bn_forward_infer(dev(c.x), dev(rm), dev(rv), dev(g) if affine else None, dev(b) if affine else None,
                            c.eps, act=act, slope=0.1)
    torch.cuda.synchronize()
    check("y", host(y), want, io)
