"""GPU parity of the generic backward row kernels against the CPU oracle.

Shapes the register-resident row kernels do not take -- rows of up to 64
columns with an odd width or a misaligned tensor (the narrow kernel, a lane
subgroup per row), and wider rows that are odd, misaligned or wider than a
512-thread team holds (the per-row coefficient kernel followed by the
column-strip kernel) -- through LayerNorm, RMSNorm and the bias + dropout +
add + LayerNorm backward.  Every output is compared with the oracle at the
parity tolerances; the per-kernel timing records show which path ran."""
import numpy as np
import pytest

from bwd_bn_stats_amd import workloads as wl

from helpers import check, host, place

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

F32, BF16 = wl.F32, wl.BF16


@pytest.fixture(scope="module")
def nh():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bwd_bn_stats_amd import normhip
    return normhip


def _tdt(t):
    return torch.float32 if t == F32 else torch.bfloat16


# rows, cols, x, dy, weight dtypes, element offset of the row tensors, path
CASES = [
    (3001, 1, F32, F32, F32, 1, "narrow"),
    (2500, 5, BF16, BF16, BF16, 0, "narrow"),       # odd width, aligned
    (4099, 33, F32, BF16, BF16, 2, "narrow"),
    (1000, 64, BF16, F32, F32, 1, "narrow"),        # widest narrow row, misaligned
    (777, 63, F32, F32, BF16, 0, "narrow"),
    (2000, 128, BF16, BF16, BF16, 0, "narrow"),     # aligned short rows: vector groups, 16 lanes per row
    (777, 256, F32, BF16, BF16, 0, "narrow"),       # 64 groups of 4: the widest fp32 narrow row
    (1000, 512, BF16, BF16, BF16, 0, "narrow"),     # 64 groups of 8
    (5003, 16, BF16, BF16, BF16, 0, "narrow"),      # two lanes per row
    (300, 65, F32, BF16, F32, 1, "strip"),          # narrowest strip row
    (513, 1601, BF16, BF16, BF16, 0, "strip"),      # odd width: scalar groups
    (100, 5000, F32, F32, BF16, 1, "strip"),        # few long rows: 8 team segments per row
    (1100, 1100, F32, BF16, F32, 1, "strip"),       # one team per row
    (2000, 700, BF16, F32, BF16, 1, "strip"),       # one wave per row
    (37, 20000, BF16, F32, F32, 3, "strip"),
    (200, 20000, BF16, BF16, BF16, 0, "strip"),     # aligned, too wide: 8-element groups
    (70, 40960, F32, F32, F32, 0, "strip"),         # aligned fp32: 4-element groups
    (40, 24576, F32, BF16, BF16, 0, "strip"),
]


def _path_ran(nh, path):
    _, n = nh.timing_read("rows_coef")
    assert (n > 0) == (path == "strip"), f"expected the {path} path, rows_coef launches: {n}"


def _run_case(nh, oracle_mod, case, blocks=0):
    rows, cols, xt, dyt, wt, offset, path = case
    print(f"[generic] rows={rows} cols={cols} x={xt} dy={dyt} w={wt} offset={offset} path={path} "
          f"blocks={blocks or 'auto'}", flush=True)
    c = wl.bda_case(rows, cols, x_t=xt, dy_t=dyt, w_t=wt, seed=rows * 7 + cols, p_drop=0.25)
    ln = c.ln
    x, dy, w = place(ln.x, offset), place(ln.dy, offset), place(ln.w, offset)
    mean, rstd = oracle_mod.layernorm_stats(ln.x.value, eps=ln.eps)
    m32, r32 = mean.astype(np.float32), rstd.astype(np.float32)
    dm, dr = torch.from_numpy(m32).cuda(), torch.from_numpy(r32).cuda()
    if blocks:
        nh.plan_override("rows_blocks", blocks)
    nh.timing_enable(True)
    try:
        # LayerNorm backward, dx in x's dtype
        wdx, wdw, wdb = oracle_mod.layernorm_backward(ln.x.value, ln.dy.value, m32, r32, ln.w.value)
        dx, dw, db = nh.layernorm_backward(dy, x, dm, dr, w, dx_dtype=_tdt(xt))
        torch.cuda.synchronize()
        check("ln dx", host(dx), wdx, xt)
        check("ln dweight", host(dw), wdw, wt)
        check("ln dbias", host(db), wdb, wt)
        _path_ran(nh, path)
        # bias + dropout + add + LayerNorm backward on the same rows
        mask = torch.from_numpy(c.mask).cuda()
        dres = torch.from_numpy(c.dresidual).cuda()
        want = oracle_mod.bda_layernorm_backward(ln.x.value, ln.dy.value, m32, r32, ln.w.value,
                                                 c.dresidual, c.mask, c.scale)
        got = nh.bda_layernorm_backward(dy, x, dm, dr, w, dres, mask, c.scale)
        torch.cuda.synchronize()
        for name, g, wv, dt in zip(("dh", "da", "dweight", "dbias", "dbias_in"), got, want,
                                   (F32, dyt, wt, wt, wt)):
            check(f"bda {name}", host(g), wv, dt)
        # RMSNorm backward, one dtype (x's) for x, dy, weight; rms saved and recomputed
        r = wl.rows_case(rows, cols, x_t=xt, dy_t=xt, w_t=xt, seed=rows * 11 + cols)
        rx, rdy, rw = place(r.x, offset), place(r.dy, offset), place(r.w, offset)
        _, wrms = oracle_mod.rmsnorm_forward(r.x.value, r.w.value, eps=r.eps)
        rms32 = wrms.astype(np.float32)
        for saved in (True, False):
            wdx, wdw = oracle_mod.rmsnorm_backward(r.x.value, r.dy.value, r.w.value,
                                                   rms32 if saved else None, eps=r.eps)
            dx, dw = nh.rmsnorm_backward(rdy, rx, torch.from_numpy(rms32).cuda() if saved else None,
                                         rw, r.eps)
            torch.cuda.synchronize()
            check(f"rms dx (saved={saved})", host(dx), wdx, xt)
            check(f"rms dweight (saved={saved})", host(dw), wdw, xt)
    finally:
        nh.timing_enable(False)
        if blocks:
            nh.plan_override("rows_blocks", 0)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}x{c[1]}-{c[6]}-off{c[5]}")
def test_generic_rows(nh, oracle_mod, case):
    _run_case(nh, oracle_mod, case)


@pytest.mark.parametrize("case,blocks", [
    ((513, 1601, BF16, BF16, BF16, 0, "strip"), 1),     # one chunk of all rows
    ((513, 1601, BF16, BF16, BF16, 0, "strip"), 7),     # ragged last chunk
    ((513, 1601, F32, F32, F32, 1, "strip"), 513),      # a chunk per row
    ((3001, 5, F32, BF16, F32, 1, "narrow"), 1),        # one block walks every row
    ((3001, 5, F32, BF16, F32, 1, "narrow"), 1000),     # fewer rows than row slots
])
def test_generic_forced_blocks(nh, oracle_mod, case, blocks):
    _run_case(nh, oracle_mod, case, blocks=blocks)


@pytest.mark.parametrize("rows,cols,offset", [(2000, 17, 1), (300, 3000, 1), (64, 20000, 0)])
def test_generic_bit_identical_runs(nh, rows, cols, offset):
    """Two calls on the same inputs give the same bits (no atomics, fixed
    summation order on the generic path too)."""
    c = wl.rows_case(rows, cols, x_t=BF16, dy_t=BF16, w_t=BF16, seed=rows + cols)
    x, dy, w = place(c.x, offset), place(c.dy, offset), place(c.w, offset)
    m = torch.zeros(rows, device="cuda")
    r = torch.ones(rows, device="cuda")
    a = nh.layernorm_backward(dy, x, m, r, w, dx_dtype=torch.float32)
    b = nh.layernorm_backward(dy, x, m, r, w, dx_dtype=torch.float32)
    ra = nh.rmsnorm_backward(dy, x, None, w, 1e-5)
    rb = nh.rmsnorm_backward(dy, x, None, w, 1e-5)
    torch.cuda.synchronize()
    for u, v in zip(list(a) + list(ra), list(b) + list(rb)):
        bits = (lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32))
        assert torch.equal(bits(u), bits(v))


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}x{c[1]}-{c[6]}-off{c[5]}")
def test_generic_forward(nh, oracle_mod, case):
    """LayerNorm forward (y in x's dtype, and fp32 y from bf16 x) and RMSNorm
    forward on the same shapes and layouts: the narrow kernel for rows of at
    most 64 columns, a team per row (256 or 1024 threads) beyond."""
    rows, cols, xt, _, wt, offset, _ = case
    print(f"[generic fwd] rows={rows} cols={cols} x={xt} w={wt} offset={offset}", flush=True)
    c = wl.rows_case(rows, cols, x_t=xt, dy_t=xt, w_t=wt, seed=rows * 5 + cols, with_bias=True)
    x, w, b = place(c.x, offset), place(c.w, offset), place(c.b, offset)
    wy, wm, wr = oracle_mod.layernorm_forward(c.x.value, c.w.value, c.b.value, eps=c.eps)
    for yt in sorted({xt, F32}):
        y, m, r = nh.layernorm_forward(x, w, b, c.eps, y_dtype=_tdt(yt))
        torch.cuda.synchronize()
        check(f"ln y ({yt})", host(y), wy, yt)
        check("ln mean", host(m), wm, F32)
        check("ln rstd", host(r), wr, F32)
    rc = wl.rows_case(rows, cols, x_t=xt, dy_t=xt, w_t=xt, seed=rows * 13 + cols)
    rx, rw = place(rc.x, offset), place(rc.w, offset)
    wy, wrms = oracle_mod.rmsnorm_forward(rc.x.value, rc.w.value, eps=rc.eps)
    y, rms = nh.rmsnorm_forward(rx, rw, rc.eps)
    torch.cuda.synchronize()
    check("rms y", host(y), wy, xt)
    check("rms rms", host(rms), wrms, F32)


@pytest.mark.parametrize("rows,cols,dt", [(2000, 128, BF16), (1001, 64, F32), (300, 512, BF16)])
def test_short_aligned_rows_on_team_kernels(nh, oracle_mod, rows, cols, dt):
    """With the "rows_narrow" override the aligned short rows stay on the
    256-thread team kernels: still the oracle's results."""
    nh.plan_override("rows_narrow", 1)
    try:
        c = wl.bda_case(rows, cols, x_t=dt, dy_t=dt, w_t=dt, seed=rows + cols, p_drop=0.2)
        ln = c.ln
        mean, rstd = oracle_mod.layernorm_stats(ln.x.value, eps=ln.eps)
        m32, r32 = mean.astype(np.float32), rstd.astype(np.float32)
        from helpers import dev
        x, dy, w = dev(ln.x), dev(ln.dy), dev(ln.w)
        wdx, wdw, wdb = oracle_mod.layernorm_backward(ln.x.value, ln.dy.value, m32, r32, ln.w.value)
        dx, dw, db = nh.layernorm_backward(dy, x, torch.from_numpy(m32).cuda(), torch.from_numpy(r32).cuda(), w,
                                           dx_dtype=_tdt(dt))
        y, fm, fr = nh.layernorm_forward(x, w, None, ln.eps)
        torch.cuda.synchronize()
        check("ln dx", host(dx), wdx, dt)
        check("ln dweight", host(dw), wdw, dt)
        check("ln dbias", host(db), wdb, dt)
        wy, wm, wr = oracle_mod.layernorm_forward(ln.x.value, ln.w.value, eps=ln.eps)
        check("ln y", host(y), wy, dt)
        check("ln mean", host(fm), wm, F32)
    finally:
        nh.plan_override("rows_narrow", 0)
