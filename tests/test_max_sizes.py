"""Largest inputs the ABI accepts (element counts just below 2^31), checked
against closed forms on every element.

The oracle cannot run 2^31 elements in a test, so these inputs are built so
that the exact results are known: each channel (or row) alternates between
a + b and a - b along its planes (or columns), with dyadic a and b exact in
bf16.  Then mean = a and var = b^2 exactly (the odd-length case shifts the
mean by b/M), every normalized value is +-b/sqrt(b^2 + eps), and with a
constant incoming gradient the parameter gradients are closed-form sums.
The results are compared on the GPU with torch elementwise ops against
those values, at the parity tolerances (normwise 2e-5 fp32, 8e-3 bf16).

The inputs are structured, not random: 16-30 GB of device memory per test,
built on the device.
"""
import math

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

EPS = 1e-5


@pytest.fixture(scope="module")
def nh():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bwd_bn_stats_amd import normhip
    return normhip


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _alt(n, dtype):
    """+1, -1, +1, ... of length n on the device."""
    s = torch.ones(n, dtype=dtype, device="cuda")
    s[1::2] = -1
    return s


def _check_two_valued(t, v_even, v_odd, tol, name):
    """Elements at even positions of t's last dimension against v_even, odd
    positions against v_odd (scalars); normwise error over the tensor."""
    scale = max(abs(v_even), abs(v_odd))
    err = max(float((t[..., 0::2].float() - v_even).abs().max()),
              float((t[..., 1::2].float() - v_odd).abs().max()))
    print(f"  {name}: normwise error {err / scale:.2e} (tol {tol:.0e})", flush=True)
    assert err <= tol * scale, name


@pytest.mark.parametrize("shape,io", [((2, 4, (1 << 28) - 8), "bf16"),   # vector units
                                      ((1, 1, (1 << 31) - 1), "bf16")])  # one channel, scalar units
def test_bn_max_size(nh, shape, io):
    N, C, HW = shape
    M = N * HW
    tdt = torch.bfloat16
    print(f"[max size] BatchNorm N={N} C={C} HW={HW} ({N * C * HW} elements) io={io}", flush=True)
    a = torch.tensor([0.5, -1.0, 2.0, 3.0][:C], dtype=torch.float64)
    b = torch.tensor([0.25, 0.5, 1.0, 2.0][:C], dtype=torch.float64)
    d = torch.tensor([1.0, -0.5, 2.0, 0.25][:C], dtype=torch.float64)
    gamma = torch.tensor([1.25, 0.75, 1.0, 0.5][:C], dtype=torch.float32)
    beta = torch.tensor([0.1, -0.2, 0.3, 0.0][:C], dtype=torch.float32)
    s = _alt(HW, tdt)
    x = torch.empty((N, C, HW), dtype=tdt, device="cuda")
    for c in range(C):
        x[:, c, :] = (a[c].item() + b[c].item() * s).to(tdt)
    del s
    # exact statistics: mean a + b*k/M, where k = (#even - #odd) per plane * N
    k = N * (HW % 2)
    mean = a + b * k / M
    ex2 = (a + b) ** 2 * (N * ((HW + 1) // 2)) / M + (a - b) ** 2 * (N * (HW // 2)) / M
    var = ex2 - mean ** 2
    inv = 1.0 / torch.sqrt(var + EPS)
    g64, b64 = gamma.double(), beta.double()
    rm, rv = torch.zeros(C, device="cuda"), torch.ones(C, device="cuda")
    y, stats = nh.bn_forward_train(x, gamma.cuda(), beta.cuda(), rm, rv, 0.1, EPS)
    torch.cuda.synchronize()
    st = stats.cpu().double()
    for i, (name, want) in enumerate((("mean", mean), ("var", var), ("inv_std", inv),
                                      ("scale", g64 * inv))):
        err = float((st[i] - want).abs().max() / want.abs().max())
        print(f"  stats.{name}: {err:.2e}", flush=True)
        assert err <= 2e-5
    want_rm, want_rv = 0.1 * mean, 0.9 + 0.1 * var * M / (M - 1)
    assert float((rm.cpu().double() - want_rm).abs().max() / want_rm.abs().max()) <= 2e-5
    assert float((rv.cpu().double() - want_rv).abs().max() / want_rv.abs().max()) <= 2e-5
    for c in range(C):
        vp = float(g64[c] * (a[c] + b[c] - mean[c]) * inv[c] + b64[c])
        vn = float(g64[c] * (a[c] - b[c] - mean[c]) * inv[c] + b64[c])
        _check_two_valued(y[:, c, :], vp, vn, 8e-3, f"y[c={c}]")
    del y
    # backward with dy = d_c everywhere: dbeta = M*d, dgamma = inv*d*sum(x - mean) = 0,
    # dx = 0 (dy*scale + k2 cancel)
    dy = torch.empty_like(x)
    for c in range(C):
        dy[:, c, :] = d[c].item()
    dx, grads = nh.bn_backward(dy, x, stats)
    torch.cuda.synchronize()
    gr = grads.cpu().double()
    want_db = M * d
    assert float((gr[1] - want_db).abs().max() / want_db.abs().max()) <= 2e-5
    # |dgamma| is 0 up to one element's worth of rounding of x - mean
    dg_scale = (inv * d.abs() * b).max() * M
    assert float(gr[0].abs().max()) <= 2e-5 * float(dg_scale)
    dx_scale = float((d.abs() * g64 * inv).max())
    dx_err = float(dx.float().abs().max())
    print(f"  dx: max |dx| {dx_err:.2e} vs |dy*scale| {dx_scale:.2e}", flush=True)
    assert dx_err <= 2e-5 * dx_scale


@pytest.mark.parametrize("N,C,dtype", [((1 << 31) // 256 - 1, 256, torch.bfloat16),  # 32 column lanes
                                        ((1 << 31) // 64 - 1, 64, torch.float32)])    # 16 column lanes
def test_bn_rows_layout_max_size(nh, N, C, dtype):
    """BatchNorm over [N, C] (the row layout, HW = 1) just below 2^31
    elements.  Channel c alternates a_c + b_c, a_c - b_c along the N rows
    (N odd: the mean moves by b_c/N), and dy = d_c everywhere."""
    tol = 8e-3 if dtype == torch.bfloat16 else 2e-5
    print(f"[max size] BatchNorm row layout N={N} C={C} ({N * C} elements) {dtype}", flush=True)
    cyc = torch.arange(C) % 4
    a = torch.tensor([0.5, -1.0, 2.0, 3.0], dtype=torch.float64)[cyc]
    b = torch.tensor([0.25, 0.5, 1.0, 2.0], dtype=torch.float64)[cyc]
    d = torch.tensor([1.0, -0.5, 2.0, 0.25], dtype=torch.float64)[cyc]
    gamma = torch.tensor([1.25, 0.75, 1.0, 0.5], dtype=torch.float32)[cyc]
    beta = torch.tensor([0.1, -0.2, 0.3, 0.0], dtype=torch.float32)[cyc]
    x = torch.empty((N, C, 1, 1), dtype=dtype, device="cuda")
    a_d, b_d = a.float().cuda(), b.float().cuda()
    step = 1 << 20
    for r0 in range(0, N, step):
        r1 = min(N, r0 + step)
        sgn = 1.0 - 2.0 * (torch.arange(r0, r1, device="cuda") % 2).float()
        x[r0:r1, :, 0, 0] = (a_d[None, :] + b_d[None, :] * sgn[:, None]).to(dtype)
    M = N
    mean = a + b * (N % 2) / M
    ex2 = (a + b) ** 2 * ((N + 1) // 2) / M + (a - b) ** 2 * (N // 2) / M
    var = ex2 - mean ** 2
    inv = 1.0 / torch.sqrt(var + EPS)
    g64, b64 = gamma.double(), beta.double()
    rm, rv = torch.zeros(C, device="cuda"), torch.ones(C, device="cuda")
    y, stats = nh.bn_forward_train(x, gamma.cuda(), beta.cuda(), rm, rv, 0.1, EPS)
    torch.cuda.synchronize()
    st = stats.cpu().double()
    for i, (name, want) in enumerate((("mean", mean), ("var", var), ("inv_std", inv),
                                      ("scale", g64 * inv))):
        err = float((st[i] - want).abs().max() / want.abs().max())
        print(f"  stats.{name}: {err:.2e}", flush=True)
        assert err <= 2e-5
    want_rm, want_rv = 0.1 * mean, 0.9 + 0.1 * var * M / (M - 1)
    assert float((rm.cpu().double() - want_rm).abs().max() / want_rm.abs().max()) <= 2e-5
    assert float((rv.cpu().double() - want_rv).abs().max() / want_rv.abs().max()) <= 2e-5
    vp = (g64 * (a + b - mean) * inv + b64).float().cuda()
    vn = (g64 * (a - b - mean) * inv + b64).float().cuda()
    y2 = y.view(N, C)
    scale = float(torch.maximum(vp.abs(), vn.abs()).max())
    err = max(float((y2[0::2].float() - vp[None, :]).abs().max()),
              float((y2[1::2].float() - vn[None, :]).abs().max()))
    print(f"  y: normwise error {err / scale:.2e} (tol {tol:.0e})", flush=True)
    assert err <= tol * scale
    del y, y2
    dy = torch.empty_like(x)
    dy.view(N, C)[:] = d.to(dtype).cuda()[None, :]
    dx, grads = nh.bn_backward(dy, x, stats)
    torch.cuda.synchronize()
    gr = grads.cpu().double()
    want_db = M * d
    assert float((gr[1] - want_db).abs().max() / want_db.abs().max()) <= 2e-5
    dg_scale = (inv * d.abs() * b).max() * M
    assert float(gr[0].abs().max()) <= 2e-5 * float(dg_scale)
    dx_scale = float((d.abs() * g64 * inv).max())
    dx_err = float(dx.float().abs().max())
    print(f"  dx: max |dx| {dx_err:.2e} vs |dy*scale| {dx_scale:.2e}", flush=True)
    assert dx_err <= 2e-5 * dx_scale


def _rows_input(rows, cols, a_of_row, b, dtype):
    """x[r, j] = a_r + b*(+1, -1, ...)_j on the device."""
    s = _alt(cols, torch.float32)
    a = a_of_row(torch.arange(rows, device="cuda")).float()
    return (a[:, None] + b * s[None, :]).to(dtype)


def test_layernorm_max_size(nh):
    rows, cols = (1 << 18) - 1, 8192          # 2^31 - 8192 elements
    print(f"[max size] LayerNorm rows={rows} cols={cols} bf16", flush=True)
    b = 0.5
    a_of_row = lambda r: (r % 4).float() - 1.5
    x = _rows_input(rows, cols, a_of_row, b, torch.bfloat16)
    w = torch.ones(cols, dtype=torch.bfloat16, device="cuda")
    rstd_exact = 1.0 / math.sqrt(b * b + EPS)
    # forward: mean = a_r, rstd, y = +-b*rstd
    y, mean, rstd = nh.layernorm_forward(x, w, None, EPS)
    torch.cuda.synchronize()
    want_mean = a_of_row(torch.arange(rows, device="cuda")).float()
    assert float((mean - want_mean).abs().max()) <= 2e-5 * 1.5
    assert float((rstd.double() - rstd_exact).abs().max()) <= 2e-5 * rstd_exact
    v = b * rstd_exact
    _check_two_valued(y, v, -v, 8e-3, "y")
    del y
    # backward with dy = 1: dx = 0, dweight_j = rows*(+-b*rstd), dbias_j = rows
    dy = torch.ones_like(x)
    dx, dw, db = nh.layernorm_backward(dy, x, mean, rstd, w)
    torch.cuda.synchronize()
    dx_err = float(dx.float().abs().max())
    print(f"  dx: max |dx| {dx_err:.2e}", flush=True)
    assert dx_err <= 2e-5 * rstd_exact
    vw = rows * b * rstd_exact
    _check_two_valued(dw, vw, -vw, 8e-3, "dweight")
    assert float((db.float() - rows).abs().max()) <= 8e-3 * rows


def test_rmsnorm_max_size(nh):
    rows, cols = (1 << 18) - 1, 8192
    print(f"[max size] RMSNorm rows={rows} cols={cols} bf16", flush=True)
    b = 0.5
    x = _rows_input(rows, cols, lambda r: r.float() * 0, b, torch.bfloat16)
    w = torch.ones(cols, dtype=torch.bfloat16, device="cuda")
    rms_exact = math.sqrt(b * b + EPS)
    y, rms = nh.rmsnorm_forward(x, w, EPS)
    torch.cuda.synchronize()
    assert float((rms.double() - rms_exact).abs().max()) <= 2e-5 * rms_exact
    v = b / rms_exact
    _check_two_valued(y, v, -v, 8e-3, "y")
    del y
    # dy = 1, w = 1: sum g*x = 0, so dx = 1/rms; dweight_j = rows*(+-b/rms)
    dy = torch.ones_like(x)
    dx, dw = nh.rmsnorm_backward(dy, x, rms, w, EPS)
    torch.cuda.synchronize()
    dx_err = float((dx.float() - 1.0 / rms_exact).abs().max())
    print(f"  dx: max error {dx_err:.2e}", flush=True)
    assert dx_err <= 8e-3 / rms_exact
    vw = rows * b / rms_exact
    _check_two_valued(dw, vw, -vw, 8e-3, "dweight")


def test_bda_max_size(nh):
    rows, cols = (1 << 18) - 1, 8192
    print(f"[max size] bias+dropout+add LayerNorm backward rows={rows} cols={cols}", flush=True)
    b = 0.5
    a_of_row = lambda r: (r % 4).float() - 1.5
    x = _rows_input(rows, cols, a_of_row, b, torch.bfloat16)
    w = torch.ones(cols, dtype=torch.bfloat16, device="cuda")
    rstd_exact = 1.0 / math.sqrt(b * b + EPS)
    mean = a_of_row(torch.arange(rows, device="cuda")).float()
    rstd = torch.full((rows,), rstd_exact, dtype=torch.float32, device="cuda")
    dy = torch.ones_like(x)
    dres = torch.full((rows, cols), 0.25, dtype=torch.float32, device="cuda")
    mask = torch.zeros((rows, cols), dtype=torch.bool, device="cuda")
    mask[:, 0::2] = True
    # dx_ln = 0, so dh = 0.25, da = 0.5 on kept (even) columns, 0 elsewhere;
    # dbias_in_j = rows*0.5 on even columns
    dh, da, dw, db, dbi = nh.bda_layernorm_backward(dy, x, mean, rstd, w, dres, mask, 2.0)
    torch.cuda.synchronize()
    assert float((dh - 0.25).abs().max()) <= 2e-5 * 0.25
    _check_two_valued(da, 0.5, 0.0, 8e-3, "da")
    _check_two_valued(dbi, rows * 0.5, 0.0, 8e-3, "dbias_in")
    vw = rows * b * rstd_exact
    _check_two_valued(dw, vw, -vw, 8e-3, "dweight")
    assert float((db.float() - rows).abs().max()) <= 8e-3 * rows
