"""GPU parity of layernorm_backward / rmsnorm_backward against the CPU fp64
oracle, element by element: normwise relative error <= 2e-5 for fp32
outputs and <= 8e-3 for bf16 outputs."""
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


TDT = {wl.F32: "f32", wl.BF16: "bf16"}


def _torch_dtype(t):
    return torch.float32 if t == wl.F32 else torch.bfloat16


# ---------------------------------------------------------------- LayerNorm
def _ln_case(nh, oracle_mod, c: wl.RowsCase, dx_t, *, weight=True, need=(True, True, True),
             override_blocks=0):
    mean, rstd = oracle_mod.layernorm_stats(c.x.value, eps=c.eps)
    mean32, rstd32 = mean.astype(np.float32), rstd.astype(np.float32)
    w = c.w.value if weight else None
    want_dx, want_dw, want_db = oracle_mod.layernorm_backward(
        c.x.value, c.dy.value, mean32.astype(np.float64), rstd32.astype(np.float64), w)
    print(f"[ln parity] {c.name} rows={c.rows} cols={c.cols} x={c.x.dtype} dy={c.dy.dtype} "
          f"w={c.w.dtype if weight else None} dx={dx_t} blocks={nh.rows_plan(c.rows, c.cols)}",
          flush=True)
    if override_blocks:
        nh.plan_override("rows_blocks", override_blocks)
    try:
        dx, dw, db = nh.layernorm_backward(
            dev(c.dy), dev(c.x), dev(mean32), dev(rstd32), dev(c.w) if weight else None,
            dx_dtype=_torch_dtype(dx_t), w_dtype=_torch_dtype(c.w.dtype),
            need_dx=need[0], need_dweight=need[1], need_dbias=need[2])
        torch.cuda.synchronize()
    finally:
        if override_blocks:
            nh.plan_override("rows_blocks", 0)
    if need[0]:
        check("dx", host(dx), want_dx, dx_t)
    if need[1]:
        check("dweight", host(dw), want_dw, c.w.dtype)
    if need[2]:
        check("dbias", host(db), want_db, c.w.dtype)
    return dx, dw, db


def test_ln_full_config(nh, oracle_mod):
    """(16,512,1600): x fp32, dy bf16, weight bf16, saved mean/rstd fp32;
    dx fp32, dweight/dbias bf16."""
    _ln_case(nh, oracle_mod, wl.ln_bwd(), wl.F32)


@pytest.mark.parametrize("xt,dyt,wt,dxt", list(itertools.product((wl.F32, wl.BF16), repeat=4)))
def test_ln_dtype_mix(nh, oracle_mod, xt, dyt, wt, dxt):
    c = wl.rows_case(300, 1600, x_t=xt, dy_t=dyt, w_t=wt, seed=51)
    _ln_case(nh, oracle_mod, c, dxt)


@pytest.mark.parametrize("rows,cols,xt", [
    (1, 1600, wl.F32),        # one row
    (7, 4, wl.F32),           # one group per row
    (513, 4096, wl.F32),      # 4 groups per thread, teams of 4
    (100, 8192, wl.F32),      # 8 groups per thread, teams of 2
    (77, 8196, wl.F32),       # wider than a 256-thread team: 512-thread team
    (64, 1001, wl.F32),       # width not a multiple of the group: generic
    (50, 2050, wl.BF16),      # bf16 rows, ragged groups per thread
    (33, 16384, wl.BF16),     # all-bf16 row too wide for LayerNorm's vector path
    (1000, 64, wl.BF16),      # many short rows
])
def test_ln_shapes(nh, oracle_mod, rows, cols, xt):
    c = wl.rows_case(rows, cols, x_t=xt, dy_t=wl.BF16, w_t=wl.BF16, seed=rows + cols)
    _ln_case(nh, oracle_mod, c, xt)


def test_ln_no_weight_and_partial_outputs(nh, oracle_mod):
    c = wl.rows_case(129, 1600, x_t=wl.F32, dy_t=wl.BF16, w_t=wl.F32, seed=52)
    _ln_case(nh, oracle_mod, c, wl.F32, weight=False)
    _ln_case(nh, oracle_mod, c, wl.F32, need=(True, False, False))
    _ln_case(nh, oracle_mod, c, wl.F32, need=(False, True, False))
    _ln_case(nh, oracle_mod, c, wl.F32, need=(False, False, True))


@pytest.mark.parametrize("blocks", [1, 5, 300])
def test_ln_forced_blocks(nh, oracle_mod, blocks):
    c = wl.rows_case(300, 1600, x_t=wl.F32, dy_t=wl.BF16, w_t=wl.BF16, seed=53)
    _ln_case(nh, oracle_mod, c, wl.F32, override_blocks=blocks)


def test_ln_zero_rows_gives_zero_grads(nh):
    x = torch.empty((0, 40), device="cuda")
    dy = torch.empty((0, 40), device="cuda")
    mean = torch.empty(0, device="cuda")
    dx, dw, db = nh.layernorm_backward(dy, x, mean, mean, torch.ones(40, device="cuda"))
    torch.cuda.synchronize()
    assert dx.numel() == 0 and bool(torch.all(dw == 0)) and bool(torch.all(db == 0))


def test_ln_bit_identical_runs(nh, oracle_mod):
    c = wl.ln_bwd()
    mean, rstd = oracle_mod.layernorm_stats(c.x.value, eps=c.eps)
    args = (dev(c.dy), dev(c.x), dev(mean.astype(np.float32)), dev(rstd.astype(np.float32)), dev(c.w))
    a = nh.layernorm_backward(*args, dx_dtype=torch.float32)
    b = nh.layernorm_backward(*args, dx_dtype=torch.float32)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.int16) if u.dtype == torch.bfloat16 else u.view(torch.int32),
                           v.view(torch.int16) if v.dtype == torch.bfloat16 else v.view(torch.int32))


# ------------------------------------------------------------------ RMSNorm
def _rms_case(nh, oracle_mod, c: wl.RowsCase, *, saved=True, weight=True, need=(True, True),
              override_blocks=0):
    rms = oracle_mod.rmsnorm_rms(c.x.value, eps=c.eps)
    rms32 = rms.astype(np.float32)
    w = c.w.value if weight else np.ones(c.cols)
    want_dx, want_dw = oracle_mod.rmsnorm_backward(
        c.x.value, c.dy.value, w, rms32.astype(np.float64) if saved else None, eps=c.eps)
    print(f"[rms parity] {c.name} rows={c.rows} cols={c.cols} t={c.x.dtype} saved={saved} "
          f"weight={weight}", flush=True)
    if override_blocks:
        nh.plan_override("rows_blocks", override_blocks)
    try:
        dx, dw = nh.rmsnorm_backward(dev(c.dy), dev(c.x), dev(rms32) if saved else None,
                                     dev(c.w) if weight else None, c.eps,
                                     need_dx=need[0], need_dweight=need[1])
        torch.cuda.synchronize()
    finally:
        if override_blocks:
            nh.plan_override("rows_blocks", 0)
    if need[0]:
        check("dx", host(dx), want_dx, c.x.dtype)
    if need[1]:
        check("dweight", host(dw), want_dw, c.x.dtype)
    return dx, dw


@pytest.mark.parametrize("dt", [wl.BF16, wl.F32])
@pytest.mark.parametrize("saved", [True, False])
def test_rms_full_config(nh, oracle_mod, dt, saved):
    """(2048, 8192) bf16 and fp32, saved rms and recompute mode."""
    _rms_case(nh, oracle_mod, wl.rms_bwd(dt), saved=saved)


@pytest.mark.parametrize("rows,cols,dt", [
    (1, 8192, wl.BF16),
    (3, 8, wl.BF16),
    (257, 1024, wl.F32),
    (100, 2048, wl.BF16),
    (40, 16384, wl.BF16),   # 64 elements per thread: generic path
    (20, 12288, wl.F32),    # wider than the fp32 vector path: generic
    (31, 999, wl.F32),      # ragged width: generic
    (17, 4100, wl.BF16),    # ragged groups per thread
])
def test_rms_shapes(nh, oracle_mod, rows, cols, dt):
    c = wl.rows_case(rows, cols, x_t=dt, dy_t=dt, w_t=dt, seed=rows * 7 + cols)
    _rms_case(nh, oracle_mod, c, saved=(rows % 2 == 1))


def test_rms_no_weight_and_partial_outputs(nh, oracle_mod):
    c = wl.rows_case(64, 4096, x_t=wl.BF16, dy_t=wl.BF16, w_t=wl.BF16, seed=61)
    _rms_case(nh, oracle_mod, c, weight=False, need=(True, False))
    _rms_case(nh, oracle_mod, c, need=(False, True))


@pytest.mark.parametrize("blocks", [1, 7, 2048])
def test_rms_forced_blocks(nh, oracle_mod, blocks):
    _rms_case(nh, oracle_mod, wl.rms_bwd(wl.BF16, rows=512, cols=8192), override_blocks=blocks)


@pytest.mark.parametrize("dt", [wl.BF16, wl.F32])
def test_rms_bit_identical_runs(nh, oracle_mod, dt):
    c = wl.rms_bwd(dt)
    rms = dev(oracle_mod.rmsnorm_rms(c.x.value, eps=c.eps).astype(np.float32))
    args = (dev(c.dy), dev(c.x), rms, dev(c.w), c.eps)
    a = nh.rmsnorm_backward(*args)
    b = nh.rmsnorm_backward(*args)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        iv = torch.int16 if u.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(u.view(iv), v.view(iv))


def test_rows_error_paths(nh):
    x = torch.randn(4, 8, device="cuda")
    with pytest.raises(nh.NormHipError) as ei:
        nh.rmsnorm_backward(x, x, None, None, eps=-1.0)
    assert ei.value.status == 6
    with pytest.raises(nh.NormHipError) as ei:
        nh.rmsnorm_backward(x, x, None, None, workspace=torch.empty(4, dtype=torch.uint8, device="cuda"))
    assert ei.value.status == 4


@pytest.mark.parametrize("depth", [1, 2, 3, 4])
def test_rows_pipeline_depths(nh, oracle_mod, depth):
    """Every row-pipeline depth of the vector kernels (forced through the
    plan override) gives the oracle's results, for rows that do not divide
    evenly among the teams."""
    nh.plan_override("rows_depth", depth)
    try:
        c = wl.rows_case(1037, 1600, x_t=wl.F32, dy_t=wl.BF16, w_t=wl.BF16, seed=91)
        _ln_case(nh, oracle_mod, c, wl.F32, override_blocks=100)
        r = wl.rows_case(333, 4096, x_t=wl.BF16, dy_t=wl.BF16, w_t=wl.BF16, seed=92)
        _rms_case(nh, oracle_mod, r, saved=True, override_blocks=50)
    finally:
        nh.plan_override("rows_depth", 0)


@pytest.mark.parametrize("cx", [8, 16, 64])
def test_rows_colsum_widths(nh, oracle_mod, cx):
    """Every column-finalize block width gives the oracle's column sums."""
    nh.plan_override("colsum_cols", cx)
    try:
        c = wl.rows_case(777, 1000, x_t=wl.F32, dy_t=wl.F32, w_t=wl.F32, seed=93)
        _ln_case(nh, oracle_mod, c, wl.F32, override_blocks=300)
    finally:
        nh.plan_override("colsum_cols", 0)


@pytest.mark.parametrize("rows,cols,xt,dyt", [(64, 16384, wl.F32, wl.BF16), (96, 12288, wl.BF16, wl.BF16),
                                              (40, 16384, wl.F32, wl.F32), (70, 10240, wl.BF16, wl.F32),
                                              (9, 32768, wl.BF16, wl.BF16)])
def test_wide_rows(nh, oracle_mod, rows, cols, xt, dyt):
    """Rows too wide for a 256-thread team: 512-thread teams up to 16384
    columns, the generic coefficient + strip kernels beyond (32768)."""
    c = wl.rows_case(rows, cols, x_t=xt, dy_t=dyt, w_t=wl.BF16, seed=rows + cols)
    _ln_case(nh, oracle_mod, c, wl.F32)
    r = wl.rows_case(rows, cols, x_t=xt, dy_t=xt, w_t=xt, seed=rows * 3 + cols)
    _rms_case(nh, oracle_mod, r, saved=True)
    _rms_case(nh, oracle_mod, r, saved=False)


@pytest.mark.parametrize("rows,cols,dt,blocks", [(2048, 8192, wl.BF16, 0), (1001, 8192, wl.F32, 0),
                                                 (777, 1000, wl.BF16, 0), (37, 4096, wl.F32, 5),
                                                 (3, 2048, wl.BF16, 0)])
def test_rms_two_team_blocks(nh, oracle_mod, rows, cols, dt, blocks):
    """RMSNorm with two row teams per block (rows_teams = 2): interleaved rows,
    the teams' column sums added through LDS; odd row counts leave one team
    a row short on the last iteration."""
    c = wl.rows_case(rows, cols, x_t=dt, dy_t=dt, w_t=dt, seed=rows + 5 * cols)
    nh.plan_override("rows_teams", 2)
    try:
        for saved in (True, False):
            _rms_case(nh, oracle_mod, c, saved=saved, override_blocks=blocks)
        _rms_case(nh, oracle_mod, c, need=(False, True))
    finally:
        nh.plan_override("rows_teams", 0)


@pytest.mark.parametrize("rows,cols,xt,dyt,teams", [(8192, 1600, wl.BF16, wl.BF16, 0), (1001, 1024, wl.F32, wl.BF16, 2),
                                                    (777, 1600, wl.F32, wl.F32, 2), (3, 512, wl.BF16, wl.BF16, 2),
                                                    (2048, 8192, wl.BF16, wl.BF16, 0), (300, 1600, wl.F32, wl.BF16, 1),
                                                    (1000, 4096, wl.BF16, wl.BF16, 0), (600, 2048, wl.F32, wl.F32, 0),
                                                    (777, 1600, wl.F32, wl.BF16, 0)])
def test_ln_team_plans(nh, oracle_mod, rows, cols, xt, dyt, teams):
    """LayerNorm with one or two row teams per block (automatic or forced by
    rows_teams), one or two blocks per CU: the oracle's results either way."""
    c = wl.rows_case(rows, cols, x_t=xt, dy_t=dyt, w_t=wl.BF16, seed=rows + 3 * cols)
    nh.plan_override("rows_teams", teams)
    try:
        _ln_case(nh, oracle_mod, c, xt)
        _ln_case(nh, oracle_mod, c, wl.F32, need=(False, True, True))
    finally:
        nh.plan_override("rows_teams", 0)
