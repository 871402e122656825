"""GPU parity of bda_layernorm_backward (the backward of bias + dropout + add
+ LayerNorm) against the CPU fp64 oracle, element by element: normwise
relative error <= 2e-5 for fp32 outputs (dh, and da when dy is fp32) and
<= 8e-3 for bf16 outputs."""
import itertools

import numpy as np
import pytest

from bwd_bn_stats_amd import workloads as wl

from helpers import check, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

NAMES = ("dh", "da", "dweight", "dbias", "dbias_in")


@pytest.fixture(scope="module")
def nh():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bwd_bn_stats_amd import normhip
    return normhip


def _stats(oracle_mod, c):
    mean, rstd = oracle_mod.layernorm_stats(c.ln.x.value, eps=c.ln.eps)
    return mean.astype(np.float32), rstd.astype(np.float32)


def _bda_case(nh, oracle_mod, c: wl.BdaCase, *, weight=True, dres=True, mask=True, scale=None,
              need=(True,) * 5, override_blocks=0, mask_dev=None):
    ln = c.ln
    scale = c.scale if scale is None else scale
    mean32, rstd32 = _stats(oracle_mod, c)
    want = oracle_mod.bda_layernorm_backward(
        ln.x.value, ln.dy.value, mean32.astype(np.float64), rstd32.astype(np.float64),
        ln.w.value if weight else None, c.dresidual if dres else None, c.mask if mask else None,
        scale)
    print(f"[bda parity] rows={ln.rows} cols={ln.cols} x={ln.x.dtype} dy={ln.dy.dtype} "
          f"w={ln.w.dtype if weight else None} dres={dres} mask={mask} scale={scale} need={need} "
          f"blocks={override_blocks or nh.rows_plan(ln.rows, ln.cols)}", flush=True)
    if mask and mask_dev is None:
        mask_dev = torch.from_numpy(c.mask).cuda().bool()
    if override_blocks:
        nh.plan_override("rows_blocks", override_blocks)
    try:
        got = nh.bda_layernorm_backward(
            dev(ln.dy), dev(ln.x), dev(mean32), dev(rstd32), dev(ln.w) if weight else None,
            dev(c.dresidual) if dres else None, mask_dev if mask else None, scale,
            w_dtype=torch.float32 if ln.w.dtype == wl.F32 else torch.bfloat16,
            need_dh=need[0], need_da=need[1], need_dweight=need[2], need_dbias=need[3],
            need_dbias_in=need[4])
        torch.cuda.synchronize()
    finally:
        if override_blocks:
            nh.plan_override("rows_blocks", 0)
    dts = (wl.F32, ln.dy.dtype, ln.w.dtype, ln.w.dtype, ln.w.dtype)
    for name, g, w, dt, n in zip(NAMES, got, want, dts, need):
        if n:
            check(name, host(g), w, dt)
        else:
            assert g is None
    return got


def test_bda_full_config(nh, oracle_mod):
    """(16,512,1600): x fp32, dy bf16, weight bf16, fp32 incoming gradient,
    keep-mask with p = 0.1; dh fp32, da bf16, column gradients bf16."""
    _bda_case(nh, oracle_mod, wl.bda_bwd())


def test_bda_width_4096(nh, oracle_mod):
    """The fusion example's tensor width, 4096 columns."""
    _bda_case(nh, oracle_mod, wl.bda_case(512, 4096, seed=81))


@pytest.mark.parametrize("xt,dyt,wt", list(itertools.product((wl.F32, wl.BF16), repeat=3)))
def test_bda_dtype_mix(nh, oracle_mod, xt, dyt, wt):
    _bda_case(nh, oracle_mod, wl.bda_case(300, 1600, x_t=xt, dy_t=dyt, w_t=wt, seed=82))


@pytest.mark.parametrize("rows,cols,xt", [
    (1, 1600, wl.F32),        # one row
    (7, 4, wl.F32),           # one group per row
    (513, 2048, wl.BF16),     # bf16 x and dy: 8-element groups
    (100, 8192, wl.F32),      # wider than a 256-thread team: 512-thread team
    (77, 8196, wl.F32),       # wider than the vector path: generic strip kernels
    (64, 1001, wl.F32),       # odd width: generic strip kernels, scalar groups
    (2000, 64, wl.BF16),      # narrow rows, many per block
])
def test_bda_shapes(nh, oracle_mod, rows, cols, xt):
    c = wl.bda_case(rows, cols, x_t=xt, dy_t=xt, w_t=wl.BF16, seed=rows + 5 * cols, p_drop=0.25)
    _bda_case(nh, oracle_mod, c)


def test_bda_options(nh, oracle_mod):
    c = wl.bda_case(129, 1600, seed=83, p_drop=0.5)
    _bda_case(nh, oracle_mod, c, dres=False)
    _bda_case(nh, oracle_mod, c, mask=False, scale=1.0)
    _bda_case(nh, oracle_mod, c, weight=False)
    _bda_case(nh, oracle_mod, c, need=(False, True, False, False, True))
    _bda_case(nh, oracle_mod, c, need=(True, False, True, True, False))
    _bda_case(nh, oracle_mod, c, need=(False, False, False, False, True))


def test_bda_misaligned_mask(nh, oracle_mod):
    """A mask at an odd address takes the generic path; same results."""
    c = wl.bda_case(64, 1600, seed=84)
    buf = torch.zeros(c.mask.size + 1, dtype=torch.uint8, device="cuda")
    buf[1:] = torch.from_numpy(c.mask.reshape(-1)).cuda()
    _bda_case(nh, oracle_mod, c, mask_dev=buf[1:])


@pytest.mark.parametrize("blocks", [1, 7, 2048])
def test_bda_forced_blocks(nh, oracle_mod, blocks):
    _bda_case(nh, oracle_mod, wl.bda_case(4099, 1024, seed=85), override_blocks=blocks)


def test_bda_zero_rows(nh):
    w = torch.ones(96, dtype=torch.bfloat16, device="cuda")
    e = torch.empty(0, 96, device="cuda")
    got = nh.bda_layernorm_backward(e.bfloat16(), e, torch.empty(0, device="cuda"),
                                    torch.empty(0, device="cuda"), w, None, None, 1.0)
    torch.cuda.synchronize()
    for t in got[2:]:
        assert t.shape == (96,) and bool((t == 0).all())


def test_bda_without_extras_is_layernorm_backward(nh, oracle_mod):
    """No incoming gradient, no mask, scale 1: dh and da equal
    layernorm_backward's dx and the shared column gradients agree bit for bit
    (same block count, one row team per block in both)."""
    c = wl.bda_case(1000, 1600, x_t=wl.F32, dy_t=wl.F32, w_t=wl.F32, seed=86)
    mean32, rstd32 = _stats(oracle_mod, c)
    args = (dev(c.ln.dy), dev(c.ln.x), dev(mean32), dev(rstd32), dev(c.ln.w))
    nh.plan_override("rows_blocks", 256)
    nh.plan_override("rows_teams", 1)
    try:
        dh, da, dw, db, dbi = nh.bda_layernorm_backward(*args, None, None, 1.0)
        dx, dw0, db0 = nh.layernorm_backward(*args, dx_dtype=torch.float32)
        torch.cuda.synchronize()
    finally:
        nh.plan_override("rows_blocks", 0)
        nh.plan_override("rows_teams", 0)
    assert torch.equal(dh, dx) and torch.equal(da, dx)
    assert torch.equal(dw.view(torch.int32), dw0.view(torch.int32))
    assert torch.equal(db.view(torch.int32), db0.view(torch.int32))
    check("dbias_in vs column sums of dx", host(dbi), host(dx).sum(axis=0), wl.F32)


def test_bda_bit_identical_runs(nh, oracle_mod):
    c = wl.bda_bwd()
    mean32, rstd32 = _stats(oracle_mod, c)
    args = (dev(c.ln.dy), dev(c.ln.x), dev(mean32), dev(rstd32), dev(c.ln.w), dev(c.dresidual),
            torch.from_numpy(c.mask).cuda().bool(), c.scale)
    a = nh.bda_layernorm_backward(*args)
    b = nh.bda_layernorm_backward(*args)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        iv = torch.int16 if u.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(u.view(iv), v.view(iv))


@pytest.mark.parametrize("depth", [1, 2, 3, 4])
def test_bda_pipeline_depths(nh, oracle_mod, depth):
    nh.plan_override("rows_depth", depth)
    try:
        _bda_case(nh, oracle_mod, wl.bda_case(1037, 1600, seed=87), override_blocks=100)
    finally:
        nh.plan_override("rows_depth", 0)


@pytest.mark.parametrize("rows,cols,xt", [(64, 8192, wl.BF16), (50, 6144, wl.F32), (33, 8192, wl.F32)])
def test_bda_wide_rows(nh, oracle_mod, rows, cols, xt):
    """Rows too wide for 16 elements per thread in a 256-thread team take a
    512-thread team."""
    _bda_case(nh, oracle_mod, wl.bda_case(rows, cols, x_t=xt, dy_t=xt, w_t=wl.BF16, seed=rows + cols))
