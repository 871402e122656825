"""The library through its C ABI alone: tests/c/abi_client.c is a plain C
program (gcc -std=c11 -Werror) that includes include/normhip.h, links
libnormhip.so and the HIP runtime, and allocates its own device buffers.

CPU: the client's host-only checks (status strings, self test, validation
of every entry point).  GPU: the client runs BatchNorm forward+backward and
LayerNorm forward+backward on inputs from the seeded generators, and its
outputs are compared with the oracle at the fp32 tolerance."""
import os
import subprocess
import sys

import numpy as np
import pytest

from bwd_bn_stats_amd import workloads as wl

from helpers import check

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "c"))
import build_client  # noqa: E402


@pytest.fixture(scope="module")
def client():
    return build_client.build()


def _run(client, *args):
    r = subprocess.run([client, *args], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    return r.stdout


def test_c_client_host_checks(client):
    assert "check: ok" in _run(client, "check")


def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.gpu
def test_c_client_batchnorm(client, oracle_mod, tmp_path):
    _gpu()
    c = wl.bn_case(3, 37, 41, 40, wl.F32, seed=1001, x_mean=5.0, x_std=0.5, beta_std=1.0)
    N, C, HW = c.N, c.C, c.hw
    inp = tmp_path / "bn_in.bin"
    with open(inp, "wb") as f:
        f.write(np.array([N, C, HW], np.int64).tobytes())
        for a in (c.x.store, c.dy.store, c.gamma, c.beta):
            f.write(np.ascontiguousarray(a, np.float32).tobytes())
    out = tmp_path / "bn_out.bin"
    print(f"[c client] bn N={N} C={C} HW={HW}", flush=True)
    _run(client, "bn", str(inp), str(out))
    got = np.fromfile(out, np.float32).astype(np.float64)
    E = N * C * HW
    y, stats, dx, grads = np.split(got, [E, E + 4 * C, 2 * E + 4 * C])
    wy, wstats, _, _ = oracle_mod.bn_forward_train(c.x.value, c.gamma, c.beta, eps=c.eps)
    wdx, wgrads = oracle_mod.bn_backward(c.x.value, c.dy.value, c.gamma, eps=c.eps)
    check("y", y, wy.reshape(-1), wl.F32)
    check("dx", dx, wdx.reshape(-1), wl.F32)
    for i in range(4):
        check(f"stats[{i}]", stats.reshape(4, C)[i], wstats[i], wl.F32)
        check(f"grads[{i}]", grads.reshape(4, C)[i], wgrads[i], wl.F32)


@pytest.mark.gpu
def test_c_client_layernorm(client, oracle_mod, tmp_path):
    _gpu()
    c = wl.rows_case(301, 1600, x_t=wl.F32, dy_t=wl.F32, w_t=wl.F32, seed=61)
    R, H = c.rows, c.cols
    inp = tmp_path / "ln_in.bin"
    with open(inp, "wb") as f:
        f.write(np.array([R, H], np.int64).tobytes())
        for a in (c.x.store, c.dy.store, c.w.store):
            f.write(np.ascontiguousarray(a, np.float32).tobytes())
    out = tmp_path / "ln_out.bin"
    print(f"[c client] ln rows={R} cols={H}", flush=True)
    _run(client, "ln", str(inp), str(out))
    got = np.fromfile(out, np.float32).astype(np.float64)
    E = R * H
    y, mean, rstd, dx, dw, db = np.split(got, np.cumsum([E, R, R, E, H]))
    wy, wmean, wrstd = oracle_mod.layernorm_forward(c.x.value, c.w.value, eps=c.eps)
    wdx, wdw, wdb = oracle_mod.layernorm_backward(c.x.value, c.dy.value, wmean, wrstd, c.w.value)
    check("y", y, wy.reshape(-1), wl.F32)
    check("mean", mean, wmean, wl.F32)
    check("rstd", rstd, wrstd, wl.F32)
    check("dx", dx, wdx.reshape(-1), wl.F32)
    check("dweight", dw, wdw, wl.F32)
    check("dbias", db, wdb, wl.F32)
