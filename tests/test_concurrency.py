"""Calls from several host threads, each on its own stream with its own
outputs and workspace, run concurrently on the GPU and give the same bits as
sequential calls.  The library's shared state (device-property and
occupancy caches, per-thread error messages) must tolerate this."""
import threading

import pytest

from bwd_bn_stats_amd import workloads as wl

from helpers import dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def nh():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bwd_bn_stats_amd import normhip
    return normhip


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_threads_and_streams(nh):
    c = wl.bn_case(16, 32, 32, 32, wl.F32, seed=8001)
    r = wl.ln_bwd(rows=1024)
    m = wl.rms_bwd(wl.BF16, rows=512, cols=4096)
    o = wl.rows_case(700, 2001, x_t=wl.F32, dy_t=wl.BF16, w_t=wl.F32, seed=8002)  # generic path
    x, dy, g, b = dev(c.x), dev(c.dy), dev(c.gamma), dev(c.beta)
    lx, ldy, lw = dev(r.x), dev(r.dy), dev(r.w)
    mx, mdy, mw = dev(m.x), dev(m.dy), dev(m.w)
    ox, ody, ow = dev(o.x), dev(o.dy), dev(o.w)

    def work():
        y, stats = nh.bn_forward_train(x, g, b, act="leaky_relu", slope=0.05)
        dx, grads = nh.bn_backward(dy, x, stats, beta=b, act="leaky_relu", slope=0.05)
        ly, mean, rstd = nh.layernorm_forward(lx, lw, None, 1e-5)
        ldx, ldw, ldb = nh.layernorm_backward(ldy, lx, mean, rstd, lw, dx_dtype=torch.float32)
        my, rms = nh.rmsnorm_forward(mx, mw, 1e-5)
        mdx, mdw = nh.rmsnorm_backward(mdy, mx, rms, mw, 1e-5)
        oy, om, orr = nh.layernorm_forward(ox, ow, None, 1e-5)
        odx, odw, odb = nh.layernorm_backward(ody, ox, om, orr, ow, dx_dtype=torch.float32)
        return [y, stats, dx, grads, ly, mean, rstd, ldx, ldw, ldb, my, rms, mdx, mdw, oy, om, orr, odx,
                odw, odb]

    ref = [t.clone() for t in work()]
    torch.cuda.synchronize()

    n_threads, reps = 4, 5
    results, errors = [None] * n_threads, []

    def body(k):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                out = None
                for _ in range(reps):
                    out = work()
                s.synchronize()
            results[k] = out
        except Exception as e:  # reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=body, args=(k,)) for k in range(n_threads)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    print(f"[concurrency] {n_threads} threads x {reps} reps of BN+LeakyReLU, LN, RMS and odd-width LN fwd/bwd",
          flush=True)
    for k, out in enumerate(results):
        for i, (u, v) in enumerate(zip(out, ref)):
            assert torch.equal(_bits(u), _bits(v)), f"thread {k} output {i} differs"
