"""Benchmark of the normalization hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--quick] [--no-cpu-baseline]
                    [--workloads NAME,...] [--list]

A step is one BatchNorm2d training forward + backward (bn_forward_train, then
bn_backward) over the CIFAR-shaped NCHW (256,32,32,32) fp32 batch, the
workload of the Aether-ML BatchNorm PR's kernel measurements.  Inputs are
resident in HBM before any timed region.

Cold protocol: every call reads inputs that were last touched more than 1 GiB
of traffic earlier.  The buffer sets rotate, and a step's backward runs on a
different set than its forward (the set whose forward ran half a rotation
earlier), so neither call finds its inputs in the 256 MB Infinity Cache.

Timing: every figure comes from a region of K back-to-back calls bracketed by
one pair of HIP events on the stream the kernels run on.  No event sits
between the kernels of a region: an event pair on a dispatch inserts a
multi-microsecond gap into the queue (measured on MI355X, about 4.5 us), while
back-to-back dispatches follow each other with no gap.  Per-kernel durations
come from regions of whole calls: the BatchNorm calls' two stages
(bn_forward_train_stage / bn_backward_stage: the reduction pass alone, then
the full call) give the reduction kernel's duration and, by difference, the
finalize+elementwise kernel's.  Each region is repeated; the line reports the
median and the p10/p90 over the repetitions.

Printed: ONE JSON line.  `value` is the step's minimal HBM traffic (forward:
read x, write y; backward: read x and dy, write dx) divided by the step time.
The algorithmic rate (each kernel's reads and writes, including the method's
re-reads of x and dy, which the Infinity Cache serves) is reported beside it.
`roofline` is for the dominant kernel among those whose inputs come from HBM
(the reduction passes; the elementwise passes re-read through the Infinity
Cache and are listed, not used, for the roofline).  `others` holds the other
workloads, measured the same way, and `floors` the bandwidth of independent
streams of the same sizes (hipMemcpyAsync device-to-device, torch's add and
sum) and of at least 1 GiB.  `cpu_baseline` is the CPU oracle on this host.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "norm fwd+bwd µs/call and achieved HBM GB/s (% of MI355X peak) at 1 GPU"
HBM_PEAK_GBS = 8000.0
COLD_BYTES = 1 << 30   # traffic between two touches of the same buffer set
GiB = 1 << 30
P = ctypes.c_void_p


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _dev(t, device):
    import torch
    from bwd_bn_stats_amd import workloads as wl
    if isinstance(t, wl.Tensor):
        if t.dtype == wl.F32:
            return torch.from_numpy(np.ascontiguousarray(t.store)).to(device)
        return torch.from_numpy(np.ascontiguousarray(t.store).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(t, dtype=np.float32)).to(device)


def _nsets(set_bytes, even=False):
    r = max(2, int(-(-COLD_BYTES // max(set_bytes, 1))) + 1)
    if even and r % 2:
        r += 1
    return r


def _q(vals):
    a = np.asarray(vals, dtype=np.float64)
    p10, med, p90 = np.percentile(a, [10, 50, 90])
    return {"median_us": round(float(med), 3), "p10_us": round(float(p10), 3), "p90_us": round(float(p90), 3)}


class Regions:
    """Times regions of back-to-back calls.  A region's K calls are captured
    once into a HIP graph on torch's capture stream and replayed `reps` times,
    each replay bracketed by one pair of HIP events on the stream it runs on:
    the device runs the captured kernels back to back, with no host launch
    cost between them (host-issued calls of a few microseconds of GPU work
    each would leave the device idle between kernels)."""

    SPIN_US = 300.0
    MIN_CALLS = 100      # calls per timed sample: the replays of one sample share one event pair
    EAGER = False        # issue every region call by call (for counter runs)
    _spin_cycles = None

    def __init__(self, torch, reps):
        self.torch, self.reps = torch, reps
        if Regions._spin_cycles is None:
            Regions._spin_cycles = self._calibrate_spin()

    def _calibrate_spin(self):
        """Cycles of torch.cuda._sleep (a bounded spin kernel) that take about
        SPIN_US microseconds."""
        torch = self.torch
        torch.cuda._sleep(1000)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cyc = 1 << 20
        e0.record()
        torch.cuda._sleep(cyc)
        e1.record()
        e1.synchronize()
        us = max(1.0, 1000.0 * e0.elapsed_time(e1))
        return max(1000, int(cyc * self.SPIN_US / us))

    def _busy(self):
        """Keeps the device busy for about SPIN_US while the host submits the
        region: the start event then fires only when the region's first
        kernel is already queued, so host submission latency stays out of the
        timed region."""
        self.torch.cuda._sleep(Regions._spin_cycles)

    def run(self, make_call, K, start=0):
        """make_call(stream) -> call(i) issuing call i on `stream` (a void*
        hipStream_t).  Captures call(start + i) for i in [0, K) in a graph.
        Each of the `reps` samples replays it M = ceil(MIN_CALLS / K) times
        between one event pair (the pair's fixed cost, about 10 us, then adds
        at most a tenth of a microsecond per call); returns the per-call
        microseconds of each sample."""
        torch = self.torch
        if Regions.EAGER:
            return self.run_eager(make_call(P(torch.cuda.current_stream().cuda_stream)), K, start)
        M = max(1, -(-self.MIN_CALLS // K))
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call = make_call(P(torch.cuda.current_stream().cuda_stream))
            call(start)  # one eager call on this stream before capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            call = make_call(P(torch.cuda.current_stream().cuda_stream))
            for i in range(K):
                call(start + i)
        graph.replay()  # untimed: first replay
        torch.cuda.synchronize()
        out = []
        for _ in range(self.reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            self._busy()
            e0.record()
            for _ in range(M):
                graph.replay()
            e1.record()
            e1.synchronize()
            out.append(1000.0 * e0.elapsed_time(e1) / (M * K))
        del graph
        return out

    def run_eager(self, call, K, start=0):
        """The same region issued call by call from the host (no graph): on
        short calls this times the host's issue rate, not the device."""
        torch = self.torch
        K = max(K, self.MIN_CALLS)
        out = []
        base = start
        for _ in range(self.reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            self._busy()
            e0.record()
            for i in range(K):
                call(base + i)
            e1.record()
            e1.synchronize()
            out.append(1000.0 * e0.elapsed_time(e1) / K)
            base += K
        return out


def _round_up(K, R):
    return -(-K // R) * R


def _chk(st, nh, what):
    if st:
        raise RuntimeError(f"{what}: {nh.status_string(st)}: {nh.last_error()}")


# ---- BatchNorm ---------------------------------------------------------------------
ACT_IDS = {"none": 0, "relu": 1, "leaky_relu": 2}


def bench_bn(nh, torch, case, K, W, reps, act="none", slope=0.01, stages=True):
    """BatchNorm2d training forward + backward, cold per call.  With `stages`,
    also the reduction passes alone (stage 1) for the per-kernel split."""
    device = torch.device("cuda:0")
    x0, dy0 = _dev(case.x, device), _dev(case.dy, device)
    g, b = _dev(case.gamma, device), _dev(case.beta, device)
    io = 0 if case.io == "f32" else 1
    N, C, HW = case.N, case.C, case.hw
    s = x0.element_size()
    E = N * C * HW
    wsb = max(16, nh.bn_forward_train_workspace(N, C, HW))
    R = _nsets(4 * E * s, even=True)
    half = R // 2
    K = _round_up(K, R)
    sets = [dict(x=x0.clone(), dy=dy0.clone(), y=torch.empty_like(x0), dx=torch.empty_like(x0),
                 rm=torch.zeros(C, device=device), rv=torch.ones(C, device=device),
                 stats=torch.empty(4, C, device=device), grads=torch.empty(4, C, device=device),
                 ws=torch.empty(wsb, dtype=torch.uint8, device=device)) for _ in range(R)]
    torch.cuda.synchronize()
    lib = nh.lib
    pg, pb = P(g.data_ptr()), P(b.data_ptr())
    a = ACT_IDS[act]
    mom, eps = case.momentum, case.eps
    ptrs = [{k: P(v.data_ptr()) for k, v in t.items()} for t in sets]

    def args_for(stream):
        fa, ba = [], []
        for p in ptrs:
            if act == "none":
                fa.append((p["x"], p["y"], io, N, C, HW, pg, pb, p["rm"], p["rv"], mom, eps, p["stats"], p["ws"],
                           wsb, stream))
                ba.append((p["dy"], p["x"], io, N, C, HW, p["stats"], p["dx"], p["grads"], p["ws"], wsb, stream))
            else:
                fa.append((p["x"], p["y"], io, N, C, HW, pg, pb, p["rm"], p["rv"], mom, eps, a, slope, p["stats"],
                           p["ws"], wsb, stream))
                ba.append((p["dy"], p["x"], io, N, C, HW, p["stats"], pb, a, slope, p["dx"], p["grads"], p["ws"],
                           wsb, stream))
        return fa, ba

    fwd_fn = lib.bn_forward_train if act == "none" else lib.bn_act_forward_train
    bwd_fn = lib.bn_backward if act == "none" else lib.bn_act_backward
    fst, bst = lib.bn_forward_train_stage, lib.bn_backward_stage

    def maker(kind):
        def make(stream):
            fa, ba = args_for(stream)
            if kind == "step":
                return lambda i: (fwd_fn(*fa[i % R]), bwd_fn(*ba[(i + half) % R]))
            if kind == "fwd":
                return lambda i: fwd_fn(*fa[i % R])
            if kind == "bwd":
                return lambda i: bwd_fn(*ba[(i + half) % R])
            if kind == "fwd1":
                return lambda i: fst(1, *fa[i % R])
            return lambda i: bst(1, *ba[(i + half) % R])
        return make

    stream0 = P(torch.cuda.current_stream(device).cuda_stream)
    fa0, ba0 = args_for(stream0)
    # every set gets statistics before any backward reads them; check codes once
    for i in range(R):
        _chk(fwd_fn(*fa0[i]), nh, "forward")
    _chk(bwd_fn(*ba0[0]), nh, "backward")
    if stages and act == "none":
        _chk(fst(1, *fa0[0]), nh, "forward stage 1")
        _chk(bst(1, *ba0[0]), nh, "backward stage 1")
    step0 = maker("step")(stream0)
    for i in range(W):
        step0(i)
    torch.cuda.synchronize()
    rg = Regions(torch, reps)
    t_step = rg.run(maker("step"), K)
    t_eager = rg.run_eager(step0, K)
    t_fwd = rg.run(maker("fwd"), K)
    t_bwd = rg.run(maker("bwd"), K)
    res = {"buffer_sets": R, "calls_per_region": K, "grid_y": nh.bn_plan(N, C, HW, io)}
    res["step"] = _q(t_step)
    res["step_host_issued"] = _q(t_eager)
    res["calls"] = {"bn_forward_train": _q(t_fwd), "bn_backward": _q(t_bwd)}
    step_us = res["step"]["median_us"]
    one_touch = 5 * E * s
    algo = {"bn_stats": E * s, "bn_apply": 2 * E * s, "bn_grad_sums": 2 * E * s, "bn_dx": 3 * E * s}
    res["one_touch_bytes"] = one_touch
    res["algorithmic_bytes"] = sum(algo.values())
    res["one_touch_gbs"] = round(one_touch / (step_us * 1e3), 1)
    res["algorithmic_gbs"] = round(sum(algo.values()) / (step_us * 1e3), 1)
    if stages and act == "none":
        t_f1 = rg.run(maker("fwd1"), K)
        t_b1 = rg.run(maker("bwd1"), K)
        f1, b1 = float(np.median(t_f1)), float(np.median(t_b1))
        fm, bm = float(np.median(t_fwd)), float(np.median(t_bwd))
        if f1 < 1.0 or b1 < 1.0:
            # the shape runs each direction as one kernel (stage 1 launches nothing)
            res["kernels"] = {"bn_fwd_channel": {"avg_us": round(fm, 3), "bytes": 3 * E * s},
                              "bn_bwd_channel": {"avg_us": round(bm, 3), "bytes": 5 * E * s}}
        else:
            res["kernels"] = {"bn_stats": {"avg_us": round(f1, 3)}, "bn_apply": {"avg_us": round(fm - f1, 3)},
                              "bn_grad_sums": {"avg_us": round(b1, 3)}, "bn_dx": {"avg_us": round(bm - b1, 3)}}
            res["stage1_calls"] = {"bn_forward_train_stage1": _q(t_f1), "bn_backward_stage1": _q(t_b1)}
            for k, v in res["kernels"].items():
                v["bytes"] = algo[k]
                v["input_from"] = "hbm" if k in ("bn_stats", "bn_grad_sums") else "infinity_cache+hbm"
        for k, v in res["kernels"].items():
            v["gbs"] = round(v["bytes"] / (v["avg_us"] * 1e3), 1)
            if v.get("input_from") == "infinity_cache+hbm":
                # x (and dy) come back from the Infinity Cache, where the
                # reduction pass just left them: only the output write must
                # reach HBM, so the algorithmic rate is no HBM fraction
                v["hbm_bytes"] = E * s
                v["hbm_gbs"] = round(E * s / (v["avg_us"] * 1e3), 1)
                v["algorithmic_over_hbm_peak"] = round(v["gbs"] / HBM_PEAK_GBS, 4)
            else:
                v["frac_of_peak"] = round(v["gbs"] / HBM_PEAK_GBS, 4)
    del sets, fa0, ba0
    torch.cuda.empty_cache()
    return res


def _single(nh, torch, f, args_for, R, K, W, reps, what):
    """Times a call that is one kernel (or one call) over R rotating sets:
    args_for(stream) -> list of R argument tuples for f."""
    stream0 = P(torch.cuda.current_stream().cuda_stream)
    a0 = args_for(stream0)
    _chk(f(*a0[0]), nh, what)
    for i in range(W):
        f(*a0[i % R])
    torch.cuda.synchronize()
    K = _round_up(K, R)

    def make(stream):
        a = args_for(stream)
        return lambda i: f(*a[i % R])
    rg = Regions(torch, reps)
    return rg.run(make, K), K


def bench_bn_infer(nh, torch, case, K, W, reps, act="relu", slope=0.01):
    """BatchNorm2d inference (+ activation): one elementwise pass, x read and
    y written once (one kernel: the call time is the kernel time)."""
    device = torch.device("cuda:0")
    x0 = _dev(case.x, device)
    g, b = _dev(case.gamma, device), _dev(case.beta, device)
    io = 0 if case.io == "f32" else 1
    N, C, HW = case.N, case.C, case.hw
    rm = torch.linspace(-0.5, 0.5, C, device=device)
    rv = torch.linspace(0.5, 2.0, C, device=device)
    byt = 2 * x0.numel() * x0.element_size()
    R = _nsets(byt)
    sets = [(x0.clone(), torch.empty_like(x0)) for _ in range(R)]
    torch.cuda.synchronize()
    ptrs = [(P(x.data_ptr()), P(y.data_ptr())) for x, y in sets]

    def args_for(stream):
        return [(x, y, io, N, C, HW, P(g.data_ptr()), P(b.data_ptr()), P(rm.data_ptr()), P(rv.data_ptr()),
                 case.eps, ACT_IDS[act], slope, stream) for x, y in ptrs]
    t, K = _single(nh, torch, nh.lib.bn_forward_infer, args_for, R, K, W, reps, "bn_forward_infer")
    del sets
    torch.cuda.empty_cache()
    us = float(np.median(t))
    return {"call": _q(t), "bytes": byt, "gbs": round(byt / (us * 1e3), 1),
            "kernels": {"bn_infer": {"avg_us": round(us, 3), "bytes": byt, "gbs": round(byt / (us * 1e3), 1),
                                     "frac_of_peak": round(byt / (us * 1e3) / HBM_PEAK_GBS, 4)}},
            "buffer_sets": R, "calls_per_region": K}


# ---- LayerNorm / RMSNorm -----------------------------------------------------------
def bench_rows(nh, torch, case, kind, K, W, reps, saved=True):
    """LayerNorm / RMSNorm backward: the row kernel (dx + column partials) and
    the column finalize, timed as a call."""
    device = torch.device("cuda:0")
    x0, dy0, w = _dev(case.x, device), _dev(case.dy, device), _dev(case.w, device)
    R_, H = case.rows, case.cols
    xf = x0.float()
    if kind == "ln":
        var, mean = torch.var_mean(xf, dim=1, unbiased=False)
        sa, sb = mean.contiguous(), torch.rsqrt(var + case.eps).contiguous()
        wsb = nh.layernorm_backward_workspace(R_, H)
    else:
        sa, sb = torch.sqrt((xf * xf).mean(dim=1) + case.eps).contiguous(), None
        wsb = nh.rmsnorm_backward_workspace(R_, H)
    del xf
    wsb = max(16, wsb)
    dx_dtype = x0.dtype
    E = R_ * H
    dxs = torch.empty(0, dtype=dx_dtype).element_size()
    set_bytes = E * (x0.element_size() + dy0.element_size() + dxs)
    R = _nsets(set_bytes)
    sets = [dict(x=x0.clone(), dy=dy0.clone(), dx=torch.empty(x0.shape, dtype=dx_dtype, device=device),
                 dw=torch.empty(H, dtype=w.dtype, device=device), db=torch.empty(H, dtype=w.dtype, device=device),
                 ws=torch.empty(wsb, dtype=torch.uint8, device=device)) for _ in range(R)]
    torch.cuda.synchronize()
    dt = {torch.float32: 0, torch.bfloat16: 1}
    pa, pw = P(sa.data_ptr()), P(w.data_ptr())
    pb = P(sb.data_ptr()) if sb is not None else None
    ptrs = [{k: P(v.data_ptr()) for k, v in t.items()} for t in sets]

    def args_for(stream):
        out = []
        for p in ptrs:
            if kind == "ln":
                out.append((p["dy"], dt[dy0.dtype], p["x"], dt[x0.dtype], pa, pb, pw, dt[w.dtype], R_, H, p["dx"],
                            dt[dx_dtype], p["dw"], p["db"], p["ws"], wsb, stream))
            else:
                out.append((p["dy"], p["x"], dt[x0.dtype], pa if saved else None, case.eps, pw, R_, H, p["dx"],
                            p["dw"], p["ws"], wsb, stream))
        return out
    f = nh.lib.layernorm_backward if kind == "ln" else nh.lib.rmsnorm_backward
    t, K = _single(nh, torch, f, args_for, R, K, W, reps, kind + " backward")
    byt = set_bytes + R_ * 4 * (2 if kind == "ln" else (1 if saved else 0)) + H * w.element_size() * (
        3 if kind == "ln" else 2)
    del sets
    torch.cuda.empty_cache()
    us = float(np.median(t))
    return {"call": _q(t), "bytes": byt, "gbs": round(byt / (us * 1e3), 1),
            "frac_of_peak": round(byt / (us * 1e3) / HBM_PEAK_GBS, 4), "buffer_sets": R, "calls_per_region": K,
            "blocks_max": nh.rows_plan(R_, H)}


def bench_bda(nh, torch, case, K, W, reps):
    """Backward of bias + dropout + add + LayerNorm: reads x, dy, the incoming
    gradient and the mask, writes dh (fp32) and da, plus the column sums."""
    device = torch.device("cuda:0")
    ln = case.ln
    x0, dy0, w = _dev(ln.x, device), _dev(ln.dy, device), _dev(ln.w, device)
    dres0 = torch.from_numpy(case.dresidual).to(device)
    mask0 = torch.from_numpy(case.mask).to(device)
    R_, H = ln.rows, ln.cols
    var, mean = torch.var_mean(x0.float(), dim=1, unbiased=False)
    mean, rstd = mean.contiguous(), torch.rsqrt(var + ln.eps).contiguous()
    wsb = max(16, nh.bda_layernorm_backward_workspace(R_, H))
    E = R_ * H
    per_elem = x0.element_size() + dy0.element_size() + 4 + 1 + 4 + dy0.element_size()
    R = _nsets(E * per_elem)
    sets = [dict(x=x0.clone(), dy=dy0.clone(), dres=dres0.clone(), mask=mask0.clone(),
                 dh=torch.empty(x0.shape, dtype=torch.float32, device=device),
                 da=torch.empty(x0.shape, dtype=dy0.dtype, device=device),
                 dw=torch.empty(H, dtype=w.dtype, device=device), db=torch.empty(H, dtype=w.dtype, device=device),
                 dbi=torch.empty(H, dtype=w.dtype, device=device),
                 ws=torch.empty(wsb, dtype=torch.uint8, device=device)) for _ in range(R)]
    torch.cuda.synchronize()
    dt = {torch.float32: 0, torch.bfloat16: 1}
    pm, pr, pw = P(mean.data_ptr()), P(rstd.data_ptr()), P(w.data_ptr())
    ptrs = [{k: P(v.data_ptr()) for k, v in t.items()} for t in sets]

    def args_for(stream):
        return [(p["dy"], dt[dy0.dtype], p["x"], dt[x0.dtype], pm, pr, pw, dt[w.dtype], p["dres"], p["mask"],
                 case.scale, R_, H, p["dh"], p["da"], p["dw"], p["db"], p["dbi"], p["ws"], wsb, stream) for p in ptrs]
    t, K = _single(nh, torch, nh.lib.bda_layernorm_backward, args_for, R, K, W, reps, "bda_layernorm_backward")
    byt = E * per_elem + R_ * 8 + H * w.element_size() * 4
    del sets
    torch.cuda.empty_cache()
    us = float(np.median(t))
    return {"call": _q(t), "bytes": byt, "gbs": round(byt / (us * 1e3), 1),
            "frac_of_peak": round(byt / (us * 1e3) / HBM_PEAK_GBS, 4), "buffer_sets": R, "calls_per_region": K}


def bench_rows_fwd(nh, torch, case, kind, K, W, reps):
    """LayerNorm / RMSNorm training forward (one kernel): read x (+ weight,
    bias once), write y and the per-row statistics."""
    device = torch.device("cuda:0")
    x0, w = _dev(case.x, device), _dev(case.w, device)
    b = _dev(case.b, device) if (kind == "ln" and case.b is not None) else None
    R_, H = case.rows, case.cols
    E = R_ * H
    R = _nsets(2 * E * x0.element_size())
    sets = [dict(x=x0.clone(), y=torch.empty_like(x0), s0=torch.empty(R_, device=device),
                 s1=torch.empty(R_, device=device)) for _ in range(R)]
    torch.cuda.synchronize()
    dt = {torch.float32: 0, torch.bfloat16: 1}
    pw, pb = P(w.data_ptr()), (P(b.data_ptr()) if b is not None else None)
    xt = dt[x0.dtype]
    ptrs = [{k: P(v.data_ptr()) for k, v in t.items()} for t in sets]

    def args_for(stream):
        if kind == "ln":
            return [(p["x"], xt, pw, pb, dt[w.dtype], R_, H, case.eps, p["y"], xt, p["s0"], p["s1"], stream)
                    for p in ptrs]
        return [(p["x"], xt, pw, R_, H, case.eps, p["y"], p["s0"], stream) for p in ptrs]
    f = nh.lib.layernorm_forward if kind == "ln" else nh.lib.rmsnorm_forward
    t, K = _single(nh, torch, f, args_for, R, K, W, reps, kind + " forward")
    byt = 2 * E * x0.element_size() + R_ * 4 * (2 if kind == "ln" else 1) + H * w.element_size() * (
        2 if b is not None else 1)
    del sets
    torch.cuda.empty_cache()
    us = float(np.median(t))
    k = "ln_fwd" if kind == "ln" else "rms_fwd"
    return {"call": _q(t), "bytes": byt, "gbs": round(byt / (us * 1e3), 1),
            "kernels": {k: {"avg_us": round(us, 3), "bytes": byt, "gbs": round(byt / (us * 1e3), 1),
                            "frac_of_peak": round(byt / (us * 1e3) / HBM_PEAK_GBS, 4)}},
            "buffer_sets": R, "calls_per_region": K}


# ---- independent bandwidth floors ---------------------------------------------------------
def _hip():
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpyAsync.argtypes = [P, P, ctypes.c_size_t, ctypes.c_int, P]
    hip.hipMemcpyAsync.restype = ctypes.c_int
    return hip


def floor_memcpy(torch, nbytes, K, W, reps):
    """hipMemcpyAsync device-to-device of `nbytes` (cold rotating buffers);
    GB/s counts the bytes read plus written."""
    hip = _hip()
    device = torch.device("cuda:0")
    R = _nsets(2 * nbytes)
    sets = [(torch.ones(nbytes // 4, device=device), torch.empty(nbytes // 4, device=device)) for _ in range(R)]
    torch.cuda.synchronize()
    t, _ = _single_fn(torch, lambda st: [(P(d.data_ptr()), P(s.data_ptr()), nbytes, 3, st) for s, d in sets],
                      hip.hipMemcpyAsync, R, K, W, reps)
    del sets
    torch.cuda.empty_cache()
    us = float(np.median(t))
    return {"bytes": 2 * nbytes, "avg_us": round(us, 3), "gbs": round(2 * nbytes / (us * 1e3), 1)}


def _single_fn(torch, args_for, f, R, K, W, reps):
    stream0 = P(torch.cuda.current_stream().cuda_stream)
    a0 = args_for(stream0)
    for i in range(max(W, 1)):
        f(*a0[i % R])
    torch.cuda.synchronize()
    K = _round_up(K, R)

    def make(stream):
        a = args_for(stream)
        return lambda i: f(*a[i % R])
    return Regions(torch, reps).run(make, K), K


def _torch_region(torch, fn, R, K, W, reps):
    """fn(i) issues a torch op on the current stream."""
    for i in range(max(W, 1)):
        fn(i)
    torch.cuda.synchronize()
    K = _round_up(K, R)
    return Regions(torch, reps).run(lambda stream: fn, K), K


def floor_torch_add(torch, n_floats, K, W, reps):
    """torch.add(a, b, out=o) over n fp32 (two reads, one write), cold."""
    device = torch.device("cuda:0")
    R = _nsets(12 * n_floats)
    sets = [(torch.ones(n_floats, device=device), torch.ones(n_floats, device=device),
             torch.empty(n_floats, device=device)) for _ in range(R)]
    torch.cuda.synchronize()

    def call(i):
        a, b, o = sets[i % R]
        torch.add(a, b, out=o)
    t, _ = _torch_region(torch, call, R, K, W, reps)
    del sets
    torch.cuda.empty_cache()
    us = float(np.median(t))
    return {"bytes": 12 * n_floats, "avg_us": round(us, 3), "gbs": round(12 * n_floats / (us * 1e3), 1)}


def floor_torch_sum(torch, n_floats, K, W, reps):
    """torch.sum over n fp32 (one read), cold."""
    device = torch.device("cuda:0")
    R = _nsets(4 * n_floats)
    sets = [torch.ones(n_floats, device=device) for _ in range(R)]
    out = torch.empty((), device=device)
    torch.cuda.synchronize()
    t, _ = _torch_region(torch, lambda i: torch.sum(sets[i % R], dim=0, out=out), R, K, W, reps)
    del sets
    torch.cuda.empty_cache()
    us = float(np.median(t))
    return {"bytes": 4 * n_floats, "avg_us": round(us, 3), "gbs": round(4 * n_floats / (us * 1e3), 1)}


def floor_read(nh, torch, n_floats, K, W, reps):
    """A plain read stream of n fp32 (nh_calib_read: cacheable 16-byte loads,
    a block sum each), cold: the read floor the reduction passes, whose loads
    must stay cacheable, are held against."""
    device = torch.device("cuda:0")
    R = _nsets(4 * n_floats)
    sets = [torch.ones(n_floats, device=device) for _ in range(R)]
    sums = torch.empty(4096, device=device)
    torch.cuda.synchronize()
    t, _ = _single_fn(torch, lambda st: [(P(a.data_ptr()), n_floats, P(sums.data_ptr()), 4096, st) for a in sets],
                      nh.lib.nh_calib_read, R, K, W, reps)
    del sets
    torch.cuda.empty_cache()
    us = float(np.median(t))
    return {"bytes": 4 * n_floats, "avg_us": round(us, 3), "gbs": round(4 * n_floats / (us * 1e3), 1)}


def floor_warm(nh, torch, n_floats, kind, K, W, reps):
    """hipMemcpyAsync (kind "copy") or torch.add (kind "add") whose sources a
    plain read stream (nh_calib_read) read just before, so that they come from
    the Infinity Cache while the output goes to HBM: the floor of the
    elementwise passes, which re-read x (and dy) right after the reduction
    pass read them.  Cold buffer sets; the op's time is a region of
    (reads, op) calls less a region of the reads alone.  GB/s counts the
    bytes read plus written."""
    hip = _hip()
    device = torch.device("cuda:0")
    nsrc = 1 if kind == "copy" else 2
    R = _nsets(4 * n_floats * (nsrc + 1))
    sets = [[torch.ones(n_floats, device=device) for _ in range(nsrc)] + [torch.empty(n_floats, device=device)]
            for _ in range(R)]
    sums = torch.empty(4096, device=device)
    ps = P(sums.data_ptr())
    torch.cuda.synchronize()

    def make(with_op):
        def mk(stream):
            def call(i):
                t = sets[i % R]
                for a in t[:nsrc]:
                    nh.lib.nh_calib_read(P(a.data_ptr()), n_floats, ps, 4096, stream)
                if not with_op:
                    return
                if kind == "copy":
                    hip.hipMemcpyAsync(P(t[1].data_ptr()), P(t[0].data_ptr()), 4 * n_floats, 3, stream)
                else:
                    torch.add(t[0], t[1], out=t[2])
            return call
        return mk
    for i in range(max(W, 1)):
        make(True)(P(torch.cuda.current_stream().cuda_stream))(i)
    torch.cuda.synchronize()
    K = _round_up(K, R)
    full = float(np.median(Regions(torch, reps).run(make(True), K)))
    base = float(np.median(Regions(torch, reps).run(make(False), K)))
    del sets
    torch.cuda.empty_cache()
    us = full - base
    nb = 4 * n_floats * (nsrc + 1)
    return {"bytes": nb, "avg_us": round(us, 3), "gbs": round(nb / (us * 1e3), 1),
            "with_reads_us": round(full, 3), "reads_us": round(base, 3)}


def floors_for(nh, torch, read_bytes, add_bytes, copy_bytes, K, W, reps):
    out = {}
    if read_bytes:
        out["read_stream"] = floor_read(nh, torch, read_bytes // 4 // 4 * 4, K, W, reps)
        out["torch_sum"] = floor_torch_sum(torch, read_bytes // 4, K, W, reps)
    if add_bytes:
        out["torch_add"] = floor_torch_add(torch, add_bytes // 12 // 4 * 4, K, W, reps)
    if copy_bytes:
        out["hip_memcpy_d2d"] = floor_memcpy(torch, copy_bytes // 2 // 16 * 16, K, W, reps)
    for v in out.values():
        v["frac_of_peak"] = round(v["gbs"] / HBM_PEAK_GBS, 4)
    return out


# ---- CPU baseline: the oracle on this host ----------------------------------------------
def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def _host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(case, budget_s=10.0):
    """The oracle's BatchNorm forward + backward on the main workload, single
    thread (the oracle as it stands) and across the host's cores (the same
    oracle code with OpenMP over channels: bit-identical results), each timed
    for about `budget_s` seconds.  GB/s counts the step's minimal traffic, as
    the GPU line's value does."""
    import oracle
    oracle.build(force=False)
    x, dy = case.x.value, case.dy.value
    g, b = case.gamma.astype(np.float64), case.beta.astype(np.float64)
    E = case.N * case.C * case.hw
    one_touch = 5 * E * (4 if case.io == "f32" else 2)
    res = {}
    cores = _host_cores()
    for threads in (1, cores):
        reps, t_total = 0, 0.0
        while t_total < budget_s and reps < 200:
            t0 = time.perf_counter()
            oracle.bn_forward_train(x, g, b, eps=case.eps, momentum=case.momentum, running_mean=case.running_mean,
                                    running_var=case.running_var, threads=threads)
            oracle.bn_backward(x, dy, g, eps=case.eps, threads=threads)
            t_total += time.perf_counter() - t0
            reps += 1
        res[threads] = (1000.0 * t_total / reps, reps)
    ms_n, reps_n = res[cores]
    ms_1, reps_1 = res[1]
    return {"value": round(one_touch / (ms_n * 1e6), 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "ms_per_step": round(ms_n, 3),
            "sample": f"the full {case.N}x{case.C}x{case.hw // 32}x32 {case.io} forward+backward step in fp64, "
                      f"{reps_n} repetitions at {cores} threads (OpenMP over channels); minimal bytes as the GPU value",
            "single_thread": {"value": round(one_touch / (ms_1 * 1e6), 3), "ms_per_step": round(ms_1, 3),
                              "repetitions": reps_1, "cores": 1},
            "cpu_model": _cpu_model()}


def cpu_oracle_times(budget_s=4.0):
    """The oracle at the host's cores on the other configurations: ms per
    call (forward + backward for BatchNorm; the backward for LayerNorm and
    RMSNorm), each timed for about `budget_s` seconds."""
    import oracle
    from bwd_bn_stats_amd import workloads as wl
    oracle.build(force=False)
    cores = _host_cores()
    out = {}

    def timed(fn):
        reps, t = 0, 0.0
        while t < budget_s and reps < 100:
            t0 = time.perf_counter()
            fn()
            t += time.perf_counter() - t0
            reps += 1
        return round(1000.0 * t / reps, 3), reps

    c = wl.bn_resnet()
    g = c.gamma.astype(np.float64)
    out["bn2d_train_fwd_bwd_nchw_64x256x56x56_bf16"] = timed(lambda: (
        oracle.bn_forward_train(c.x.value, g, c.beta.astype(np.float64), eps=c.eps, momentum=c.momentum,
                                running_mean=c.running_mean, running_var=c.running_var, threads=cores),
        oracle.bn_backward(c.x.value, c.dy.value, g, eps=c.eps, threads=cores)))
    r = wl.ln_bwd()
    mean, rstd = oracle.layernorm_stats(r.x.value, eps=r.eps)
    m32, r32 = mean.astype(np.float32), rstd.astype(np.float32)
    out["ln_bwd_16x512x1600"] = timed(lambda: oracle.layernorm_backward(r.x.value, r.dy.value, m32, r32, r.w.value,
                                                                        threads=cores))
    for dt in (wl.BF16, wl.F32):
        q = wl.rms_bwd(dt)
        rms = oracle.rmsnorm_rms(q.x.value, eps=q.eps).astype(np.float32)
        out[f"rms_bwd_2048x8192_{dt}"] = timed(lambda q=q, rms=rms: oracle.rmsnorm_backward(
            q.x.value, q.dy.value, q.w.value, rms, eps=q.eps, threads=cores))
    return {k: {"ms_per_call": v[0], "repetitions": v[1], "cores": cores} for k, v in out.items()}


# ---- workloads ------------------------------------------------------------------------------
MAIN = "bn2d_train_fwd_bwd_nchw_256x32x32x32_f32"
BIG = "bn2d_train_fwd_bwd_nchw_64x256x56x56_bf16"


def workload_table(wl):
    """name -> (kind, factory, extra).  Names carry the shape and dtypes."""
    return {
        MAIN: ("bn", lambda: wl.bn_cifar(wl.F32), {}),
        BIG: ("bn", wl.bn_resnet, {}),
        "bn2d_train_fwd_bwd_nchw_256x32x32x32_bf16": ("bn", lambda: wl.bn_cifar(wl.BF16), {}),
        "bn2d_train_fwd_bwd_nchw_3x37x41x40_f32": ("bn", wl.bn_ragged, {}),
        "ln_bwd_16x512x1600_xf32_dybf16_wbf16": ("rows", wl.ln_bwd, {"kind": "ln"}),
        "rms_bwd_2048x8192_bf16_saved_rms": ("rows", lambda: wl.rms_bwd(wl.BF16), {"kind": "rms", "saved": True}),
        "rms_bwd_2048x8192_bf16_recompute_rms": ("rows", lambda: wl.rms_bwd(wl.BF16),
                                                 {"kind": "rms", "saved": False}),
        "rms_bwd_2048x8192_f32_saved_rms": ("rows", lambda: wl.rms_bwd(wl.F32), {"kind": "rms", "saved": True}),
        "rms_bwd_2048x8192_f32_recompute_rms": ("rows", lambda: wl.rms_bwd(wl.F32), {"kind": "rms", "saved": False}),
        "ln_fwd_16x512x1600_xf32_wbf16": ("rows_fwd", wl.ln_bwd, {"kind": "ln"}),
        "rms_fwd_2048x8192_bf16": ("rows_fwd", lambda: wl.rms_bwd(wl.BF16), {"kind": "rms"}),
        "rms_fwd_2048x8192_f32": ("rows_fwd", lambda: wl.rms_bwd(wl.F32), {"kind": "rms"}),
        "bn2d_relu_train_fwd_bwd_nchw_256x32x32x32_f32": ("bn", lambda: wl.bn_cifar(wl.F32), {"act": "relu"}),
        "bn2d_relu_train_fwd_bwd_nchw_64x256x56x56_bf16": ("bn", wl.bn_resnet, {"act": "relu"}),
        "bn2d_infer_relu_nchw_256x32x32x32_f32": ("bn_infer", lambda: wl.bn_cifar(wl.F32), {}),
        "bn2d_infer_relu_nchw_64x256x56x56_bf16": ("bn_infer", wl.bn_resnet, {}),
        "bda_ln_bwd_16x512x1600": ("bda", wl.bda_bwd, {}),
    }


def run_workload(nh, torch, wl, name, K, W, reps):
    kind, factory, extra = workload_table(wl)[name]
    case = factory()
    if kind == "bn":
        return bench_bn(nh, torch, case, K, W, reps, act=extra.get("act", "none"))
    if kind == "bn_infer":
        return bench_bn_infer(nh, torch, case, K, W, reps)
    if kind == "rows":
        return bench_rows(nh, torch, case, extra["kind"], K, W, reps, saved=extra.get("saved", True))
    if kind == "rows_fwd":
        return bench_rows_fwd(nh, torch, case, extra["kind"], K, W, reps)
    if kind == "bda":
        return bench_bda(nh, torch, case, K, W, reps)
    raise KeyError(name)


def _floors_for_bn(nh, torch, res, K, W, reps):
    """Independent streams of the BatchNorm kernels' sizes: the reduction
    passes' reads (x; x and dy), the dx pass's two reads and one write, and a
    copy of x (the apply pass's read + write), the last two both cold and with
    their sources just read (as the elementwise passes find x and dy)."""
    k = res.get("kernels", {})
    if "bn_stats" not in k:
        return None
    E_s = k["bn_stats"]["bytes"]
    fl = {"stats_read": floors_for(nh, torch, E_s, 0, 0, K, W, reps),
          "grad_sums_read": floors_for(nh, torch, 2 * E_s, 0, 0, K, W, reps),
          "dx_add": floors_for(nh, torch, 0, 3 * E_s, 0, K, W, reps),
          "apply_copy": floors_for(nh, torch, 0, 0, 2 * E_s, K, W, reps)}
    n = E_s // 4 // 4 * 4
    fl["apply_copy"]["hip_memcpy_d2d_cached_src"] = floor_warm(nh, torch, n, "copy", K, W, reps)
    fl["dx_add"]["torch_add_cached_srcs"] = floor_warm(nh, torch, n, "add", K, W, reps)
    for v in (fl["apply_copy"]["hip_memcpy_d2d_cached_src"], fl["dx_add"]["torch_add_cached_srcs"]):
        v["frac_of_peak"] = round(v["gbs"] / HBM_PEAK_GBS, 4)
    for kname, fkey, skey in (("bn_stats", "stats_read", "read_stream"), ("bn_grad_sums", "grad_sums_read",
                                                                           "read_stream")):
        k[kname]["frac_of_read_stream"] = round(k[kname]["gbs"] / fl[fkey][skey]["gbs"], 4)
    return fl


def _roofline(res, traffic_tag):
    k = res["kernels"]
    hbm = [n for n, v in k.items() if v.get("input_from") == "hbm"]
    dom = max(hbm, key=lambda n: k[n]["avg_us"])
    v = k[dom]
    return {"kernel": dom, "bound": "hbm", "achieved": v["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": v["frac_of_peak"], "traffic": _traffic_for(dom, traffic_tag), "avg_us": v["avg_us"],
            "algorithmic_bytes": v["bytes"], "input_from": "hbm (cold per call)",
            "timing": "HIP event pair around K back-to-back stage-1 calls on the launch stream"}


# ---- rocprofv3 summaries (text files under profiles/) ---------------------------------------
KERNEL_SOURCES = ["bn_kernels.hip", "nh_device.hpp", "nh_internal.hpp", "nh_bn.hpp", "rows_kernels.hip",
                  "rows_common.hpp", "nh_rows.hpp", "rows_fwd_kernels.hip", "rows_bda_kernels.hip",
                  "rows_generic_kernels.hip", "calib_kernels.hip"]
_COMMON_SOURCES = ["nh_device.hpp", "nh_internal.hpp"]
_BN_SOURCES = ["bn_kernels.hip", "nh_bn.hpp"] + _COMMON_SOURCES
_ROWS_SOURCES = ["rows_kernels.hip", "rows_common.hpp", "nh_rows.hpp", "rows_fwd_kernels.hip",
                 "rows_bda_kernels.hip", "rows_generic_kernels.hip"] + _COMMON_SOURCES


def workload_sources(workload):
    """The kernel sources a workload's kernels are compiled from: a counter
    summary stays valid until one of these changes."""
    return _BN_SOURCES if workload.startswith("bn") else _ROWS_SOURCES
PROFILE_TRACE = ("rocprofv3 --kernel-trace --stats -f csv -d <dir> -o {w} -- python3 bench.py --workloads {w} "
                 "--steps 20 --warmup 3 --reps 3 --no-cpu-baseline --no-floors")
PROFILE_PMC = ("rocprofv3 --pmc {counter} -f csv -d <dir> -o {w} -- python3 bench.py --workloads {w} --steps 4 "
               "--warmup 1 --reps 1 --no-cpu-baseline --no-floors --no-calib --eager")
PROFILE_CALIB = ("rocprofv3 --pmc {counter} -f csv -d <dir> -o calib -- python3 bench.py --calib-only")


def _short_kernel(name):
    import re
    return re.sub(r"\(.*", "", name).replace("void ", "").strip()


def sources_digest(files=KERNEL_SOURCES):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "bwd_bn_stats_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def calib_run(nh, torch):
    """Known-size streams for scaling the HBM byte counters: nh_calib_add of
    two 32 MiB reads and one 32 MiB write, cold, ten times."""
    device = torch.device("cuda:0")
    n = 8 * 1024 * 1024
    R = _nsets(12 * n)
    sets = [(torch.ones(n, device=device), torch.ones(n, device=device), torch.empty(n, device=device))
            for _ in range(R)]
    torch.cuda.synchronize()
    for i in range(10):
        a, b, o = sets[i % R]
        nh.calib_add(a, b, o)
    torch.cuda.synchronize()


def summarize_workload(workload, trace_csv, fetch_csv, write_csv, calib_fetch_csv, calib_write_csv, out_path):
    """One workload's kernels: calls and mean duration (kernel trace), and
    data-fabric bytes per dispatch (FETCH_SIZE / WRITE_SIZE, each scaled by
    the same counter on the calibration add of known size).  The counters
    see the L2's traffic to the fabric, so reads the Infinity Cache serves
    count as well as HBM reads; no counter separates the two."""
    import collections
    import csv

    def per_kernel(path, value):
        d = collections.OrderedDict()
        for r in csv.DictReader(open(path)):
            name = _short_kernel(r["Kernel_Name"])
            d.setdefault(name, []).append(value(r))
        return d

    dur = per_kernel(trace_csv, lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    ctx = _context_split(trace_csv)
    fet = per_kernel(fetch_csv, lambda r: float(r["Counter_Value"])) if fetch_csv else {}
    wri = per_kernel(write_csv, lambda r: float(r["Counter_Value"])) if write_csv else {}
    cf = per_kernel(calib_fetch_csv, lambda r: float(r["Counter_Value"])) if calib_fetch_csv else {}
    cw = per_kernel(calib_write_csv, lambda r: float(r["Counter_Value"])) if calib_write_csv else {}
    n = 8 * 1024 * 1024
    ck = next((k for k in cf if "calib_add" in k), None)
    fscale = (2 * n * 4) / (np.mean(cf[ck]) * 1024) if ck else None
    wscale = (n * 4) / (np.mean(cw[ck]) * 1024) if ck and ck in cw else None
    lines = [f"# {workload}: MI355X kernel durations (rocprofv3 kernel trace) and data-fabric bytes per dispatch",
             f"command_trace: {PROFILE_TRACE.format(w=workload)}",
             f"command_fetch: {PROFILE_PMC.format(counter='FETCH_SIZE', w=workload)}",
             f"command_write: {PROFILE_PMC.format(counter='WRITE_SIZE', w=workload)}",
             f"command_calib: {PROFILE_CALIB.format(counter='FETCH_SIZE')} (and WRITE_SIZE)",
             f"summarized by: python bench.py --summarize {workload} <trace.csv> <fetch.csv> <write.csv> "
             "<calib_fetch.csv> <calib_write.csv>",
             "protocol: every call cold (inputs last touched > 1 GiB earlier); no warm steps",
             f"fetch_scale: {fscale:.5f}" if fscale else "fetch_scale: none",
             f"write_scale: {wscale:.5f}" if wscale else "write_scale: none",
             "note: read_MB / write_MB are the L2's traffic to the data fabric (FETCH_SIZE / WRITE_SIZE): reads "
             "the Infinity Cache serves count as well as HBM reads; the PMC passes run eagerly (no graph replay)",
             f"sources: {','.join(workload_sources(workload))}",
             f"source_sha256_16: {sources_digest(workload_sources(workload))}",
             "",
             f"{'kernel':70s} {'calls':>6s} {'avg_us':>8s} {'min_us':>8s} {'max_us':>8s} {'read_MB':>9s} {'write_MB':>9s}"]
    for k, ds in dur.items():
        if not k.startswith("nh::"):
            continue
        rd = f"{np.mean(fet[k]) * 1024 * fscale / 1e6:9.2f}" if fscale and k in fet else f"{'-':>9s}"
        wr = f"{np.mean(wri[k]) * 1024 * wscale / 1e6:9.2f}" if wscale and k in wri else f"{'-':>9s}"
        lines.append(f"{k[:70]:70s} {len(ds):6d} {np.mean(ds):8.3f} {np.min(ds):8.3f} {np.max(ds):8.3f} {rd} {wr}")
        lines += _context_lines(ctx.get(k, {}), 57)
    open(out_path, "w").write("\n".join(lines) + "\n")


def _context_split(trace_csv):
    """Each dispatch's duration grouped by kernel, then by the kernel
    dispatched just before it (the same kernel in a reduction-only region,
    the other passes in a step)."""
    import collections
    import csv
    ctx = collections.OrderedDict()
    prev = None
    for r in sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Dispatch_Id"])):
        name = _short_kernel(r["Kernel_Name"])
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        ctx.setdefault(name, collections.OrderedDict()).setdefault(prev, []).append(d)
        prev = name
    return ctx


def _context_lines(by_prev, width):
    out = []
    for p, v in by_prev.items():
        if len(v) >= 5:
            out.append(f"    after {(p or '(first)').replace('nh::', '')[:width]:{width}s} {len(v):6d} {np.mean(v):8.3f}")
    return out


def summarize_stats(stats_csv, trace_csv, out_path, command):
    """rocprofv3 --stats kernel table of one command -> short text, with each
    library kernel's durations split by the kernel dispatched before it when
    the kernel trace is given."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    ctx = _context_split(trace_csv) if trace_csv else {}
    lines = ["# rocprofv3 kernel-trace statistics (MI355X)", f"command: {command}",
             f"source_sha256_16: {sources_digest()}", "",
             f"{'kernel':80s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
    for r in rows:
        name = _short_kernel(r['Name'])
        lines.append(f"{name[:80]:80s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.3f} "
                     f"{float(r['MinNs']) / 1e3:9.3f} {float(r['MaxNs']) / 1e3:9.3f}")
        if name.startswith("nh::"):
            lines += _context_lines(ctx.get(name, {}), 67)
    open(out_path, "w").write("\n".join(lines) + "\n")


PROFILE_UTIL_COUNTERS = "VALUBusy MemUnitStalled SQ_INSTS_VALU SQ_INSTS_VMEM_RD SQ_WAVES"
PROFILE_UTIL = ("rocprofv3 --pmc " + PROFILE_UTIL_COUNTERS + " -f csv -d <dir> -o {w} -- python3 bench.py "
                "--workloads {w} --steps 4 --warmup 1 --reps 1 --no-cpu-baseline --no-floors --no-calib --eager")


def summarize_util(workload, counter_csv, out_path):
    """One workload's library kernels: the mean per dispatch of each counter of
    one rocprofv3 --pmc pass (VALUBusy: % of GPU time the vector ALUs issue;
    MemUnitStalled: % of GPU time the memory unit stalls; instruction and
    wave counts per dispatch)."""
    import collections
    import csv
    vals = collections.OrderedDict()
    for r in csv.DictReader(open(counter_csv)):
        name = _short_kernel(r["Kernel_Name"])
        if name.startswith("nh::"):
            vals.setdefault(name, collections.OrderedDict()).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
    names = PROFILE_UTIL_COUNTERS.split()
    lines = [f"# {workload}: MI355X per-kernel utilisation counters (one rocprofv3 --pmc pass, eager calls)",
             f"command: {PROFILE_UTIL.format(w=workload)}",
             f"summarized by: python bench.py --summarize-util {workload} <counter_collection.csv>",
             "note: VALUBusy = % of GPU time the vector ALUs issue instructions; MemUnitStalled = % of GPU time "
             "the memory unit is stalled; the other columns are per-dispatch totals",
             f"sources: {','.join(workload_sources(workload))}",
             f"source_sha256_16: {sources_digest(workload_sources(workload))}",
             "",
             f"{'kernel':70s} {'calls':>6s} " + " ".join(f"{n:>16s}" for n in names)]
    for k, d in vals.items():
        calls = max(len(v) for v in d.values())
        cols = " ".join(f"{np.mean(d[n]):16.2f}" if n in d else f"{'-':>16s}" for n in names)
        lines.append(f"{k[:70]:70s} {calls:6d} {cols}")
    open(out_path, "w").write("\n".join(lines) + "\n")


def _traffic_for(kernel_key, workload):
    """Data-fabric bytes per launch (read + write) of a kernel from the
    committed counter summary of `workload`, if it was taken on the current kernel
    sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"{workload}.txt")
    if not os.path.exists(path):
        return None
    digest, rows = None, []
    for line in open(path):
        if line.startswith("source_sha256_16:"):
            digest = line.split(":", 1)[1].strip()
        elif line.startswith("nh::"):
            rows.append((line[:70].strip(), line[70:].split()))
    if digest != sources_digest(workload_sources(workload)):
        return None
    want = "nh::" + {"bn_stats": "bn_stats_kernel", "bn_grad_sums": "bn_grad_sums_kernel",
                     "bn_apply": "bn_apply_kernel", "bn_dx": "bn_dx_kernel"}.get(kernel_key, kernel_key)
    for name, f in rows:
        if name.startswith(want) and len(f) == 6:
            try:
                return round((float(f[4]) + float(f[5])) * 1e6)
            except ValueError:
                return None
    return None


# ---- main ------------------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40, help="calls per timed region")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--reps", type=int, default=5, help="repetitions of every timed region")
    ap.add_argument("--quick", action="store_true", help="main workload only")
    ap.add_argument("--workloads", default="", help="comma-separated workload names (default: all)")
    ap.add_argument("--list", action="store_true", help="print the workload names and exit")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-floors", action="store_true")
    ap.add_argument("--no-calib", action="store_true")
    ap.add_argument("--calib-only", action="store_true", help="run the counter-scaling streams only")
    ap.add_argument("--eager", action="store_true",
                    help="issue every timed call from the host instead of replaying captured graphs")
    ap.add_argument("--summarize", nargs=6, metavar=("WORKLOAD", "TRACE", "FETCH", "WRITE", "CALIB_FETCH",
                                                     "CALIB_WRITE"),
                    help="write profiles/<WORKLOAD>.txt from rocprofv3 csv files and exit")
    ap.add_argument("--summarize-util", nargs=2, metavar=("WORKLOAD", "COUNTER_CSV"),
                    help="write profiles/<WORKLOAD>_util.txt from a rocprofv3 --pmc csv and exit")
    ap.add_argument("--summarize-stats", nargs=3, metavar=("STATS_CSV", "TRACE_CSV", "OUT"),
                    help="write a profiles/ summary of a rocprofv3 --stats table (TRACE_CSV may be -) and exit")
    args = ap.parse_args()
    if args.summarize:
        w = args.summarize[0]
        files = [f if f != "-" else None for f in args.summarize[1:]]
        summarize_workload(w, *files, os.path.join(ROOT, "profiles", f"{w}.txt"))
        return
    if args.summarize_util:
        w = args.summarize_util[0]
        summarize_util(w, args.summarize_util[1], os.path.join(ROOT, "profiles", f"{w}_util.txt"))
        return
    if args.summarize_stats:
        cmd = "rocprofv3 --kernel-trace --stats -f csv -d <dir> -o bench -- python3 bench.py"
        tr = args.summarize_stats[1]
        summarize_stats(args.summarize_stats[0], tr if tr != "-" else None, args.summarize_stats[2], cmd)
        return
    from bwd_bn_stats_amd import workloads as wl
    if args.list:
        print("\n".join(workload_table(wl)))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "this library has no multi-GPU path to time.", file=sys.stderr)
        sys.exit(2)

    import torch
    from bwd_bn_stats_amd import normhip as nh

    torch.cuda.set_device(0)
    K, W, reps = args.steps, args.warmup, args.reps
    Regions.EAGER = args.eager
    if args.calib_only:
        calib_run(nh, torch)
        return
    log(f"[bench] device: {torch.cuda.get_device_name(0)}")
    names = [n for n in args.workloads.split(",") if n] if args.workloads else (
        [MAIN] if args.quick else list(workload_table(wl)))
    results = {}
    for name in names:
        log(f"[bench] {name}")
        results[name] = run_workload(nh, torch, wl, name, K, W, reps)
        r = results[name]
        t = r.get("step", r.get("call", {})).get("median_us")
        log(f"[bench]   {t} us/call")
    if not args.no_calib and not args.workloads:
        calib_run(nh, torch)   # counter-scaling streams, also in the default run's kernel trace

    floors = {}
    if not args.no_floors:
        for name in (MAIN, BIG):
            if name in results and "kernels" in results[name]:
                log(f"[bench] independent floors at {name}'s sizes")
                floors[name] = _floors_for_bn(nh, torch, results[name], K, W, reps)
        if not args.workloads:
            log("[bench] independent floors at >= 1 GiB")
            kk = max(5, K // 4)
            floors["ge_1GiB"] = {"hip_memcpy_d2d_2GiB": floor_memcpy(torch, GiB, kk, 2, reps),
                                 "torch_add_1.2GB": floor_torch_add(torch, 100663296, kk, 2, reps),
                                 "read_stream_1GiB": floor_read(nh, torch, GiB // 4, kk, 2, reps),
                                 "torch_sum_1GiB": floor_torch_sum(torch, GiB // 4, kk, 2, reps)}
            for v in floors["ge_1GiB"].values():
                v["frac_of_peak"] = round(v["gbs"] / HBM_PEAK_GBS, 4)
            for wname, key, nb in (("rms_bwd_2048x8192_bf16_saved_rms", "add", 100663296),
                                   ("rms_bwd_2048x8192_f32_saved_rms", "add", 201326592),
                                   ("ln_bwd_16x512x1600_xf32_dybf16_wbf16", "add", 131072000),
                                   ("ln_fwd_16x512x1600_xf32_wbf16", "copy", 104857600),
                                   ("rms_fwd_2048x8192_bf16", "copy", 67108864)):
                if wname in results:
                    log(f"[bench] independent floors at {wname}'s size")
                    floors[wname] = floors_for(nh, torch, 0, nb if key == "add" else 0,
                                               nb if key == "copy" else 0, K, W, reps)

    if MAIN not in results:
        print(json.dumps({"workloads": results, "floors": floors}), flush=True)
        return
    main_r = results[MAIN]
    step_us = main_r["step"]["median_us"]
    out = {
        "metric": METRIC,
        "value": main_r["one_touch_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(step_us / 1000.0, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": MAIN, "shape_nchw": [256, 32, 32, 32], "io": "f32", "stats": "f32",
                   "step": "bn_forward_train + bn_backward", "cache": "cold per call",
                   "value_bytes": "minimal: read x, write y; read x and dy, write dx", "parallelism": "single GPU"},
        "us_per_call": step_us,
        "frac_of_peak": round(main_r["one_touch_gbs"] / HBM_PEAK_GBS, 4),
        "algorithmic_gbs": main_r["algorithmic_gbs"],
        "step": main_r["step"],
        "per_call": main_r["calls"],
        "roofline": _roofline(main_r, MAIN),
        "kernels": main_r["kernels"],
    }
    if BIG in results:
        big = dict(results[BIG])
        big["roofline"] = _roofline(big, BIG)
        big["frac_of_peak"] = round(big["one_touch_gbs"] / HBM_PEAK_GBS, 4)
        out[BIG] = big
    out["others"] = {k: v for k, v in results.items() if k not in (MAIN, BIG)}
    out["floors"] = floors
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline: the oracle on the host")
        out["cpu_baseline"] = cpu_baseline(wl.bn_cifar(wl.F32))
        if not args.quick and not args.workloads:
            out["cpu_baseline"]["other_configs"] = cpu_oracle_times()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
