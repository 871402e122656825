"""Benchmark of the normalization hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--quick] [--no-cpu-baseline]

A step is one BatchNorm2d training forward + backward (bn_forward_train then
bn_backward) over the CIFAR-shaped NCHW (256,32,32,32) fp32 batch, the
workload of the Aether-ML BatchNorm PR's kernel measurements.  Inputs are
resident in HBM before the timed region.  To time HBM rather than the 256 MB
Infinity Cache, consecutive steps rotate through enough independent buffer
sets that each step's tensors were last touched more than 1 GiB of traffic
earlier ("cold"); back-to-back steps on one set ("warm") are reported too.

Printed: ONE JSON line with the step throughput (algorithmic bytes of the
forward + backward / step time), the roofline of the dominant kernel (its
average duration from hipExtLaunchKernel start/stop events recorded during
the timed region), the per-kernel breakdown, a calibration floor (a plain
two-read/one-write stream of the same size) and the CPU oracle's throughput
on this host.  The other workloads (bf16 BatchNorm shapes, LayerNorm and
RMSNorm backward) are measured the same way and reported under "others".
"""
from __future__ import annotations

import argparse
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
COLD_BYTES = 1 << 30  # traffic between two touches of the same buffer set


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------------
def _dev(t, device):
    import numpy as np
    import torch
    from bwd_bn_stats_amd import workloads as wl
    if isinstance(t, wl.Tensor):
        if t.dtype == wl.F32:
            return torch.from_numpy(np.ascontiguousarray(t.store)).to(device)
        return torch.from_numpy(np.ascontiguousarray(t.store).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(t, dtype=np.float32)).to(device)


def _nsets(set_bytes, cold):
    if not cold:
        return 1
    return max(2, int(-(-COLD_BYTES // max(set_bytes, 1))) + 1)


class Timed:
    """Runs `step(i)` K times after W warmups; returns host-clock ms/step and
    per-kernel event durations recorded during the timed region."""

    def __init__(self, nh, torch):
        self.nh, self.torch = nh, torch

    def run(self, step, K, W, kernels, launches_per_step=8):
        """Returns (ms per step of the un-instrumented timed region, per-kernel
        event durations of an identical instrumented region run right after).

        The per-kernel start/stop events ride on the dispatch packets
        (hipExtLaunchKernel) and time each kernel exactly, but they stop the
        queue from overlapping one kernel's drain with the next one's launch,
        so the step time is taken from a region without them."""
        nh, torch = self.nh, self.torch
        nh.timing_reserve(K * launches_per_step)
        for i in range(W):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            step(W + i)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        nh.timing_enable(True)
        t2 = time.perf_counter()
        for i in range(K):
            step(W + K + i)
        torch.cuda.synchronize()
        self.events_ms = 1000.0 * (time.perf_counter() - t2) / K
        nh.timing_enable(False)
        per = {}
        for k in kernels:
            ms, n = nh.timing_read(k)
            if n:
                per[k] = {"launches": n, "avg_us": 1000.0 * ms / n}
        return 1000.0 * (t1 - t0) / K, per

    def per_call(self, parts, K, start):
        """Times each call of `parts` ([(name, fn(i))], run in order as one
        step) with stream events around it, over K cold steps; returns
        p10/median/p90 in microseconds per part and for their sum."""
        torch = self.torch
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)] for _ in range(K)]
        torch.cuda.synchronize()
        for i in range(K):
            ev[i][0].record()
            for j, (_, fn) in enumerate(parts):
                fn(start + i)
                ev[i][j + 1].record()
        torch.cuda.synchronize()
        out = {}
        cols = [[1000.0 * ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(K)] for j in range(len(parts))]
        if len(parts) > 1:
            cols.append([sum(c[i] for c in cols) for i in range(K)])
        names = [n for n, _ in parts] + (["sum"] if len(parts) > 1 else [])
        for n, c in zip(names, cols):
            q = np.percentile(np.asarray(c), [10, 50, 90])
            out[n] = {"p10_us": round(float(q[0]), 2), "median_us": round(float(q[1]), 2),
                      "p90_us": round(float(q[2]), 2)}
        return out


# ---- BatchNorm --------------------------------------------------------------------
BN_KERNELS = ["bn_stats", "bn_fwd_finalize", "bn_apply", "bn_grad_sums", "bn_bwd_finalize", "bn_dx",
              "bn_fwd_channel", "bn_bwd_channel"]
ACT_IDS = {"none": 0, "relu": 1, "leaky_relu": 2}


def bn_bytes(case):
    """Algorithmic bytes per launch: inputs read once, outputs written once."""
    s = 4 if case.io == "f32" else 2
    E = case.N * case.C * case.hw
    # The one-block-per-channel kernels do both passes of a direction: the
    # reduction's reads and the elementwise pass's reads and writes.
    return {"bn_stats": E * s, "bn_apply": 2 * E * s, "bn_grad_sums": 2 * E * s, "bn_dx": 3 * E * s,
            "bn_fwd_finalize": None, "bn_bwd_finalize": None,
            "bn_fwd_channel": 3 * E * s, "bn_bwd_channel": 5 * E * s}


BN_STEP_KERNELS = ("bn_stats", "bn_apply", "bn_grad_sums", "bn_dx")


def bench_bn(nh, torch, case, K, W, cold=True, act="none", slope=0.01):
    import ctypes
    device = torch.device("cuda:0")
    x0, dy0 = _dev(case.x, device), _dev(case.dy, device)
    g, b = _dev(case.gamma, device), _dev(case.beta, device)
    io = 0 if case.io == "f32" else 1
    N, C, HW = case.N, case.C, case.hw
    wsb = nh.bn_forward_train_workspace(N, C, HW)
    set_bytes = 4 * x0.numel() * x0.element_size()
    R = _nsets(set_bytes, cold)
    sets = []
    for _ in range(R):
        s = dict(x=x0.clone(), dy=dy0.clone(), y=torch.empty_like(x0), dx=torch.empty_like(x0),
                 rm=torch.zeros(C, device=device), rv=torch.ones(C, device=device),
                 stats=torch.empty(4, C, device=device), grads=torch.empty(4, C, device=device),
                 ws=torch.empty(max(wsb, 16), dtype=torch.uint8, device=device))
        sets.append(s)
    torch.cuda.synchronize()
    P = ctypes.c_void_p
    stream = P(torch.cuda.current_stream(device).cuda_stream)
    calls = []
    for s in sets:
        p = {k: P(v.data_ptr()) for k, v in s.items()}
        calls.append((p, s["ws"].numel()))
    lib = nh.lib

    a = ACT_IDS[act]

    def fwd(i):
        p, nb = calls[i % R]
        if act == "none":
            st = lib.bn_forward_train(p["x"], p["y"], io, N, C, HW, P(g.data_ptr()), P(b.data_ptr()),
                                      p["rm"], p["rv"], case.momentum, case.eps, p["stats"], p["ws"],
                                      nb, stream)
        else:
            st = lib.bn_act_forward_train(p["x"], p["y"], io, N, C, HW, P(g.data_ptr()),
                                          P(b.data_ptr()), p["rm"], p["rv"], case.momentum, case.eps,
                                          a, slope, p["stats"], p["ws"], nb, stream)
        if st:
            raise RuntimeError(nh.last_error())

    def bwd(i):
        p, nb = calls[i % R]
        if act == "none":
            st = lib.bn_backward(p["dy"], p["x"], io, N, C, HW, p["stats"], p["dx"], p["grads"],
                                 p["ws"], nb, stream)
        else:
            st = lib.bn_act_backward(p["dy"], p["x"], io, N, C, HW, p["stats"], P(b.data_ptr()), a,
                                     slope, p["dx"], p["grads"], p["ws"], nb, stream)
        if st:
            raise RuntimeError(nh.last_error())

    def step(i):
        fwd(i)
        bwd(i)

    tm = Timed(nh, torch)
    ms, per = tm.run(step, K, W, BN_KERNELS)
    calls_pct = tm.per_call([("bn_forward_train", fwd), ("bn_backward", bwd)], K, W + 2 * K)
    byt = bn_bytes(case)
    for k, v in per.items():
        if byt.get(k):
            v["bytes"] = byt[k]
            v["gbs"] = byt[k] / (v["avg_us"] * 1e3)
            v["frac_of_peak"] = v["gbs"] / HBM_PEAK_GBS
    step_bytes = sum(byt[k] for k in BN_STEP_KERNELS)  # the same on either path
    del sets, calls
    torch.cuda.empty_cache()
    # one-touch minimum: forward x + y, backward x + dy + dx
    one_touch = 5 * N * C * HW * (4 if case.io == "f32" else 2)
    return {"ms_per_step": ms, "us_per_call": 1000.0 * ms,
            "us_per_call_with_kernel_events": 1000.0 * tm.events_ms, "step_bytes": step_bytes,
            "gbs": step_bytes / (ms * 1e6), "one_touch_bytes": one_touch,
            "one_touch_gbs": one_touch / (ms * 1e6), "buffer_sets": R, "kernels": per,
            "per_call": calls_pct, "grid_y": nh.bn_plan(N, C, HW, io)}


def bench_bn_graph(nh, torch, case, K, W):
    """A launch-bound step (small shape): fwd+bwd issued eagerly, one call
    at a time, against the same two calls captured once in a HIP graph and
    replayed.  Buffers stay warm (the shape fits in cache)."""
    device = torch.device("cuda:0")
    x, dy = _dev(case.x, device), _dev(case.dy, device)
    g, b = _dev(case.gamma, device), _dev(case.beta, device)
    ws = torch.empty(max(16, nh.bn_forward_train_workspace(case.N, case.C, case.hw)), dtype=torch.uint8,
                     device=device)
    y, dx = torch.empty_like(x), torch.empty_like(x)
    stats = torch.empty(4, case.C, device=device)
    grads = torch.empty(4, case.C, device=device)

    def step():
        nh.bn_forward_train(x, g, b, None, None, case.momentum, case.eps, y=y, stats=stats,
                            workspace=ws)
        nh.bn_backward(dy, x, stats, dx=dx, grads=grads, workspace=ws)

    for _ in range(W):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    eager_us = 1e6 * (time.perf_counter() - t0) / K
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    res = {"eager_us_per_step": round(eager_us, 2), "kernels_per_step": 4}
    for inner in (1, 10):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(inner):
                step()
        for _ in range(W):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            graph.replay()
        torch.cuda.synchronize()
        res[f"graph_{inner}_steps_us_per_step"] = round(1e6 * (time.perf_counter() - t0) / (K * inner), 2)
        del graph
    return res


def bench_bn_infer(nh, torch, case, K, W, act="relu", slope=0.01):
    """BatchNorm2d inference (+ activation): one elementwise pass, x read and
    y written once."""
    import ctypes
    device = torch.device("cuda:0")
    x0 = _dev(case.x, device)
    g, b = _dev(case.gamma, device), _dev(case.beta, device)
    io = 0 if case.io == "f32" else 1
    N, C, HW = case.N, case.C, case.hw
    rm = torch.linspace(-0.5, 0.5, C, device=device)
    rv = torch.linspace(0.5, 2.0, C, device=device)
    R = _nsets(2 * x0.numel() * x0.element_size(), True)
    sets = [(x0.clone(), torch.empty_like(x0)) for _ in range(R)]
    torch.cuda.synchronize()
    P = ctypes.c_void_p
    stream = P(torch.cuda.current_stream(device).cuda_stream)
    ptrs = [(P(x.data_ptr()), P(y.data_ptr())) for x, y in sets]
    a = ACT_IDS[act]

    def step(i):
        x, y = ptrs[i % R]
        if nh.lib.bn_forward_infer(x, y, io, N, C, HW, P(g.data_ptr()), P(b.data_ptr()),
                                   P(rm.data_ptr()), P(rv.data_ptr()), case.eps, a, slope, stream):
            raise RuntimeError(nh.last_error())

    tm = Timed(nh, torch)
    ms, per = tm.run(step, K, W, ["bn_infer"], launches_per_step=1)
    byt = 2 * x0.numel() * x0.element_size()
    for v in per.values():
        v["bytes"] = byt
        v["gbs"] = byt / (v["avg_us"] * 1e3)
        v["frac_of_peak"] = v["gbs"] / HBM_PEAK_GBS
    del sets, ptrs
    torch.cuda.empty_cache()
    return {"ms_per_step": ms, "us_per_call": 1000.0 * ms, "step_bytes": byt,
            "gbs": byt / (ms * 1e6), "buffer_sets": R, "kernels": per}


# ---- LayerNorm / RMSNorm -----------------------------------------------------------
def bench_rows(nh, torch, case, kind, K, W, cold=True, saved=True):
    import ctypes
    device = torch.device("cuda:0")
    x0, dy0, w = _dev(case.x, device), _dev(case.dy, device), _dev(case.w, device)
    R_, H = case.rows, case.cols
    xf = x0.float()
    if kind == "ln":
        var, mean = torch.var_mean(xf, dim=1, unbiased=False)
        stat_a, stat_b = mean.contiguous(), torch.rsqrt(var + case.eps).contiguous()
        wsb = nh.layernorm_backward_workspace(R_, H)
    else:
        stat_a = torch.sqrt((xf * xf).mean(dim=1) + case.eps).contiguous()
        stat_b = None
        wsb = nh.rmsnorm_backward_workspace(R_, H)
    del xf
    dx_dtype = x0.dtype
    set_bytes = x0.numel() * (x0.element_size() * 2 + dy0.element_size())
    R = _nsets(set_bytes, cold)
    sets = [dict(x=x0.clone(), dy=dy0.clone(), dx=torch.empty(x0.shape, dtype=dx_dtype, device=device),
                 dw=torch.empty(H, dtype=w.dtype, device=device),
                 db=torch.empty(H, dtype=w.dtype, device=device),
                 ws=torch.empty(max(wsb, 16), dtype=torch.uint8, device=device)) for _ in range(R)]
    torch.cuda.synchronize()
    P = ctypes.c_void_p
    stream = P(torch.cuda.current_stream(device).cuda_stream)
    dt = {torch.float32: 0, torch.bfloat16: 1}
    calls = [({k: P(v.data_ptr()) for k, v in s.items()}, s["ws"].numel()) for s in sets]
    lib = nh.lib
    pa, pb, pw = P(stat_a.data_ptr()), (P(stat_b.data_ptr()) if stat_b is not None else None), P(w.data_ptr())

    if kind == "ln":
        def step(i):
            p, nb = calls[i % R]
            st = lib.layernorm_backward(p["dy"], dt[dy0.dtype], p["x"], dt[x0.dtype], pa, pb, pw,
                                        dt[w.dtype], R_, H, p["dx"], dt[dx_dtype], p["dw"], p["db"],
                                        p["ws"], nb, stream)
            if st:
                raise RuntimeError(nh.last_error())
        kernels = ["ln_rows", "ln_colsum", "rows_coef"]
    else:
        rms_p = pa if saved else None

        def step(i):
            p, nb = calls[i % R]
            st = lib.rmsnorm_backward(p["dy"], p["x"], dt[x0.dtype], rms_p, case.eps, pw, R_, H,
                                      p["dx"], p["dw"], p["ws"], nb, stream)
            if st:
                raise RuntimeError(nh.last_error())
        kernels = ["rms_rows", "rms_colsum", "rows_coef"]

    tm = Timed(nh, torch)
    ms, per = tm.run(step, K, W, kernels)
    calls_pct = tm.per_call([("layernorm_backward" if kind == "ln" else "rmsnorm_backward", step)], K,
                            W + 2 * K)
    E = R_ * H
    row_bytes = E * (x0.element_size() + dy0.element_size() + torch.empty(0, dtype=dx_dtype).element_size())
    row_bytes += R_ * 4 * (2 if kind == "ln" else (1 if saved else 0)) + H * w.element_size()
    rk = kernels[0]
    if rk in per:
        per[rk]["bytes"] = row_bytes
        per[rk]["gbs"] = row_bytes / (per[rk]["avg_us"] * 1e3)
        per[rk]["frac_of_peak"] = per[rk]["gbs"] / HBM_PEAK_GBS
    G = nh.rows_plan(R_, H)
    del sets, calls
    torch.cuda.empty_cache()
    return {"ms_per_call": ms, "us_per_call": 1000.0 * ms, "bytes": row_bytes,
            "gbs": row_bytes / (ms * 1e6), "buffer_sets": R, "kernels": per, "blocks_max": G,
            "per_call": calls_pct}


def bench_bda(nh, torch, case, K, W, cold=True):
    """Backward of bias + dropout + add + LayerNorm: reads x, dy, the incoming
    gradient and the mask, writes dh (fp32) and da, plus the column sums."""
    import ctypes
    device = torch.device("cuda:0")
    ln = case.ln
    x0, dy0, w = _dev(ln.x, device), _dev(ln.dy, device), _dev(ln.w, device)
    dres0 = torch.from_numpy(case.dresidual).to(device)
    mask0 = torch.from_numpy(case.mask).to(device)
    R_, H = ln.rows, ln.cols
    var, mean = torch.var_mean(x0.float(), dim=1, unbiased=False)
    mean, rstd = mean.contiguous(), torch.rsqrt(var + ln.eps).contiguous()
    wsb = nh.bda_layernorm_backward_workspace(R_, H)
    E = R_ * H
    per_elem = x0.element_size() + dy0.element_size() + 4 + 1 + 4 + dy0.element_size()
    R = _nsets(E * per_elem, cold)
    sets = [dict(x=x0.clone(), dy=dy0.clone(), dres=dres0.clone(), mask=mask0.clone(),
                 dh=torch.empty(x0.shape, dtype=torch.float32, device=device),
                 da=torch.empty(x0.shape, dtype=dy0.dtype, device=device),
                 dw=torch.empty(H, dtype=w.dtype, device=device),
                 db=torch.empty(H, dtype=w.dtype, device=device),
                 dbi=torch.empty(H, dtype=w.dtype, device=device),
                 ws=torch.empty(max(wsb, 16), dtype=torch.uint8, device=device)) for _ in range(R)]
    torch.cuda.synchronize()
    P = ctypes.c_void_p
    stream = P(torch.cuda.current_stream(device).cuda_stream)
    dt = {torch.float32: 0, torch.bfloat16: 1}
    calls = [({k: P(v.data_ptr()) for k, v in s.items()}, s["ws"].numel()) for s in sets]
    pm, pr, pw = P(mean.data_ptr()), P(rstd.data_ptr()), P(w.data_ptr())

    def step(i):
        p, nb = calls[i % R]
        st = nh.lib.bda_layernorm_backward(p["dy"], dt[dy0.dtype], p["x"], dt[x0.dtype], pm, pr, pw,
                                           dt[w.dtype], p["dres"], p["mask"], case.scale, R_, H,
                                           p["dh"], p["da"], p["dw"], p["db"], p["dbi"], p["ws"], nb,
                                           stream)
        if st:
            raise RuntimeError(nh.last_error())

    kernels = ["bda_rows", "bda_colsum"]
    ms, per = Timed(nh, torch).run(step, K, W, kernels)
    row_bytes = E * per_elem + R_ * 8 + H * w.element_size()
    if "bda_rows" in per:
        per["bda_rows"]["bytes"] = row_bytes
        per["bda_rows"]["gbs"] = row_bytes / (per["bda_rows"]["avg_us"] * 1e3)
        per["bda_rows"]["frac_of_peak"] = per["bda_rows"]["gbs"] / HBM_PEAK_GBS
    G = nh.rows_plan(R_, H)
    del sets, calls
    torch.cuda.empty_cache()
    return {"ms_per_call": ms, "us_per_call": 1000.0 * ms, "bytes": row_bytes,
            "gbs": row_bytes / (ms * 1e6), "buffer_sets": R, "kernels": per, "blocks_max": G}


def bench_rows_fwd(nh, torch, case, kind, K, W, cold=True):
    """LayerNorm / RMSNorm training forward: read x (+ weight, bias once),
    write y and the per-row statistics."""
    import ctypes
    device = torch.device("cuda:0")
    x0, w = _dev(case.x, device), _dev(case.w, device)
    b = _dev(case.b, device) if (kind == "ln" and case.b is not None) else None
    R_, H = case.rows, case.cols
    set_bytes = 2 * x0.numel() * x0.element_size()
    R = _nsets(set_bytes, cold)
    sets = [dict(x=x0.clone(), y=torch.empty_like(x0), s0=torch.empty(R_, device=device),
                 s1=torch.empty(R_, device=device)) for _ in range(R)]
    torch.cuda.synchronize()
    P = ctypes.c_void_p
    stream = P(torch.cuda.current_stream(device).cuda_stream)
    dt = {torch.float32: 0, torch.bfloat16: 1}
    calls = [{k: P(v.data_ptr()) for k, v in s.items()} for s in sets]
    lib = nh.lib
    pw, pb = P(w.data_ptr()), (P(b.data_ptr()) if b is not None else None)
    xt = dt[x0.dtype]
    if kind == "ln":
        def step(i):
            p = calls[i % R]
            st = lib.layernorm_forward(p["x"], xt, pw, pb, dt[w.dtype], R_, H, case.eps, p["y"], xt,
                                       p["s0"], p["s1"], stream)
            if st:
                raise RuntimeError(nh.last_error())
        kernels = ["ln_fwd"]
    else:
        def step(i):
            p = calls[i % R]
            st = lib.rmsnorm_forward(p["x"], xt, pw, R_, H, case.eps, p["y"], p["s0"], stream)
            if st:
                raise RuntimeError(nh.last_error())
        kernels = ["rms_fwd"]
    ms, per = Timed(nh, torch).run(step, K, W, kernels)
    E = R_ * H
    byt = 2 * E * x0.element_size() + R_ * 4 * (2 if kind == "ln" else 1)
    k = kernels[0]
    if k in per:
        per[k]["bytes"] = byt
        per[k]["gbs"] = byt / (per[k]["avg_us"] * 1e3)
        per[k]["frac_of_peak"] = per[k]["gbs"] / HBM_PEAK_GBS
    del sets, calls
    torch.cuda.empty_cache()
    return {"us_per_call": 1000.0 * ms, "bytes": byt, "gbs": byt / (ms * 1e6), "buffer_sets": R,
            "kernels": per}


# ---- calibration floor ---------------------------------------------------------------
def bench_calib(nh, torch, n_floats, K, W):
    device = torch.device("cuda:0")
    set_bytes = 3 * n_floats * 4
    R = _nsets(set_bytes, True)
    sets = [(torch.randn(n_floats, device=device), torch.randn(n_floats, device=device),
             torch.empty(n_floats, device=device)) for _ in range(R)]
    torch.cuda.synchronize()

    def step(i):
        a, b, o = sets[i % R]
        nh.calib_add(a, b, o)

    ms, per = Timed(nh, torch).run(step, K, W, ["calib"])
    byt = 3 * n_floats * 4
    avg = per["calib"]["avg_us"]
    del sets
    torch.cuda.empty_cache()
    return {"bytes": byt, "avg_us": avg, "gbs": byt / (avg * 1e3), "frac_of_peak": byt / (avg * 1e3) / HBM_PEAK_GBS}


def bench_copy(nh, torch, nbytes, K, W):
    """Calibration floor of a one-read/one-write stream: nh_calib_copy of
    nbytes (cold rotating buffers); GB/s counts the bytes read plus written."""
    device = torch.device("cuda:0")
    R = _nsets(2 * nbytes, True)
    sets = [(torch.empty(nbytes, dtype=torch.uint8, device=device),
             torch.empty(nbytes, dtype=torch.uint8, device=device)) for _ in range(R)]
    for a, _ in sets:
        a.fill_(1)
    torch.cuda.synchronize()

    def step(i):
        a, b = sets[i % R]
        nh.calib_copy(a, b)

    ms, per = Timed(nh, torch).run(step, K, W, ["calib"])
    avg = per["calib"]["avg_us"]
    del sets
    torch.cuda.empty_cache()
    return {"bytes": 2 * nbytes, "avg_us": avg, "gbs": 2 * nbytes / (avg * 1e3)}


def bench_read(nh, torch, n_floats, K, W):
    """Calibration floor of a read-only reduction shaped like the stats pass
    (nh_calib_read over n fp32, cold rotating buffers)."""
    device = torch.device("cuda:0")
    R = _nsets(4 * n_floats, True)
    sets = [torch.ones(n_floats, device=device) for _ in range(R)]
    sums = torch.empty(4096, device=device)
    torch.cuda.synchronize()

    def step(i):
        nh.calib_read(sets[i % R], sums)

    ms, per = Timed(nh, torch).run(step, K, W, ["calib"])
    avg = per["calib"]["avg_us"]
    del sets
    torch.cuda.empty_cache()
    return {"bytes": 4 * n_floats, "avg_us": avg, "gbs": 4 * n_floats / (avg * 1e3)}


# ---- CPU baseline: the oracle on this host ----------------------------------------------
def cpu_baseline(case, budget_s=12.0):
    import numpy as np
    import oracle
    oracle.build(force=False)
    x, dy = case.x.value, case.dy.value
    g, b = case.gamma.astype(np.float64), case.beta.astype(np.float64)
    reps, t_total = 0, 0.0
    while t_total < budget_s and reps < 50:
        t0 = time.perf_counter()
        oracle.bn_forward_train(x, g, b, eps=case.eps, momentum=case.momentum,
                                running_mean=case.running_mean, running_var=case.running_var)
        oracle.bn_backward(x, dy, g, eps=case.eps)
        t_total += time.perf_counter() - t0
        reps += 1
    step_bytes = sum(bn_bytes(case)[k] for k in BN_STEP_KERNELS)
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": step_bytes * reps / t_total / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "ms_per_step": 1000.0 * t_total / reps, "cpu_model": model,
            "host_cores_available": os.cpu_count(),
            "sample": f"full {case.N}x{case.C}x{case.hw // 32}x32 {case.io} forward+backward step, "
                      f"{reps} repetitions (fp64, single thread, same algorithmic bytes as the GPU step)"}


# ---- rocprofv3 summaries (text files under profiles/) ------------------------------
PROFILE_CMD_TRACE = ("rocprofv3 --kernel-trace --stats -f csv --kernel-include-regex \"nh::\" "
                     "-d <dir> -o bench_quick -- python3 bench.py --quick --steps 20 --warmup 5 "
                     "--no-cpu-baseline")
PROFILE_CMD_PMC = ("rocprofv3 --pmc {counter} -f csv --kernel-include-regex \"nh::\" -d <dir> "
                   "-o bench_quick -- python3 bench.py --quick --steps 5 --warmup 2 --no-cpu-baseline")
BN_SOURCES = ["bn_kernels.hip", "nh_device.hpp", "nh_internal.hpp", "nh_bn.hpp"]
PROFILE_CMD_ALL_TRACE = ("rocprofv3 --kernel-trace --stats -f csv -d <dir> -o bench_all -- "
                         "python3 bench.py --steps 10 --warmup 2 --no-cpu-baseline")
PROFILE_CMD_ALL_PMC = ("rocprofv3 --pmc {counter} -f csv --kernel-include-regex \"nh::\" -d <dir> "
                       "-o bench_all -- python3 bench.py --steps 4 --warmup 1 --no-cpu-baseline")


def _short_kernel(name):
    import re
    return re.sub(r"\(.*", "", name).replace("void ", "").strip()


def sources_digest(files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "bwd_bn_stats_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def summarize_trace(stats_csv, out_path):
    """Kernel-trace statistics (rocprofv3 --stats) -> short text table."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    lines = ["# rocprofv3 kernel-trace statistics: BatchNorm2d (256,32,32,32) fp32 fwd+bwd",
             "# (cold and warm steps of bench.py --quick plus the calibration add)",
             f"command: {PROFILE_CMD_TRACE}",
             "summarized by: python bench.py --summarize-trace <dir>/bench_quick_kernel_stats.csv",
             "",
             f"{'kernel':60s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
    for r in rows:
        lines.append(f"{_short_kernel(r['Name'])[:60]:60s} {int(r['Calls']):6d} "
                     f"{float(r['AverageNs']) / 1e3:9.3f} {float(r['MinNs']) / 1e3:9.3f} "
                     f"{float(r['MaxNs']) / 1e3:9.3f}")
    open(out_path, "w").write("\n".join(lines) + "\n")


def summarize_counters(fetch_csv, write_csv, out_dir):
    """FETCH_SIZE / WRITE_SIZE per dispatch (first half of each kernel's
    dispatches = the cold steps), scaled by the calibration add of known size
    (two 32 MiB reads, one 32 MiB write).  Writes one file per BN kernel."""
    import collections
    import csv

    def load(path):
        d = collections.OrderedDict()
        for r in csv.DictReader(open(path)):
            d.setdefault(_short_kernel(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        return d

    f, w = load(fetch_csv), load(write_csv)
    cold = {k: sum(v[:max(1, len(v) // 2)]) / max(1, len(v) // 2) for k, v in f.items()}
    coldw = {k: sum(v[:max(1, len(v) // 2)]) / max(1, len(v) // 2) for k, v in w.items()}
    calib = next(k for k in cold if "calib_add4" in k)
    n = 256 * 32 * 32 * 32
    fscale = (2 * n * 4) / (cold[calib] * 1024)
    wscale = (n * 4) / (coldw[calib] * 1024)
    digest = sources_digest(BN_SOURCES)
    alg = {"bn_stats": n * 4, "bn_apply": 2 * n * 4, "bn_grad_sums": 2 * n * 4, "bn_dx": 3 * n * 4}
    for k in cold:
        tag = next((a for a in alg if f"{a}_kernel" in k), None)
        if tag is None:
            continue
        fb = cold[k] * 1024 * fscale
        wb = coldw.get(k, 0.0) * 1024 * wscale
        text = "\n".join([
            f"# HBM-side traffic of {k}: BatchNorm2d (256,32,32,32) fp32, cold steps",
            f"command_fetch: {PROFILE_CMD_PMC.format(counter='FETCH_SIZE')}",
            f"command_write: {PROFILE_CMD_PMC.format(counter='WRITE_SIZE')}",
            "summarized by: python bench.py --summarize-counters <fetch_dir>/bench_quick_counter_collection.csv "
            "<write_dir>/bench_quick_counter_collection.csv",
            f"fetch_kib_per_dispatch: {cold[k]:.1f}",
            f"write_kib_per_dispatch: {coldw.get(k, 0.0):.1f}",
            f"calib_add fetch_kib / write_kib: {cold[calib]:.1f} / {coldw[calib]:.1f} "
            f"(known: {2 * n * 4 // 1024} / {n * 4 // 1024})",
            f"fetch_scale: {fscale:.5f}",
            f"write_scale: {wscale:.5f}",
            f"hbm_bytes_per_launch: {fb + wb:.0f}",
            f"algorithmic_bytes_per_launch: {alg[tag]}",
            f"traffic_over_algorithmic: {(fb + wb) / alg[tag]:.4f}",
            f"sources: {','.join(BN_SOURCES)}",
            f"source_sha256_16: {digest}",
            "note: FETCH_SIZE counts L2 misses served by the data fabric, so reads that hit the "
            "256 MB Infinity Cache are included",
        ])
        open(os.path.join(out_dir, f"{tag}_bn_cifar_f32_counters.txt"), "w").write(text + "\n")


def summarize_all(trace_csv, fetch_csv, write_csv, out_path):
    """Every normhip kernel of a full bench.py run, one line per (kernel,
    grid): dispatches and mean duration from the kernel trace, and HBM-side
    bytes per dispatch from FETCH_SIZE / WRITE_SIZE scaled by the calibration
    add of known size.  Lines follow the order of the bench's workloads."""
    import collections
    import csv

    def grid_blocks(r, x_key, wg_key):
        return int(float(r[x_key])) // max(1, int(float(r[wg_key])))

    trace = collections.OrderedDict()
    for r in csv.DictReader(open(trace_csv)):
        name = _short_kernel(r["Kernel_Name"])
        if not name.startswith("nh::"):
            continue
        key = (name, grid_blocks(r, "Grid_Size_X", "Workgroup_Size_X") * int(r["Grid_Size_Y"]))
        trace.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)

    def counters(path):
        d = collections.OrderedDict()
        for r in csv.DictReader(open(path)):
            key = (_short_kernel(r["Kernel_Name"]), int(float(r["Grid_Size"])) // max(1, int(r["Workgroup_Size"])))
            d.setdefault(key, []).append(float(r["Counter_Value"]))
        return d

    f, w = counters(fetch_csv), counters(write_csv)
    n = 256 * 32 * 32 * 32
    calib = next(k for k in f if "calib_add4" in k[0])

    def leading(vals):
        # the run's first calibration add is the (256,32,32,32) one; later
        # ones (the row backwards' floors) have other sizes
        out = [v for v in vals[:1]]
        for v in vals[1:]:
            if abs(v - vals[0]) > 0.1 * vals[0]:
                break
            out.append(v)
        return out

    fc, wc = leading(f[calib]), leading(w[calib])
    fscale = (2 * n * 4) / (sum(fc) / len(fc) * 1024)
    wscale = (n * 4) / (sum(wc) / len(wc) * 1024)
    lines = ["# normhip kernels over every bench.py workload (MI355X): duration and HBM-side traffic",
             f"command_trace: {PROFILE_CMD_ALL_TRACE}",
             f"command_fetch: {PROFILE_CMD_ALL_PMC.format(counter='FETCH_SIZE')}",
             f"command_write: {PROFILE_CMD_ALL_PMC.format(counter='WRITE_SIZE')}",
             "summarized by: python bench.py --summarize-all <trace_dir>/bench_all_kernel_trace.csv "
             "<fetch_dir>/bench_all_counter_collection.csv <write_dir>/bench_all_counter_collection.csv",
             f"fetch_scale: {fscale:.5f} (FETCH_SIZE of the calibration add vs its known reads)",
             f"write_scale: {wscale:.5f}",
             "note: FETCH_SIZE counts L2 misses served by the data fabric, so reads served by the "
             "256 MB Infinity Cache are included",
             "note: the BatchNorm (256,32,32,32) fp32 lines average its cold and warm steps; every "
             "other workload runs cold only",
             "note: the calib_add4 line averages every calibration add of the run (the (256,32,32,32) "
             "one and the row backwards' floors); the scales above use the first",
             "",
             f"{'kernel':64s} {'blocks':>7s} {'calls':>6s} {'avg_us':>8s} {'read_MB':>9s} {'write_MB':>9s}"]
    for key, durs in trace.items():
        fk, wk = f.get(key), w.get(key)
        rd = f"{sum(fk) / len(fk) * 1024 * fscale / 1e6:9.2f}" if fk else f"{'-':>9s}"
        wr = f"{sum(wk) / len(wk) * 1024 * wscale / 1e6:9.2f}" if wk else f"{'-':>9s}"
        lines.append(f"{key[0][:64]:64s} {key[1]:7d} {len(durs):6d} {sum(durs) / len(durs):8.2f} {rd} {wr}")
    open(out_path, "w").write("\n".join(lines) + "\n")


def _traffic_for(kernel_name, workload_tag):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"{kernel_name}_{workload_tag}_counters.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    srcs = [x for x in fields.get("sources", "").split(",") if x]
    if not srcs or not all(os.path.exists(os.path.join(ROOT, "bwd_bn_stats_amd", "csrc", x)) for x in srcs):
        return None
    if sources_digest(srcs) != fields.get("source_sha256_16"):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--quick", action="store_true", help="main workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--summarize-trace", metavar="KERNEL_STATS_CSV",
                    help="write profiles/ summary of a rocprofv3 --stats run and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/ traffic summaries of two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-all", nargs=3, metavar=("TRACE_CSV", "FETCH_CSV", "WRITE_CSV"),
                    help="write the profiles/ summary of every kernel of a full run and exit")
    args = ap.parse_args()
    if args.summarize_all:
        summarize_all(*args.summarize_all, os.path.join(ROOT, "profiles", "norm_kernels_all_workloads.txt"))
        return
    if args.summarize_trace or args.summarize_counters:
        os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
        if args.summarize_trace:
            summarize_trace(args.summarize_trace,
                            os.path.join(ROOT, "profiles", "bn_cifar_f32_kernel_trace.txt"))
        if args.summarize_counters:
            summarize_counters(*args.summarize_counters, os.path.join(ROOT, "profiles"))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "this library has no multi-GPU path to time.", file=sys.stderr)
        sys.exit(2)

    import torch
    from bwd_bn_stats_amd import normhip as nh
    from bwd_bn_stats_amd import workloads as wl

    torch.cuda.set_device(0)
    K, W = args.steps, args.warmup
    log(f"[bench] device: {torch.cuda.get_device_name(0)}")

    main_case = wl.bn_cifar(wl.F32)
    log("[bench] main: BatchNorm2d (256,32,32,32) fp32 fwd+bwd, cold")
    cold = bench_bn(nh, torch, main_case, K, W, cold=True)
    log(f"[bench]   {cold['us_per_call']:.1f} us/step, {cold['gbs']:.0f} GB/s")
    log("[bench] main: warm")
    warm = bench_bn(nh, torch, main_case, K, W, cold=False)
    log("[bench] calibration floor (two reads, one write, bn_dx-sized)")
    calib = bench_calib(nh, torch, main_case.N * main_case.C * main_case.hw, K, W)
    log("[bench] read-only floors (stats-sized and grad_sums-sized)")
    E = main_case.N * main_case.C * main_case.hw
    read1, read2 = bench_read(nh, torch, E, K, W), bench_read(nh, torch, 2 * E, K, W)
    for k, rd in (("bn_stats", read1), ("bn_grad_sums", read2)):
        if k in cold["kernels"]:
            cold["kernels"][k]["read_floor_gbs"] = round(rd["gbs"], 1)
            cold["kernels"][k]["frac_of_read_floor"] = round(cold["kernels"][k]["gbs"] / rd["gbs"], 4)

    others = {}
    if not args.quick:
        kk = max(10, K // 2)
        for name, fn in (("bn_cifar_256x32x32x32_bf16", lambda: wl.bn_cifar(wl.BF16)),
                         ("bn_resnet_64x256x56x56_bf16", wl.bn_resnet),
                         ("bn_ragged_3x37x41x40_f32", wl.bn_ragged)):
            log(f"[bench] {name}")
            others[name] = bench_bn(nh, torch, fn(), kk, W, cold=True)
        log("[bench] bn_ragged_3x37x41x40_f32 eager vs HIP graph replay (launch-bound)")
        others["bn_ragged_3x37x41x40_f32_graph"] = bench_bn_graph(nh, torch, wl.bn_ragged(), max(50, K), W)
        for name, fn, act in (("bn_relu_cifar_256x32x32x32_f32", lambda: wl.bn_cifar(wl.F32), "relu"),
                              ("bn_leaky_relu_cifar_256x32x32x32_f32", lambda: wl.bn_cifar(wl.F32),
                               "leaky_relu"),
                              ("bn_relu_resnet_64x256x56x56_bf16", wl.bn_resnet, "relu")):
            log(f"[bench] {name}")
            others[name] = bench_bn(nh, torch, fn(), kk, W, cold=True, act=act)
        for name, fn in (("bn_infer_relu_cifar_256x32x32x32_f32", lambda: wl.bn_cifar(wl.F32)),
                         ("bn_infer_relu_resnet_64x256x56x56_bf16", wl.bn_resnet)):
            log(f"[bench] {name}")
            others[name] = bench_bn_infer(nh, torch, fn(), kk, W)
        log("[bench] ln_bwd_16x512x1600 (x f32, dy bf16, w bf16, dx f32)")
        others["ln_bwd_16x512x1600"] = bench_rows(nh, torch, wl.ln_bwd(), "ln", kk, W)
        log("[bench] bda_bwd_16x512x1600 (bias+dropout+add+LayerNorm backward)")
        others["bda_bwd_16x512x1600"] = bench_bda(nh, torch, wl.bda_bwd(), kk, W)
        for dt in (wl.BF16, wl.F32):
            for saved in (True, False):
                name = f"rms_bwd_2048x8192_{dt}_{'saved' if saved else 'recompute'}_rms"
                log(f"[bench] {name}")
                others[name] = bench_rows(nh, torch, wl.rms_bwd(dt), "rms", kk, W, saved=saved)
        log("[bench] ln_fwd_16x512x1600 (x f32, w/b bf16, y f32)")
        others["ln_fwd_16x512x1600"] = bench_rows_fwd(nh, torch, wl.ln_bwd(), "ln", kk, W)
        for dt in (wl.BF16, wl.F32):
            log(f"[bench] rms_fwd_2048x8192_{dt}")
            others[f"rms_fwd_2048x8192_{dt}"] = bench_rows_fwd(nh, torch, wl.rms_bwd(dt), "rms", kk, W)
        # shapes beyond the configs, one per planner path: late ResNet BatchNorm
        # layers (one fused block per channel; 8-byte bf16 units), BatchNorm over
        # [N, C] (the row layout), RMSNorm over a 128-wide head dimension
        # (lane-subgroup rows) and 32768-wide rows (row-sum + column-strip kernels)
        for name, fn in (("bn_late_64x2048x7x7_bf16",
                          lambda: wl.bn_case(64, 2048, 7, 7, wl.BF16, seed=1011, x_mean=3.0)),
                         ("bn_64x1024x14x14_bf16",
                          lambda: wl.bn_case(64, 1024, 14, 14, wl.BF16, seed=1012, x_mean=3.0))):
            log(f"[bench] {name}")
            others[name] = bench_bn(nh, torch, fn(), kk, W, cold=True)
        log("[bench] bn_16384x2048x1x1_bf16 (BatchNorm over [N, C]: the row layout)")
        others["bn_16384x2048x1x1_bf16"] = bench_bn(
            nh, torch, wl.bn_case(16384, 2048, 1, 1, wl.BF16, seed=1015), kk, W, cold=True)
        log("[bench] rms_bwd_131072x128_bf16 (head-dimension rows)")
        others["rms_bwd_131072x128_bf16"] = bench_rows(
            nh, torch, wl.rows_case(131072, 128, x_t=wl.BF16, dy_t=wl.BF16, w_t=wl.BF16, seed=1013), "rms", kk, W)
        log("[bench] ln_bwd_512x32768_bf16 (rows wider than a 512-thread team)")
        others["ln_bwd_512x32768_bf16"] = bench_rows(
            nh, torch, wl.rows_case(512, 32768, x_t=wl.BF16, dy_t=wl.BF16, w_t=wl.BF16, seed=1014, with_bias=True),
            "ln", kk, W)

    if not args.quick:
        # one-read/one-write kernels against a plain copy of the same bytes
        for name, kern in (("bn_infer_relu_cifar_256x32x32x32_f32", "bn_infer"),
                           ("bn_infer_relu_resnet_64x256x56x56_bf16", "bn_infer"),
                           ("ln_fwd_16x512x1600", "ln_fwd"), ("rms_fwd_2048x8192_bf16", "rms_fwd"),
                           ("rms_fwd_2048x8192_f32", "rms_fwd")):
            o = others.get(name)
            if not o or kern not in o["kernels"] or not o["kernels"][kern].get("bytes"):
                continue
            log(f"[bench] copy floor for {name}")
            cp = bench_copy(nh, torch, o["kernels"][kern]["bytes"] // 32 * 16, max(10, K // 2), W)
            o["copy_floor"] = {"gbs": round(cp["gbs"], 1), "avg_us": round(cp["avg_us"], 3)}
            o["kernels"][kern]["frac_of_copy_floor"] = round(o["kernels"][kern]["gbs"] / cp["gbs"], 4)
        # the row backwards (two reads, one write per element) against the
        # calibration add (two fp32 reads, one write) of the same total bytes
        for name, kern in (("ln_bwd_16x512x1600", "ln_rows"), ("rms_bwd_2048x8192_bf16_saved_rms", "rms_rows"),
                           ("rms_bwd_2048x8192_f32_saved_rms", "rms_rows")):
            o = others.get(name)
            if not o or kern not in o["kernels"] or not o["kernels"][kern].get("bytes"):
                continue
            log(f"[bench] add floor for {name}")
            ad = bench_calib(nh, torch, o["kernels"][kern]["bytes"] // 12 // 1024 * 1024, max(10, K // 2), W)
            o["add_floor"] = {"gbs": round(ad["gbs"], 1), "avg_us": round(ad["avg_us"], 3)}
            o["kernels"][kern]["frac_of_add_floor"] = round(o["kernels"][kern]["gbs"] / ad["gbs"], 4)
            o["call_frac_of_add_floor"] = round(o["gbs"] / ad["gbs"], 4)

    # dominant kernel of the step: the largest share of the step's kernel time
    per = cold["kernels"]
    dom = max((k for k in per if per[k].get("bytes")), key=lambda k: per[k]["avg_us"] * per[k]["launches"])
    traffic = _traffic_for(dom, "bn_cifar_f32")
    roofline = {"kernel": dom, "bound": "hbm", "achieved": round(per[dom]["gbs"], 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(per[dom]["gbs"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                "avg_us": round(per[dom]["avg_us"], 3), "algorithmic_bytes": per[dom]["bytes"]}

    out = {
        "metric": METRIC,
        "value": round(cold["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(cold["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "batchnorm2d_train_fwd_bwd", "shape_nchw": [256, 32, 32, 32],
                   "io": "f32", "stats": "f32", "cache": "cold (rotating buffer sets)",
                   "step": "bn_forward_train + bn_backward", "parallelism": "single GPU"},
        "us_per_call": round(cold["us_per_call"], 2),
        "us_per_call_with_kernel_events": round(cold["us_per_call_with_kernel_events"], 2),
        "frac_of_peak": round(cold["gbs"] / HBM_PEAK_GBS, 4),
        "frac_of_calib_floor": round(cold["gbs"] / calib["gbs"], 4),
        "one_touch": {"bytes": cold["one_touch_bytes"], "gbs": round(cold["one_touch_gbs"], 1),
                      "frac_of_peak": round(cold["one_touch_gbs"] / HBM_PEAK_GBS, 4)},
        "per_call": cold["per_call"],
        "roofline": roofline,
        "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in per.items()},
        "warm": {"us_per_call": round(warm["us_per_call"], 2), "gbs": round(warm["gbs"], 1)},
        "calib_read2_write1": {k: round(v, 4) if isinstance(v, float) else v for k, v in calib.items()},
        "others": others,
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline: oracle on the host")
        out["cpu_baseline"] = cpu_baseline(main_case)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
