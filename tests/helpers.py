"""Shared test helpers: host <-> device transfer of workload tensors and the
normwise comparison used by every parity test."""
from __future__ import annotations

import sys

import numpy as np

from bwd_bn_stats_amd import workloads as wl

# Tolerances (normwise: max|gpu - oracle| / max|oracle| per output tensor).
TOL = {wl.F32: 2e-5, wl.BF16: 8e-3}


def dev(t, device="cuda"):
    """workloads.Tensor (or a float32 numpy array) -> torch device tensor."""
    import torch
    if isinstance(t, wl.Tensor):
        if t.dtype == wl.F32:
            return torch.from_numpy(np.ascontiguousarray(t.store)).to(device)
        bits = np.ascontiguousarray(t.store).view(np.int16)
        return torch.from_numpy(bits).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(t, dtype=np.float32)).to(device)


def host(t) -> np.ndarray:
    """torch tensor (float32 or bfloat16) -> exact float64 values on the host."""
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return wl.bf16_bits_to_f32(bits).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def rel_err(got, want) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = float(np.max(np.abs(want))) if want.size else 0.0
    num = float(np.max(np.abs(got - want))) if want.size else 0.0
    if den == 0.0:
        return num
    return num / den


def ulp_histogram(got, want) -> dict:
    """Element-wise distance, in bf16 ulps of the exact value, between a bf16
    result and the exact value (reported, not asserted)."""
    want = np.asarray(want, np.float64)
    got = np.asarray(got, np.float64)
    mag = np.maximum(np.abs(want), 1e-30)
    ulp = 2.0 ** (np.floor(np.log2(mag)) - 7)
    d = np.abs(got - want) / ulp
    bins = [0.0, 0.5, 1.0, 2.0, 4.0, np.inf]
    counts, _ = np.histogram(d, bins=bins)
    return {f"<={b}": int(c) for b, c in zip(bins[1:], counts)}


def check(name, got, want, dtype, tol=None, report=True):
    tol = TOL[dtype] if tol is None else tol
    e = rel_err(got, want)
    if report:
        extra = ""
        if dtype == wl.BF16:
            extra = f" ulp-hist={ulp_histogram(got, want)}"
        print(f"  {name}: rel_err={e:.3e} (tol {tol:.0e}){extra}", flush=True)
        sys.stdout.flush()
    assert e <= tol, f"{name}: normwise relative error {e:.3e} > {tol:.0e}"
    return e
