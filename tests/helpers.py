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


def _next_toward(v: np.ndarray, up: np.ndarray, dtype) -> np.ndarray:
    """The neighbouring representable value of each v (fp32 values of dtype
    storage), upwards where `up`, else downwards."""
    v32 = np.asarray(v, np.float32)
    if dtype == wl.F32:
        return np.nextafter(v32, np.where(up, np.float32(np.inf), np.float32(-np.inf))).astype(np.float32)
    bits = wl.f32_to_bf16_bits(v32).astype(np.int32)
    mag_up = up == (v32 > 0)
    nb = np.where(v32 == 0, np.where(up, 0x0001, 0x8001),
                  np.where(mag_up, bits + 1, bits - 1))
    return wl.bf16_bits_to_f32(nb.astype(np.uint16))


def clear_of_kink(oracle_mod, t, gamma, beta, eps, delta, max_iter=8):
    """Moves the few elements of x whose BatchNorm output z lies within
    `delta` of 0 (the kink of ReLU/LeakyReLU) away from it, in x's storage
    type, until every |z| >= delta as the fp64 oracle computes it.  There the
    fp32 kernel and the fp64 oracle take the same activation branch for
    every element, since the kernel's error in z is far below delta."""
    x32 = (t.store.astype(np.float32) if t.dtype == wl.F32
           else wl.bf16_bits_to_f32(t.store)).copy()
    for _ in range(max_iter):
        z, stats, _, _ = oracle_mod.bn_forward_train(x32.astype(np.float64), gamma, beta, eps=eps)
        near = np.abs(z) < delta
        if not near.any():
            return wl.make_tensor(x32.astype(np.float64), t.dtype)
        scale = np.broadcast_to(stats[3].reshape((1, -1) + (1,) * (x32.ndim - 2)), x32.shape)
        up = (z >= 0) == (scale >= 0)             # the direction of x that moves z away from 0
        step = np.where(up, 1.0, -1.0) * 3.0 * delta / np.maximum(np.abs(scale), 1e-30)
        cand = wl.make_tensor(x32.astype(np.float64) + step, t.dtype)
        c32 = cand.store.astype(np.float32) if t.dtype == wl.F32 else wl.bf16_bits_to_f32(cand.store)
        stuck = c32 == x32
        c32 = np.where(stuck, _next_toward(x32, up, t.dtype), c32)
        x32 = np.where(near, c32, x32)
    raise AssertionError("could not move x clear of the activation kink")


def place(t: wl.Tensor, offset: int):
    """Device copy of t starting `offset` elements into a larger buffer, so
    that an offset of 1-3 leaves the tensor misaligned for 16-byte access."""
    import torch
    if t.dtype == wl.F32:
        flat = torch.from_numpy(np.ascontiguousarray(t.store).reshape(-1))
        buf = torch.zeros(flat.numel() + offset, dtype=torch.float32, device="cuda")
        buf[offset:] = flat.cuda()
    else:
        flat = torch.from_numpy(np.ascontiguousarray(t.store).reshape(-1).view(np.int16))
        buf = torch.zeros(flat.numel() + offset, dtype=torch.int16, device="cuda")
        buf[offset:] = flat.cuda()
        buf = buf.view(torch.bfloat16)
    return buf[offset:].view(t.shape)
