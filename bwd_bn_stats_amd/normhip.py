"""Python binding of libnormhip (include/normhip.h): argument marshalling only.

Every computation runs in the library's HIP kernels.  PyTorch supplies device
memory (torch tensors) and the stream (torch.cuda.current_stream()).  There is
no fallback: importing the binding without the built library raises.

Functions carry the C ABI's names:
    bn_forward_train, bn_backward, layernorm_backward, rmsnorm_backward
plus the workspace queries and measurement helpers.
"""
from __future__ import annotations

import ctypes
import functools
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# NORMHIP_LIBRARY names another build of the same library (the host-sanitizer
# build of the test suite); by default the in-tree one.
LIB_PATH = os.environ.get("NORMHIP_LIBRARY") or os.path.join(_HERE, "libnormhip.so")

F32, BF16 = 0, 1
_DT = {torch.float32: F32, torch.bfloat16: BF16}

KERNELS = ["bn_stats", "bn_fwd_finalize", "bn_apply", "bn_grad_sums", "bn_bwd_finalize", "bn_dx",
           "ln_rows", "ln_colsum", "rms_rows", "rms_colsum", "calib", "ln_fwd", "rms_fwd", "bn_infer",
           "bda_rows", "bda_colsum", "rows_coef", "bn_fwd_channel", "bn_bwd_channel"]

ACTS = {"none": 0, "relu": 1, "leaky_relu": 2}

EXPORTS = [
    "nh_status_string", "nh_last_error", "nh_kernel_name",
    "bn_forward_train_workspace", "bn_backward_workspace", "bn_forward_train", "bn_backward",
    "bn_forward_train_stage", "bn_backward_stage", "bn_forward_train_noalloc",
    "bn_act_forward_train", "bn_act_backward", "bn_forward_infer",
    "layernorm_backward_workspace", "layernorm_backward",
    "bda_layernorm_backward_workspace", "bda_layernorm_backward",
    "rmsnorm_backward_workspace", "rmsnorm_backward", "layernorm_forward", "rmsnorm_forward",
    "nh_timing_enable", "nh_timing_reserve", "nh_timing_read",
    "nh_calib_copy", "nh_calib_add", "nh_calib_read",
    "nh_bn_plan", "nh_rows_plan", "nh_plan_override", "nh_selftest_host",
]


class NormHipError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)}: {msg}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m bwd_bn_stats_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    i64, sz, f32, p, i32 = ctypes.c_int64, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p, ctypes.c_int
    psz = ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "nh_status_string": (ctypes.c_char_p, [i32]),
        "nh_last_error": (ctypes.c_char_p, []),
        "nh_kernel_name": (ctypes.c_char_p, [i32]),
        "bn_forward_train_workspace": (i32, [i64, i64, i64, psz]),
        "bn_backward_workspace": (i32, [i64, i64, i64, psz]),
        "bn_forward_train": (i32, [p, p, i32, i64, i64, i64, p, p, p, p, f32, f32, p, p, sz, p]),
        "bn_backward": (i32, [p, p, i32, i64, i64, i64, p, p, p, p, sz, p]),
        "bn_forward_train_stage": (i32, [i32, p, p, i32, i64, i64, i64, p, p, p, p, f32, f32, p, p, sz, p]),
        "bn_forward_train_noalloc": (i32, [p, p, i32, i64, i64, i64, p, p, p, p, f32, f32, p, p]),
        "bn_backward_stage": (i32, [i32, p, p, i32, i64, i64, i64, p, p, p, p, sz, p]),
        "bn_act_forward_train": (i32, [p, p, i32, i64, i64, i64, p, p, p, p, f32, f32, i32, f32, p, p,
                                       sz, p]),
        "bn_act_backward": (i32, [p, p, i32, i64, i64, i64, p, p, i32, f32, p, p, p, sz, p]),
        "bn_forward_infer": (i32, [p, p, i32, i64, i64, i64, p, p, p, p, f32, i32, f32, p]),
        "layernorm_backward_workspace": (i32, [i64, i64, psz]),
        "layernorm_backward": (i32, [p, i32, p, i32, p, p, p, i32, i64, i64, p, i32, p, p, p, sz, p]),
        "bda_layernorm_backward_workspace": (i32, [i64, i64, psz]),
        "bda_layernorm_backward": (i32, [p, i32, p, i32, p, p, p, i32, p, p, f32, i64, i64, p, p, p, p, p,
                                         p, sz, p]),
        "rmsnorm_backward_workspace": (i32, [i64, i64, psz]),
        "rmsnorm_backward": (i32, [p, p, i32, p, f32, p, i64, i64, p, p, p, sz, p]),
        "layernorm_forward": (i32, [p, i32, p, p, i32, i64, i64, f32, p, i32, p, p, p]),
        "rmsnorm_forward": (i32, [p, i32, p, i64, i64, f32, p, p, p]),
        "nh_timing_enable": (i32, [i32]),
        "nh_timing_reserve": (i32, [i64]),
        "nh_timing_read": (i32, [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
        "nh_calib_copy": (i32, [p, p, sz, p]),
        "nh_calib_add": (i32, [p, p, p, i64, p]),
        "nh_calib_read": (i32, [p, i64, p, i64, p]),
        "nh_bn_plan": (i32, [i64, i64, i64, i32, ctypes.POINTER(ctypes.c_int)]),
        "nh_rows_plan": (i32, [i64, i64, ctypes.POINTER(ctypes.c_int)]),
        "nh_plan_override": (i32, [ctypes.c_char_p, i64]),
        "nh_selftest_host": (i32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.nh_status_string(status).decode()


def last_error() -> str:
    return lib.nh_last_error().decode()


def _check(status: int, fn: str):
    if status != 0:
        raise NormHipError(status, fn, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}; float32 or bfloat16 only")
    return _DT[t.dtype]


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev_tensor(t, name, dtype=None, numel=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    return t


def _workspace(nbytes: int, device, workspace):
    """The caller's workspace tensor (device memory, contiguous; the library
    checks its size and alignment), or a new one of the queried size."""
    if workspace is None and nbytes > 0:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    return _dev_tensor(workspace, "workspace")


def common_device(tensors):
    """The one device of the device tensors among `tensors` (None when there
    are none); ValueError when they span several.  The library runs on the
    current HIP device and takes every pointer and the stream on it."""
    devs = []
    for t in tensors:
        d = getattr(t, "device", None)
        if getattr(t, "is_cuda", False) and d not in devs:
            devs.append(d)
    if len(devs) > 1:
        raise ValueError(f"all tensors must be on one device, got {', '.join(str(d) for d in devs)}")
    return devs[0] if devs else None


def _on_tensor_device(f):
    """Runs f with the device of its tensor arguments current (all on one
    device), so that the library's current device, the stream and every
    pointer agree."""
    @functools.wraps(f)
    def g(*args, **kw):
        d = common_device([a for a in list(args) + list(kw.values()) if isinstance(a, torch.Tensor)])
        if d is None:
            return f(*args, **kw)
        with torch.cuda.device(d):
            return f(*args, **kw)
    return g


def _nchw(x: torch.Tensor):
    if x.dim() < 2:
        raise ValueError("BatchNorm input must be [N, C, ...]")
    N, C = x.shape[0], x.shape[1]
    HW = 1
    for s in x.shape[2:]:
        HW *= s
    return N, C, HW


# ---- workspace queries ----------------------------------------------------------
def bn_forward_train_workspace(N: int, C: int, HW: int) -> int:
    out = ctypes.c_size_t()
    _check(lib.bn_forward_train_workspace(N, C, HW, ctypes.byref(out)), "bn_forward_train_workspace")
    return out.value


def bn_backward_workspace(N: int, C: int, HW: int) -> int:
    out = ctypes.c_size_t()
    _check(lib.bn_backward_workspace(N, C, HW, ctypes.byref(out)), "bn_backward_workspace")
    return out.value


def layernorm_backward_workspace(rows: int, cols: int) -> int:
    out = ctypes.c_size_t()
    _check(lib.layernorm_backward_workspace(rows, cols, ctypes.byref(out)), "layernorm_backward_workspace")
    return out.value


def bda_layernorm_backward_workspace(rows: int, cols: int) -> int:
    out = ctypes.c_size_t()
    _check(lib.bda_layernorm_backward_workspace(rows, cols, ctypes.byref(out)),
           "bda_layernorm_backward_workspace")
    return out.value


def rmsnorm_backward_workspace(rows: int, cols: int) -> int:
    out = ctypes.c_size_t()
    _check(lib.rmsnorm_backward_workspace(rows, cols, ctypes.byref(out)), "rmsnorm_backward_workspace")
    return out.value


# ---- BatchNorm ---------------------------------------------------------------------
def _act(act):
    return ACTS[act] if isinstance(act, str) else int(act)


@_on_tensor_device
def bn_forward_train(x, gamma=None, beta=None, running_mean=None, running_var=None,
                     momentum: float = 0.1, eps: float = 1e-5, *, act="none", slope: float = 0.01,
                     y=None, stats=None, workspace=None):
    """BatchNorm2d training forward (bn_forward_train, or bn_act_forward_train
    when act is not "none").  Returns (y, stats[4, C])."""
    _dev_tensor(x, "x")
    N, C, HW = _nchw(x)
    f32 = torch.float32
    for t, n in ((gamma, "gamma"), (beta, "beta"), (running_mean, "running_mean"),
                 (running_var, "running_var")):
        _dev_tensor(t, n, f32, C)
    y = torch.empty_like(x) if y is None else _dev_tensor(y, "y", x.dtype, x.numel())
    stats = torch.empty((4, C), dtype=f32, device=x.device) if stats is None else \
        _dev_tensor(stats, "stats", f32, 4 * C)
    ws = _workspace(bn_forward_train_workspace(N, C, HW), x.device, workspace)
    nb = 0 if ws is None else ws.numel() * ws.element_size()
    if act == "none":
        _check(lib.bn_forward_train(_ptr(x), _ptr(y), _dt(x), N, C, HW, _ptr(gamma), _ptr(beta),
                                    _ptr(running_mean), _ptr(running_var), momentum, eps,
                                    _ptr(stats), _ptr(ws), nb, _stream(x.device)), "bn_forward_train")
    else:
        _check(lib.bn_act_forward_train(_ptr(x), _ptr(y), _dt(x), N, C, HW, _ptr(gamma), _ptr(beta),
                                        _ptr(running_mean), _ptr(running_var), momentum, eps,
                                        _act(act), slope, _ptr(stats), _ptr(ws), nb,
                                        _stream(x.device)), "bn_act_forward_train")
    return y, stats


@_on_tensor_device
def bn_backward(dy, x, stats, *, beta=None, act="none", slope: float = 0.01, dx=None, grads=None,
                need_dx=True, workspace=None):
    """BatchNorm2d training backward (bn_backward, or bn_act_backward when act
    is not "none").  Returns (dx or None, grads[4, C])."""
    _dev_tensor(x, "x")
    _dev_tensor(dy, "dy", x.dtype, x.numel())
    N, C, HW = _nchw(x)
    f32 = torch.float32
    _dev_tensor(stats, "stats", f32, 4 * C)
    _dev_tensor(beta, "beta", f32, C)
    if need_dx:
        dx = torch.empty_like(x) if dx is None else _dev_tensor(dx, "dx", x.dtype, x.numel())
    else:
        dx = None
    grads = torch.empty((4, C), dtype=f32, device=x.device) if grads is None else \
        _dev_tensor(grads, "grads", f32, 4 * C)
    ws = _workspace(bn_backward_workspace(N, C, HW), x.device, workspace)
    nb = 0 if ws is None else ws.numel() * ws.element_size()
    if act == "none":
        _check(lib.bn_backward(_ptr(dy), _ptr(x), _dt(x), N, C, HW, _ptr(stats), _ptr(dx),
                               _ptr(grads), _ptr(ws), nb, _stream(x.device)), "bn_backward")
    else:
        _check(lib.bn_act_backward(_ptr(dy), _ptr(x), _dt(x), N, C, HW, _ptr(stats), _ptr(beta),
                                   _act(act), slope, _ptr(dx), _ptr(grads), _ptr(ws), nb,
                                   _stream(x.device)), "bn_act_backward")
    return dx, grads


@_on_tensor_device
def bn_forward_train_stage(stage: int, x, y, stats, workspace, gamma=None, beta=None, running_mean=None,
                           running_var=None, momentum: float = 0.1, eps: float = 1e-5):
    """One stage of the BatchNorm2d training forward (bn_forward_train_stage):
    1 = the statistics pass into `workspace`, 2 = finalize + apply from it.
    Both stages take the same tensors; stage 1 then stage 2 equals
    bn_forward_train."""
    _dev_tensor(x, "x")
    N, C, HW = _nchw(x)
    f32 = torch.float32
    for t, n in ((gamma, "gamma"), (beta, "beta"), (running_mean, "running_mean"),
                 (running_var, "running_var")):
        _dev_tensor(t, n, f32, C)
    _dev_tensor(y, "y", x.dtype, x.numel())
    _dev_tensor(stats, "stats", f32, 4 * C)
    _dev_tensor(workspace, "workspace")
    nb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.bn_forward_train_stage(int(stage), _ptr(x), _ptr(y), _dt(x), N, C, HW, _ptr(gamma), _ptr(beta),
                                      _ptr(running_mean), _ptr(running_var), momentum, eps, _ptr(stats),
                                      _ptr(workspace), nb, _stream(x.device)), "bn_forward_train_stage")


@_on_tensor_device
def bn_backward_stage(stage: int, dy, x, stats, dx, grads, workspace):
    """One stage of the BatchNorm2d training backward (bn_backward_stage): 1 =
    the grad_sums pass into `workspace`, 2 = finalize + dx from it (dx may be
    None).  Both stages take the same tensors."""
    _dev_tensor(x, "x")
    _dev_tensor(dy, "dy", x.dtype, x.numel())
    N, C, HW = _nchw(x)
    f32 = torch.float32
    _dev_tensor(stats, "stats", f32, 4 * C)
    _dev_tensor(dx, "dx", x.dtype, x.numel())
    _dev_tensor(grads, "grads", f32, 4 * C)
    _dev_tensor(workspace, "workspace")
    nb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.bn_backward_stage(int(stage), _ptr(dy), _ptr(x), _dt(x), N, C, HW, _ptr(stats), _ptr(dx),
                                 _ptr(grads), _ptr(workspace), nb, _stream(x.device)), "bn_backward_stage")


@_on_tensor_device
def bn_forward_infer(x, running_mean, running_var, gamma=None, beta=None, eps: float = 1e-5, *,
                     act="none", slope: float = 0.01, y=None):
    """BatchNorm2d inference from the running statistics (+ activation).  Returns y."""
    _dev_tensor(x, "x")
    N, C, HW = _nchw(x)
    f32 = torch.float32
    for t, n in ((gamma, "gamma"), (beta, "beta"), (running_mean, "running_mean"),
                 (running_var, "running_var")):
        _dev_tensor(t, n, f32, C)
    y = torch.empty_like(x) if y is None else _dev_tensor(y, "y", x.dtype, x.numel())
    _check(lib.bn_forward_infer(_ptr(x), _ptr(y), _dt(x), N, C, HW, _ptr(gamma), _ptr(beta),
                                _ptr(running_mean), _ptr(running_var), eps, _act(act), slope,
                                _stream(x.device)), "bn_forward_infer")
    return y


# ---- LayerNorm / RMSNorm ---------------------------------------------------------------
def _rows(x):
    cols = x.shape[-1] if x.dim() > 0 else 1
    rows = x.numel() // cols if cols else 0
    return rows, cols


@_on_tensor_device
def layernorm_backward(dy, x, mean, rstd, weight=None, *, dx_dtype=None, w_dtype=None,
                       need_dx=True, need_dweight=True, need_dbias=True, dx=None,
                       dweight=None, dbias=None, workspace=None):
    """LayerNorm backward over the last dim.  Returns (dx, dweight, dbias)
    (None for the outputs not requested).  dweight/dbias take the weight's
    dtype (w_dtype when there is no weight, default float32)."""
    _dev_tensor(x, "x")
    _dev_tensor(dy, "dy", None, x.numel())
    rows, cols = _rows(x)
    f32 = torch.float32
    _dev_tensor(mean, "mean", f32, rows)
    _dev_tensor(rstd, "rstd", f32, rows)
    _dev_tensor(weight, "weight", None, cols)
    wdt = weight.dtype if weight is not None else (w_dtype or f32)
    dxdt = dx_dtype or x.dtype
    if need_dx:
        dx = torch.empty(x.shape, dtype=dxdt, device=x.device) if dx is None else \
            _dev_tensor(dx, "dx", dxdt, x.numel())
    else:
        dx = None
    dweight = (torch.empty(cols, dtype=wdt, device=x.device) if dweight is None else
               _dev_tensor(dweight, "dweight", wdt, cols)) if need_dweight else None
    dbias = (torch.empty(cols, dtype=wdt, device=x.device) if dbias is None else
             _dev_tensor(dbias, "dbias", wdt, cols)) if need_dbias else None
    ws = _workspace(layernorm_backward_workspace(rows, cols), x.device, workspace)
    nb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.layernorm_backward(_ptr(dy), _dt(dy), _ptr(x), _dt(x), _ptr(mean), _ptr(rstd),
                                  _ptr(weight), _DT[wdt], rows, cols, _ptr(dx), _DT[dxdt],
                                  _ptr(dweight), _ptr(dbias), _ptr(ws), nb, _stream(x.device)),
           "layernorm_backward")
    return dx, dweight, dbias


@_on_tensor_device
def bda_layernorm_backward(dy, x, mean, rstd, weight=None, dresidual=None, mask=None,
                           scale: float = 1.0, *, w_dtype=None, need_dh=True, need_da=True,
                           need_dweight=True, need_dbias=True, need_dbias_in=True, workspace=None):
    """Backward of bias + dropout + add + LayerNorm over the last dim.
    mask: bool or uint8 tensor (nonzero = kept) or None.  Returns
    (dh fp32, da in dy's dtype, dweight, dbias, dbias_in), None where not
    requested; the column gradients take the weight's dtype."""
    _dev_tensor(x, "x")
    _dev_tensor(dy, "dy", None, x.numel())
    rows, cols = _rows(x)
    f32 = torch.float32
    _dev_tensor(mean, "mean", f32, rows)
    _dev_tensor(rstd, "rstd", f32, rows)
    _dev_tensor(weight, "weight", None, cols)
    _dev_tensor(dresidual, "dresidual", f32, x.numel())
    if mask is not None:
        _dev_tensor(mask, "mask", None, x.numel())
        if mask.dtype not in (torch.bool, torch.uint8):
            raise TypeError("mask must be bool or uint8")
    wdt = weight.dtype if weight is not None else (w_dtype or f32)
    dh = torch.empty(x.shape, dtype=f32, device=x.device) if need_dh else None
    da = torch.empty(x.shape, dtype=dy.dtype, device=x.device) if need_da else None
    cols_out = [torch.empty(cols, dtype=wdt, device=x.device) if need else None
                for need in (need_dweight, need_dbias, need_dbias_in)]
    ws = _workspace(bda_layernorm_backward_workspace(rows, cols), x.device, workspace)
    nb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.bda_layernorm_backward(_ptr(dy), _dt(dy), _ptr(x), _dt(x), _ptr(mean), _ptr(rstd),
                                      _ptr(weight), _DT[wdt], _ptr(dresidual), _ptr(mask), scale,
                                      rows, cols, _ptr(dh), _ptr(da), *[_ptr(t) for t in cols_out],
                                      _ptr(ws), nb, _stream(x.device)), "bda_layernorm_backward")
    return (dh, da, *cols_out)


@_on_tensor_device
def rmsnorm_backward(dy, x, rms=None, weight=None, eps: float = 1e-5, *, need_dx=True,
                     need_dweight=True, dx=None, dweight=None, workspace=None):
    """RMSNorm backward over the last dim.  rms=None recomputes rms from x
    with eps.  Returns (dx, dweight) (None for outputs not requested)."""
    _dev_tensor(x, "x")
    _dev_tensor(dy, "dy", x.dtype, x.numel())
    rows, cols = _rows(x)
    _dev_tensor(rms, "rms", torch.float32, rows)
    _dev_tensor(weight, "weight", x.dtype, cols)
    if need_dx:
        dx = torch.empty_like(x) if dx is None else _dev_tensor(dx, "dx", x.dtype, x.numel())
    else:
        dx = None
    dweight = (torch.empty(cols, dtype=x.dtype, device=x.device) if dweight is None else
               _dev_tensor(dweight, "dweight", x.dtype, cols)) if need_dweight else None
    ws = _workspace(rmsnorm_backward_workspace(rows, cols), x.device, workspace)
    nb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.rmsnorm_backward(_ptr(dy), _ptr(x), _dt(x), _ptr(rms), eps, _ptr(weight), rows, cols,
                                _ptr(dx), _ptr(dweight), _ptr(ws), nb, _stream(x.device)),
           "rmsnorm_backward")
    return dx, dweight


@_on_tensor_device
def layernorm_forward(x, weight=None, bias=None, eps: float = 1e-5, *, y_dtype=None, w_dtype=None,
                      y=None, mean=None, rstd=None, need_rstd=True):
    """LayerNorm training forward over the last dim.  Returns (y, mean, rstd)
    (rstd None when not requested)."""
    _dev_tensor(x, "x")
    rows, cols = _rows(x)
    f32 = torch.float32
    wdt = weight.dtype if weight is not None else (bias.dtype if bias is not None else (w_dtype or f32))
    _dev_tensor(weight, "weight", wdt, cols)
    _dev_tensor(bias, "bias", wdt, cols)
    ydt = y_dtype or x.dtype
    y = torch.empty(x.shape, dtype=ydt, device=x.device) if y is None else _dev_tensor(y, "y", ydt, x.numel())
    mean = torch.empty(rows, dtype=f32, device=x.device) if mean is None else _dev_tensor(mean, "mean", f32, rows)
    if need_rstd:
        rstd = torch.empty(rows, dtype=f32, device=x.device) if rstd is None else _dev_tensor(rstd, "rstd", f32, rows)
    else:
        rstd = None
    _check(lib.layernorm_forward(_ptr(x), _dt(x), _ptr(weight), _ptr(bias), _DT[wdt], rows, cols, eps,
                                 _ptr(y), _DT[ydt], _ptr(mean), _ptr(rstd), _stream(x.device)),
           "layernorm_forward")
    return y, mean, rstd


@_on_tensor_device
def rmsnorm_forward(x, weight=None, eps: float = 1e-5, *, y=None, rms=None, need_rms=True):
    """RMSNorm forward over the last dim.  Returns (y, rms or None)."""
    _dev_tensor(x, "x")
    rows, cols = _rows(x)
    _dev_tensor(weight, "weight", x.dtype, cols)
    y = torch.empty_like(x) if y is None else _dev_tensor(y, "y", x.dtype, x.numel())
    if need_rms:
        rms = torch.empty(rows, dtype=torch.float32, device=x.device) if rms is None else \
            _dev_tensor(rms, "rms", torch.float32, rows)
    else:
        rms = None
    _check(lib.rmsnorm_forward(_ptr(x), _dt(x), _ptr(weight), rows, cols, eps, _ptr(y), _ptr(rms),
                               _stream(x.device)), "rmsnorm_forward")
    return y, rms


# ---- measurement --------------------------------------------------------------------------
def timing_enable(on: bool):
    _check(lib.nh_timing_enable(1 if on else 0), "nh_timing_enable")


def timing_reserve(launches: int):
    _check(lib.nh_timing_reserve(launches), "nh_timing_reserve")


def timing_read(kernel) -> tuple[float, int]:
    """(total ms, launches) recorded for a kernel id or name."""
    kid = KERNELS.index(kernel) if isinstance(kernel, str) else int(kernel)
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib.nh_timing_read(kid, ctypes.byref(ms), ctypes.byref(n)), "nh_timing_read")
    return ms.value, n.value


@_on_tensor_device
def calib_copy(src, dst):
    _dev_tensor(src, "src")
    _dev_tensor(dst, "dst")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError(f"dst holds fewer than the {nbytes} bytes of src")
    _check(lib.nh_calib_copy(_ptr(src), _ptr(dst), nbytes, _stream(src.device)), "nh_calib_copy")


@_on_tensor_device
def calib_read(a, block_sums):
    _dev_tensor(a, "a", torch.float32)
    _dev_tensor(block_sums, "block_sums", torch.float32)
    _check(lib.nh_calib_read(_ptr(a), a.numel(), _ptr(block_sums), block_sums.numel(),
                             _stream(a.device)), "nh_calib_read")


@_on_tensor_device
def calib_add(a, b, out):
    _dev_tensor(a, "a", torch.float32)
    _dev_tensor(b, "b", torch.float32, a.numel())
    _dev_tensor(out, "out", torch.float32, a.numel())
    _check(lib.nh_calib_add(_ptr(a), _ptr(b), _ptr(out), a.numel(), _stream(a.device)), "nh_calib_add")


def bn_plan(N, C, HW, io=F32) -> int:
    g = ctypes.c_int()
    _check(lib.nh_bn_plan(N, C, HW, io, ctypes.byref(g)), "nh_bn_plan")
    return g.value


def rows_plan(rows, cols) -> int:
    g = ctypes.c_int()
    _check(lib.nh_rows_plan(rows, cols, ctypes.byref(g)), "nh_rows_plan")
    return g.value


def plan_override(key: str, value: int):
    _check(lib.nh_plan_override(key.encode(), value), "nh_plan_override")
