"""Seeded synthetic inputs for the normalization workloads.

This module only draws random numbers and rounds them to the storage type
(fp32, or bf16 with round-to-nearest-even).  It holds none of the
normalization arithmetic: both the HIP path and the CPU oracle consume the
arrays it returns, so the two sides see bit-identical inputs.

Workloads (shapes and distributions follow the pages' benchmark settings):

* ``bn_ragged``  -- BatchNorm2d NCHW (3,37,41,40) fp32, x ~ N(5, 0.5^2): the
  ragged parity shape of the Aether-ML BatchNorm PR ("Testing" section).
* ``bn_cifar``   -- BatchNorm2d NCHW (256,32,32,32), fp32 or bf16 I/O: the
  CIFAR-10 activation shape of the same PR ("Results" section).
* ``ln_bwd``     -- LayerNorm backward (16,512,1600): x fp32, dy bf16,
  weight bf16 (nvFuser issue 1473, the layer_norm backward definition).
* ``rms_bwd``    -- RMSNorm backward (2048,8192), bf16 or fp32 (nvFuser
  issue 3629, the rmsnorm_bwd benchmark size).
* ``bn_resnet``  -- BatchNorm2d NCHW (64,256,56,56) bf16 I/O, x ~ N(3, 1).
* ``bda_bwd``    -- bias + dropout + add + LayerNorm backward (16,512,1600):
  the LayerNorm inputs of ``ln_bwd`` plus an fp32 incoming gradient and a
  dropout keep-mask (nvFuser issue 1473, its one-kernel fusion example).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F32 = "f32"
BF16 = "bf16"


def round_f32(a: np.ndarray) -> np.ndarray:
    """fp64 draws -> nearest fp32 (numpy's cast is round-to-nearest-even)."""
    return np.asarray(a, dtype=np.float64).astype(np.float32)


def f32_to_bf16_bits(a32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round-to-nearest-even (finite inputs only)."""
    u = np.ascontiguousarray(a32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Tensor:
    """One input array in its storage type.

    ``store`` is what goes to the device (float32 array, or uint16 bf16 bit
    patterns); ``value`` is the exact numeric value of every element as
    float64, which is what the oracle consumes.
    """

    dtype: str
    store: np.ndarray

    @property
    def value(self) -> np.ndarray:
        if self.dtype == F32:
            return self.store.astype(np.float64)
        return bf16_bits_to_f32(self.store).astype(np.float64)

    @property
    def shape(self):
        return self.store.shape


def make_tensor(draw: np.ndarray, dtype: str) -> Tensor:
    a32 = round_f32(draw)
    if dtype == F32:
        return Tensor(F32, np.ascontiguousarray(a32))
    if dtype == BF16:
        return Tensor(BF16, f32_to_bf16_bits(a32))
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclass
class BNCase:
    name: str
    N: int
    C: int
    HW: tuple
    io: str
    x: Tensor
    dy: Tensor
    gamma: np.ndarray  # fp32 [C]
    beta: np.ndarray   # fp32 [C]
    running_mean: np.ndarray  # fp32 [C]
    running_var: np.ndarray   # fp32 [C]
    eps: float = 1e-5
    momentum: float = 0.1
    meta: dict = field(default_factory=dict)

    @property
    def hw(self) -> int:
        return int(np.prod(self.HW))


def bn_case(N, C, H, W, io=F32, *, seed, x_mean=0.0, x_std=1.0,
            beta_std=0.1, dy_std=1.0, name="bn") -> BNCase:
    """BatchNorm2d training inputs: x ~ N(x_mean, x_std^2) i.i.d. for every
    element, gamma ~ U(0.5, 1.5), beta ~ N(0, beta_std^2), dy ~ N(0, dy_std^2);
    running_mean = 0, running_var = 1 (PyTorch's initial buffers)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = make_tensor(rng.normal(x_mean, x_std, size=(N, C, H, W)), io)
    gamma = round_f32(rng.uniform(0.5, 1.5, size=C))
    beta = round_f32(rng.normal(0.0, beta_std, size=C))
    dy = make_tensor(rng.normal(0.0, dy_std, size=(N, C, H, W)), io)
    return BNCase(name, N, C, (H, W), io, x, dy, gamma, beta,
                  np.zeros(C, np.float32), np.ones(C, np.float32))


@dataclass
class RowsCase:
    name: str
    rows: int
    cols: int
    x: Tensor
    dy: Tensor
    w: Tensor
    b: Tensor | None
    eps: float = 1e-5


def rows_case(rows, cols, *, x_t, dy_t, w_t, seed, with_bias=False,
              name="rows") -> RowsCase:
    """LayerNorm/RMSNorm backward inputs: x ~ N(0,1), dy ~ N(0,1),
    weight ~ U(0.5, 1.5), bias ~ N(0, 0.1^2) (the bias is not read by the
    backward; it is drawn so the stream of draws matches the forward)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = make_tensor(rng.normal(0.0, 1.0, size=(rows, cols)), x_t)
    dy = make_tensor(rng.normal(0.0, 1.0, size=(rows, cols)), dy_t)
    w = make_tensor(rng.uniform(0.5, 1.5, size=cols), w_t)
    b = make_tensor(rng.normal(0.0, 0.1, size=cols), w_t) if with_bias else None
    return RowsCase(name, rows, cols, x, dy, w, b)


@dataclass
class BdaCase:
    """Inputs of the bias + dropout + add + LayerNorm backward: a LayerNorm
    case plus the gradient reaching h from elsewhere (fp32), the dropout
    keep-mask (uint8 0/1, drawn here: it is random state of the forward) and
    the dropout scale 1/(1 - p) rounded to fp32."""
    ln: RowsCase
    dresidual: np.ndarray   # fp32 [rows, cols]
    mask: np.ndarray        # uint8 [rows, cols]
    scale: float
    p_drop: float


def bda_case(rows, cols, *, x_t=F32, dy_t=BF16, w_t=BF16, seed, p_drop=0.1,
             name="bda") -> BdaCase:
    """rows_case inputs, then dresidual ~ N(0, 1) and mask ~ Bernoulli(1 - p_drop)."""
    ln = rows_case(rows, cols, x_t=x_t, dy_t=dy_t, w_t=w_t, seed=seed, name=name)
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    dres = round_f32(rng.normal(0.0, 1.0, size=(rows, cols)))
    mask = (rng.random(size=(rows, cols)) >= p_drop).astype(np.uint8)
    scale = float(np.float32(1.0 / (1.0 - p_drop)))
    return BdaCase(ln, dres, mask, scale, p_drop)


# ---- the workloads ----------------------------------------------------------

def bn_ragged(seed=1001) -> BNCase:
    return bn_case(3, 37, 41, 40, F32, seed=seed, x_mean=5.0, x_std=0.5,
                   beta_std=1.0, name="bn_ragged_3x37x41x40_f32")


def bn_cifar(io=F32, seed=1002) -> BNCase:
    return bn_case(256, 32, 32, 32, io, seed=seed, x_mean=0.0, x_std=1.0,
                   beta_std=0.1, name=f"bn_cifar_256x32x32x32_{io}")


def ln_bwd(seed=1003, rows=16 * 512, cols=1600) -> RowsCase:
    return rows_case(rows, cols, x_t=F32, dy_t=BF16, w_t=BF16, seed=seed,
                     with_bias=True, name=f"ln_bwd_{rows}x{cols}")


def rms_bwd(dtype=BF16, seed=1004, rows=2048, cols=8192) -> RowsCase:
    return rows_case(rows, cols, x_t=dtype, dy_t=dtype, w_t=dtype, seed=seed,
                     name=f"rms_bwd_{rows}x{cols}_{dtype}")


def bn_resnet(seed=1005) -> BNCase:
    return bn_case(64, 256, 56, 56, BF16, seed=seed, x_mean=3.0, x_std=1.0,
                   beta_std=0.1, name="bn_resnet_64x256x56x56_bf16")


def bda_bwd(seed=1006, rows=16 * 512, cols=1600) -> BdaCase:
    return bda_case(rows, cols, x_t=F32, dy_t=BF16, w_t=BF16, seed=seed, p_drop=0.1,
                    name=f"bda_bwd_{rows}x{cols}")
