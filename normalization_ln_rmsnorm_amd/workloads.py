"""Seeded synthetic workloads for the normalization family.

This module only draws random inputs; it holds none of the normalization
arithmetic, so the HIP path and the float64 oracle can both consume its
arrays.  Every array is produced on the host with numpy's PCG64 generator,
seeded per workload, in a fixed draw order:

    x, per-channel parameters, outlier columns, weight, bias, residual, dy.

Values are drawn in float32; bf16 workloads round each float32 value to the
nearest bf16 (ties to even) once and hand out the 16-bit patterns as uint16;
fp16 variants (same recipe, dtype "f16") round to float16 arrays.
"N(a, s)" means mean a, standard deviation s.

The six workloads (sizes as the benchmark runs them):

  ln_f32_64x256          LayerNorm fwd+bwd, fp32, 64 x 256;
                         x ~ N(0,1), w = 1 + 0.1 N(0,1), b = 0.1 N(0,1),
                         dy ~ N(0,1), eps = 1e-5
  rms_bf16_16384x4096    RMSNorm fwd+bwd, bf16 I/O, 16384 tokens x 4096
                         hidden; x ~ N(0,1) with 8 distinct random columns
                         scaled by 20, w = 1 + 0.05 N(0,1), dy ~ N(0,1),
                         eps = 1e-6
  ln_bf16_25216x768      LayerNorm fwd+bwd, bf16, 128 x 197 tokens x 768;
                         x ~ N(0.5, 2), w/b as the fp32 LayerNorm case,
                         dy ~ N(0,1), eps = 1e-5
  ln_bf16_4096x1000      as above with 4096 x 1000 (a width that is not a
                         power of two)
  bn_f32_64x256x56x56    BatchNorm2d training fwd+bwd, fp32, NCHW
                         64 x 256 x 56 x 56, residual add + ReLU; channel c
                         has x = mu_c + sd_c N(0,1), mu_c ~ U(-2,2),
                         sd_c ~ U(0.5,3); res ~ N(0,1); w/b as above;
                         dy ~ N(0,1); momentum 0.1, eps 1e-5; running mean
                         0 and running variance 1 at the start
  bn_bf16_256x64x112x112 BatchNorm2d bf16, NCHW 256 x 64 x 112 x 112, exact
                         GELU, training fwd+bwd then eval fwd from the
                         updated running statistics; mu_c ~ U(-1,1),
                         sd_c ~ U(0.2,4); no residual; dy ~ N(0,1); w/b as
                         above; momentum 0.1, eps 1e-5; running mean 0 and
                         running variance 1 at the start

EXTRA_WORKLOADS adds fp16 variants of the RMSNorm and bf16 BatchNorm
workloads, two BatchNorm1d workloads (same recipe as the BatchNorm2d ones):
(N, C) = 8192 x 2048 fp32 with ReLU, and (N, C, L) = 2048 x 512 x 32 bf16
with residual + GELU and an eval step, and an activation + dropout workload:
x, dy ~ N(0, 1) of 16384 x 4096 bf16, GELU, drop probability 0.1, a fixed
64-bit dropout seed.
"""
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "ln", "rms", "bn" or "ad" (activation + dropout)
    dtype: str           # "f32", "bf16" or "f16" (I/O dtype)
    shape: tuple         # (M, N) for ln/rms, (N, C, H, W) for bn
    seed: int
    eps: float
    momentum: float = 0.1
    act: str = "none"
    residual: bool = False
    eval_after_train: bool = False
    extra: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        """Rows for ln/rms; (n, c) planes for BatchNorm."""
        if self.kind == "bn":
            return self.shape[0] * self.shape[1]
        return self.shape[0]


WORKLOADS = {
    w.name: w
    for w in [
        Workload("ln_f32_64x256", "ln", "f32", (64, 256), 1000, 1e-5,
                 extra=dict(x_mean=0.0, x_std=1.0)),
        Workload("rms_bf16_16384x4096", "rms", "bf16", (16384, 4096), 1001, 1e-6,
                 extra=dict(outlier_cols=8, outlier_scale=20.0)),
        Workload("ln_bf16_25216x768", "ln", "bf16", (25216, 768), 1002, 1e-5,
                 extra=dict(x_mean=0.5, x_std=2.0)),
        Workload("ln_bf16_4096x1000", "ln", "bf16", (4096, 1000), 1012, 1e-5,
                 extra=dict(x_mean=0.5, x_std=2.0)),
        Workload("bn_f32_64x256x56x56", "bn", "f32", (64, 256, 56, 56), 1003, 1e-5,
                 momentum=0.1, act="relu", residual=True,
                 extra=dict(mu_range=(-2.0, 2.0), sd_range=(0.5, 3.0))),
        Workload("bn_bf16_256x64x112x112", "bn", "bf16", (256, 64, 112, 112), 1004,
                 1e-5, momentum=0.1, act="gelu", residual=False, eval_after_train=True,
                 extra=dict(mu_range=(-1.0, 1.0), sd_range=(0.2, 4.0))),
    ]
}

# The workload the headline benchmark line is quoted on: the largest
# single-GPU configuration (BatchNorm2d bf16 256 x 64 x 112 x 112, GELU;
# 411 MB per activation tensor).
HEADLINE = "bn_bf16_256x64x112x112"


def _variant(base: str, name: str, **changes) -> Workload:
    from dataclasses import replace
    return replace(WORKLOADS[base], name=name, **changes)


# Variants beyond the six above, measured alongside them: the same recipes
# with fp16 I/O, and BatchNorm1d inputs -- (N, C) with HW = 1 and (N, C, L)
# -- whose planes are too short for the plane path.  Shapes stored as
# (N, C, L, 1).
EXTRA_WORKLOADS = {
    w.name: w
    for w in [
        _variant("rms_bf16_16384x4096", "rms_f16_16384x4096", dtype="f16"),
        _variant("bn_bf16_256x64x112x112", "bn_f16_256x64x112x112", dtype="f16"),
        Workload("bn1d_f32_8192x2048", "bn", "f32", (8192, 2048, 1, 1), 1005, 1e-5,
                 momentum=0.1, act="relu", residual=False,
                 extra=dict(mu_range=(-2.0, 2.0), sd_range=(0.5, 3.0))),
        Workload("bn1d_bf16_2048x512x32", "bn", "bf16", (2048, 512, 32, 1), 1006, 1e-5,
                 momentum=0.1, act="gelu", residual=True, eval_after_train=True,
                 extra=dict(mu_range=(-1.0, 1.0), sd_range=(0.2, 4.0))),
        Workload("actdrop_bf16_16384x4096", "ad", "bf16", (16384, 4096), 1007, 0.0,
                 act="gelu", extra=dict(drop_p=0.1, dropout_seed=0x5EED1234ABCD, x_std=1.0)),
    ]
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); uint16 bits.

    Input preparation only (finite values)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def to_io(a: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> the I/O representation: float32, bf16 bits (uint16)
    or float16, each rounded to nearest-even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(a)
    if dtype == "f16":
        return a.astype(np.float16)
    return a



def _normal(rng, size, mean=0.0, std=1.0):
    v = rng.standard_normal(size=size, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    if mean != 0.0:
        v += np.float32(mean)
    return v


def gen_rowwise(wl: Workload, M: int = None, N: int = None, seed: int = None):
    """Inputs for a LayerNorm / RMSNorm workload, optionally at another shape.

    Returns dict(x, w, b, dy) (b is None for RMSNorm) in the workload's I/O
    dtype (float32 arrays, uint16 bf16 bit patterns, or float16 arrays)."""
    M = wl.shape[0] if M is None else M
    N = wl.shape[1] if N is None else N
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    if wl.kind == "rms":
        x = _normal(rng, (M, N))
        k = min(wl.extra.get("outlier_cols", 0), N)
        cols = rng.choice(N, size=k, replace=False) if k else np.zeros(0, np.int64)
        x[:, cols] *= np.float32(wl.extra.get("outlier_scale", 1.0))
        w = np.float32(1.0) + _normal(rng, (N,), std=0.05)
        b = None
    else:
        x = _normal(rng, (M, N), wl.extra.get("x_mean", 0.0), wl.extra.get("x_std", 1.0))
        w = np.float32(1.0) + _normal(rng, (N,), std=0.1)
        b = _normal(rng, (N,), std=0.1)
    dy = _normal(rng, (M, N))
    out = dict(x=to_io(x, wl.dtype), w=to_io(w, wl.dtype), dy=to_io(dy, wl.dtype),
               b=to_io(b, wl.dtype) if b is not None else None)
    return out


def gen_bn(wl: Workload, Nb: int = None, C: int = None, HW: int = None, seed: int = None):
    """Inputs for a BatchNorm workload as [Nb, C, HW] arrays (NCHW, H*W = HW).

    Returns dict(x, res, w, b, dy, running_mean, running_var); res is None
    when the workload has no residual.  Running statistics are float32."""
    Nb = wl.shape[0] if Nb is None else Nb
    C = wl.shape[1] if C is None else C
    HW = wl.shape[2] * wl.shape[3] if HW is None else HW
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    x = _normal(rng, (Nb, C, HW))
    lo, hi = wl.extra["mu_range"]
    mu = rng.uniform(lo, hi, size=C).astype(np.float32)
    lo, hi = wl.extra["sd_range"]
    sd = rng.uniform(lo, hi, size=C).astype(np.float32)
    x *= sd[None, :, None]
    x += mu[None, :, None]
    w = np.float32(1.0) + _normal(rng, (C,), std=0.1)
    b = _normal(rng, (C,), std=0.1)
    res = _normal(rng, (Nb, C, HW)) if wl.residual else None
    dy = _normal(rng, (Nb, C, HW))
    return dict(x=to_io(x, wl.dtype), res=to_io(res, wl.dtype) if res is not None else None,
                w=to_io(w, wl.dtype), b=to_io(b, wl.dtype), dy=to_io(dy, wl.dtype),
                running_mean=np.zeros(C, np.float32), running_var=np.ones(C, np.float32))


def gen_act_dropout(wl: Workload, n: int = None, seed: int = None):
    """Inputs for an activation + dropout workload: dict(x, dy), flat, in the
    workload's I/O dtype; x ~ N(0, x_std), dy ~ N(0, 1)."""
    n = wl.shape[0] * wl.shape[1] if n is None else n
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    x = _normal(rng, (n,), std=wl.extra.get("x_std", 1.0))
    dy = _normal(rng, (n,))
    return dict(x=to_io(x, wl.dtype), dy=to_io(dy, wl.dtype))
