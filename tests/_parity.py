"""Helpers for GPU-vs-oracle parity checks.

Tolerances (fixed for the normalization family):
  float32 I/O  every element satisfies |got - ref| <= 1e-5 + 1e-5 * |ref|
               (statistics, running statistics and parameter gradients too);
  bf16 / fp16  every element satisfies |got - ref| <= 2 ulp(max(|ref|, F))
  I/O          with ulp_bf16(v) = 2^(floor(log2 v) - 7),
               ulp_f16(v) = 2^(max(floor(log2 v), -14) - 10), and the floor
               F = 2^-12 * max(largest |ref| of that row, channel or vector,
                               the scale of the terms the output is formed
                               from, when given -- e.g. rstd * |dy * w| for
                               a row's dx).
               The floor only matters where cancellation leaves a result
               twelve binades below the scale of its terms, which float32
               arithmetic cannot resolve; the strict (unfloored) ulp error
               is reported alongside.
The reference values are the oracle's float64 results on exactly the inputs
the GPU consumed.  Nothing here computes an expected value itself.
"""
import numpy as np
import torch

F32_ATOL = 1e-5
F32_RTOL = 1e-5
BF16_ULPS = 2.0


TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def to_dev(a, dtype, device="cuda"):
    """numpy float32 array, uint16 bf16 bits or float16 array -> device tensor."""
    if a is None:
        return None
    if dtype == "bf16":
        assert a.dtype == np.uint16
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    if dtype == "f16":
        assert a.dtype == np.float16
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def to_f64(t):
    """Device tensor (float32, bf16 or fp16) -> exact float64 numpy array."""
    if t.dtype == torch.bfloat16:
        bits = t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


def ulp_bf16(v):
    v = np.maximum(np.abs(v), np.finfo(np.float64).tiny)
    return np.exp2(np.floor(np.log2(v)) - 7.0)


def ulp_f16(v):
    v = np.maximum(np.abs(v), np.finfo(np.float64).tiny)
    return np.exp2(np.maximum(np.floor(np.log2(v)), -14.0) - 10.0)


def check(name, got, ref, dtype, group_axis=None, report=None, scale=None):
    """Assert the tolerance for `dtype`; returns a summary dict.

    group_axis: axes over which the bf16 floor's row/channel maximum is taken
    (None = the whole array).  scale: optional array broadcastable to ref,
    the magnitude of the terms each output is formed from (oracle values)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    if dtype == "f32":
        bound = F32_ATOL + F32_RTOL * np.abs(ref)
        bad = err > bound
        summary = dict(name=name, max_abs=float(err.max(initial=0)),
                       max_ratio=float((err / bound).max(initial=0)), n_bad=int(bad.sum()))
    else:
        if group_axis is None:
            R = np.abs(ref).max(initial=0)
        else:
            R = np.abs(ref).max(axis=group_axis, keepdims=True, initial=0)
        if scale is not None:
            R = np.maximum(R, np.abs(scale))
        ulp = ulp_bf16 if dtype == "bf16" else ulp_f16
        floor = np.exp2(-12.0) * R
        u = ulp(np.maximum(np.abs(ref), floor))
        bad = err > BF16_ULPS * u
        strict = err / ulp(ref)
        summary = dict(name=name, max_ulp=float((err / u).max(initial=0)),
                       max_strict_ulp=float(strict.max(initial=0)),
                       n_strict_over_2=int((strict > 2).sum()), n_bad=int(bad.sum()))
    if report is not None:
        report.append(summary)
    if summary["n_bad"]:
        idx = np.argwhere(bad)[:5]
        detail = [(tuple(int(i) for i in ix), float(got[tuple(ix)]), float(ref[tuple(ix)])) for ix in idx]
        raise AssertionError(f"{name}: {summary} first offenders (index, got, ref): {detail}")
    return summary


def round_bf16_f32(a):
    """float32 array -> bf16 bits (nearest-even), for test-side input edits."""
    from normalization_ln_rmsnorm_amd.workloads import f32_to_bf16_bits
    return f32_to_bf16_bits(a)


def to_io(a, dtype):
    """float32 values -> the I/O representation of `dtype` (nearest-even)."""
    from normalization_ln_rmsnorm_amd.workloads import to_io as _to_io
    return _to_io(a, dtype)


# Pre-activation values where an activation's derivative jumps (PyTorch's
# definitions; CELU and the smooth ones have none, softplus's switch to the
# identity at 20 moves values by about 2e-9 only).
KINKS = {"relu": (0.0,), "leaky_relu": (0.0,), "elu": (0.0,), "selu": (0.0,),
         "relu6": (0.0, 6.0), "hardsigmoid": (-3.0, 3.0), "hardswish": (-3.0, 3.0)}


def avoid_kinks(orc, inp, dtype, eps, act, delta=1e-3, step=None):
    """Move the residual (or x) so no pre-activation lies within `delta` of a
    kink of `act`.

    Where the derivative jumps, an element whose z is within rounding
    distance of the kink has two valid gradients (the GPU's float32 z and the
    oracle's float64 z may fall on different sides).  The test inputs are
    shifted away from every kink, using the oracle's z, so the choice is
    unique.  Returns the edited copy of `inp` and the number of elements
    moved."""
    kinks = np.asarray(KINKS.get(act, ()), dtype=np.float64)
    out = dict(inp)
    if kinks.size == 0:
        return out, 0
    bf16 = dtype == "bf16"
    step = step if step is not None else {"bf16": 0.0625, "f16": 1.0 / 64}.get(dtype, 4 * delta)
    moved = 0
    for _ in range(6):
        y, _, _, _, _ = orc.bn_fwd_train(out["x"], out["res"], out["w"], out["b"], eps=eps,
                                         act="none", bf16=bf16)
        d = y[..., None] - kinks
        j = np.abs(d).argmin(axis=-1)
        nearest = np.take_along_axis(d, j[..., None], axis=-1)[..., 0]
        near = np.abs(nearest) < delta
        if not near.any():
            return out, moved
        moved += int(near.sum())
        shift = np.where(nearest >= 0, step, -step)
        key = "res" if out["res"] is not None else "x"
        base = orc.widen(out[key], bf16=bf16)
        edited = (base + np.where(near, shift, 0.0)).astype(np.float32)
        out[key] = to_io(edited, dtype)
    raise AssertionError(f"could not move the pre-activations away from the {act} kinks")


def avoid_relu_kink(orc, inp, dtype, eps, delta=1e-3, step=None):
    return avoid_kinks(orc, inp, dtype, eps, "relu", delta, step)
