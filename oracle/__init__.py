"""Float64 CPU oracle for LayerNorm, RMSNorm and BatchNorm.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and
the benchmark's ``cpu_baseline`` leg may import this package.  The product
library never imports, links or calls it, and it shares no code with the HIP
kernels.  The arithmetic lives in ``norm_oracle.c`` (plain loops, double
accumulators); this module only converts arrays and calls it through ctypes.

Inputs may be float32 arrays, float64 arrays or bf16 bit patterns held in
uint16 arrays (pass ``bf16=True``); each is widened exactly to float64, so
the oracle sees precisely the values the GPU path consumes.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# NORM_ORACLE_LIB points the module at another build of norm_oracle.c (the
# mutation test loads copies with one planted mistake each).
_LIB_PATH = os.environ.get("NORM_ORACLE_LIB") or os.path.join(_HERE, "libnorm_oracle.so")
_lib = None

ACT = {"none": 0, "relu": 1, "gelu": 2, "sigmoid": 3, "tanh": 4, "silu": 5, "mish": 6,
       "leaky_relu": 7, "elu": 8, "selu": 9, "celu": 10, "softplus": 11, "relu6": 12,
       "hardsigmoid": 13, "hardswish": 14}

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.c_int64
_U32P = ctypes.POINTER(ctypes.c_uint32)
_U8P = ctypes.POINTER(ctypes.c_uint8)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    sigs = {
        "orc_act_vec": [ctypes.c_int, ctypes.c_double, ctypes.c_int, _I64, _D, _D],
        "orc_ln_fwd": [_I64, _I64, ctypes.c_double, _D, _D, _D, _D, _D, _D],
        "orc_ln_bwd": [_I64, _I64, ctypes.c_double, _D, _D, _D, _D, _D, _D],
        "orc_rms_fwd": [_I64, _I64, ctypes.c_double, _D, _D, _D, _D],
        "orc_rms_bwd": [_I64, _I64, ctypes.c_double, _D, _D, _D, _D, _D],
        "orc_bn_stats": [_I64, _I64, _I64, _D, _D, _D],
        "orc_bn_fwd_train": [_I64, _I64, _I64, ctypes.c_double, ctypes.c_double,
                             ctypes.c_int, ctypes.c_double, _D, _D, _D, _D, _D, _D, _D, _D, _D],
        "orc_bn_fwd_eval": [_I64, _I64, _I64, ctypes.c_double, ctypes.c_int, ctypes.c_double,
                            _D, _D, _D, _D, _D, _D, _D],
        "orc_bn_bwd": [_I64, _I64, _I64, ctypes.c_double, ctypes.c_int, ctypes.c_double,
                       _D, _D, _D, _D, _D, _D, _D, _D, _D, _D],
        "orc_welford": [_I64, _D, _D],
        "orc_philox4x32_10": [_U32P, _U32P, _U32P],
        "orc_dropout_keep": [_I64, ctypes.c_double, ctypes.c_uint64, ctypes.c_uint64, _U8P],
        "orc_act_dropout_fwd": [_I64, ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                ctypes.c_uint64, ctypes.c_uint64, _D, _D],
        "orc_act_dropout_bwd": [_I64, ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                ctypes.c_uint64, ctypes.c_uint64, _D, _D, _D],
        "orc_chan_merge": [_D, _D, _D],
    }
    for name, argtypes in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = None
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_dropout_threshold.argtypes = [ctypes.c_double]
    lib.orc_dropout_threshold.restype = ctypes.c_uint32
    _lib = lib
    return lib


def num_threads() -> int:
    return int(_load().orc_num_threads())


def widen(a, bf16: bool = False) -> np.ndarray:
    """Exact widening to a contiguous float64 array.

    bf16=True reads ``a`` as uint16 bf16 bit patterns: a bf16 value is the
    upper half of the float32 with the same bits, so shifting left by 16 and
    reinterpreting gives the exact value."""
    if a is None:
        return None
    a = np.asarray(a)
    if bf16:
        if a.dtype != np.uint16:
            raise TypeError("bf16 input must be uint16 bit patterns")
        f32 = (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
        return np.ascontiguousarray(f32, dtype=np.float64)
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(_D)


def _f(a, bf16):
    return widen(a, bf16) if a is not None else None


def act(name, z, grad=False, param=0.0):
    """act(z), or act'(z) with grad=True; `param` is the leaky slope or the
    elu / celu alpha."""
    z = widen(z)
    out = np.empty_like(z)
    _load().orc_act_vec(ACT[name], float(param), int(bool(grad)), z.size, _p(z), _p(out))
    return out


# ---------------------------------------------------------------- LayerNorm
def ln_fwd(x, w=None, b=None, eps=1e-5, bf16=False):
    """Returns (y, mean, rstd) in float64; x is [M, N]."""
    x = _f(x, bf16); w = _f(w, bf16); b = _f(b, bf16)
    M, N = x.shape
    y = np.empty_like(x); mean = np.empty(M); rstd = np.empty(M)
    _load().orc_ln_fwd(M, N, eps, _p(x), _p(w), _p(b), _p(y), _p(mean), _p(rstd))
    return y, mean, rstd


def ln_bwd(dy, x, w=None, eps=1e-5, bf16=False):
    """Returns (dx, dw, db) in float64."""
    dy = _f(dy, bf16); x = _f(x, bf16); w = _f(w, bf16)
    M, N = x.shape
    dx = np.empty_like(x); dw = np.empty(N); db = np.empty(N)
    _load().orc_ln_bwd(M, N, eps, _p(dy), _p(x), _p(w), _p(dx), _p(dw), _p(db))
    return dx, dw, db


# ------------------------------------------------------------------ RMSNorm
def rms_fwd(x, w=None, eps=1e-6, bf16=False):
    """Returns (y, rstd) in float64."""
    x = _f(x, bf16); w = _f(w, bf16)
    M, N = x.shape
    y = np.empty_like(x); rstd = np.empty(M)
    _load().orc_rms_fwd(M, N, eps, _p(x), _p(w), _p(y), _p(rstd))
    return y, rstd


def rms_bwd(dy, x, w=None, eps=1e-6, bf16=False):
    """Returns (dx, dw) in float64."""
    dy = _f(dy, bf16); x = _f(x, bf16); w = _f(w, bf16)
    M, N = x.shape
    dx = np.empty_like(x); dw = np.empty(N)
    _load().orc_rms_bwd(M, N, eps, _p(dy), _p(x), _p(w), _p(dx), _p(dw))
    return dx, dw


# ---------------------------------------------------------------- BatchNorm
def bn_stats(x, bf16=False):
    """Per-channel (mean, biased variance); x is [Nb, C, HW]."""
    x = _f(x, bf16)
    Nb, C, HW = x.shape
    mean = np.empty(C); var = np.empty(C)
    _load().orc_bn_stats(Nb, C, HW, _p(x), _p(mean), _p(var))
    return mean, var


def bn_fwd_train(x, res=None, w=None, b=None, running_mean=None, running_var=None,
                 eps=1e-5, momentum=0.1, act="none", bf16=False, act_param=0.0):
    """Returns (y, save_mean, save_rstd, new_running_mean, new_running_var).

    The running statistics are float32 on the GPU side; pass them as they
    stand and they are widened here.  The inputs are not modified."""
    x = _f(x, bf16); res = _f(res, bf16); w = _f(w, bf16); b = _f(b, bf16)
    rm = widen(running_mean).copy() if running_mean is not None else None
    rv = widen(running_var).copy() if running_var is not None else None
    Nb, C, HW = x.shape
    y = np.empty_like(x); sm = np.empty(C); sr = np.empty(C)
    _load().orc_bn_fwd_train(Nb, C, HW, eps, momentum, ACT[act], float(act_param), _p(x), _p(res),
                             _p(w), _p(b), _p(rm), _p(rv), _p(y), _p(sm), _p(sr))
    return y, sm, sr, rm, rv


def bn_fwd_eval(x, running_mean, running_var, res=None, w=None, b=None, eps=1e-5,
                act="none", bf16=False, act_param=0.0):
    x = _f(x, bf16); res = _f(res, bf16); w = _f(w, bf16); b = _f(b, bf16)
    rm = widen(running_mean); rv = widen(running_var)
    Nb, C, HW = x.shape
    y = np.empty_like(x)
    _load().orc_bn_fwd_eval(Nb, C, HW, eps, ACT[act], float(act_param), _p(x), _p(res), _p(w), _p(b),
                            _p(rm), _p(rv), _p(y))
    return y


def bn_bwd(dy, x, res=None, w=None, b=None, eps=1e-5, act="none", bf16=False, act_param=0.0,
           grad_at=None):
    """Returns (dx, dres, dw, db); dres is None when there is no residual.

    grad_at: optional float64 array of x's shape; where it is not NaN, the
    activation's derivative of that element is taken at that point instead
    of at z (selects a one-sided derivative at a kink)."""
    dy = _f(dy, bf16); x = _f(x, bf16); res = _f(res, bf16)
    w = _f(w, bf16); b = _f(b, bf16)
    if grad_at is not None:
        grad_at = widen(grad_at)
        assert grad_at.shape == x.shape
    Nb, C, HW = x.shape
    dx = np.empty_like(x)
    dres = np.empty_like(x) if res is not None else None
    dw = np.empty(C); db = np.empty(C)
    _load().orc_bn_bwd(Nb, C, HW, eps, ACT[act], float(act_param), _p(dy), _p(x), _p(res), _p(w), _p(b),
                       _p(grad_at), _p(dx), _p(dres), _p(dw), _p(db))
    return dx, dres, dw, db


# ------------------------------------------------- activation + dropout
def philox4x32_10(ctr, key):
    """The four output words of Philox4x32-10 for a 4-word counter and a
    2-word key."""
    c = (ctypes.c_uint32 * 4)(*[int(v) & 0xFFFFFFFF for v in ctr])
    k = (ctypes.c_uint32 * 2)(*[int(v) & 0xFFFFFFFF for v in key])
    o = (ctypes.c_uint32 * 4)()
    _load().orc_philox4x32_10(c, k, o)
    return [int(v) for v in o]


def dropout_threshold(p):
    return int(_load().orc_dropout_threshold(float(p)))


def dropout_keep(n, p, seed, offset=0):
    """uint8 keep mask of elements offset .. offset + n - 1."""
    keep = np.empty(int(n), dtype=np.uint8)
    _load().orc_dropout_keep(int(n), float(p), int(seed), int(offset),
                             keep.ctypes.data_as(_U8P))
    return keep


def act_dropout_fwd(x, act="none", p=0.0, seed=0, offset=0, act_param=0.0, bf16=False):
    """y = keep ? act(x) / (1 - p) : 0 over the flattened x (float64)."""
    x = _f(x, bf16)
    y = np.empty_like(x)
    _load().orc_act_dropout_fwd(x.size, ACT[act], float(act_param), float(p), int(seed), int(offset),
                                _p(x), _p(y))
    return y


def act_dropout_bwd(dy, x, act="none", p=0.0, seed=0, offset=0, act_param=0.0, bf16=False):
    """dx = keep ? dy * act'(x) / (1 - p) : 0 (float64)."""
    dy = _f(dy, bf16); x = _f(x, bf16)
    dx = np.empty_like(x)
    _load().orc_act_dropout_bwd(x.size, ACT[act], float(act_param), float(p), int(seed), int(offset),
                                _p(dy), _p(x), _p(dx))
    return dx


# ------------------------------------------------------ one-pass statistics
def welford(x):
    """(count, mean, M2) by Welford's per-value update."""
    x = widen(x).ravel()
    out = np.empty(3)
    _load().orc_welford(x.size, _p(x), _p(out))
    return out


def chan_merge(a, b):
    """Merge of two (count, mean, M2) triples."""
    a = widen(a); b = widen(b)
    out = np.empty(3)
    _load().orc_chan_merge(_p(a), _p(b), _p(out))
    return out
