"""Thin ctypes binding over libmi355norm.so (the C ABI in include/mi355norm.h).

Argument marshalling only: every step of every operation runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the current
stream.  There is no fallback: if the library is missing or a call fails,
an exception is raised.

Functions keep the C names (ln_fwd, ln_bwd, rms_fwd, rms_bwd, bn_fwd_train,
bn_fwd_eval, bn_bwd).  Tensors must be contiguous CUDA (HIP) tensors of
dtype float32, bfloat16 or float16; statistics are float32.  Outputs that are not
passed in are allocated with torch.
"""
import ctypes
import os

import torch  # loaded first so the library binds to torch's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmi355norm.so")

NORM_F32, NORM_BF16, NORM_F16 = 0, 1, 2
ACT = {"none": 0, "relu": 1, "gelu": 2, "sigmoid": 3, "tanh": 4, "silu": 5, "mish": 6,
       "leaky_relu": 7, "elu": 8, "selu": 9, "celu": 10, "softplus": 11, "relu6": 12,
       "hardsigmoid": 13, "hardswish": 14}
STATUS = {0: "NORM_OK", -1: "NORM_ERR_NULL", -2: "NORM_ERR_SHAPE", -3: "NORM_ERR_DTYPE",
          -4: "NORM_ERR_ACT", -5: "NORM_ERR_ARG", -6: "NORM_ERR_WORKSPACE", -7: "NORM_ERR_HIP"}

_V = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t
_U64 = ctypes.c_uint64

SIGNATURES = {
    "ln_fwd": (_I, [_I, _I64, _I64, _F, _V, _V, _V, _V, _V, _V, _V]),
    "ln_bwd_workspace_bytes": (_SZ, [_I, _I64, _I64]),
    "ln_bwd": (_I, [_I, _I64, _I64, _V, _V, _V, _V, _V, _V, _V, _V, _V, _SZ, _V]),
    "rms_fwd": (_I, [_I, _I64, _I64, _F, _V, _V, _V, _V, _V]),
    "rms_bwd_workspace_bytes": (_SZ, [_I, _I64, _I64]),
    "rms_bwd": (_I, [_I, _I64, _I64, _V, _V, _V, _V, _V, _V, _V, _SZ, _V]),
    "rms_bwd_noalloc": (_I, [_I, _I64, _I64, _V, _V, _V, _V, _V, _V, _V]),
    "bn_workspace_bytes": (_SZ, [_I, _I64, _I64, _I64]),
    "bn_fwd_train": (_I, [_I, _I64, _I64, _I64, _F, _F, _I, _F, _V, _V, _V, _V, _V, _V, _V, _V,
                          _V, _V, _SZ, _V]),
    "bn_fwd_eval": (_I, [_I, _I64, _I64, _I64, _F, _I, _F, _V, _V, _V, _V, _V, _V, _V, _V]),
    "bn_bwd": (_I, [_I, _I64, _I64, _I64, _I, _F, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V,
                    _SZ, _V]),
    "act_dropout_fwd": (_I, [_I, _I64, _I, _F, _F, _U64, _U64, _V, _V, _V]),
    "act_dropout_bwd": (_I, [_I, _I64, _I, _F, _F, _U64, _U64, _V, _V, _V, _V]),
    "norm_status_str": (ctypes.c_char_p, [_I]),
    "norm_arm_kernel_events": (None, [ctypes.POINTER(ctypes.c_void_p), _I]),
    "norm_last_kernel_count": (_I, []),
    "norm_last_kernel_name": (ctypes.c_char_p, [_I]),
    "norm_last_main_kernel": (_I, []),
    "norm_bn_force_path": (_I, [_I]),
}

_lib = None


def lib():
    """Load libmi355norm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m normalization_ln_rmsnorm_amd.build` (hipcc, gfx950)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


class NormError(RuntimeError):
    def __init__(self, fn, code):
        msg = lib().norm_status_str(code).decode()
        super().__init__(f"{fn}: {STATUS.get(code, code)} ({msg})")
        self.code = code


def _check(fn, code):
    if code != 0:
        raise NormError(fn, code)


def _dt(t):
    if t.dtype == torch.float32:
        return NORM_F32
    if t.dtype == torch.bfloat16:
        return NORM_BF16
    if t.dtype == torch.float16:
        return NORM_F16
    raise TypeError(f"unsupported dtype {t.dtype}: use float32, bfloat16 or float16")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _same(t, ref, name):
    if t is not None and t.dtype != ref.dtype:
        raise TypeError(f"{name} must have dtype {ref.dtype}")


def _stat(t, n, device, name):
    if t is None:
        return torch.empty(n, dtype=torch.float32, device=device)
    if t.dtype != torch.float32 or t.numel() != n:
        raise ValueError(f"{name} must be float32 with {n} elements")
    return t


def _workspace(nbytes, device, ws):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    return ws, ws.numel() * ws.element_size()


def arm_kernel_events(events):
    """Arm hipEvent_t handles for the next call: kernel i of that call is
    launched with events[2i] / events[2i+1] attached to its dispatch (None
    leaves that side unrecorded)."""
    arr = (ctypes.c_void_p * len(events))(
        *[ctypes.c_void_p(None if e is None else getattr(e, "value", e)) for e in events])
    lib().norm_arm_kernel_events(arr, len(events) // 2)


BN_PATHS = {"auto": 0, "plane": 1, "cols": 2}


def bn_force_path(path):
    """Pin BatchNorm's data path ("auto", "plane" or "cols") for every later
    call in this process; returns the previous setting's name (a test hook:
    both paths compute the same results)."""
    prev = lib().norm_bn_force_path(BN_PATHS[path])
    return {v: k for k, v in BN_PATHS.items()}[prev]


def last_kernels():
    """(names of the kernels the last call launched, index of its main kernel)."""
    n = lib().norm_last_kernel_count()
    return [lib().norm_last_kernel_name(i).decode() for i in range(n)], lib().norm_last_main_kernel()


# ---------------------------------------------------------------- LayerNorm
def ln_fwd(x, w=None, b=None, eps=1e-5, *, y=None, mean=None, rstd=None):
    """LayerNorm over the last axis.  Returns (y, mean, rstd)."""
    N = x.shape[-1]
    M = x.numel() // N if N else 0
    _same(w, x, "w"); _same(b, x, "b")
    y = torch.empty_like(x) if y is None else y
    mean = _stat(mean, M, x.device, "mean")
    rstd = _stat(rstd, M, x.device, "rstd")
    _check("ln_fwd", lib().ln_fwd(_dt(x), M, N, float(eps), _ptr(x), _ptr(w), _ptr(b), _ptr(y),
                                  _ptr(mean), _ptr(rstd), _stream(x.device)))
    return y, mean, rstd


def ln_bwd_workspace_bytes(dtype, M, N):
    return int(lib().ln_bwd_workspace_bytes(_dt(torch.empty(0, dtype=dtype)), M, N))


def ln_bwd(dy, x, w, mean, rstd, *, want_dw=True, want_db=True, dx=None, dw=None, db=None,
           ws=None):
    """Returns (dx, dw, db); dw/db are None when not wanted."""
    N = x.shape[-1]
    M = x.numel() // N if N else 0
    _same(dy, x, "dy"); _same(w, x, "w")
    dx = torch.empty_like(x) if dx is None else dx
    if want_dw and dw is None:
        dw = torch.empty(N, dtype=x.dtype, device=x.device)
    if want_db and db is None:
        db = torch.empty(N, dtype=x.dtype, device=x.device)
    need = lib().ln_bwd_workspace_bytes(_dt(x), M, N) if (dw is not None or db is not None) else 0
    ws, nbytes = _workspace(need, x.device, ws)
    _check("ln_bwd", lib().ln_bwd(_dt(x), M, N, _ptr(dy), _ptr(x), _ptr(w), _ptr(mean), _ptr(rstd),
                                  _ptr(dx), _ptr(dw), _ptr(db), _ptr(ws), nbytes,
                                  _stream(x.device)))
    return dx, dw, db


# ------------------------------------------------------------------ RMSNorm
def rms_fwd(x, w=None, eps=1e-6, *, y=None, rstd=None):
    """RMSNorm over the last axis.  Returns (y, rstd)."""
    N = x.shape[-1]
    M = x.numel() // N if N else 0
    _same(w, x, "w")
    y = torch.empty_like(x) if y is None else y
    rstd = _stat(rstd, M, x.device, "rstd")
    _check("rms_fwd", lib().rms_fwd(_dt(x), M, N, float(eps), _ptr(x), _ptr(w), _ptr(y),
                                    _ptr(rstd), _stream(x.device)))
    return y, rstd


def rms_bwd_workspace_bytes(dtype, M, N):
    return int(lib().rms_bwd_workspace_bytes(_dt(torch.empty(0, dtype=dtype)), M, N))


def rms_bwd(dy, x, w, rstd, *, want_dw=True, dx=None, dw=None, ws=None):
    """Returns (dx, dw); dw is None when not wanted."""
    N = x.shape[-1]
    M = x.numel() // N if N else 0
    _same(dy, x, "dy"); _same(w, x, "w")
    dx = torch.empty_like(x) if dx is None else dx
    if want_dw and dw is None:
        dw = torch.empty(N, dtype=x.dtype, device=x.device)
    need = lib().rms_bwd_workspace_bytes(_dt(x), M, N) if dw is not None else 0
    ws, nbytes = _workspace(need, x.device, ws)
    _check("rms_bwd", lib().rms_bwd(_dt(x), M, N, _ptr(dy), _ptr(x), _ptr(w), _ptr(rstd), _ptr(dx),
                                    _ptr(dw), _ptr(ws), nbytes, _stream(x.device)))
    return dx, dw


def rms_bwd_noalloc(dy, x, w, rstd, *, dx, dw=None):
    """rms_bwd through the entry point that allocates nothing (the dw partial
    rows live in the library's static per-GPU scratch).  dx (and dw, if
    wanted) must be passed in; nothing is allocated here either.  Calls that
    overlap on one GPU race on the scratch.  Returns (dx, dw)."""
    N = x.shape[-1]
    M = x.numel() // N if N else 0
    _same(dy, x, "dy"); _same(w, x, "w"); _same(dx, x, "dx"); _same(dw, x, "dw")
    _check("rms_bwd_noalloc", lib().rms_bwd_noalloc(_dt(x), M, N, _ptr(dy), _ptr(x), _ptr(w), _ptr(rstd),
                                                    _ptr(dx), _ptr(dw), _stream(x.device)))
    return dx, dw


# ---------------------------------------------------------------- BatchNorm
def bn_shape(x):
    """(Nb, C, HW) of an (N, C), (N, C, L) or (N, C, H, W) tensor."""
    if x.dim() < 2:
        raise ValueError("BatchNorm input needs at least (N, C)")
    Nb, C = x.shape[0], x.shape[1]
    HW = 1
    for s in x.shape[2:]:
        HW *= s
    return Nb, C, HW


def bn_workspace_bytes(dtype, Nb, C, HW):
    return int(lib().bn_workspace_bytes(_dt(torch.empty(0, dtype=dtype)), Nb, C, HW))


def bn_fwd_train(x, w=None, b=None, running_mean=None, running_var=None, eps=1e-5, momentum=0.1,
                 act="none", res=None, *, act_param=0.0, y=None, save_mean=None, save_rstd=None,
                 ws=None):
    """Training forward; updates running stats in place.  Returns (y, save_mean, save_rstd).

    act_param: negative slope for leaky_relu, alpha for elu / celu."""
    Nb, C, HW = bn_shape(x)
    _same(res, x, "res"); _same(w, x, "w"); _same(b, x, "b")
    y = torch.empty_like(x) if y is None else y
    save_mean = _stat(save_mean, C, x.device, "save_mean")
    save_rstd = _stat(save_rstd, C, x.device, "save_rstd")
    ws, nbytes = _workspace(lib().bn_workspace_bytes(_dt(x), Nb, C, HW), x.device, ws)
    _check("bn_fwd_train", lib().bn_fwd_train(
        _dt(x), Nb, C, HW, float(eps), float(momentum), ACT[act], float(act_param), _ptr(x),
        _ptr(res), _ptr(w),
        _ptr(b), _ptr(running_mean), _ptr(running_var), _ptr(save_mean), _ptr(save_rstd), _ptr(y),
        _ptr(ws), nbytes, _stream(x.device)))
    return y, save_mean, save_rstd


def bn_fwd_eval(x, w, b, running_mean, running_var, eps=1e-5, act="none", res=None, *,
                act_param=0.0, y=None):
    Nb, C, HW = bn_shape(x)
    _same(res, x, "res"); _same(w, x, "w"); _same(b, x, "b")
    y = torch.empty_like(x) if y is None else y
    _check("bn_fwd_eval", lib().bn_fwd_eval(
        _dt(x), Nb, C, HW, float(eps), ACT[act], float(act_param), _ptr(x), _ptr(res), _ptr(w),
        _ptr(b),
        _ptr(running_mean), _ptr(running_var), _ptr(y), _stream(x.device)))
    return y


def bn_bwd(dy, x, w, b, save_mean, save_rstd, act="none", res=None, *, act_param=0.0,
           want_dw=True, want_db=True, dx=None, dres=None, dw=None, db=None, ws=None):
    """Returns (dx, dres, dw, db); dres is None without a residual."""
    Nb, C, HW = bn_shape(x)
    _same(dy, x, "dy"); _same(res, x, "res"); _same(w, x, "w"); _same(b, x, "b")
    dx = torch.empty_like(x) if dx is None else dx
    if res is not None and dres is None:
        dres = torch.empty_like(x)
    if want_dw and dw is None:
        dw = torch.empty(C, dtype=x.dtype, device=x.device)
    if want_db and db is None:
        db = torch.empty(C, dtype=x.dtype, device=x.device)
    ws, nbytes = _workspace(lib().bn_workspace_bytes(_dt(x), Nb, C, HW), x.device, ws)
    _check("bn_bwd", lib().bn_bwd(
        _dt(x), Nb, C, HW, ACT[act], float(act_param), _ptr(dy), _ptr(x), _ptr(res), _ptr(w),
        _ptr(b),
        _ptr(save_mean), _ptr(save_rstd), _ptr(dx), _ptr(dres), _ptr(dw), _ptr(db), _ptr(ws),
        nbytes, _stream(x.device)))
    return dx, dres, dw, db


# ------------------------------------------------------ activation + dropout
def act_dropout_fwd(x, act="none", drop_p=0.0, seed=0, offset=0, *, act_param=0.0, y=None):
    """y = act(x) with inverted dropout (probability drop_p), element-wise;
    the mask is a function of (seed, offset + element index).  offset must
    be a multiple of 8 (one generator call serves eight elements)."""
    y = torch.empty_like(x) if y is None else y
    _same(y, x, "y")
    if y.numel() != x.numel():
        raise ValueError("y must have x's size")
    _check("act_dropout_fwd", lib().act_dropout_fwd(
        _dt(x), x.numel(), ACT[act], float(act_param), float(drop_p), int(seed), int(offset),
        _ptr(x), _ptr(y), _stream(x.device)))
    return y


def act_dropout_bwd(dy, x, act="none", drop_p=0.0, seed=0, offset=0, *, act_param=0.0, dx=None):
    """dx = dy * act'(x) through the same dropout mask as the forward."""
    _same(dy, x, "dy")
    dx = torch.empty_like(x) if dx is None else dx
    if dy.numel() != x.numel() or dx.numel() != x.numel():
        raise ValueError("dy, x and dx must have the same size")
    _check("act_dropout_bwd", lib().act_dropout_bwd(
        _dt(x), x.numel(), ACT[act], float(act_param), float(drop_p), int(seed), int(offset),
        _ptr(dy), _ptr(x), _ptr(dx), _stream(x.device)))
    return dx
