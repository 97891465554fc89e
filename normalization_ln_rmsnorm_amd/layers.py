"""Drop-in PyTorch layers over the C ABI: LayerNorm, RMSNorm, BatchNorm1d and
BatchNorm2d with a fused residual add and activation, and a fused
activation + dropout.

Pages (by title):
  [NormPage] "How attorch implements LayerNorm, BatchNorm and RMSNorm: the
             three normalization Triton kernels explained" -- the LayerNorm
             layer (an autograd Function behind an nn.LayerNorm subclass,
             with an autocast_to_fp32 switch), the BatchNorm layers (AMP
             custom_fwd / custom_bwd, a residual added before the activation,
             act_func strings, (N, C) inputs viewed as three-dimensional) and
             the RMSNorm layer.
  [ActPage]  "Operator fusion in practice: attorch's activation and dropout
             fusion kernels", section 6 (activation names carrying their
             parameter, e.g. leaky_relu_0.01) and section 7 (output dtype
             following PyTorch's autocast).

Every forward and backward runs in the HIP kernels through normlib; these
classes only reshape, pick dtypes and keep module state.  There is no
fallback: CPU tensors, or a missing library, raise.

Dtypes.  The kernels take the parameters in the activation dtype, so a
float32 weight meeting a bf16 / fp16 activation is cast to it for the call
and its gradient cast back.  Statistics and running statistics are float32.
Under autocast, LayerNorm and RMSNorm with autocast_to_fp32=True (the
default) run in float32 as PyTorch's autocast runs layer normalization, and
return float32; with autocast_to_fp32=False they keep the input's precision
(half the activation memory).  BatchNorm keeps the input dtype, as PyTorch's
autocast does.
"""
import math

import torch
from torch import nn

from . import normlib as nl

# Activations that take a parameter, with PyTorch's defaults.
_PARAM_DEFAULT = {"leaky_relu": 0.01, "elu": 1.0, "celu": 1.0}


def parse_act(act_func):
    """Activation name -> (kernel name, parameter).

    None or "none" is the identity; a parametric activation may carry its
    parameter after the last underscore ("leaky_relu_0.2", "elu_0.5"),
    otherwise PyTorch's default is used."""
    if act_func is None:
        return "none", 0.0
    if not isinstance(act_func, str):
        raise TypeError("act_func must be a string or None")
    name = act_func.strip().lower()
    if name in nl.ACT:
        return name, _PARAM_DEFAULT.get(name, 0.0)
    base, sep, tail = name.rpartition("_")
    if sep and base in _PARAM_DEFAULT:
        try:
            p = float(tail)
        except ValueError:
            p = None
        if p is not None and math.isfinite(p) and not (base == "celu" and p == 0.0):
            return base, p
    raise ValueError(f"unknown activation {act_func!r}; expected one of {sorted(nl.ACT)} "
                     f"(parametric ones may end in _<value>: {sorted(_PARAM_DEFAULT)})")


def _autocast_on(t):
    return torch.is_autocast_enabled(t.device.type) if t.is_cuda else False


def _as(t, dtype):
    return None if t is None else t.to(dtype).contiguous()


def _grad_back(g, like):
    """Kernel gradient (activation dtype) -> the parameter's dtype."""
    return None if g is None else g.to(like.dtype)


# ---------------------------------------------------------------- LayerNorm
class _LayerNormFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, weight, bias, n, eps):
        x2 = x.contiguous().view(-1, n)
        w = _as(weight, x.dtype)
        b = _as(bias, x.dtype)
        y, mean, rstd = nl.ln_fwd(x2, w, b, eps)
        ctx.save_for_backward(x2, w, mean, rstd)
        ctx.shapes = (x.shape, weight, bias)
        return y.view(x.shape)

    @staticmethod
    def backward(ctx, dy):
        x2, w, mean, rstd = ctx.saved_tensors
        shape, weight, bias = ctx.shapes
        want_w = weight is not None and ctx.needs_input_grad[1]
        want_b = bias is not None and ctx.needs_input_grad[2]
        dy2 = dy.to(x2.dtype).contiguous().view(x2.shape)
        dx, dw, db = nl.ln_bwd(dy2, x2, w, mean, rstd, want_dw=want_w, want_db=want_b)
        dw = _grad_back(dw, weight).view(weight.shape) if want_w else None
        db = _grad_back(db, bias).view(bias.shape) if want_b else None
        return dx.view(shape), dw, db, None, None


class LayerNorm(nn.LayerNorm):
    """nn.LayerNorm whose forward and backward run in the HIP kernels.

    autocast_to_fp32: under autocast, compute (and return) float32 like
    PyTorch (True), or keep the input's precision (False)."""

    def __init__(self, normalized_shape, eps=1e-5, elementwise_affine=True, bias=True,
                 device=None, dtype=None, autocast_to_fp32=True):
        super().__init__(normalized_shape, eps=eps, elementwise_affine=elementwise_affine,
                         bias=bias, device=device, dtype=dtype)
        self.autocast_to_fp32 = autocast_to_fp32

    def forward(self, x):
        if tuple(x.shape[x.dim() - len(self.normalized_shape):]) != tuple(self.normalized_shape):
            raise ValueError(f"input's trailing shape {tuple(x.shape)} does not end in "
                             f"{tuple(self.normalized_shape)}")
        if _autocast_on(x) and self.autocast_to_fp32:
            x = x.float()
        n = math.prod(self.normalized_shape)
        with torch.autocast(x.device.type, enabled=False):
            return _LayerNormFn.apply(x, self.weight, self.bias, n, self.eps)

    def extra_repr(self):
        return super().extra_repr() + f", autocast_to_fp32={self.autocast_to_fp32}"


# ------------------------------------------------------------------ RMSNorm
class _RMSNormFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, weight, n, eps):
        x2 = x.contiguous().view(-1, n)
        w = _as(weight, x.dtype)
        y, rstd = nl.rms_fwd(x2, w, eps)
        ctx.save_for_backward(x2, w, rstd)
        ctx.shapes = (x.shape, weight)
        return y.view(x.shape)

    @staticmethod
    def backward(ctx, dy):
        x2, w, rstd = ctx.saved_tensors
        shape, weight = ctx.shapes
        want_w = weight is not None and ctx.needs_input_grad[1]
        dy2 = dy.to(x2.dtype).contiguous().view(x2.shape)
        dx, dw = nl.rms_bwd(dy2, x2, w, rstd, want_dw=want_w)
        dw = _grad_back(dw, weight).view(weight.shape) if want_w else None
        return dx.view(shape), dw, None, None


class RMSNorm(nn.RMSNorm):
    """nn.RMSNorm whose forward and backward run in the HIP kernels.

    eps=None takes the input dtype's machine epsilon, as PyTorch does;
    autocast_to_fp32 as for LayerNorm."""

    def __init__(self, normalized_shape, eps=None, elementwise_affine=True, device=None,
                 dtype=None, autocast_to_fp32=True):
        super().__init__(normalized_shape, eps=eps, elementwise_affine=elementwise_affine,
                         device=device, dtype=dtype)
        self.autocast_to_fp32 = autocast_to_fp32

    def forward(self, x):
        if tuple(x.shape[x.dim() - len(self.normalized_shape):]) != tuple(self.normalized_shape):
            raise ValueError(f"input's trailing shape {tuple(x.shape)} does not end in "
                             f"{tuple(self.normalized_shape)}")
        if _autocast_on(x) and self.autocast_to_fp32:
            x = x.float()
        eps = self.eps if self.eps is not None else torch.finfo(x.dtype).eps
        n = math.prod(self.normalized_shape)
        with torch.autocast(x.device.type, enabled=False):
            return _RMSNormFn.apply(x, self.weight, n, eps)


# ---------------------------------------------------------------- BatchNorm
class _BatchNormFn(torch.autograd.Function):
    @staticmethod
    @torch.amp.custom_fwd(device_type="cuda")
    def forward(ctx, x, res, weight, bias, running_mean, running_var, training, momentum, eps,
                act, act_param):
        x = x.contiguous()
        res = _as(res, x.dtype)
        w = _as(weight, x.dtype)
        b = _as(bias, x.dtype)
        if training:
            # `training` means "normalize by the batch"; the running
            # statistics (when tracked) are updated then.  They are float32
            # for the kernels; other dtypes go through a float32 copy.
            rm, rv = running_mean, running_var
            tmp = rm is not None and rm.dtype != torch.float32
            if tmp:
                rm, rv = rm.float(), rv.float()
            y, sm, sr = nl.bn_fwd_train(x, w, b, rm, rv, eps, momentum, act, res, act_param=act_param)
            if tmp:
                running_mean.copy_(rm)
                running_var.copy_(rv)
            ctx.save_for_backward(x, res, w, b, sm, sr)
        else:
            y = nl.bn_fwd_eval(x, w, b, running_mean.float(), running_var.float(), eps, act, res,
                               act_param=act_param)
        ctx.training = training
        ctx.act = (act, act_param)
        ctx.params = (weight, bias)
        return y

    @staticmethod
    @torch.amp.custom_bwd(device_type="cuda")
    def backward(ctx, dy):
        if not ctx.training:
            raise NotImplementedError(
                "backward through BatchNorm in eval mode (running statistics) is not provided; "
                "use training mode or freeze the layer")
        x, res, w, b, sm, sr = ctx.saved_tensors
        weight, bias = ctx.params
        act, act_param = ctx.act
        want_w = weight is not None and ctx.needs_input_grad[2]
        want_b = bias is not None and ctx.needs_input_grad[3]
        dx, dres, dw, db = nl.bn_bwd(dy.to(x.dtype).contiguous(), x, w, b, sm, sr, act, res,
                                     act_param=act_param, want_dw=want_w, want_db=want_b)
        dw = _grad_back(dw, weight) if want_w else None
        db = _grad_back(db, bias) if want_b else None
        dres = dres if (res is not None and ctx.needs_input_grad[1]) else None
        return dx, dres, dw, db, None, None, None, None, None, None, None


class _FusedBatchNorm:
    """Shared forward of the BatchNorm layers: act_func after the
    normalization, pre_act_add (a tensor of the input's shape) added before
    it.  Running statistics follow PyTorch: momentum=None takes the
    cumulative average, track_running_stats=False always normalizes by the
    batch."""

    def _init_act(self, act_func):
        self.act_func = act_func
        self._act, self._act_param = parse_act(act_func)

    def forward(self, x, pre_act_add=None):
        self._check_input_dim(x)
        if pre_act_add is not None and pre_act_add.shape != x.shape:
            raise ValueError(f"pre_act_add has shape {tuple(pre_act_add.shape)}, input "
                             f"{tuple(x.shape)}")
        use_batch = self.training or not self.track_running_stats
        factor = 0.0 if self.momentum is None else self.momentum
        if self.training and self.track_running_stats and self.num_batches_tracked is not None:
            self.num_batches_tracked.add_(1)
            if self.momentum is None:
                factor = 1.0 / float(self.num_batches_tracked.item())
        # Batch statistics: the running ones are updated only in training
        # (and absent when not tracked); otherwise the running ones are read.
        return _BatchNormFn.apply(
            x, pre_act_add, self.weight, self.bias, self.running_mean, self.running_var,
            use_batch, factor, self.eps, self._act, self._act_param)

    def extra_repr(self):
        return super().extra_repr() + f", act_func={self.act_func!r}"


class BatchNorm1d(_FusedBatchNorm, nn.BatchNorm1d):
    """nn.BatchNorm1d ((N, C) or (N, C, L) inputs) with a fused residual add
    and activation, forward and backward in the HIP kernels."""

    def __init__(self, num_features, eps=1e-5, momentum=0.1, affine=True,
                 track_running_stats=True, device=None, dtype=None, act_func=None):
        nn.BatchNorm1d.__init__(self, num_features, eps=eps, momentum=momentum, affine=affine,
                                track_running_stats=track_running_stats, device=device,
                                dtype=dtype)
        self._init_act(act_func)


class BatchNorm2d(_FusedBatchNorm, nn.BatchNorm2d):
    """nn.BatchNorm2d (NCHW inputs) with a fused residual add and
    activation, forward and backward in the HIP kernels; e.g.
    BatchNorm2d(64, act_func="relu")(x, pre_act_add=shortcut)."""

    def __init__(self, num_features, eps=1e-5, momentum=0.1, affine=True,
                 track_running_stats=True, device=None, dtype=None, act_func=None):
        nn.BatchNorm2d.__init__(self, num_features, eps=eps, momentum=momentum, affine=affine,
                                track_running_stats=track_running_stats, device=device,
                                dtype=dtype)
        self._init_act(act_func)


# ------------------------------------------------------ activation + dropout
class _ActDropoutFn(torch.autograd.Function):
    @staticmethod
    @torch.amp.custom_fwd(device_type="cuda")
    def forward(ctx, x, act, act_param, p, seed):
        x = x.contiguous()
        y = nl.act_dropout_fwd(x, act, p, seed, 0, act_param=act_param)
        ctx.save_for_backward(x)
        ctx.cfg = (act, act_param, p, seed)
        return y

    @staticmethod
    @torch.amp.custom_bwd(device_type="cuda")
    def backward(ctx, dy):
        (x,) = ctx.saved_tensors
        act, act_param, p, seed = ctx.cfg
        dx = nl.act_dropout_bwd(dy.to(x.dtype).contiguous(), x, act, p, seed, 0, act_param=act_param)
        return dx, None, None, None, None


class ActDropout(nn.Module):
    """An activation followed by inverted dropout in one kernel ([ActPage]
    sections 3-5), e.g. ActDropout("gelu", drop_p=0.1).  Training draws a
    64-bit seed from PyTorch's default CPU generator per call (kept in
    `last_seed`); the backward regenerates the mask from it instead of
    storing it.  In eval mode (or with drop_p = 0) it is the plain
    activation."""

    def __init__(self, act_func="relu", drop_p=0.5):
        super().__init__()
        if not 0.0 <= drop_p <= 1.0:
            raise ValueError("drop_p must be in [0, 1]")
        self.act_func = act_func
        self._act, self._act_param = parse_act(act_func)
        self.drop_p = float(drop_p)
        self.last_seed = None

    def forward(self, x):
        p = self.drop_p if self.training else 0.0
        seed = int(torch.randint(0, 1 << 62, (1,)).item()) if p > 0.0 else 0
        self.last_seed = seed
        return _ActDropoutFn.apply(x, self._act, self._act_param, p, seed)

    def extra_repr(self):
        return f"act_func={self.act_func!r}, drop_p={self.drop_p}"


def output_dtype(input_dtype, autocast_enabled, autocast_to_fp32=True, kind="layer_norm"):
    """The dtype these layers return ([ActPage] section 7: outputs follow
    PyTorch's autocast): LayerNorm / RMSNorm return float32 under autocast
    unless autocast_to_fp32=False; BatchNorm and everything outside
    autocast return the input dtype."""
    if kind in ("layer_norm", "rms_norm") and autocast_enabled and autocast_to_fp32:
        return torch.float32
    return input_dtype
