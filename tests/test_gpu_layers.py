"""GPU tests of the PyTorch layers (LayerNorm, RMSNorm, BatchNorm1d/2d with
a fused residual and activation): forward values and autograd gradients
against the float64 oracle on the same inputs, and module semantics
(running statistics, momentum=None, eval mode, autocast dtypes) against
torch.nn's modules."""
import dataclasses

import numpy as np
import pytest
import torch

from tests._parity import TORCH_DTYPE, avoid_kinks, check, to_dev, to_f64

pytestmark = pytest.mark.gpu

nm = pytest.importorskip("normalization_ln_rmsnorm_amd")
from normalization_ln_rmsnorm_amd.workloads import WORKLOADS, gen_bn, gen_rowwise  # noqa: E402


def _param(a, dtype, param_dtype):
    """Generated parameter -> a module parameter tensor of param_dtype
    (values exactly representable in the activation dtype)."""
    return torch.nn.Parameter(to_dev(a, dtype).to(param_dtype))


def _bf(dtype):
    return dtype == "bf16"


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("param_f32", [False, True])
def test_layernorm_layer(orc, dtype, param_f32):
    wl = WORKLOADS["ln_bf16_25216x768"] if dtype != "f32" else WORKLOADS["ln_f32_64x256"]
    wl = dataclasses.replace(wl, dtype=dtype)
    B, T, N = 3, 37, 768
    inp = gen_rowwise(wl, M=B * T, N=N, seed=7)
    pdt = torch.float32 if param_f32 else TORCH_DTYPE[dtype]
    m = nm.LayerNorm(N, eps=wl.eps).cuda().to(pdt)
    m.weight = _param(inp["w"], dtype, pdt)
    m.bias = _param(inp["b"], dtype, pdt)
    x = to_dev(inp["x"], dtype).view(B, T, N).requires_grad_(True)
    y = m(x)
    assert y.dtype == x.dtype and y.shape == x.shape
    y.backward(to_dev(inp["dy"], dtype).view(B, T, N))
    torch.cuda.synchronize()
    ry, _, _ = orc.ln_fwd(inp["x"], inp["w"], inp["b"], eps=wl.eps, bf16=_bf(dtype))
    rdx, rdw, rdb = orc.ln_bwd(inp["dy"], inp["x"], inp["w"], eps=wl.eps, bf16=_bf(dtype))
    check("layer y", to_f64(y).reshape(-1, N), ry, dtype, group_axis=1)
    g = np.abs(orc.widen(inp["dy"], bf16=_bf(dtype)) * orc.widen(inp["w"], bf16=_bf(dtype)))
    _, _, rrstd = orc.ln_fwd(inp["x"], inp["w"], inp["b"], eps=wl.eps, bf16=_bf(dtype))
    check("layer dx", to_f64(x.grad).reshape(-1, N), rdx, dtype, group_axis=1,
          scale=rrstd[:, None] * g.max(axis=1, keepdims=True))
    # The gradient is produced in the activation dtype, then cast to the
    # parameter's dtype.
    check("layer dw", to_f64(m.weight.grad), rdw, dtype)
    check("layer db", to_f64(m.bias.grad), rdb, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rmsnorm_layer(orc, dtype):
    wl = dataclasses.replace(WORKLOADS["rms_bf16_16384x4096"], dtype=dtype)
    M, N = 96, 4096
    inp = gen_rowwise(wl, M=M, N=N, seed=11)
    m = nm.RMSNorm(N, eps=wl.eps).cuda().to(TORCH_DTYPE[dtype])
    m.weight = _param(inp["w"], dtype, TORCH_DTYPE[dtype])
    x = to_dev(inp["x"], dtype).view(2, M // 2, N).requires_grad_(True)
    y = m(x)
    y.backward(to_dev(inp["dy"], dtype).view(2, M // 2, N))
    torch.cuda.synchronize()
    ry, rrstd = orc.rms_fwd(inp["x"], inp["w"], eps=wl.eps, bf16=_bf(dtype))
    rdx, rdw = orc.rms_bwd(inp["dy"], inp["x"], inp["w"], eps=wl.eps, bf16=_bf(dtype))
    check("rms layer y", to_f64(y).reshape(M, N), ry, dtype, group_axis=1)
    g = np.abs(orc.widen(inp["dy"], bf16=_bf(dtype)) * orc.widen(inp["w"], bf16=_bf(dtype)))
    check("rms layer dx", to_f64(x.grad).reshape(M, N), rdx, dtype, group_axis=1,
          scale=rrstd[:, None] * g.max(axis=1, keepdims=True))
    check("rms layer dw", to_f64(m.weight.grad), rdw, dtype)


def test_rmsnorm_default_eps_is_machine_epsilon(orc):
    wl = dataclasses.replace(WORKLOADS["rms_bf16_16384x4096"], dtype="f32")
    inp = gen_rowwise(wl, M=8, N=256, seed=3)
    m = nm.RMSNorm(256).cuda()
    m.weight = _param(inp["w"], "f32", torch.float32)
    y = m(to_dev(inp["x"], "f32"))
    ry, _ = orc.rms_fwd(inp["x"], inp["w"], eps=float(np.finfo(np.float32).eps))
    check("rms default eps", to_f64(y), ry, "f32")


def _bn_case(orc, cls, dtype, shape, act, residual, seed=5):
    """One training step and one eval step of a BatchNorm layer against the
    oracle.  shape is the module input's shape."""
    Nb, C = shape[0], shape[1]
    HW = int(np.prod(shape[2:])) if len(shape) > 2 else 1
    base = WORKLOADS["bn_f32_64x256x56x56"] if dtype == "f32" else WORKLOADS["bn_bf16_256x64x112x112"]
    wl = dataclasses.replace(base, dtype=dtype, residual=residual)
    inp = gen_bn(wl, Nb=Nb, C=C, HW=HW, seed=seed)
    name, p = nm.parse_act(act)
    inp, _ = avoid_kinks(orc, inp, dtype, wl.eps, name)
    pdt = TORCH_DTYPE[dtype]
    m = cls(C, eps=wl.eps, momentum=wl.momentum, act_func=act).cuda().to(pdt)
    m.weight = _param(inp["w"], dtype, pdt)
    m.bias = _param(inp["b"], dtype, pdt)
    m.running_mean = m.running_mean.float()
    m.running_var = m.running_var.float()
    x = to_dev(inp["x"], dtype).view(shape).requires_grad_(True)
    res = to_dev(inp["res"], dtype).view(shape).requires_grad_(True) if residual else None
    y = m(x, pre_act_add=res)
    y.backward(to_dev(inp["dy"], dtype).view(shape))
    m.eval()
    with torch.no_grad():
        ye = m(x, pre_act_add=res)
    torch.cuda.synchronize()
    bf = _bf(dtype)
    res_np = inp["res"] if residual else None
    ry, rsm, rsr, rrm, rrv = orc.bn_fwd_train(inp["x"], res_np, inp["w"], inp["b"],
                                              inp["running_mean"], inp["running_var"],
                                              eps=wl.eps, momentum=wl.momentum, act=name, bf16=bf,
                                              act_param=p)
    rdx, rdres, rdw, rdb = orc.bn_bwd(inp["dy"], inp["x"], res_np, inp["w"], inp["b"], eps=wl.eps,
                                      act=name, bf16=bf, act_param=p)
    rye = orc.bn_fwd_eval(inp["x"], to_f64(m.running_mean), to_f64(m.running_var), res_np,
                          inp["w"], inp["b"], eps=wl.eps, act=name, bf16=bf, act_param=p)
    ch = (0, 2)
    as3 = lambda t: to_f64(t).reshape(Nb, C, HW)
    check("bn layer y", as3(y), ry, dtype, group_axis=ch)
    check("bn layer running_mean", to_f64(m.running_mean), rrm, "f32")
    check("bn layer running_var", to_f64(m.running_var), rrv, "f32")
    assert int(m.num_batches_tracked) == 1
    z, _, _, _, _ = orc.bn_fwd_train(inp["x"], res_np, inp["w"], inp["b"], eps=wl.eps, act="none",
                                     bf16=bf)
    dz = orc.widen(inp["dy"], bf16=bf) * orc.act(name, z, grad=True, param=p)
    wabs = np.abs(orc.widen(inp["w"], bf16=bf))
    check("bn layer dx", as3(x.grad), rdx, dtype, group_axis=ch,
          scale=(wabs * rsr * np.abs(dz).max(axis=(0, 2)))[None, :, None])
    if residual:
        check("bn layer dres", as3(res.grad), rdres, dtype, group_axis=ch)
    check("bn layer dw", to_f64(m.weight.grad), rdw, dtype)
    check("bn layer db", to_f64(m.bias.grad), rdb, dtype)
    check("bn layer y_eval", as3(ye), rye, dtype, group_axis=ch)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_batchnorm2d_relu_residual(orc, dtype):
    print(f"case BatchNorm2d {dtype} relu+res", flush=True)
    _bn_case(orc, nm.BatchNorm2d, dtype, (4, 16, 28, 28), "relu", True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape,act", [((512, 64), "leaky_relu_0.2"), ((64, 32, 20), "gelu"),
                                       ((33, 7), "silu"), ((16, 24, 49), "elu_0.5")])
def test_batchnorm1d(orc, dtype, shape, act):
    print(f"case BatchNorm1d {dtype} {shape} {act}", flush=True)
    _bn_case(orc, nm.BatchNorm1d, dtype, shape, act, residual=len(shape) == 3)


def test_batchnorm_semantics_match_torch():
    """momentum=None (cumulative average), track_running_stats=False and the
    eval path behave as torch.nn.BatchNorm2d (float32, GPU)."""
    torch.manual_seed(0)
    for kw in (dict(momentum=None), dict(momentum=0.3), dict(track_running_stats=False),
               dict(affine=False)):
        ours = nm.BatchNorm2d(6, **kw).cuda()
        ref = torch.nn.BatchNorm2d(6, **kw).cuda()
        for step in range(3):
            x = torch.randn(5, 6, 7, 9, device="cuda") * 2 + 0.5
            torch.testing.assert_close(ours(x), ref(x), rtol=1e-4, atol=1e-5)
        if ref.track_running_stats:
            torch.testing.assert_close(ours.running_mean, ref.running_mean, rtol=1e-5, atol=1e-6)
            torch.testing.assert_close(ours.running_var, ref.running_var, rtol=1e-5, atol=1e-6)
            assert int(ours.num_batches_tracked) == int(ref.num_batches_tracked) == 3
        ours.eval(); ref.eval()
        x = torch.randn(5, 6, 7, 9, device="cuda")
        torch.testing.assert_close(ours(x), ref(x), rtol=1e-4, atol=1e-5)


def test_layers_match_torch_modules():
    """Forward and gradients agree with torch.nn in float32 (a semantic
    check; exactness is pinned against the oracle above)."""
    torch.manual_seed(1)
    x = torch.randn(8, 50, 96, device="cuda", requires_grad=True)
    dy = torch.randn_like(x)
    for ours, ref in ((nm.LayerNorm(96), torch.nn.LayerNorm(96)), (nm.RMSNorm(96), torch.nn.RMSNorm(96))):
        ours, ref = ours.cuda(), ref.cuda()
        with torch.no_grad():
            ref.weight.copy_(torch.randn(96) * 0.1 + 1)
            ours.weight.copy_(ref.weight)
        gx = []
        for m in (ours, ref):
            x.grad = None
            m(x).backward(dy)
            gx.append(x.grad.clone())
        torch.testing.assert_close(gx[0], gx[1], rtol=1e-4, atol=1e-5)
        torch.testing.assert_close(ours.weight.grad, ref.weight.grad, rtol=1e-4, atol=1e-4)
    xb = torch.randn(4, 8, 10, 10, device="cuda", requires_grad=True)
    ours = nm.BatchNorm2d(8, act_func="relu").cuda()
    ref = torch.nn.BatchNorm2d(8).cuda()
    dyb = torch.randn_like(xb)
    g = []
    for f in (lambda t: ours(t), lambda t: torch.relu(ref(t))):
        xb.grad = None
        f(xb).backward(dyb)
        g.append(xb.grad.clone())
    torch.testing.assert_close(g[0], g[1], rtol=1e-4, atol=1e-5)


def test_autocast_dtypes():
    x = torch.randn(4, 64, device="cuda", dtype=torch.bfloat16)
    with torch.autocast("cuda", dtype=torch.bfloat16):
        assert nm.LayerNorm(64).cuda()(x).dtype == torch.float32
        assert nm.LayerNorm(64, autocast_to_fp32=False).cuda()(x).dtype == torch.bfloat16
        assert nm.RMSNorm(64, autocast_to_fp32=False).cuda()(x).dtype == torch.bfloat16
        xb = torch.randn(4, 8, 5, 5, device="cuda", dtype=torch.bfloat16, requires_grad=True)
        bn = nm.BatchNorm2d(8, act_func="gelu").cuda()
        y = bn(xb)
        assert y.dtype == torch.bfloat16
        y.float().sum().backward()
    assert xb.grad.dtype == torch.bfloat16 and bn.weight.grad.dtype == torch.float32


def test_eval_mode_backward_is_refused():
    bn = nm.BatchNorm2d(4).cuda().eval()
    x = torch.randn(2, 4, 3, 3, device="cuda", requires_grad=True)
    with pytest.raises(NotImplementedError):
        bn(x).sum().backward()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_act_dropout_layer(orc, dtype):
    from normalization_ln_rmsnorm_amd.workloads import EXTRA_WORKLOADS, gen_act_dropout
    wl = dataclasses.replace(EXTRA_WORKLOADS["actdrop_bf16_16384x4096"], dtype=dtype)
    inp = gen_act_dropout(wl, n=6 * 1000, seed=4)
    torch.manual_seed(123)
    m = nm.ActDropout("leaky_relu_0.1", drop_p=0.3)
    x = to_dev(inp["x"], dtype).view(6, 1000).requires_grad_(True)
    y = m(x)
    y.backward(to_dev(inp["dy"], dtype).view(6, 1000))
    torch.cuda.synchronize()
    p32 = float(np.float32(0.3))
    ry = orc.act_dropout_fwd(inp["x"], "leaky_relu", p32, m.last_seed, 0, act_param=0.1, bf16=_bf(dtype))
    rdx = orc.act_dropout_bwd(inp["dy"], inp["x"], "leaky_relu", p32, m.last_seed, 0, act_param=0.1,
                              bf16=_bf(dtype))
    check("ActDropout y", to_f64(y).ravel(), ry, dtype)
    check("ActDropout dx", to_f64(x.grad).ravel(), rdx, dtype)
    m.eval()
    ye = m(x.detach())
    torch.cuda.synchronize()
    check("ActDropout eval", to_f64(ye).ravel(),
          orc.act("leaky_relu", orc.widen(inp["x"], bf16=_bf(dtype)), param=0.1), dtype)
