"""Pins for the float64 oracle, checked against things other than itself.

Each oracle function is pinned by at least one of: hand-derived closed forms
(tests/golden/*.json), invariants the definitions imply, an independent
library implementation (PyTorch float64 on the CPU, numpy), central finite
differences of the forward, and the exact relation between one-pass and
two-pass statistics.  These run on the CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _arr(v):
    return None if v is None else np.asarray(v, dtype=np.float64)


# ----------------------------------------------------------- closed forms
def test_ln_closed_form(orc):
    g = _golden("layernorm_closed_form.json")
    for c in g["cases"]:
        y, mean, rstd = orc.ln_fwd(_arr(c["x"]), _arr(c["w"]), _arr(c["b"]), eps=c["eps"])
        np.testing.assert_allclose(y, c["y"], rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(mean, c["mean"], rtol=1e-14)
        np.testing.assert_allclose(rstd, c["rstd"], rtol=1e-14)
    for c in g["backward_cases"]:
        dx, dw, db = orc.ln_bwd(_arr(c["dy"]), _arr(c["x"]), _arr(c["w"]), eps=c["eps"])
        np.testing.assert_allclose(dx, c["dx"], atol=1e-14)
        np.testing.assert_allclose(dw, c["dw"], rtol=1e-14)
        np.testing.assert_allclose(db, c["db"], rtol=1e-14)


def test_rms_closed_form(orc):
    g = _golden("rmsnorm_closed_form.json")
    for c in g["cases"]:
        y, rstd = orc.rms_fwd(_arr(c["x"]), _arr(c["w"]), eps=c["eps"])
        np.testing.assert_allclose(y, c["y"], rtol=1e-14)
        np.testing.assert_allclose(rstd, c["rstd"], rtol=1e-14)
    for c in g["backward_cases"]:
        dx, dw = orc.rms_bwd(_arr(c["dy"]), _arr(c["x"]), _arr(c["w"]), eps=c["eps"])
        np.testing.assert_allclose(dx, c["dx"], atol=1e-14)
        np.testing.assert_allclose(dw, c["dw"], rtol=1e-14)


def test_bn_closed_form(orc):
    g = _golden("batchnorm_closed_form.json")
    for c in g["cases"]:
        y, sm, sr, rm, rv = orc.bn_fwd_train(
            _arr(c["x"]), _arr(c["res"]), _arr(c["w"]), _arr(c["b"]),
            _arr(c["running_mean"]), _arr(c["running_var"]),
            eps=c["eps"], momentum=c["momentum"], act=c["act"])
        np.testing.assert_allclose(y, c["y"], atol=1e-14)
        np.testing.assert_allclose(sm, c["save_mean"], rtol=1e-14)
        np.testing.assert_allclose(sr, c["save_rstd"], rtol=1e-14)
        np.testing.assert_allclose(rm, c["new_running_mean"], rtol=1e-14)
        np.testing.assert_allclose(rv, c["new_running_var"], rtol=1e-14)
    for c in g["backward_cases"]:
        dx, dres, dw, db = orc.bn_bwd(_arr(c["dy"]), _arr(c["x"]), None, _arr(c["w"]),
                                      _arr(c["b"]), eps=c["eps"], act=c["act"])
        np.testing.assert_allclose(dx, c["dx"], atol=1e-14)
        np.testing.assert_allclose(dw, c["dw"], rtol=1e-14)
        np.testing.assert_allclose(db, c["db"], rtol=1e-14)


def test_activation_table(orc):
    g = _golden("activations_table.json")
    for c in g["cases"]:
        f = orc.act(c["act"], np.array([c["z"]]), param=c.get("p", 0.0))[0]
        df = orc.act(c["act"], np.array([c["z"]]), grad=True, param=c.get("p", 0.0))[0]
        assert f == pytest.approx(c["f"], rel=1e-14, abs=1e-15), c
        assert df == pytest.approx(c["df"], rel=1e-14, abs=1e-15), c


def test_gelu_limits_and_library(orc):
    z = np.linspace(-8, 8, 1601)
    f = orc.act("gelu", z)
    ref = F.gelu(torch.from_numpy(z), approximate="none").numpy()
    np.testing.assert_allclose(f, ref, rtol=1e-14, atol=1e-15)
    # Far tails: GELU(z) -> z for large z and -> 0 for very negative z.
    big = orc.act("gelu", np.array([10.0, 40.0, -40.0]))
    assert big[0] == pytest.approx(10.0, rel=1e-15) and big[1] == 40.0 and big[2] == 0.0
    # Derivative against central differences of the oracle's own GELU.
    h = 1e-6
    zz = np.linspace(-5, 5, 101)
    fd = (orc.act("gelu", zz + h) - orc.act("gelu", zz - h)) / (2 * h)
    np.testing.assert_allclose(orc.act("gelu", zz, grad=True), fd, atol=1e-8)


# Activation family against PyTorch float64 (values, derivatives by autograd,
# and PyTorch's conventions at the kinks).  CELU takes alpha = 2: with an
# alpha such as 0.8, PyTorch's float64 CELU gradient differs from the
# definition by ~3e-7 relative (its 1/alpha input scale is not carried in
# double precision), while alpha = 2 makes 1/alpha exact.
TORCH_ACTS = {
    "sigmoid": (lambda t, p: torch.sigmoid(t), 0.0),
    "tanh": (lambda t, p: torch.tanh(t), 0.0),
    "silu": (lambda t, p: F.silu(t), 0.0),
    "mish": (lambda t, p: F.mish(t), 0.0),
    "leaky_relu": (lambda t, p: F.leaky_relu(t, p), 0.07),
    "elu": (lambda t, p: F.elu(t, p), 1.3),
    "selu": (lambda t, p: F.selu(t), 0.0),
    "celu": (lambda t, p: F.celu(t, p), 2.0),  # alpha exact in binary (see below)
    "softplus": (lambda t, p: F.softplus(t), 0.0),
    "relu6": (lambda t, p: F.relu6(t), 0.0),
    "hardsigmoid": (lambda t, p: F.hardsigmoid(t), 0.0),
    "hardswish": (lambda t, p: F.hardswish(t), 0.0),
    "relu": (lambda t, p: F.relu(t), 0.0),
    "gelu": (lambda t, p: F.gelu(t, approximate="none"), 0.0),
}


@pytest.mark.parametrize("name", sorted(TORCH_ACTS))
def test_activation_family_matches_torch(orc, name):
    fn, p = TORCH_ACTS[name]
    # A grid with the kinks (0, +-3, 6, 20) on it, plus tails.
    z = np.concatenate([np.linspace(-30, 30, 6001), [0.0, -3.0, 3.0, 6.0, 20.0, -20.0]])
    t = torch.tensor(z, requires_grad=True)
    y = fn(t, p)
    y.sum().backward()
    np.testing.assert_allclose(orc.act(name, z, param=p), y.detach().numpy(), rtol=1e-14, atol=1e-15)
    # PyTorch's hardsigmoid gradient uses a float32 literal for 1/6.
    rtol = 1e-7 if name == "hardsigmoid" else 1e-13
    np.testing.assert_allclose(orc.act(name, z, grad=True, param=p), t.grad.numpy(), rtol=rtol,
                               atol=1e-15)


# ------------------------------------------------------------- invariants
def test_ln_invariants(orc):
    rng = np.random.default_rng(1)
    x = rng.normal(0.3, 2.0, size=(37, 129))
    y, mean, rstd = orc.ln_fwd(x, eps=0.0)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-14)
    np.testing.assert_allclose((y * y).mean(axis=1), 1.0, rtol=1e-13)
    eps = 0.7
    y, mean, rstd = orc.ln_fwd(x, eps=eps)
    var = np.var(x, axis=1)
    np.testing.assert_allclose((y * y).mean(axis=1), var / (var + eps), rtol=1e-13)
    np.testing.assert_allclose(mean, np.mean(x, axis=1), rtol=1e-13)


def test_rms_invariants(orc):
    rng = np.random.default_rng(2)
    x = rng.normal(0.0, 3.0, size=(33, 77))
    y, rstd = orc.rms_fwd(x, eps=0.0)
    np.testing.assert_allclose(np.sqrt((y * y).mean(axis=1)), 1.0, rtol=1e-13)
    eps = 0.3
    y, rstd = orc.rms_fwd(x, eps=eps)
    ms = np.mean(x * x, axis=1)
    np.testing.assert_allclose((y * y).mean(axis=1), ms / (ms + eps), rtol=1e-13)


def test_ln_backward_invariants(orc):
    rng = np.random.default_rng(3)
    M, N, eps = 9, 50, 0.2
    x = rng.normal(size=(M, N)); dy = rng.normal(size=(M, N)); w = rng.normal(1, 0.3, N)
    dx, dw, db = orc.ln_bwd(dy, x, w, eps=eps)
    # The gradient is orthogonal to the constant vector (sum_j dx = 0 for any eps).
    np.testing.assert_allclose(dx.sum(axis=1), 0.0, atol=1e-12)
    # sum_j dx * xhat = rstd * sum_j g * xhat * eps / (var + eps).
    mu = x.mean(axis=1, keepdims=True); var = x.var(axis=1, keepdims=True)
    r = 1 / np.sqrt(var + eps); xhat = (x - mu) * r; g = dy * w
    lhs = (dx * xhat).sum(axis=1)
    rhs = (r[:, 0] * (g * xhat).sum(axis=1) * eps / (var[:, 0] + eps))
    np.testing.assert_allclose(lhs, rhs, rtol=1e-10, atol=1e-12)


def test_rms_backward_invariant(orc):
    rng = np.random.default_rng(4)
    M, N = 7, 40
    x = rng.normal(size=(M, N)); dy = rng.normal(size=(M, N)); w = rng.normal(1, 0.3, N)
    dx, dw = orc.rms_bwd(dy, x, w, eps=0.0)
    # At eps = 0 the output is scale invariant in x, so dx is orthogonal to x.
    np.testing.assert_allclose((dx * x).sum(axis=1), 0.0, atol=1e-11)


# ------------------------------------------------- independent library check
def test_ln_matches_torch_float64(orc):
    rng = np.random.default_rng(5)
    M, N, eps = 13, 96, 1e-5
    x = rng.normal(0.5, 2, size=(M, N)); w = rng.normal(1, .1, N); b = rng.normal(0, .1, N)
    dy = rng.normal(size=(M, N))
    tx = torch.tensor(x, requires_grad=True); tw = torch.tensor(w, requires_grad=True)
    tb = torch.tensor(b, requires_grad=True)
    ty = F.layer_norm(tx, (N,), tw, tb, eps)
    ty.backward(torch.tensor(dy))
    y, mean, rstd = orc.ln_fwd(x, w, b, eps=eps)
    dx, dw, db = orc.ln_bwd(dy, x, w, eps=eps)
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dw, tw.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(db, tb.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_rms_matches_torch_float64(orc):
    rng = np.random.default_rng(6)
    M, N, eps = 11, 64, 1e-6
    x = rng.normal(size=(M, N)); x[:, 3] *= 20; w = rng.normal(1, .05, N)
    dy = rng.normal(size=(M, N))
    tx = torch.tensor(x, requires_grad=True); tw = torch.tensor(w, requires_grad=True)
    ty = F.rms_norm(tx, (N,), tw, eps)
    ty.backward(torch.tensor(dy))
    y, rstd = orc.rms_fwd(x, w, eps=eps)
    dx, dw = orc.rms_bwd(dy, x, w, eps=eps)
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dw, tw.grad.numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("act,res", [("none", False), ("relu", True), ("gelu", False),
                                     ("gelu", True)])
def test_bn_matches_torch_float64(orc, act, res):
    rng = np.random.default_rng(7)
    Nb, C, HW, eps, mom = 4, 5, 9, 1e-5, 0.1
    x = rng.normal(size=(Nb, C, HW)) * rng.uniform(.5, 3, C)[None, :, None] \
        + rng.uniform(-2, 2, C)[None, :, None]
    w = rng.normal(1, .1, C); b = rng.normal(0, .1, C)
    r = rng.normal(size=(Nb, C, HW)) if res else None
    dy = rng.normal(size=(Nb, C, HW))
    rm0 = rng.normal(size=C); rv0 = rng.uniform(.5, 2, C)
    tx = torch.tensor(x, requires_grad=True); tw = torch.tensor(w, requires_grad=True)
    tb = torch.tensor(b, requires_grad=True)
    tr = torch.tensor(r, requires_grad=True) if res else None
    trm = torch.tensor(rm0.copy()); trv = torch.tensor(rv0.copy())
    z = F.batch_norm(tx, trm, trv, tw, tb, training=True, momentum=mom, eps=eps)
    if res:
        z = z + tr
    ty = {"none": lambda t: t, "relu": F.relu,
          "gelu": lambda t: F.gelu(t, approximate="none")}[act](z)
    ty.backward(torch.tensor(dy))
    y, sm, sr, rm, rv = orc.bn_fwd_train(x, r, w, b, rm0, rv0, eps=eps, momentum=mom, act=act)
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(rm, trm.numpy(), rtol=1e-13)
    np.testing.assert_allclose(rv, trv.numpy(), rtol=1e-13)
    np.testing.assert_allclose(sm, x.mean(axis=(0, 2)), rtol=1e-13)
    np.testing.assert_allclose(sr, 1 / np.sqrt(x.var(axis=(0, 2)) + eps), rtol=1e-13)
    dx, dres, dw, db = orc.bn_bwd(dy, x, r, w, b, eps=eps, act=act)
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dw, tw.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(db, tb.grad.numpy(), rtol=1e-10, atol=1e-12)
    if res:
        np.testing.assert_allclose(dres, tr.grad.numpy(), rtol=1e-12, atol=1e-13)
    # Eval mode against PyTorch with the updated running statistics.
    te = F.batch_norm(torch.tensor(x), torch.tensor(rm), torch.tensor(rv), torch.tensor(w),
                      torch.tensor(b), training=False, eps=eps)
    if res:
        te = te + torch.tensor(r)
    te = {"none": lambda t: t, "relu": F.relu,
          "gelu": lambda t: F.gelu(t, approximate="none")}[act](te)
    ye = orc.bn_fwd_eval(x, rm, rv, r, w, b, eps=eps, act=act)
    np.testing.assert_allclose(ye, te.numpy(), rtol=1e-12, atol=1e-13)


# --------------------------------------------------- finite differences
def _fd(f, arr, h=1e-6):
    g = np.zeros_like(arr)
    it = np.nditer(arr, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = arr[i]
        arr[i] = old + h; fp = f()
        arr[i] = old - h; fm = f()
        arr[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


def test_ln_finite_differences(orc):
    rng = np.random.default_rng(8)
    x = rng.normal(size=(3, 7)); w = rng.normal(1, .3, 7); b = rng.normal(0, .3, 7)
    dy = rng.normal(size=(3, 7)); eps = 1e-3
    L = lambda: float((orc.ln_fwd(x, w, b, eps=eps)[0] * dy).sum())
    dx, dw, db = orc.ln_bwd(dy, x, w, eps=eps)
    np.testing.assert_allclose(dx, _fd(L, x), atol=1e-7)
    np.testing.assert_allclose(dw, _fd(L, w), atol=1e-7)
    np.testing.assert_allclose(db, _fd(L, b), atol=1e-7)


def test_rms_finite_differences(orc):
    rng = np.random.default_rng(9)
    x = rng.normal(size=(3, 7)); w = rng.normal(1, .3, 7)
    dy = rng.normal(size=(3, 7)); eps = 1e-3
    L = lambda: float((orc.rms_fwd(x, w, eps=eps)[0] * dy).sum())
    dx, dw = orc.rms_bwd(dy, x, w, eps=eps)
    np.testing.assert_allclose(dx, _fd(L, x), atol=1e-7)
    np.testing.assert_allclose(dw, _fd(L, w), atol=1e-7)


@pytest.mark.parametrize("act,res", [("relu", True), ("gelu", False), ("gelu", True),
                                     ("none", False), ("silu", True), ("mish", False),
                                     ("elu", True), ("tanh", False)])
def test_bn_finite_differences(orc, act, res):
    rng = np.random.default_rng(10)
    shape = (2, 3, 5)
    x = rng.normal(size=shape) * 2 + 0.5; w = rng.normal(1, .3, 3); b = rng.normal(0, .3, 3)
    r = rng.normal(size=shape) if res else None
    dy = rng.normal(size=shape); eps = 1e-3
    if act == "relu":
        # Keep every pre-activation away from the kink so the central
        # difference sees a differentiable function.
        _, sm, sr, _, _ = orc.bn_fwd_train(x, None, w, b, eps=eps)
        z = (x - sm[None, :, None]) * sr[None, :, None] * w[None, :, None] + b[None, :, None] + r
        r = r + np.where(np.abs(z) < 0.05, np.sign(z) * 0.1 + (z == 0) * 0.1, 0.0)
    p = 1.3 if act == "elu" else 0.0
    L = lambda: float((orc.bn_fwd_train(x, r, w, b, eps=eps, act=act, act_param=p)[0] * dy).sum())
    dx, dres, dw, db = orc.bn_bwd(dy, x, r, w, b, eps=eps, act=act, act_param=p)
    np.testing.assert_allclose(dx, _fd(L, x), atol=2e-7)
    np.testing.assert_allclose(dw, _fd(L, w), atol=2e-7)
    np.testing.assert_allclose(db, _fd(L, b), atol=2e-7)
    if res:
        np.testing.assert_allclose(dres, _fd(L, r), atol=2e-7)


# --------------------------------------------------- one-pass statistics
def test_welford_equals_two_pass(orc):
    rng = np.random.default_rng(11)
    for mu, sd, n in [(0.0, 1.0, 1000), (1e3, 1e-2, 5000), (-2.0, 3.0, 1), (5.0, 0.5, 2)]:
        x = rng.normal(mu, sd, size=n)
        cnt, mean, m2 = orc.welford(x)
        assert cnt == n
        assert mean == pytest.approx(np.mean(x), rel=1e-12, abs=1e-14)
        assert m2 / n == pytest.approx(np.var(x), rel=1e-10, abs=1e-14)


def test_chan_merge_equals_two_pass(orc):
    rng = np.random.default_rng(12)
    x = rng.normal(3.0, 2.0, size=3001)
    # Split at random points, merge the pieces in order and as a tree.
    cuts = np.sort(rng.choice(np.arange(1, x.size), size=9, replace=False))
    parts = [orc.welford(p) for p in np.split(x, cuts)]
    acc = parts[0]
    for p in parts[1:]:
        acc = orc.chan_merge(acc, p)
    while len(parts) > 1:
        parts = [orc.chan_merge(parts[i], parts[i + 1]) if i + 1 < len(parts) else parts[i]
                 for i in range(0, len(parts), 2)]
    for t in (acc, parts[0]):
        assert t[0] == x.size
        assert t[1] == pytest.approx(np.mean(x), rel=1e-13)
        assert t[2] / x.size == pytest.approx(np.var(x), rel=1e-12)
    # Merging with an empty triple is the identity.
    e = orc.chan_merge(np.zeros(3), acc)
    np.testing.assert_allclose(e, acc, rtol=0)


def test_bn_stats_two_pass_and_invariants(orc):
    rng = np.random.default_rng(13)
    x = rng.normal(size=(3, 4, 10)) * 4 + 1
    mean, var = orc.bn_stats(x)
    np.testing.assert_allclose(mean, x.mean(axis=(0, 2)), rtol=1e-13)
    np.testing.assert_allclose(var, x.var(axis=(0, 2)), rtol=1e-13)
    y, sm, sr, _, _ = orc.bn_fwd_train(x, eps=0.0)
    np.testing.assert_allclose(y.mean(axis=(0, 2)), 0.0, atol=1e-14)
    np.testing.assert_allclose((y * y).mean(axis=(0, 2)), 1.0, rtol=1e-13)
    # Welford over one channel's values, in memory order, equals the two-pass result.
    for c in range(4):
        cnt, m, m2 = orc.welford(x[:, c, :])
        assert m == pytest.approx(mean[c], rel=1e-12)
        assert m2 / cnt == pytest.approx(var[c], rel=1e-12)


def test_bn_running_stats_unbiased_factor(orc):
    # n = 2 makes the unbiased factor n/(n-1) = 2, so a biased-variance
    # running update would be off by a factor visible at any tolerance.
    x = np.array([[[1.0]], [[4.0]]])
    for m in (0.1, 0.5, 1.0, 0.0):
        _, sm, sr, rm, rv = orc.bn_fwd_train(x, running_mean=np.array([0.0]),
                                             running_var=np.array([1.0]), eps=0.0, momentum=m)
        assert rm[0] == pytest.approx(m * 2.5, abs=1e-15)
        assert rv[0] == pytest.approx((1 - m) * 1.0 + m * 4.5, rel=1e-15)
        assert sr[0] == pytest.approx(1 / 1.5, rel=1e-15)


# ------------------------------------------------ one-sided derivatives
def test_grad_at_selects_the_one_sided_limit(orc):
    """grad_at picks the derivative's side at a kink.  A channel [-1, 0, 1]
    (w = 1, b = 0, no shift) puts z of its middle element exactly on the
    ReLU kink.  The result with the right side selected must be the limit
    of the plain backward as that element's residual moves up from 0 (z just
    right of the kink), and the left side the limit from below; NaN entries
    leave the plain backward unchanged bit for bit."""
    x = np.array([[[-1.0, 0.0, 1.0], [-2.0, 0.0, 2.0]]])
    dy = np.array([[[0.3, -0.7, 0.5], [1.1, 0.9, -0.4]]])
    w, b = np.ones(2), np.zeros(2)
    r = np.zeros_like(x)
    eps = 1e-5
    plain = orc.bn_bwd(dy, x, r, w, b, eps=eps, act="relu")
    nan = np.full(x.shape, np.nan)
    same = orc.bn_bwd(dy, x, r, w, b, eps=eps, act="relu", grad_at=nan)
    for a, c in zip(plain, same):
        assert np.array_equal(a, c)
    for side in (1.0, -1.0):
        at = nan.copy()
        at[0, :, 1] = side * 2.0 ** -60
        got = orc.bn_bwd(dy, x, r, w, b, eps=eps, act="relu", grad_at=at)
        r2 = r.copy()
        r2[0, :, 1] = side * 1e-9
        lim = orc.bn_bwd(dy, x, r2, w, b, eps=eps, act="relu")
        for a, c in zip(got, lim):
            np.testing.assert_allclose(a, c, atol=1e-12)
    # The right side passes the gradient through the kink element.
    at = nan.copy()
    at[0, :, 1] = 2.0 ** -60
    _, dres, _, db = orc.bn_bwd(dy, x, r, w, b, eps=eps, act="relu", grad_at=at)
    assert np.array_equal(dres[0, :, 1], dy[0, :, 1])
    assert plain[1][0, 0, 1] == 0.0
