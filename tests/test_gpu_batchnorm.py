"""GPU parity: BatchNorm training forward, eval forward and backward (with
the fused residual and each fused activation) through the C ABI against the
float64 oracle, element by element.

Every output (y, y_eval, dx, dres, dw, db, the saved and running statistics
and the workspace) sits between guard bands that must come back unchanged.

At a kink of the activation, an element whose exact pre-activation lies
within the kernels' float32 rounding radius of the kink has two valid
gradients.  Small cases move such elements off the kink first
(tests._parity.avoid_kinks; the radius is a few dozen float32 ulps of the
terms z is formed from, so almost none move).  The full-size ReLU workload
runs on the benchmark's unedited inputs: there the side the GPU took at each
such element is read from its forward output and handed to the oracle
(tests._parity.relu_kink_sides).
"""
import dataclasses

import numpy as np
import pytest
import torch

from tests._parity import (KINK_LOG, TORCH_DTYPE, Guarded, assert_guards, avoid_kinks, check,
                           relu_kink_sides, to_dev, to_f64, to_io)

pytestmark = pytest.mark.gpu

nl = pytest.importorskip("normalization_ln_rmsnorm_amd")
from normalization_ln_rmsnorm_amd.workloads import EXTRA_WORKLOADS, WORKLOADS, gen_bn  # noqa: E402


@pytest.fixture
def force_path():
    """Pins BatchNorm's data path for one test (restored afterwards)."""
    prev = []

    def set_path(path):
        prev.append(nl.bn_force_path(path))
    yield set_path
    if prev:
        nl.bn_force_path(prev[0])


def _wl(dtype, act, residual):
    base = WORKLOADS["bn_f32_64x256x56x56"] if dtype == "f32" else WORKLOADS["bn_bf16_256x64x112x112"]
    return dataclasses.replace(base, dtype=dtype, act=act, residual=residual)


def _scale_w(orc, inp, dtype, k):
    """Multiply the affine weight by a power of two (exact in every format)."""
    out = dict(inp)
    w = orc.widen(inp["w"], bf16=dtype == "bf16") * k
    out["w"] = to_io(w.astype(np.float32), dtype)
    return out


def run_case(orc, dtype, Nb, C, HW, act, residual, with_wb=True, eval_after=True, report=None,
             inp=None, wl=None, act_param=0.0, w_scale=1, raw=False, misalign=0):
    """raw=True keeps the inputs unedited (ReLU: the GPU's side at elements
    within rounding of the kink goes to the oracle); misalign=1 places every
    streamed output off 16-byte alignment (the scalar paths)."""
    wl = wl or _wl(dtype, act, residual)
    if inp is None:
        inp = gen_bn(wl, Nb=Nb, C=C, HW=HW)
    bf16 = dtype == "bf16"
    eps, mom = wl.eps, wl.momentum
    if w_scale != 1:
        inp = _scale_w(orc, inp, dtype, w_scale)
    inp = dict(inp)
    if not residual:
        inp["res"] = None
    if not with_wb:
        inp["w"] = inp["b"] = None
    if raw:
        assert act in ("relu", "none") and dtype in ("f32", "bf16"), "raw inputs: ReLU, f32/bf16"
        moved = 0
    else:
        inp, moved = avoid_kinks(orc, inp, dtype, eps, act)
    tdt = TORCH_DTYPE[dtype]
    shape = (Nb, C, HW)
    x = to_dev(inp["x"], dtype)
    res = to_dev(inp["res"], dtype) if residual else None
    w = to_dev(inp["w"], dtype) if with_wb else None
    b = to_dev(inp["b"], dtype) if with_wb else None
    dy = to_dev(inp["dy"], dtype)
    w_np, b_np, res_np = inp["w"], inp["b"], inp["res"]

    G = dict(y=Guarded(shape, tdt, misalign=misalign), dx=Guarded(shape, tdt, misalign=misalign),
             sm=Guarded((C,), torch.float32), sr=Guarded((C,), torch.float32),
             rm=Guarded((C,), torch.float32, fill=torch.from_numpy(inp["running_mean"].copy())),
             rv=Guarded((C,), torch.float32, fill=torch.from_numpy(inp["running_var"].copy())),
             dres=Guarded(shape, tdt, misalign=misalign) if residual else None,
             dw=Guarded((C,), tdt) if with_wb else None, db=Guarded((C,), tdt) if with_wb else None,
             ye=Guarded(shape, tdt, misalign=misalign) if eval_after else None,
             ws=Guarded((max(1, nl.bn_workspace_bytes(tdt, Nb, C, HW)),), torch.uint8))
    t = {k: (g.t if g is not None else None) for k, g in G.items()}
    rm, rv = t["rm"], t["rv"]

    ap = act_param
    y, sm, sr = nl.bn_fwd_train(x, w, b, rm, rv, eps, mom, act, res, act_param=ap, y=t["y"],
                                save_mean=t["sm"], save_rstd=t["sr"], ws=t["ws"])
    dx, dres, dw, db = nl.bn_bwd(dy, x, w, b, sm, sr, act, res, act_param=ap, want_dw=with_wb,
                                 want_db=with_wb, dx=t["dx"], dres=t["dres"], dw=t["dw"],
                                 db=t["db"], ws=t["ws"])
    ye = nl.bn_fwd_eval(x, w, b, rm, rv, eps, act, res, act_param=ap, y=t["ye"]) if eval_after else None
    assert_guards(G)

    grad_at, n_amb = None, 0
    if raw and act == "relu":
        grad_at, n_amb = relu_kink_sides(orc, inp, dtype, eps, y)
    ry, rsm, rsr, rrm, rrv = orc.bn_fwd_train(inp["x"], res_np, w_np, b_np, inp["running_mean"],
                                              inp["running_var"], eps=eps, momentum=mom, act=act,
                                              bf16=bf16, act_param=ap)
    rdx, rdres, rdw, rdb = orc.bn_bwd(inp["dy"], inp["x"], res_np, w_np, b_np, eps=eps, act=act,
                                      bf16=bf16, act_param=ap, grad_at=grad_at)
    tag = f"bn/{dtype}/{Nb}x{C}x{HW}/{act}({ap})/res={residual}"
    if moved or n_amb or raw:
        KINK_LOG.append(f"{tag}: {moved} of {x.numel()} elements moved off a kink, {n_amb} within "
                        "rounding of one on unedited inputs (the GPU's side taken)")
    ch = (0, 2)  # bf16 floor taken per channel
    check(f"{tag} y", to_f64(y), ry, dtype, group_axis=ch, report=report)
    check(f"{tag} save_mean", to_f64(sm), rsm, "f32", report=report)
    check(f"{tag} save_rstd", to_f64(sr), rsr, "f32", report=report)
    check(f"{tag} running_mean", to_f64(rm), rrm, "f32", report=report)
    check(f"{tag} running_var", to_f64(rv), rrv, "f32", report=report)
    # Scale of the terms dx is formed from: |w_c * rstd_c| * max |dz| per
    # channel, dz = dy * act'(z) (oracle values).
    wabs = np.abs(orc.widen(w_np, bf16=bf16)) if with_wb else np.ones(C)
    z, _, _, _, _ = orc.bn_fwd_train(inp["x"], res_np, w_np, b_np, eps=eps, act="none", bf16=bf16)
    if grad_at is not None:
        z = np.where(np.isnan(grad_at), z, grad_at)
    dz = orc.widen(inp["dy"], bf16=bf16) * orc.act(act, z, grad=True, param=ap)
    del z
    dx_scale = (wabs * rsr * np.abs(dz).max(axis=(0, 2)))[None, :, None]
    # L2 norms of the terms db and dw sum per channel (dz and dz * xhat).
    db_l2 = np.sqrt((dz * dz).sum(axis=(0, 2)))
    xhat = (orc.widen(inp["x"], bf16=bf16) - rsm[None, :, None]) * rsr[None, :, None]
    dz *= xhat
    del xhat
    dw_l2 = np.sqrt((dz * dz).sum(axis=(0, 2)))
    del dz
    check(f"{tag} dx", to_f64(dx), rdx, dtype, group_axis=ch, report=report, scale=dx_scale)
    if residual:
        check(f"{tag} dres", to_f64(dres), rdres, dtype, group_axis=ch, report=report)
    if with_wb:
        check(f"{tag} dw", to_f64(dw), rdw, dtype, report=report, sum_l2=dw_l2)
        check(f"{tag} db", to_f64(db), rdb, dtype, report=report, sum_l2=db_l2)
    if eval_after:
        # Eval reads the running statistics the training step just wrote
        # (float32 on the device, passed to the oracle as they stand).
        rye = orc.bn_fwd_eval(inp["x"], to_f64(rm), to_f64(rv), res_np, w_np, b_np, eps=eps,
                              act=act, bf16=bf16, act_param=ap)
        check(f"{tag} y_eval", to_f64(ye), rye, dtype, group_axis=ch, report=report)
    return n_amb


SMALL = [(2, 3, 5), (4, 8, 49), (3, 5, 1), (2, 4, 7), (5, 16, 64), (2, 2, 3136), (7, 3, 1000),
         (1, 2, 12544), (16, 4, 24)]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("act,residual", [("none", False), ("relu", True), ("gelu", False),
                                          ("gelu", True), ("relu", False), ("none", True)])
@pytest.mark.parametrize("Nb,C,HW", SMALL)
def test_small_shapes(orc, dtype, act, residual, Nb, C, HW):
    print(f"case bn {dtype} {Nb}x{C}x{HW} {act} res={residual}", flush=True)
    run_case(orc, dtype, Nb, C, HW, act, residual)


# The rest of the activation family, on the run-time-dispatched kernels.  The
# weight is scaled by 4 so z spreads over about [-16, 16] and every branch
# (both saturations of relu6 / hardsigmoid / hardswish, the exp tails) is hit.
FAMILY = [("sigmoid", 0.0), ("tanh", 0.0), ("silu", 0.0), ("mish", 0.0), ("leaky_relu", 0.01),
          ("leaky_relu", 0.2), ("elu", 1.0), ("elu", 0.5), ("selu", 0.0), ("celu", 1.0),
          ("celu", 2.0), ("softplus", 0.0), ("relu6", 0.0), ("hardsigmoid", 0.0),
          ("hardswish", 0.0)]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("act,ap", FAMILY)
@pytest.mark.parametrize("residual", [False, True])
@pytest.mark.parametrize("Nb,C,HW", [(4, 8, 49), (7, 3, 1000), (2, 2, 3136)])
def test_activation_family(orc, dtype, act, ap, residual, Nb, C, HW):
    print(f"case bn {dtype} {Nb}x{C}x{HW} {act}({ap}) res={residual}", flush=True)
    run_case(orc, dtype, Nb, C, HW, act, residual, act_param=ap, w_scale=4)


def test_softplus_threshold(orc):
    """z beyond 20 takes softplus's identity branch (weight scaled by 8)."""
    run_case(orc, "f32", 4, 4, 2000, "softplus", True, w_scale=8)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_no_affine(orc, dtype):
    run_case(orc, dtype, 4, 6, 50, "gelu", True, with_wb=False)


def test_two_values_pin_unbiased_running_var(orc):
    """n = 2 per channel: the unbiased factor is 2, visible at any tolerance."""
    run_case(orc, "f32", 2, 5, 1, "none", False)


@pytest.mark.parametrize("name", ["bn_f32_64x256x56x56", "bn_bf16_256x64x112x112"])
def test_full_size_workloads(orc, name):
    """The two BatchNorm2d workloads at full size on the benchmark's own
    (unedited) inputs and launch configuration; for ReLU the GPU's side at
    the elements within rounding of the kink is handed to the oracle."""
    wl = WORKLOADS[name]
    Nb, C, H, W = wl.shape
    print(f"case {name}", flush=True)
    report = []
    n_amb = run_case(orc, wl.dtype, Nb, C, H * W, wl.act, wl.residual, eval_after=True,
                     report=report, wl=wl, raw=wl.act in ("relu", "none"))
    for r in report:
        print(r, flush=True)
    print(f"{name}: {n_amb} elements within rounding of the ReLU kink", flush=True)


@pytest.mark.parametrize("path", ["plane", "cols"])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("Nb,C,HW", [(4, 8, 49), (7, 3, 1000), (3, 5, 1), (33, 7, 13)])
def test_unaligned_outputs_scalar_tails(orc, force_path, path, dtype, Nb, C, HW):
    """Every streamed output one element off 16-byte alignment (the scalar
    path of each kernel), on both data paths, with guard bands."""
    force_path(path)
    print(f"case bn unaligned path={path} {dtype} {Nb}x{C}x{HW}", flush=True)
    run_case(orc, dtype, Nb, C, HW, "gelu", True, misalign=1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Nb,C,HW", [(8, 16, 3136), (64, 64, 1)])
def test_relu_raw_inputs(orc, dtype, Nb, C, HW):
    """ReLU + residual on unedited inputs (the full-size workload's method at
    a size with many elements near the kink relative to the radius)."""
    print(f"case bn relu raw {dtype} {Nb}x{C}x{HW}", flush=True)
    run_case(orc, dtype, Nb, C, HW, "relu", True, raw=True)


# BatchNorm1d shapes: (N, C) with HW = 1 and (N, C, L); they take the
# column path (vector or scalar, depending on whether C * HW splits into
# 128-bit vectors).
BN1D = [(4096, 64, 1), (3, 5, 1), (1000, 333, 1), (256, 1024, 1), (64, 32, 16), (33, 7, 49),
        (16, 128, 49), (2, 3, 2), (517, 24, 3),
        # 256 row tiles x 40 columns per channel: 10240 (tile, column) entries
        # per channel, past what the finalize holds in registers (512)
        (4096, 8, 40)]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("act,residual", [("relu", True), ("gelu", False), ("silu", True)])
@pytest.mark.parametrize("Nb,C,HW", BN1D)
def test_bn1d_shapes(orc, dtype, act, residual, Nb, C, HW):
    print(f"case bn1d {dtype} {Nb}x{C}x{HW} {act} res={residual}", flush=True)
    run_case(orc, dtype, Nb, C, HW, act, residual)


@pytest.mark.parametrize("path", ["plane", "cols"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Nb,C,HW", [(4, 8, 49), (7, 3, 1000), (8, 16, 64), (300, 40, 1)])
def test_each_path_on_every_shape(orc, force_path, path, dtype, Nb, C, HW):
    """Either data path, forced, meets the tolerance on shapes that would
    normally take the other."""
    force_path(path)
    print(f"case bn path={path} {dtype} {Nb}x{C}x{HW}", flush=True)
    run_case(orc, dtype, Nb, C, HW, "gelu", True)


@pytest.mark.parametrize("name", ["bn1d_f32_8192x2048", "bn1d_bf16_2048x512x32"])
def test_full_size_bn1d(orc, name):
    wl = EXTRA_WORKLOADS[name]
    Nb, C, L, _ = wl.shape
    print(f"case {name}", flush=True)
    report = []
    run_case(orc, wl.dtype, Nb, C, L, wl.act, wl.residual, report=report, wl=wl,
             raw=wl.act in ("relu", "none") and wl.dtype in ("f32", "bf16"))
    for r in report:
        print(r, flush=True)


def test_full_size_f16(orc):
    """The bf16 BatchNorm workload's recipe and shape with fp16 I/O."""
    wl = dataclasses.replace(WORKLOADS["bn_bf16_256x64x112x112"], dtype="f16")
    Nb, C, H, W = wl.shape
    print("case bn f16 256x64x112x112 gelu", flush=True)
    report = []
    run_case(orc, "f16", Nb, C, H * W, wl.act, wl.residual, report=report, wl=wl)
    for r in report:
        print(r, flush=True)


def test_backward_bitwise_deterministic(orc):
    wl = _wl("f32", "relu", True)
    inp = gen_bn(wl, Nb=8, C=32, HW=784)
    x, res, w, b, dy = (to_dev(inp[k], "f32") for k in ("x", "res", "w", "b", "dy"))
    outs = []
    for _ in range(2):
        run = []
        for act in ("relu", "mish"):
            rm = torch.zeros(32, device="cuda"); rv = torch.ones(32, device="cuda")
            y, sm, sr = nl.bn_fwd_train(x, w, b, rm, rv, wl.eps, wl.momentum, act, res)
            run += [y, sm, sr, rm, rv] + list(nl.bn_bwd(dy, x, w, b, sm, sr, act, res))
        outs.append(run)
    torch.cuda.synchronize()
    for a, b_ in zip(outs[0], outs[1]):
        assert torch.equal(a, b_)


# ---------------------------------------------------------------- output stores past 2 GiB
# The output stores address a plane (plane path) or a row tile (column path)
# from its first element with 32-bit offsets, and fall back to non-temporal
# global stores when that region is 4 GiB or more.  Replicating an input
# block along the batch or spatial axis leaves every per-channel mean the
# statistics and the backward sums are made of unchanged, so the outputs of
# the large tensor are the oracle's outputs on the block, repeated (dw / db
# scale with the replication; the running variance's n / (n - 1) uses the
# large count).  Each repeated output is checked through its maximum and
# minimum over the copies: both within tolerance bound every copy.  The
# block's channels keep the workload recipe's ratio of mean to spread (at
# most ~4): float32 statistics cannot meet the 1e-5 tolerance on y for a
# channel whose mean is hundreds of spreads from zero.
def run_replicated(orc, dtype, small, reps, axis, act, residual, x=None):
    Nb0, C, HW0 = small
    wl = _wl(dtype, act, residual)
    inp = gen_bn(wl, Nb=Nb0, C=C, HW=HW0)
    if x is not None:
        inp["x"] = x
    eps, mom, bf16 = wl.eps, wl.momentum, dtype == "bf16"
    rep = tuple(reps if d == axis else 1 for d in range(3))

    def big(a):
        return to_dev(a, dtype).repeat(*rep)

    x, dy = big(inp["x"]), big(inp["dy"])
    res = big(inp["res"]) if residual else None
    w, b = to_dev(inp["w"], dtype), to_dev(inp["b"], dtype)
    rm = torch.from_numpy(inp["running_mean"].copy()).cuda()
    rv = torch.from_numpy(inp["running_var"].copy()).cuda()
    y, sm, sr = nl.bn_fwd_train(x, w, b, rm, rv, eps, mom, act, res)
    dx, dres, dw, db = nl.bn_bwd(dy, x, w, b, sm, sr, act, res)
    ye = nl.bn_fwd_eval(x, w, b, rm, rv, eps, act, res)
    torch.cuda.synchronize()
    del x, dy, res

    res_np = inp["res"] if residual else None
    ry, rsm, rsr, rrm, rrv = orc.bn_fwd_train(inp["x"], res_np, inp["w"], inp["b"], inp["running_mean"],
                                              inp["running_var"], eps=eps, momentum=mom, act=act, bf16=bf16)
    rdx, rdres, rdw, rdb = orc.bn_bwd(inp["dy"], inp["x"], res_np, inp["w"], inp["b"], eps=eps, act=act,
                                      bf16=bf16)
    rye = orc.bn_fwd_eval(inp["x"], to_f64(rm), to_f64(rv), res_np, inp["w"], inp["b"], eps=eps, act=act,
                          bf16=bf16)
    # Running variance with the replicated count n instead of the block's n0.
    n0, n = Nb0 * HW0, Nb0 * HW0 * reps
    rv0 = orc.widen(inp["running_var"], bf16=False)
    var = (rrv - (1.0 - mom) * rv0) / mom * (n0 - 1) / n0
    rrv_big = (1.0 - mom) * rv0 + mom * var * n / (n - 1)

    def folds(t):
        if axis == 0:
            v = t.view(reps, Nb0, C, HW0)
            return v.amax(0), v.amin(0)
        v = t.view(Nb0, C, reps, HW0)
        return v.amax(2), v.amin(2)

    tag = f"bn/{dtype}/{small}x{reps}@{axis}/{act}/res={residual}"
    ch = (0, 2)
    for name, t, ref in (("y", y, ry), ("y_eval", ye, rye), ("dx", dx, rdx)) + (
            (("dres", dres, rdres),) if residual else ()):
        hi, lo = folds(t)
        scale = None
        if name == "dx":
            scale = np.abs(rdx).max(axis=ch, keepdims=True) + np.abs(orc.widen(inp["w"], bf16=bf16)
                                                                     * rsr)[None, :, None]
        check(f"{tag} {name} max", to_f64(hi), ref, dtype, group_axis=ch, scale=scale)
        check(f"{tag} {name} min", to_f64(lo), ref, dtype, group_axis=ch, scale=scale)
    check(f"{tag} save_mean", to_f64(sm), rsm, "f32")
    check(f"{tag} save_rstd", to_f64(sr), rsr, "f32")
    check(f"{tag} running_mean", to_f64(rm), rrm, "f32")
    check(f"{tag} running_var", to_f64(rv), rrv_big, "f32")
    # dw and db add `reps` copies of the block's terms, each copy carrying
    # the same per-element rounding, so they are compared per copy.
    check(f"{tag} dw / copies", to_f64(dw) / reps, rdw, dtype)
    check(f"{tag} db / copies", to_f64(db) / reps, rdb, dtype)


@pytest.mark.parametrize("HW", [(1 << 30) - 1024, 1 << 30])
def test_plane_over_2_and_4_gib(orc, HW):
    """One float32 plane of 4 GiB - 4 KiB (buffer stores at offsets past
    2^31) and of 4 GiB (the non-temporal fallback)."""
    print(f"case bn plane f32 1x1x{HW}", flush=True)
    run_replicated(orc, "f32", (1, 1, 1024), HW // 1024, 2, "relu", True)


def two_row_block(C, seed):
    """Rows m_c + s_c and m_c - s_c with the workload recipe's channel mean
    m_c ~ U(-2, 2) and spread s_c ~ U(0.5, 3), float32 [2, C, 1].  Two free
    draws per channel would give some of millions of channels a spread so
    small that no float32 statistics reach the 1e-5 tolerance on y."""
    rng = np.random.default_rng(seed)
    m = rng.uniform(-2.0, 2.0, C)
    sp = rng.uniform(0.5, 3.0, C)
    return np.stack([m + sp, m - sp]).astype(np.float32)[:, :, None]


def test_column_tile_over_2_gib(orc):
    """Column path, float32, 256-row tiles of 2^22 - 16 columns (4 GiB -
    16 KiB: buffer stores at offsets past 2^31)."""
    C = (1 << 22) - 16
    print(f"case bn cols f32 256x{C}", flush=True)
    run_replicated(orc, "f32", (2, C, 1), 128, 0, "gelu", True, x=two_row_block(C, 20251))


@pytest.mark.parametrize("dtype,act,residual", [("f32", "relu", True), ("bf16", "none", False)])
def test_column_tile_fallback(orc, dtype, act, residual):
    """Column path with a nominal row tile of 4 GiB (2^22 columns): the
    non-temporal fallback, checked element by element.  Every channel has
    two elements, so its tolerance floor (2^-12 of the channel's largest
    output) is sound only while one of them is far from zero: float32 runs
    ReLU + residual (every store: y, dres, dx, y_eval); bf16, whose
    tolerance leans on that floor, runs the plain affine output (one element
    near +|w|, the other near -|w|)."""
    C = 1 << 22
    inp = gen_bn(_wl(dtype, act, residual), Nb=2, C=C, HW=1)
    inp["x"] = to_io(two_row_block(C, 20252), dtype)
    print(f"case bn cols fallback {dtype} 2x{C} {act} res={residual}", flush=True)
    run_case(orc, dtype, 2, C, 1, act, residual, inp=inp)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_long_planes(orc, dtype):
    """Planes of 2^21 + 512 elements: past 2^18 vectors for every I/O type,
    so the statistics (and, for 16-bit I/O, the backward reduction) move
    their float32 state into float64 between pieces of the plane; checked
    element by element."""
    HW = (1 << 21) + 512
    print(f"case bn long planes {dtype} 2x3x{HW}", flush=True)
    run_case(orc, dtype, 2, 3, HW, "gelu", True)


@pytest.mark.parametrize("path", ["plane", "cols"])
@pytest.mark.parametrize("act,residual", [("relu", True), ("gelu", False)])
def test_f32_channels_far_from_zero(orc, force_path, path, act, residual):
    """float32 channels whose mean is up to ~50 spreads from zero: the
    recipe's channels moved by a per-channel offset of 10-25 (either sign).
    The statistics fold values relative to a per-tile shift and the
    pre-activation is formed centred, so the 1e-5 tolerance holds.  The
    float32 saved mean, from which the backward recomputes z, bounds the
    range: its rounding moves every z of the channel alike, and with GELU
    db (a sum of n derivatives) reaches the tolerance near |mean| / std ~
    100."""
    force_path(path)
    Nb, C, HW = (4, 8, 3136) if path == "plane" else (256, 64, 1)
    inp = gen_bn(_wl("f32", act, residual), Nb=Nb, C=C, HW=HW)
    rng = np.random.default_rng(777)
    off = rng.uniform(10.0, 25.0, C) * rng.choice([-1.0, 1.0], C)
    inp["x"] = (inp["x"].astype(np.float64) + off[None, :, None]).astype(np.float32)
    print(f"case bn f32 far-from-zero path={path} {Nb}x{C}x{HW} {act} res={residual}", flush=True)
    run_case(orc, "f32", Nb, C, HW, act, residual, inp=inp)
