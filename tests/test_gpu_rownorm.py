"""GPU parity: LayerNorm / RMSNorm forward and backward through the C ABI
against the float64 oracle, element by element.

Shapes span every tiling the planner picks (thread groups of 1..1024 lanes,
vector and scalar paths, ragged tails) plus the four row-wise workloads at
full size, launched exactly as the benchmark launches them.
"""
import dataclasses

import numpy as np
import pytest
import torch

from tests._parity import TORCH_DTYPE, Guarded, assert_guards, check, to_dev, to_f64

pytestmark = pytest.mark.gpu

nl = pytest.importorskip("normalization_ln_rmsnorm_amd")
from normalization_ln_rmsnorm_amd.workloads import WORKLOADS, gen_rowwise  # noqa: E402

def _wl(kind, dtype):
    """The workload whose value recipe a small case borrows."""
    if kind == "rms":
        return dataclasses.replace(WORKLOADS["rms_bf16_16384x4096"], dtype=dtype)
    if dtype == "f32":
        return WORKLOADS["ln_f32_64x256"]
    return dataclasses.replace(WORKLOADS["ln_bf16_25216x768"], dtype=dtype)


def run_case(orc, kind, dtype, M, N, with_w=True, with_b=True, eps=None, seed=None, guard=True,
             report=None, inp=None):
    wl = _wl(kind, dtype)
    eps = wl.eps if eps is None else eps
    if inp is None:
        inp = gen_rowwise(wl, M=M, N=N, seed=seed)
    bf16 = dtype == "bf16"
    tdt = TORCH_DTYPE[dtype]
    x = to_dev(inp["x"], dtype)
    dy = to_dev(inp["dy"], dtype)
    w = to_dev(inp["w"], dtype) if with_w else None
    b = to_dev(inp["b"], dtype) if (with_b and kind == "ln") else None
    w_np = inp["w"] if with_w else None
    b_np = inp["b"] if (with_b and kind == "ln") else None

    # Every output between guard bands (y, dx, the statistics, dw / db and
    # the workspace).
    ln = kind == "ln"
    if guard:
        wsn = (nl.ln_bwd_workspace_bytes if ln else nl.rms_bwd_workspace_bytes)(tdt, M, N)
        G = dict(y=Guarded((M, N), tdt), dx=Guarded((M, N), tdt), rstd=Guarded((M,), torch.float32),
                 mean=Guarded((M,), torch.float32) if ln else None,
                 dw=Guarded((N,), tdt) if with_w else None,
                 db=Guarded((N,), tdt) if (ln and with_b) else None,
                 ws=Guarded((max(1, wsn),), torch.uint8))
        t = {k: (g.t if g is not None else None) for k, g in G.items()}
    else:
        G, t = {}, dict(y=None, dx=None, rstd=None, mean=None, dw=None, db=None, ws=None)
    if ln:
        y, mean, rstd = nl.ln_fwd(x, w, b, eps, y=t["y"], mean=t["mean"], rstd=t["rstd"])
        dx, dw, db = nl.ln_bwd(dy, x, w, mean, rstd, dx=t["dx"], want_dw=with_w, want_db=with_b,
                               dw=t["dw"], db=t["db"], ws=t["ws"])
        ry, rmean, rrstd = orc.ln_fwd(inp["x"], w_np, b_np, eps=eps, bf16=bf16)
        rdx, rdw, rdb = orc.ln_bwd(inp["dy"], inp["x"], w_np, eps=eps, bf16=bf16)
    else:
        y, rstd = nl.rms_fwd(x, w, eps, y=t["y"], rstd=t["rstd"])
        dx, dw = nl.rms_bwd(dy, x, w, rstd, dx=t["dx"], want_dw=with_w, dw=t["dw"], ws=t["ws"])
        db = None
        ry, rrstd = orc.rms_fwd(inp["x"], w_np, eps=eps, bf16=bf16)
        rdx, rdw = orc.rms_bwd(inp["dy"], inp["x"], w_np, eps=eps, bf16=bf16)
    torch.cuda.synchronize()
    if guard:
        assert_guards(G)
    tag = f"{kind}/{dtype}/{M}x{N}"
    check(f"{tag} y", to_f64(y), ry, dtype, group_axis=1, report=report)
    check(f"{tag} rstd", to_f64(rstd), rrstd, "f32", report=report)
    if kind == "ln":
        check(f"{tag} mean", to_f64(mean), rmean, "f32", report=report)
    # Scale of the terms dx is formed from: rstd * |dy * w| per row.
    g = np.abs(orc.widen(inp["dy"], bf16=bf16) * (orc.widen(w_np, bf16=bf16) if with_w else 1.0))
    dx_scale = rrstd[:, None] * g.max(axis=1, keepdims=True)
    check(f"{tag} dx", to_f64(dx), rdx, dtype, group_axis=1, report=report, scale=dx_scale)
    if with_w:
        check(f"{tag} dw", to_f64(dw), rdw, dtype, report=report)
    if kind == "ln" and with_b:
        check(f"{tag} db", to_f64(db), rdb, dtype, report=report)
    return dict(x=x, dy=dy, w=w, b=b, mean=mean if kind == "ln" else None, rstd=rstd, dx=dx, dw=dw, db=db)


SHAPES = [(1, 1), (3, 7), (64, 256), (37, 768), (33, 1000), (5, 1024), (130, 96), (300, 520),
          (17, 4096), (3, 16384), (9, 3000), (2, 24)]


@pytest.mark.parametrize("kind", ["ln", "rms"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,N", SHAPES)
def test_small_shapes(orc, kind, dtype, M, N):
    print(f"case {kind} {dtype} {M}x{N}", flush=True)
    run_case(orc, kind, dtype, M, N)


@pytest.mark.parametrize("kind", ["ln", "rms"])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_widest_rows(orc, kind, dtype):
    N = 32768 if dtype == "f32" else 65536
    print(f"case {kind} {dtype} 3x{N}", flush=True)
    run_case(orc, kind, dtype, 3, N)


@pytest.mark.parametrize("kind", ["ln", "rms"])
@pytest.mark.parametrize("with_w,with_b", [(False, False), (True, False), (False, True)])
def test_optional_params(orc, kind, with_w, with_b):
    print(f"case {kind} w={with_w} b={with_b}", flush=True)
    run_case(orc, kind, "bf16", 19, 768, with_w=with_w, with_b=with_b)


@pytest.mark.parametrize("kind", ["ln", "rms"])
def test_unaligned_scalar_path(orc, kind):
    """Tensors that are not 16-byte aligned take the scalar path."""
    M, N = 11, 96
    wl = _wl(kind, "f32")
    inp = gen_rowwise(wl, M=M, N=N)
    big = torch.empty(M * N + 1, dtype=torch.float32, device="cuda")
    x = big[1:].view(M, N)
    x.copy_(to_dev(inp["x"], "f32"))
    w = to_dev(inp["w"], "f32")
    if kind == "ln":
        y, mean, rstd = nl.ln_fwd(x, w, to_dev(inp["b"], "f32"), wl.eps)
        ry, _, _ = orc.ln_fwd(inp["x"], inp["w"], inp["b"], eps=wl.eps)
    else:
        y, rstd = nl.rms_fwd(x, w, wl.eps)
        ry, _ = orc.rms_fwd(inp["x"], inp["w"], eps=wl.eps)
    check(f"{kind} unaligned y", to_f64(y), ry, "f32")


@pytest.mark.parametrize("kind", ["ln", "rms"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,ws_shift", [(1100, 130, 0), (2000, 256, 4), (777, 1003, 8), (600, 4096, 4),
                                           (600, 8192, 0), (300, 8193, 0), (1000, 2048, 0)])
def test_column_sum_paths(orc, kind, dtype, M, N, ws_shift):
    """dw / db through the column-sum kernel: many partial rows, widths that
    are not a multiple of 4 (scalar columns), workspaces that are not 16-byte
    aligned (scalar loads), and rows wide enough that a block holds a single
    row slot (its partial row stored straight from registers: 16 bytes at a
    time, or one float at a time on the scalar path of an odd width), and a
    bf16 LayerNorm width whose dW and dB staging fills 64 KiB of LDS,
    checked against the oracle."""
    print(f"case colsum {kind} {dtype} {M}x{N} ws+{ws_shift}", flush=True)
    wl = _wl(kind, dtype)
    inp = gen_rowwise(wl, M=M, N=N)
    bf16 = dtype == "bf16"
    x, dy, w = (to_dev(inp[k], dtype) for k in ("x", "dy", "w"))
    need = (nl.ln_bwd_workspace_bytes if kind == "ln" else nl.rms_bwd_workspace_bytes)(x.dtype, M, N)
    big = torch.empty(need + 16, dtype=torch.uint8, device="cuda")
    ws = big[ws_shift:ws_shift + need]
    if kind == "ln":
        b = to_dev(inp["b"], dtype)
        _, mean, rstd = nl.ln_fwd(x, w, b, wl.eps)
        _, dw, db = nl.ln_bwd(dy, x, w, mean, rstd, ws=ws)
        _, rdw, rdb = orc.ln_bwd(inp["dy"], inp["x"], inp["w"], eps=wl.eps, bf16=bf16)
        check(f"colsum {kind} db", to_f64(db), rdb, dtype)
    else:
        _, rstd = nl.rms_fwd(x, w, wl.eps)
        _, dw = nl.rms_bwd(dy, x, w, rstd, ws=ws)
        _, rdw = orc.rms_bwd(inp["dy"], inp["x"], inp["w"], eps=wl.eps, bf16=bf16)
    check(f"colsum {kind} dw", to_f64(dw), rdw, dtype)


@pytest.mark.parametrize("name", ["ln_f32_64x256", "rms_bf16_16384x4096", "ln_bf16_25216x768",
                                  "ln_bf16_4096x1000"])
def test_full_size_workloads(orc, name):
    """The workloads at the sizes and launch configuration the benchmark uses."""
    wl = WORKLOADS[name]
    M, N = wl.shape
    print(f"case {name}", flush=True)
    report = []
    run_case(orc, wl.kind, wl.dtype, M, N, guard=True, report=report)
    for r in report:
        print(r, flush=True)


@pytest.mark.parametrize("kind,shape", [("rms", (16384, 4096)), ("ln", (25216, 768))])
def test_full_size_f16(orc, kind, shape):
    """The two large row-wise workloads with fp16 I/O (same recipe)."""
    print(f"case {kind} f16 {shape}", flush=True)
    report = []
    run_case(orc, kind, "f16", *shape, guard=True, report=report)
    for r in report:
        print(r, flush=True)


@pytest.mark.parametrize("kind", ["ln", "rms"])
def test_backward_bitwise_deterministic(orc, kind):
    M, N = 2048, 4096
    wl = _wl(kind, "bf16")
    inp = gen_rowwise(wl, M=M, N=N)
    x, dy, w = (to_dev(inp[k], "bf16") for k in ("x", "dy", "w"))
    outs = []
    for _ in range(2):
        if kind == "ln":
            b = to_dev(inp["b"], "bf16")
            _, mean, rstd = nl.ln_fwd(x, w, b, wl.eps)
            outs.append(nl.ln_bwd(dy, x, w, mean, rstd))
        else:
            _, rstd = nl.rms_fwd(x, w, wl.eps)
            outs.append(nl.rms_bwd(dy, x, w, rstd))
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        if a is not None:
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_empty_batch_is_noop(orc):
    x = torch.empty(0, 64, device="cuda")
    y, mean, rstd = nl.ln_fwd(x, None, None, 1e-5)
    assert y.shape == (0, 64)
    dx, dw, db = nl.ln_bwd(x, x, torch.ones(64, device="cuda"), mean, rstd)
    torch.cuda.synchronize()
    assert torch.all(dw == 0) and torch.all(db == 0)


@pytest.mark.parametrize("kind", ["ln", "rms"])
@pytest.mark.parametrize("dtype,M,N", [("f32", 5000003, 4), ("bf16", 5000003, 8)])
def test_persistent_forward_grid(orc, kind, dtype, M, N):
    """Narrow rows in so many row groups that the forward grid is capped and
    each block loops over several groups with the next one's loads issued
    ahead (the other shapes here give every block one group); a row count
    that leaves the last group partly filled."""
    print(f"case {kind} {dtype} {M}x{N} (persistent forward)", flush=True)
    run_case(orc, kind, dtype, M, N)


@pytest.mark.parametrize("kind", ["ln", "rms"])
def test_rows_past_2_32_elements(orc, kind):
    """bf16, 63 x 16646 = 1048698 rows x 4096 (past 2^32 elements, 8 GiB per
    tensor): every element index of the row path beyond 32 bits.  Rows are
    independent, so a 63-row block repeated down the rows has the oracle's
    block outputs in every copy; each output is checked through its maximum
    and minimum over the copies (both within tolerance bound every copy),
    and dw / db, which add the copies, per copy.  The period is odd on
    purpose: with a power-of-two period dividing the persistent grid's row
    step, every block would add the same two rows thousands of times and
    its float32 partial of dw would repeat one rounding coherently (a
    property of that adversarial input, not of the index arithmetic under
    test); an odd period gives every block varied rows, as data does."""
    dtype, N, B, reps = "bf16", 4096, 63, 16646
    wl = _wl(kind, dtype)
    inp = gen_rowwise(wl, M=B, N=N)
    x = to_dev(inp["x"], dtype).repeat(reps, 1)
    dy = to_dev(inp["dy"], dtype).repeat(reps, 1)
    w = to_dev(inp["w"], dtype)
    print(f"case {kind} bf16 {B * reps}x{N}", flush=True)
    if kind == "ln":
        b = to_dev(inp["b"], dtype)
        y, mean, rstd = nl.ln_fwd(x, w, b, wl.eps)
        dx, dw, db = nl.ln_bwd(dy, x, w, mean, rstd)
        ry, rmean, rrstd = orc.ln_fwd(inp["x"], inp["w"], inp["b"], eps=wl.eps, bf16=True)
        rdx, rdw, rdb = orc.ln_bwd(inp["dy"], inp["x"], inp["w"], eps=wl.eps, bf16=True)
    else:
        y, rstd = nl.rms_fwd(x, w, wl.eps)
        dx, dw = nl.rms_bwd(dy, x, w, rstd)
        mean = db = None
        ry, rrstd = orc.rms_fwd(inp["x"], inp["w"], eps=wl.eps, bf16=True)
        rdx, rdw = orc.rms_bwd(inp["dy"], inp["x"], inp["w"], eps=wl.eps, bf16=True)
    torch.cuda.synchronize()
    del x, dy

    def folds(t):
        v = t.view(reps, B, -1)
        return v.amax(0), v.amin(0)

    g = np.abs(orc.widen(inp["dy"], bf16=True) * orc.widen(inp["w"], bf16=True))
    dx_scale = rrstd[:, None] * g.max(axis=1, keepdims=True)
    tag = f"{kind}/bf16/{B}x{reps}x{N}"
    for name, t, ref, dt, scale in (("y", y, ry, dtype, None), ("dx", dx, rdx, dtype, dx_scale),
                                    ("rstd", rstd, rrstd[:, None], "f32", None)) + (
            (("mean", mean, rmean[:, None], "f32", None),) if kind == "ln" else ()):
        hi, lo = folds(t)
        for side, v in (("max", hi), ("min", lo)):
            check(f"{tag} {name} {side}", to_f64(v), ref, dt, group_axis=1 if dt != "f32" else None,
                  scale=scale)
    check(f"{tag} dw / copies", to_f64(dw) / reps, rdw, dtype)
    if kind == "ln":
        check(f"{tag} db / copies", to_f64(db) / reps, rdb, dtype)


@pytest.mark.parametrize("M,N", [(64, 256), (37, 768), (17, 4096)])
def test_f32_rows_far_from_zero(orc, M, N):
    """float32 LayerNorm rows moved by a per-row offset of 50-100 (either
    sign; the recipe's rows have spread ~1).  The row is summed relative to
    its first element, then centred exactly in registers, so the 1e-5
    tolerance holds; the float32 saved mean, from which the backward forms
    xhat, bounds the range near |mean| / std ~ 300."""
    wl = _wl("ln", "f32")
    inp = gen_rowwise(wl, M=M, N=N)
    rng = np.random.default_rng(4242)
    off = rng.uniform(50.0, 100.0, M) * rng.choice([-1.0, 1.0], M)
    inp["x"] = (inp["x"].astype(np.float64) + off[:, None]).astype(np.float32)
    print(f"case ln f32 far-from-zero {M}x{N}", flush=True)
    run_case(orc, "ln", "f32", M, N, inp=inp)


@pytest.mark.parametrize("kind", ["ln", "rms"])
def test_workspace_reused_across_shapes(orc, kind):
    """One workspace through backward calls of alternating shapes and data:
    every call's dw / db must come from its own partial rows, never from
    rows an earlier call left in the workspace (or in a cache)."""
    dtype, N = "bf16", 4096
    wl = _wl(kind, dtype)
    need = (nl.ln_bwd_workspace_bytes if kind == "ln" else nl.rms_bwd_workspace_bytes)(
        torch.bfloat16, 8192, N)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    cases = [(8192, 11), (2048, 12), (6000, 13), (2048, 14), (8192, 15), (777, 16)]
    print(f"case {kind} ws reuse {cases}", flush=True)
    for M, seed in cases:
        inp = gen_rowwise(wl, M=M, N=N, seed=seed)
        x, dy, w = (to_dev(inp[k], dtype) for k in ("x", "dy", "w"))
        if kind == "ln":
            b = to_dev(inp["b"], dtype)
            _, mean, rstd = nl.ln_fwd(x, w, b, wl.eps)
            _, dw, db = nl.ln_bwd(dy, x, w, mean, rstd, ws=ws)
            _, rdw, rdb = orc.ln_bwd(inp["dy"], inp["x"], inp["w"], eps=wl.eps, bf16=True)
            check(f"{kind} reuse {M} db", to_f64(db), rdb, dtype)
        else:
            _, rstd = nl.rms_fwd(x, w, wl.eps)
            _, dw = nl.rms_bwd(dy, x, w, rstd, ws=ws)
            _, rdw = orc.rms_bwd(inp["dy"], inp["x"], inp["w"], eps=wl.eps, bf16=True)
        check(f"{kind} reuse {M} dw", to_f64(dw), rdw, dtype)
