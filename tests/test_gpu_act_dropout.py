"""GPU parity of the fused activation + dropout against the float64 oracle:
the keep mask bit for bit (an integer decision on the generator's words,
taken identically on both sides), y and dx element by element, the edge
probabilities, split calls with offsets, unaligned tensors, and the full
16384 x 4096 bf16 workload."""
import dataclasses

import numpy as np
import pytest
import torch

from tests._parity import TORCH_DTYPE, Guarded, assert_guards, check, to_dev, to_f64, to_io

pytestmark = pytest.mark.gpu

nl = pytest.importorskip("normalization_ln_rmsnorm_amd")
from normalization_ln_rmsnorm_amd.workloads import EXTRA_WORKLOADS, gen_act_dropout  # noqa: E402

WL = EXTRA_WORKLOADS["actdrop_bf16_16384x4096"]


def _inputs(dtype, n, seed):
    return gen_act_dropout(dataclasses.replace(WL, dtype=dtype), n=n, seed=seed)


def run_case(orc, dtype, n, act, p, seed, offset, param=0.0, x_dev=None, misalign=0):
    """Outputs sit between guard bands; misalign=1 places them off 16-byte
    alignment."""
    inp = _inputs(dtype, n, seed=(seed ^ n) & 0xFFFF)
    bf16 = dtype == "bf16"
    x = to_dev(inp["x"], dtype) if x_dev is None else x_dev(inp["x"])
    dy = to_dev(inp["dy"], dtype)
    p32 = float(np.float32(p))  # the kernels see p as float32
    tdt = TORCH_DTYPE[dtype]
    G = {k: Guarded((n,), tdt, misalign=misalign) for k in ("y", "ynone", "dx")}
    y = nl.act_dropout_fwd(x, act, p, seed, offset, act_param=param, y=G["y"].t)
    ynone = nl.act_dropout_fwd(x, "none", p, seed, offset, y=G["ynone"].t)
    dx = nl.act_dropout_bwd(dy, x, act, p, seed, offset, act_param=param, dx=G["dx"].t)
    assert_guards(G)
    keep = orc.dropout_keep(n, p32, seed, offset)
    # x has no exact zeros, so the identity activation exposes the mask.
    assert (orc.widen(inp["x"], bf16=bf16) != 0).all()
    got_keep = (to_f64(ynone) != 0).astype(np.uint8)
    mism = np.flatnonzero(got_keep != keep)
    assert mism.size == 0, f"mask differs at {mism[:8]} (of {mism.size})"
    tag = f"ad/{dtype}/n={n}/{act}({param})/p={p}/seed={seed}/off={offset}"
    ry = orc.act_dropout_fwd(inp["x"], act, p32, seed, offset, act_param=param, bf16=bf16)
    rdx = orc.act_dropout_bwd(inp["dy"], inp["x"], act, p32, seed, offset, act_param=param, bf16=bf16)
    check(f"{tag} y", to_f64(y), ry, dtype)
    check(f"{tag} dx", to_f64(dx), rdx, dtype)
    return y, dx


ACTS = [("none", 0.0), ("relu", 0.0), ("gelu", 0.0), ("silu", 0.0), ("leaky_relu", 0.2),
        ("hardswish", 0.0), ("tanh", 0.0)]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("act,param", ACTS)
@pytest.mark.parametrize("n", [1, 3, 8, 1000, 4099, (1 << 16) + 5])
def test_parity(orc, dtype, act, param, n):
    print(f"case act_dropout {dtype} {act} n={n}", flush=True)
    run_case(orc, dtype, n, act, 0.1, seed=0x1234_5678_9ABC, offset=0, param=param)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("p", [0.0, 0.5, 0.9, 1.0])
@pytest.mark.parametrize("offset", [0, 8, 1 << 34])
def test_probabilities_and_offsets(orc, dtype, p, offset):
    print(f"case act_dropout {dtype} p={p} offset={offset}", flush=True)
    if p in (0.0, 1.0):
        # p = 0 keeps everything (the plain activation); p = 1 drops all.
        n = 5000
        inp = _inputs(dtype, n, 1)
        x = to_dev(inp["x"], dtype)
        y = nl.act_dropout_fwd(x, "gelu", p, 77, offset)
        torch.cuda.synchronize()
        ref = orc.act("gelu", orc.widen(inp["x"], bf16=dtype == "bf16")) if p == 0.0 else np.zeros(n)
        check(f"p={p} y", to_f64(y), ref, dtype)
        return
    run_case(orc, dtype, 20000, "gelu", p, seed=(1 << 40) + 3, offset=offset)


def test_split_calls_reproduce_the_whole(orc):
    """Two calls with offsets give the mask and values of one call."""
    n, n1 = 10000, 4096
    x = to_dev(_inputs("f32", n, 9)["x"], "f32")
    whole = nl.act_dropout_fwd(x, "silu", 0.3, 42, 0)
    a = nl.act_dropout_fwd(x[:n1].contiguous(), "silu", 0.3, 42, 0)
    b = nl.act_dropout_fwd(x[n1:].contiguous(), "silu", 0.3, 42, n1)
    torch.cuda.synchronize()
    assert torch.equal(whole, torch.cat([a, b]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unaligned_tensors_take_the_scalar_path(orc, dtype):
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]

    def shifted(a):
        t = to_dev(a, dtype)
        big = torch.empty(t.numel() + 1, dtype=tdt, device="cuda")
        big[1:].copy_(t)
        return big[1:]
    run_case(orc, dtype, 3001, "gelu", 0.25, seed=5, offset=8, x_dev=shifted, misalign=1)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("n", [1, 5, 4097, 100003])
def test_unaligned_outputs(orc, dtype, n):
    """Aligned input, outputs one element off 16-byte alignment (the scalar
    path), with guard bands."""
    print(f"case act_dropout unaligned outputs {dtype} n={n}", flush=True)
    run_case(orc, dtype, n, "silu", 0.2, seed=11, offset=24, misalign=1)


def test_full_size_workload(orc):
    M, N = WL.shape
    print("case actdrop_bf16_16384x4096", flush=True)
    inp = gen_act_dropout(WL)
    x, dy = to_dev(inp["x"], "bf16"), to_dev(inp["dy"], "bf16")
    p, seed = WL.extra["drop_p"], WL.extra["dropout_seed"]
    G = {k: Guarded((M * N,), torch.bfloat16) for k in ("y", "dx")}
    y = nl.act_dropout_fwd(x, WL.act, p, seed, 0, y=G["y"].t)
    dx = nl.act_dropout_bwd(dy, x, WL.act, p, seed, 0, dx=G["dx"].t)
    assert_guards(G)
    p32 = float(np.float32(p))
    ry = orc.act_dropout_fwd(inp["x"], WL.act, p32, seed, 0, bf16=True)
    check("full y", to_f64(y), ry, "bf16")
    del ry
    rdx = orc.act_dropout_bwd(inp["dy"], inp["x"], WL.act, p32, seed, 0, bf16=True)
    check("full dx", to_f64(dx), rdx, "bf16")
    keep = orc.dropout_keep(M * N, p32, seed, 0)
    # GELU(x) = 0 only at x = 0 (the draw holds a few exact zeros): dropped
    # elements are 0 and, wherever x != 0, kept ones are not.
    yv = to_f64(y)
    nz = orc.widen(inp["x"], bf16=True) != 0
    assert (yv[keep == 0] == 0).all()
    assert np.array_equal((yv[nz] != 0).astype(np.uint8), keep[nz])


TAIL_ACTS = [("gelu", 0.0), ("silu", 0.0), ("sigmoid", 0.0), ("tanh", 0.0), ("mish", 0.0),
             ("softplus", 0.0), ("elu", 1.0), ("selu", 0.0), ("celu", 1.3)]


def _grid(dtype, n=65536 + 5, lim=12.0):
    return to_io(np.linspace(-lim, lim, n, dtype=np.float32), dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("act,param", TAIL_ACTS)
def test_activation_over_both_tails(orc, dtype, act, param):
    """p = 0 (no dropout): the activation and its derivative on a dense grid
    over [-12, 12] -- far into both tails, where the 16-bit forms differ most
    from the exact ones -- element by element against the oracle (the
    pre-activation is x itself, so the kinks of elu / selu at 0 are decided
    on the same value on both sides)."""
    print(f"case tails {dtype} {act}", flush=True)
    bf16 = dtype == "bf16"
    xs = _grid(dtype)
    ones = to_io(np.ones(xs.shape[0], dtype=np.float32), dtype)
    x, dy = to_dev(xs, dtype), to_dev(ones, dtype)
    y = nl.act_dropout_fwd(x, act, 0.0, 5, 0, act_param=param)
    dx = nl.act_dropout_bwd(dy, x, act, 0.0, 5, 0, act_param=param)
    torch.cuda.synchronize()
    check(f"tails {dtype} {act} y", to_f64(y), orc.act_dropout_fwd(xs, act, 0.0, 5, 0, act_param=param, bf16=bf16),
          dtype)
    check(f"tails {dtype} {act} dx", to_f64(dx),
          orc.act_dropout_bwd(ones, xs, act, 0.0, 5, 0, act_param=param, bf16=bf16), dtype)


def test_fp16_gelu_forward_tail_is_relatively_accurate(orc):
    """The fp16 GELU forward keeps a small relative error in its negative
    tail (results down to fp16's subnormals): checked with the tolerance floor
    taken over each run of 64 neighbouring grid points, so every value is
    held to about 2 ulp of its own magnitude."""
    xs = _grid("f16", n=64 * 2048)
    y = nl.act_dropout_fwd(to_dev(xs, "f16"), "gelu", 0.0, 5, 0)
    torch.cuda.synchronize()
    ref = orc.act_dropout_fwd(xs, "gelu", 0.0, 5, 0)
    check("fp16 gelu tail y", to_f64(y).reshape(-1, 64), ref.reshape(-1, 64), "f16", group_axis=1)


def test_past_2_32_elements(orc):
    """bf16, 2^32 + 2^20 + 3 elements (8 GiB per tensor, a ragged scalar
    tail): the element index, the generator counter and the output offsets
    beyond 32 bits.  The input repeats a 2^20-element block; slices around
    2^31, 2^32 and the end are checked against the oracle with the offset of
    their first element (the mask depends on seed and offset + index only)."""
    B, L = 1 << 20, 8192
    n = (1 << 32) + B + 3
    reps = (n - 3) // B
    seed, off0, p = 0x5EED, 12344, 0.1  # offsets are multiples of 8
    inp = _inputs("bf16", B, seed=7)
    xb, dyb = to_dev(inp["x"], "bf16"), to_dev(inp["dy"], "bf16")
    x = torch.cat([xb.repeat(reps), xb[:3]])
    dy = torch.cat([dyb.repeat(reps), dyb[:3]])
    assert x.numel() == n
    print(f"case act_dropout bf16 n={n}", flush=True)
    y = nl.act_dropout_fwd(x, "gelu", p, seed, off0)
    dx = nl.act_dropout_bwd(dy, x, "gelu", p, seed, off0)
    torch.cuda.synchronize()
    del x, dy
    p32 = float(np.float32(p))
    xs_all = np.concatenate([inp["x"], inp["x"]])
    dys_all = np.concatenate([inp["dy"], inp["dy"]])
    for s, ln in ((0, L), ((1 << 31) - L // 2, L), ((1 << 32) - L // 2, L), (n - L - 3, L + 3)):
        k = s % B
        xs, dys = xs_all[k:k + ln], dys_all[k:k + ln]
        ry = orc.act_dropout_fwd(xs, "gelu", p32, seed, off0 + s, bf16=True)
        rdx = orc.act_dropout_bwd(dys, xs, "gelu", p32, seed, off0 + s, bf16=True)
        check(f"ad/bf16/n={n}/slice@{s} y", to_f64(y[s:s + ln]), ry, "bf16")
        check(f"ad/bf16/n={n}/slice@{s} dx", to_f64(dx[s:s + ln]), rdx, "bf16")
