"""rms_bwd_noalloc (the entry point that allocates nothing; its dw partial
rows live in the library's static per-GPU scratch) against rms_bwd (caller
workspace), through the C ABI: two calls in a row, the second smaller, each
compared with the regular entry point bit for bit and with the float64
oracle at the bf16 tolerance; shapes beyond the scratch are refused."""
import numpy as np
import pytest
import torch

from tests._parity import Guarded, assert_guards, check, to_dev, to_f64

pytestmark = pytest.mark.gpu

nl = pytest.importorskip("normalization_ln_rmsnorm_amd")
from normalization_ln_rmsnorm_amd.workloads import WORKLOADS, gen_rowwise  # noqa: E402

WL = WORKLOADS["rms_bf16_16384x4096"]


def _one(orc, M, N):
    inp = gen_rowwise(WL, M=M, N=N)
    x, dy, w = (to_dev(inp[k], "bf16") for k in ("x", "dy", "w"))
    _, rstd = nl.rms_fwd(x, w, WL.eps)
    dx_ref, dw_ref = nl.rms_bwd(dy, x, w, rstd)
    G = dict(dx=Guarded((M, N), torch.bfloat16), dw=Guarded((N,), torch.bfloat16))
    dx, dw = nl.rms_bwd_noalloc(dy, x, w, rstd, dx=G["dx"].t, dw=G["dw"].t)
    assert_guards(G)
    assert torch.equal(dx.view(torch.int16), dx_ref.view(torch.int16))
    assert torch.equal(dw.view(torch.int16), dw_ref.view(torch.int16))
    rdx, rdw = orc.rms_bwd(inp["dy"], inp["x"], inp["w"], eps=WL.eps, bf16=True)
    g = np.abs(orc.widen(inp["dy"], bf16=True) * orc.widen(inp["w"], bf16=True))
    _, rr = orc.rms_fwd(inp["x"], inp["w"], eps=WL.eps, bf16=True)
    check(f"noalloc {M}x{N} dx", to_f64(dx), rdx, "bf16", group_axis=1,
          scale=rr[:, None] * g.max(axis=1, keepdims=True))
    check(f"noalloc {M}x{N} dw", to_f64(dw), rdw, "bf16")


def test_two_calls_second_smaller(orc):
    """The full RMSNorm workload shape, then a smaller one (fewer partial
    rows and a narrower row): the scratch keeps the first call's contents,
    which the second must not pick up."""
    print("case noalloc 16384x4096 then 3000x1024", flush=True)
    _one(orc, 16384, 4096)
    _one(orc, 3000, 1024)
    torch.cuda.synchronize()


def test_shape_beyond_the_scratch_is_refused():
    """N = 16384 with many rows needs 512 partial rows of 64 KiB: more than
    the scratch; refused before any launch (outputs untouched)."""
    M, N = 8192, 16384
    x = torch.zeros(M, N, dtype=torch.bfloat16, device="cuda")
    rstd = torch.ones(M, device="cuda")
    dx = torch.full_like(x, 7.0)
    dw = torch.full((N,), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(nl.NormError, match="NORM_ERR_WORKSPACE"):
        nl.rms_bwd_noalloc(x, x, None, rstd, dx=dx, dw=dw)
    torch.cuda.synchronize()
    assert bool((dx == 7.0).all()) and bool((dw == 7.0).all())


def test_graph_capture_replays():
    """The callers this entry point is for include stream capture: an RMSNorm
    forward + no-allocation backward recorded in a graph, replayed three
    times with eager work in between (a no-allocation backward of another
    shape, which overwrites the scratch), reproduces the eager outputs bit
    for bit on every replay."""
    print("case noalloc graph capture 2000x2048", flush=True)
    gen = torch.Generator().manual_seed(7)
    bf = torch.bfloat16
    x = torch.randn(2000, 2048, generator=gen).to(bf).cuda()
    dy = torch.randn(2000, 2048, generator=gen).to(bf).cuda()
    w = (1.0 + 0.05 * torch.randn(2048, generator=gen)).to(bf).cuda()
    y, rstd = torch.empty_like(x), torch.empty(2000, device="cuda")
    dx, dw = torch.empty_like(x), torch.empty(2048, dtype=bf, device="cuda")

    def step():
        nl.rms_fwd(x, w, 1e-6, y=y, rstd=rstd)
        nl.rms_bwd_noalloc(dy, x, w, rstd, dx=dx, dw=dw)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (y, rstd, dx, dw)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    xo = torch.randn(700, 512, generator=gen).to(bf).cuda()
    wo = torch.ones(512, dtype=bf, device="cuda")
    dxo, dwo = torch.empty_like(xo), torch.empty_like(wo)
    for replay in range(3):
        for t in (y, rstd, dx, dw):
            t.fill_(float("nan"))
        _, ro = nl.rms_fwd(xo, wo, 1e-6)
        nl.rms_bwd_noalloc(xo, xo, wo, ro, dx=dxo, dw=dwo)  # eager use of the same scratch
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("y", "rstd", "dx", "dw"), (y, rstd, dx, dw), ref):
            assert torch.equal(t.view(torch.uint8), r.view(torch.uint8)), f"replay {replay}: {name}"
