"""Stream capture: every entry point enqueues only kernels on the caller's
stream (no allocation, no memset, no synchronization), so a torch / HIP graph
can record a whole forward + backward sequence.  The graph is replayed
several times, with eager work and synchronizations in between, and every
replay must reproduce the eager results bit for bit (all kernels reduce in a
fixed order).  Covers the row kernels with and without the column-sum
kernel, the empty-batch gradient fill, both BatchNorm paths with and without
a residual, the eval forward and the fused activation + dropout."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

nl = pytest.importorskip("normalization_ln_rmsnorm_amd")


def _rand(shape, dtype, gen, scale=1.0, shift=0.0):
    t = torch.randn(*shape, generator=gen, dtype=torch.float32) * scale + shift
    return t.to(dtype).cuda()


class Sequence:
    """Inputs, preallocated outputs and workspaces, and one step that runs
    every operation into them."""

    def __init__(self):
        g = torch.Generator().manual_seed(20240611)
        bf, f32 = torch.bfloat16, torch.float32
        e = lambda *s, dt=bf: torch.empty(*s, dtype=dt, device="cuda")
        ws = lambda n: torch.empty(max(1, n), dtype=torch.uint8, device="cuda")
        self.out = {}
        # LayerNorm, bf16, 300 x 768: many row groups -> column-sum kernel.
        self.ln = dict(x=_rand((300, 768), bf, g, 2.0, 0.5), dy=_rand((300, 768), bf, g),
                       w=_rand((768,), bf, g, 0.1, 1.0), b=_rand((768,), bf, g, 0.1))
        self.ln_ws = ws(nl.ln_bwd_workspace_bytes(bf, 300, 768))
        # LayerNorm, fp32, 5 x 256: one block writes dw / db directly.
        self.ln2 = dict(x=_rand((5, 256), f32, g), dy=_rand((5, 256), f32, g),
                        w=_rand((256,), f32, g, 0.1, 1.0), b=_rand((256,), f32, g, 0.1))
        self.ln2_ws = ws(nl.ln_bwd_workspace_bytes(f32, 5, 256))
        # LayerNorm backward of an empty batch: dw, db are zero-filled.
        self.ln0 = dict(x=e(0, 64), dy=e(0, 64), w=_rand((64,), bf, g, 0.1, 1.0))
        # RMSNorm, bf16, 1000 x 1024.
        self.rms = dict(x=_rand((1000, 1024), bf, g), dy=_rand((1000, 1024), bf, g),
                        w=_rand((1024,), bf, g, 0.05, 1.0))
        self.rms_ws = ws(nl.rms_bwd_workspace_bytes(bf, 1000, 1024))
        # BatchNorm2d bf16 plane path with GELU; BatchNorm1d fp32 column
        # path with a residual and ReLU.
        self.bn = dict(x=_rand((4, 8, 32, 32), bf, g, 2.0, 0.3), dy=_rand((4, 8, 32, 32), bf, g),
                       w=_rand((8,), bf, g, 0.1, 1.0), b=_rand((8,), bf, g, 0.1), res=None,
                       act="gelu")
        self.bn1 = dict(x=_rand((64, 32, 3), f32, g, 1.5, -0.2), dy=_rand((64, 32, 3), f32, g),
                        w=_rand((32,), f32, g, 0.1, 1.0), b=_rand((32,), f32, g, 0.1),
                        res=_rand((64, 32, 3), f32, g), act="relu")
        for d in (self.bn, self.bn1):
            x = d["x"]
            Nb, C = x.shape[0], x.shape[1]
            HW = x.numel() // (Nb * C)
            d["ws"] = ws(nl.bn_workspace_bytes(x.dtype, Nb, C, HW))
            d["rm0"] = torch.zeros(C, dtype=f32, device="cuda")
            d["rv0"] = torch.ones(C, dtype=f32, device="cuda")
            d["rm"], d["rv"] = d["rm0"].clone(), d["rv0"].clone()
        # Activation + dropout, bf16, GELU, p = 0.1.
        self.ad = dict(x=_rand((100003,), bf, g), dy=_rand((100003,), bf, g))
        self._alloc_outputs()

    def _alloc_outputs(self):
        o, L, L2, R = self.out, self.ln, self.ln2, self.rms
        for k, (d, f32) in {"ln": (L, False), "ln2": (L2, True)}.items():
            M, N = d["x"].shape
            o[k + ".y"] = torch.empty_like(d["x"])
            o[k + ".mean"] = torch.empty(M, device="cuda")
            o[k + ".rstd"] = torch.empty(M, device="cuda")
            o[k + ".dx"] = torch.empty_like(d["x"])
            o[k + ".dw"] = torch.empty(N, dtype=d["x"].dtype, device="cuda")
            o[k + ".db"] = torch.empty(N, dtype=d["x"].dtype, device="cuda")
        o["ln0.dx"] = torch.empty_like(self.ln0["x"])
        o["ln0.dw"] = torch.empty(64, dtype=torch.bfloat16, device="cuda")
        o["ln0.db"] = torch.empty(64, dtype=torch.bfloat16, device="cuda")
        o["rms.y"] = torch.empty_like(R["x"])
        o["rms.rstd"] = torch.empty(R["x"].shape[0], device="cuda")
        o["rms.dx"] = torch.empty_like(R["x"])
        o["rms.dw"] = torch.empty(R["x"].shape[1], dtype=R["x"].dtype, device="cuda")
        for k, d in (("bn", self.bn), ("bn1", self.bn1)):
            C = d["x"].shape[1]
            for n in ("y", "dx", "ye"):
                o[f"{k}.{n}"] = torch.empty_like(d["x"])
            o[f"{k}.dres"] = torch.empty_like(d["x"]) if d["res"] is not None else None
            for n in ("dw", "db"):
                o[f"{k}.{n}"] = torch.empty(C, dtype=d["x"].dtype, device="cuda")
            for n in ("sm", "sr"):
                o[f"{k}.{n}"] = torch.empty(C, device="cuda")
            o[f"{k}.rm"], o[f"{k}.rv"] = d["rm"], d["rv"]
        o["ad.y"] = torch.empty_like(self.ad["x"])
        o["ad.dx"] = torch.empty_like(self.ad["x"])

    def reset_running_stats(self):
        for d in (self.bn, self.bn1):
            d["rm"].copy_(d["rm0"])
            d["rv"].copy_(d["rv0"])

    def poison_outputs(self):
        for k, t in self.out.items():
            if t is not None and t.numel() and k not in ("bn.rm", "bn.rv", "bn1.rm", "bn1.rv"):
                t.fill_(float("nan"))

    def step(self):
        o = self.out
        for k, d, ws in (("ln", self.ln, self.ln_ws), ("ln2", self.ln2, self.ln2_ws)):
            nl.ln_fwd(d["x"], d["w"], d["b"], 1e-5, y=o[k + ".y"], mean=o[k + ".mean"], rstd=o[k + ".rstd"])
            nl.ln_bwd(d["dy"], d["x"], d["w"], o[k + ".mean"], o[k + ".rstd"], dx=o[k + ".dx"],
                      dw=o[k + ".dw"], db=o[k + ".db"], ws=ws)
        z = self.ln0
        empty = torch.empty(0, device="cuda")
        nl.ln_bwd(z["dy"], z["x"], z["w"], empty, empty, dx=o["ln0.dx"], dw=o["ln0.dw"], db=o["ln0.db"],
                  ws=self.ln_ws)
        R = self.rms
        nl.rms_fwd(R["x"], R["w"], 1e-6, y=o["rms.y"], rstd=o["rms.rstd"])
        nl.rms_bwd(R["dy"], R["x"], R["w"], o["rms.rstd"], dx=o["rms.dx"], dw=o["rms.dw"], ws=self.rms_ws)
        for k, d in (("bn", self.bn), ("bn1", self.bn1)):
            nl.bn_fwd_train(d["x"], d["w"], d["b"], d["rm"], d["rv"], 1e-5, 0.1, d["act"], d["res"],
                            y=o[k + ".y"], save_mean=o[k + ".sm"], save_rstd=o[k + ".sr"], ws=d["ws"])
            nl.bn_bwd(d["dy"], d["x"], d["w"], d["b"], o[k + ".sm"], o[k + ".sr"], d["act"], d["res"],
                      dx=o[k + ".dx"], dres=o[k + ".dres"], dw=o[k + ".dw"], db=o[k + ".db"], ws=d["ws"])
            nl.bn_fwd_eval(d["x"], d["w"], d["b"], d["rm"], d["rv"], 1e-5, d["act"], d["res"],
                           y=o[k + ".ye"])
        A = self.ad
        nl.act_dropout_fwd(A["x"], "gelu", 0.1, 0xC0FFEE, 8, y=o["ad.y"])
        nl.act_dropout_bwd(A["dy"], A["x"], "gelu", 0.1, 0xC0FFEE, 8, dx=o["ad.dx"])

    def snapshot(self):
        return {k: (t.clone() if t is not None else None) for k, t in self.out.items()}


def test_graph_replays_match_eager():
    print("case graph capture of the forward + backward sequence", flush=True)
    s = Sequence()
    s.reset_running_stats()
    s.poison_outputs()
    s.step()
    torch.cuda.synchronize()
    ref = s.snapshot()
    for k, t in ref.items():
        if t is not None and t.numel():
            assert torch.isfinite(t.float()).all(), f"eager {k} not finite"

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        s.step()
    torch.cuda.synchronize()

    other = torch.randn(512, 512, device="cuda")
    for replay in range(3):
        s.reset_running_stats()
        s.poison_outputs()
        # Eager work between replays, on the same device and stream.
        other = torch.tanh(other @ other.t() * 1e-3)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, t in s.out.items():
            if t is None:
                continue
            same = torch.equal(t.view(torch.uint8) if t.numel() else t, ref[k].view(torch.uint8)
                               if t.numel() else ref[k])
            assert same, f"replay {replay}: {k} differs from the eager result"
    assert float(other.abs().sum()) > 0
