"""Benchmark: normalization forward+backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-others] [--no-cpu]

A step is one forward and one backward pass of the workload (BatchNorm
workloads: training forward, backward, and the eval forward when the workload
has one) on seeded synthetic inputs already resident in HBM.  Before every
operation a 512 MiB scratch buffer is streamed (read by default, --flush
write rewrites it), so inputs come from HBM rather than the 256 MB Infinity
Cache; that flush is outside the timed spans.  Each
operation is timed on the device: the library attaches caller-created HIP
events to its kernels' own dispatches (norm_arm_kernel_events).  A span pass
with events only on the first kernel's start and the last kernel's end gives
the operation's time (events between kernels would delay the next dispatch);
a second pass with events on every kernel gives each kernel's duration, the
main streaming kernel's for the roofline -- the same quantities rocprofv3's
kernel trace reports.  Host-side events around each
call are recorded too (they add the ~6 us dispatch latency of a lone launch).

Bytes are algorithmic: what the method must move (every activation tensor in
its I/O dtype once per pass that touches it, plus the small vectors), not
what the hardware happened to move.  The default workload is the largest:
BatchNorm2d bf16 256 x 64 x 112 x 112 with exact GELU (training forward,
backward, eval forward); the other workloads are measured too and reported
under "per_workload", each with the float64 oracle timed on the host cores
beside it.  `value` is the whole step's algorithmic bytes over its summed
device time.  Rank 0 prints one JSON line.
"""
import argparse
import ctypes
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "norm fwd+bwd achieved HBM GB/s (% of peak) and rows/s at 1 MI355X"
FLUSH_BYTES = 512 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=None)
    p.add_argument("--no-others", action="store_true", help="skip the other workloads")
    p.add_argument("--other-steps", type=int, default=20)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="oracle time spent on the headline workload's CPU baseline")
    p.add_argument("--other-cpu-seconds", type=float, default=2.0,
                   help="oracle time spent on each other workload's CPU baseline")
    p.add_argument("--flush", choices=["read", "write"], default="read",
                   help="evict the caches by reading (default) or rewriting a 512 MiB buffer")
    return p.parse_args()


# ------------------------------------------------------------- HIP events
class Hip:
    """hipEvent helpers through the HIP runtime torch already loaded."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        ev = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return ev

    def destroy(self, events):
        for e in events:
            if e is not None:
                self.lib.hipEventDestroy(e)

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value


# ------------------------------------------------------ algorithmic bytes
def bytes_rowwise(kind, M, N, es):
    U = M * N * es
    if kind == "ln":
        fwd = 2 * U + 2 * N * es + 2 * M * 4
        bwd = 3 * U + N * es + 2 * M * 4 + 2 * N * es
        bwd_kernel = 3 * U + N * es + 2 * M * 4
    else:
        fwd = 2 * U + N * es + M * 4
        bwd = 3 * U + N * es + M * 4 + N * es
        bwd_kernel = 3 * U + N * es + M * 4
    return dict(fwd=fwd, bwd=bwd, bwd_kernel=bwd_kernel, fwd_kernel=fwd)


def bytes_bn(wl, es):
    Nb, C, H, W = wl.shape
    U = Nb * C * H * W * es
    small = 8 * C * 4
    res = 1 if wl.residual else 0
    fwd = (2 + res + 1) * U + small          # x twice (stats, apply), res, y
    fwd_kernel = (1 + res + 1) * U           # the apply kernel alone
    if res:
        bwd = 7 * U + small                  # pass 1: dy, x, res -> dres; pass 2: dres, x -> dx
        bwd_kernel = 4 * U                   # main kernel: pass 1
    else:
        bwd = 5 * U + small                  # pass 1: dy, x; pass 2: dy, x -> dx
        bwd_kernel = 3 * U                   # main kernel: pass 2
    ev = (2 + res) * U + small if wl.eval_after_train else 0
    return dict(fwd=fwd, bwd=bwd, eval=ev, fwd_kernel=fwd_kernel, bwd_kernel=bwd_kernel)


def bytes_act_dropout(wl, es):
    U = wl.shape[0] * wl.shape[1] * es
    return dict(fwd=2 * U, bwd=3 * U, fwd_kernel=2 * U, bwd_kernel=3 * U)


# ------------------------------------------------------------ workloads
ELEM_SIZE = {"f32": 4, "bf16": 2, "f16": 2}


def torch_dtype(torch, dtype):
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]


def to_device(torch, a, dtype):
    """Host array in the I/O representation (bf16 as uint16 bits) -> device."""
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


class RowBench:
    def __init__(self, wl, nl, torch):
        from normalization_ln_rmsnorm_amd.workloads import gen_rowwise
        self.wl, self.nl, self.torch = wl, nl, torch
        M, N = wl.shape
        self.inp = gen_rowwise(wl)
        tdt = torch_dtype(torch, wl.dtype)
        dev = lambda a: to_device(torch, a, wl.dtype)
        self.x, self.dy, self.w = dev(self.inp["x"]), dev(self.inp["dy"]), dev(self.inp["w"])
        self.b = dev(self.inp["b"]) if wl.kind == "ln" else None
        self.y = torch.empty(M, N, dtype=tdt, device="cuda")
        self.dx = torch.empty_like(self.y)
        self.mean = torch.empty(M, dtype=torch.float32, device="cuda")
        self.rstd = torch.empty(M, dtype=torch.float32, device="cuda")
        self.dw = torch.empty(N, dtype=tdt, device="cuda")
        self.db = torch.empty(N, dtype=tdt, device="cuda")
        ws_fn = nl.ln_bwd_workspace_bytes if wl.kind == "ln" else nl.rms_bwd_workspace_bytes
        self.ws = torch.empty(max(1, ws_fn(tdt, M, N)), dtype=torch.uint8, device="cuda")
        self.bytes = bytes_rowwise(wl.kind, M, N, ELEM_SIZE[wl.dtype])
        self.ops = ["fwd", "bwd"]
        self.dominant = "bwd"

    def run(self, op):
        nl, wl = self.nl, self.wl
        if wl.kind == "ln":
            if op == "fwd":
                nl.ln_fwd(self.x, self.w, self.b, wl.eps, y=self.y, mean=self.mean, rstd=self.rstd)
            else:
                nl.ln_bwd(self.dy, self.x, self.w, self.mean, self.rstd, dx=self.dx, dw=self.dw,
                          db=self.db, ws=self.ws)
        else:
            if op == "fwd":
                nl.rms_fwd(self.x, self.w, wl.eps, y=self.y, rstd=self.rstd)
            else:
                nl.rms_bwd(self.dy, self.x, self.w, self.rstd, dx=self.dx, dw=self.dw, ws=self.ws)

    def cpu_units(self):
        """Rows: the oracle is timed on groups of whole rows."""
        return self.wl.shape[0]

    def cpu_prepare(self, orc, r0, r1):
        bf16 = self.wl.dtype == "bf16"
        inp = self.inp
        return dict(x=orc.widen(inp["x"][r0:r1], bf16=bf16), dy=orc.widen(inp["dy"][r0:r1], bf16=bf16),
                    w=orc.widen(inp["w"], bf16=bf16),
                    b=orc.widen(inp["b"], bf16=bf16) if inp["b"] is not None else None)

    def cpu_step(self, orc, arrays):
        wl = self.wl
        if wl.kind == "ln":
            orc.ln_fwd(arrays["x"], arrays["w"], arrays["b"], eps=wl.eps)
            orc.ln_bwd(arrays["dy"], arrays["x"], arrays["w"], eps=wl.eps)
        else:
            orc.rms_fwd(arrays["x"], arrays["w"], eps=wl.eps)
            orc.rms_bwd(arrays["dy"], arrays["x"], arrays["w"], eps=wl.eps)


class BnBench:
    def __init__(self, wl, nl, torch):
        from normalization_ln_rmsnorm_amd.workloads import gen_bn
        self.wl, self.nl, self.torch = wl, nl, torch
        Nb, C, H, W = wl.shape
        inp = gen_bn(wl)
        tdt = torch_dtype(torch, wl.dtype)
        shape = (Nb, C, H, W)
        dev = lambda a: to_device(torch, a, wl.dtype)
        self.x = dev(inp["x"]).view(shape)
        self.dy = dev(inp["dy"]).view(shape)
        self.res = dev(inp["res"]).view(shape) if wl.residual else None
        self.w, self.b = dev(inp["w"]), dev(inp["b"])
        self.inp = inp  # host copy for the CPU oracle baseline
        self.rm = torch.zeros(C, device="cuda")
        self.rv = torch.ones(C, device="cuda")
        self.y = torch.empty(shape, dtype=tdt, device="cuda")
        self.ye = torch.empty(shape, dtype=tdt, device="cuda") if wl.eval_after_train else None
        self.dx = torch.empty(shape, dtype=tdt, device="cuda")
        self.dres = torch.empty(shape, dtype=tdt, device="cuda") if wl.residual else None
        self.sm = torch.empty(C, device="cuda")
        self.sr = torch.empty(C, device="cuda")
        self.dw = torch.empty(C, dtype=tdt, device="cuda")
        self.db = torch.empty(C, dtype=tdt, device="cuda")
        self.ws = torch.empty(nl.bn_workspace_bytes(tdt, Nb, C, H * W), dtype=torch.uint8, device="cuda")
        self.bytes = bytes_bn(wl, ELEM_SIZE[wl.dtype])
        self.ops = ["fwd", "bwd"] + (["eval"] if wl.eval_after_train else [])
        self.dominant = "bwd"

    def cpu_units(self):
        """Channels: the oracle is timed on groups of whole channels."""
        return self.wl.shape[1]

    def cpu_prepare(self, orc, c0, c1):
        """float64 copies of channels c0..c1-1 (outside the timed region)."""
        bf16 = self.wl.dtype == "bf16"
        sub = lambda a: orc.widen(np.ascontiguousarray(a[:, c0:c1, :]), bf16=bf16)
        inp = self.inp
        return dict(x=sub(inp["x"]), dy=sub(inp["dy"]),
                    res=sub(inp["res"]) if inp["res"] is not None else None,
                    w=orc.widen(inp["w"][c0:c1], bf16=bf16), b=orc.widen(inp["b"][c0:c1], bf16=bf16),
                    rm=inp["running_mean"][c0:c1].astype(np.float64),
                    rv=inp["running_var"][c0:c1].astype(np.float64))

    def cpu_step(self, orc, a):
        """One step of the oracle on a group of channels: training forward
        (statistics, EMA, activation), backward, and the eval forward."""
        wl = self.wl
        _, _, _, rm, rv = orc.bn_fwd_train(a["x"], a["res"], a["w"], a["b"], a["rm"], a["rv"],
                                           eps=wl.eps, momentum=wl.momentum, act=wl.act)
        orc.bn_bwd(a["dy"], a["x"], a["res"], a["w"], a["b"], eps=wl.eps, act=wl.act)
        if wl.eval_after_train:
            orc.bn_fwd_eval(a["x"], rm, rv, a["res"], a["w"], a["b"], eps=wl.eps, act=wl.act)

    def run(self, op):
        nl, wl = self.nl, self.wl
        if op == "fwd":
            nl.bn_fwd_train(self.x, self.w, self.b, self.rm, self.rv, wl.eps, wl.momentum, wl.act,
                            self.res, y=self.y, save_mean=self.sm, save_rstd=self.sr, ws=self.ws)
        elif op == "bwd":
            nl.bn_bwd(self.dy, self.x, self.w, self.b, self.sm, self.sr, wl.act, self.res,
                      dx=self.dx, dres=self.dres, dw=self.dw, db=self.db, ws=self.ws)
        else:
            nl.bn_fwd_eval(self.x, self.w, self.b, self.rm, self.rv, wl.eps, wl.act, self.res,
                           y=self.ye)


class AdBench:
    """Activation + dropout: forward reads x, writes y; backward reads dy and
    x, writes dx (the mask recomputed from the seed)."""

    def __init__(self, wl, nl, torch):
        from normalization_ln_rmsnorm_amd.workloads import gen_act_dropout
        self.wl, self.nl, self.torch = wl, nl, torch
        inp = gen_act_dropout(wl)
        self.x = to_device(torch, inp["x"], wl.dtype)
        self.dy = to_device(torch, inp["dy"], wl.dtype)
        self.inp = inp  # host copy for the CPU oracle baseline
        self.y = torch.empty_like(self.x)
        self.dx = torch.empty_like(self.x)
        self.p, self.seed = wl.extra["drop_p"], wl.extra["dropout_seed"]
        self.bytes = bytes_act_dropout(wl, ELEM_SIZE[wl.dtype])
        self.ops = ["fwd", "bwd"]
        self.dominant = "bwd"

    def cpu_units(self):
        """Blocks of 2^16 elements (offsets stay multiples of 8)."""
        return -(-self.x.numel() // (1 << 16))

    def cpu_prepare(self, orc, u0, u1):
        bf16 = self.wl.dtype == "bf16"
        a, b = u0 << 16, min(u1 << 16, self.x.numel())
        return dict(x=orc.widen(self.inp["x"][a:b], bf16=bf16),
                    dy=orc.widen(self.inp["dy"][a:b], bf16=bf16), offset=a)

    def cpu_step(self, orc, a):
        wl = self.wl
        orc.act_dropout_fwd(a["x"], wl.act, self.p, self.seed, a["offset"])
        orc.act_dropout_bwd(a["dy"], a["x"], wl.act, self.p, self.seed, a["offset"])

    def run(self, op):
        nl, wl = self.nl, self.wl
        if op == "fwd":
            nl.act_dropout_fwd(self.x, wl.act, self.p, self.seed, 0, y=self.y)
        else:
            nl.act_dropout_bwd(self.dy, self.x, wl.act, self.p, self.seed, 0, dx=self.dx)


def bench_class(wl):
    return {"ln": RowBench, "rms": RowBench, "bn": BnBench, "ad": AdBench}[wl.kind]


MAX_KERNELS = 4  # kernels per operation timed through the library's hook


class CacheFlush:
    """Evicts the 256 MB Infinity Cache and the L2s before each operation by
    streaming a 512 MiB buffer: read (a sum into a scalar; leaves no dirty
    lines whose write-back the next kernel would share HBM with) or
    rewritten in place."""

    def __init__(self, torch, mode):
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        self.sink = torch.empty((), dtype=torch.float32, device="cuda")
        self.mode = mode
        self.torch = torch

    def add_(self, _=None):
        if self.mode == "read":
            self.torch.sum(self.buf, dim=0, out=self.sink)
        else:
            self.buf.add_(1)


def measure(bench, steps, warmup, torch, hip, nl, flush):
    """Runs `steps` timed steps; every operation runs twice per step (each
    after the cache flush).  The span pass attaches HIP events only to the
    first kernel's start and the last kernel's end (an event attached in
    between delays the next dispatch by several microseconds, which plain
    calls do not pay), giving the operation's device time.  The kernel pass
    attaches a pair to every kernel, giving each kernel's own duration (the
    main streaming kernel's for the roofline).  Host-side events around the
    span pass are recorded too (they add the dispatch latency)."""
    nk = {}
    for op in bench.ops:  # kernel count of each operation
        bench.run(op)
        nk[op] = min(len(nl.last_kernels()[0]), MAX_KERNELS)
    torch.cuda.synchronize()

    def one_step(record):
        out = {}
        for op in bench.ops:
            flush.add_(1)
            if not record:
                bench.run(op)
                continue
            k = nk[op]
            span = [hip.event(), hip.event()]
            evs = [None] * (2 * k)
            evs[0], evs[2 * k - 1] = span
            nl.arm_kernel_events(evs)
            h0 = torch.cuda.Event(enable_timing=True)
            h1 = torch.cuda.Event(enable_timing=True)
            h0.record()
            bench.run(op)
            h1.record()
            flush.add_(1)
            kev = [hip.event() for _ in range(2 * k)]
            nl.arm_kernel_events(kev)
            # A stream event between the flush and the call, as in the span
            # pass: without it the first kernel's start event was stamped
            # ~2 us early (before the flush kernel had fully drained).
            torch.cuda.Event().record()
            bench.run(op)
            names, main = nl.last_kernels()
            out[op] = (span, kev, names, main, h0, h1)
        return out

    for _ in range(warmup):
        one_step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    recs = [one_step(True) for _ in range(steps)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dev_ms, host_ms, main_ms, kern_ms = {}, {}, {}, {}
    names_main = {}
    for op in bench.ops:
        d, h, m = [], [], []
        per_kernel = None
        for r in recs:
            span, kev, names, main, h0, h1 = r[op]
            k = nk[op]
            d.append(hip.elapsed_ms(span[0], span[1]))
            h.append(h0.elapsed_time(h1))
            m.append(hip.elapsed_ms(kev[2 * main], kev[2 * main + 1]) if main >= 0 else float("nan"))
            ks = [hip.elapsed_ms(kev[2 * i], kev[2 * i + 1]) for i in range(k)]
            per_kernel = [p + [t] for p, t in zip(per_kernel, ks)] if per_kernel else [[t] for t in ks]
            names_main[op] = (names, main)
        dev_ms[op], host_ms[op], main_ms[op] = d, h, m
        kern_ms[op] = {f"{i}:{names_main[op][0][i]}": float(np.mean(v)) * 1e3
                       for i, v in enumerate(per_kernel or [])}
    for r in recs:
        for span, kev, *_ in r.values():
            hip.destroy(span + kev)
    return dict(dev=dev_ms, host=host_ms, main=main_ms, kernels_us=kern_ms, names=names_main,
                wall=wall)


def summarize(bench, meas):
    wl = bench.wl
    res = {"workload": wl.name, "rows": wl.rows}
    tot_bytes, tot_ms = 0, 0.0
    for op in bench.ops:
        dev = meas["dev"][op]
        ms = float(np.mean(dev))
        b = bench.bytes[op]
        res[op] = {"ms_mean": ms, "ms_p10": float(np.percentile(dev, 10)),
                   "ms_p50": float(np.percentile(dev, 50)),
                   "ms_p90": float(np.percentile(dev, 90)),
                   "ms_host_events_incl_launch": float(np.mean(meas["host"][op])),
                   "bytes": b, "GBps": b / ms / 1e6, "frac_of_peak": b / ms / 1e6 / PEAK_HBM_GBPS,
                   "rows_per_s": wl.rows / (ms / 1e3), "kernels_us": meas["kernels_us"][op]}
        if op in ("fwd", "bwd"):
            tot_bytes += b
            tot_ms += ms
    res["fwd_bwd"] = {"ms": tot_ms, "bytes": tot_bytes, "GBps": tot_bytes / tot_ms / 1e6,
                      "frac_of_peak": tot_bytes / tot_ms / 1e6 / PEAK_HBM_GBPS,
                      "rows_per_s": wl.rows / (tot_ms / 1e3)}
    # The whole step: every operation of the workload (BatchNorm workloads
    # with an eval step: training forward, backward and the eval forward).
    st_bytes = sum(bench.bytes[op] for op in bench.ops)
    st_ms = sum(res[op]["ms_mean"] for op in bench.ops)
    res["step"] = {"ops": list(bench.ops), "ms": st_ms, "bytes": st_bytes,
                   "GBps": st_bytes / st_ms / 1e6, "frac_of_peak": st_bytes / st_ms / 1e6 / PEAK_HBM_GBPS,
                   "rows_per_s": wl.rows / (st_ms / 1e3)}
    names, main = meas["names"][bench.dominant]
    km = float(np.mean(meas["main"][bench.dominant]))
    kb = bench.bytes[bench.dominant + "_kernel"]
    kname = names[main] if main >= 0 else ""
    traffic = load_traffic(f"{kname}|{wl.name}")
    res["dominant_kernel"] = {"op": bench.dominant, "kernel": kname, "avg_us": km * 1e3, "bytes": kb,
                              "GBps": kb / km / 1e6, "traffic": traffic,
                              "traffic_GBps": traffic / km / 1e6 if traffic else None}
    return res


def load_traffic(kernel_key):
    """HBM traffic per launch recorded from rocprofv3 PMC runs, if the
    kernel's source files (its header and the shared headers it is compiled
    from) still match the ones profiled (else None)."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.md")
    if not os.path.exists(path):
        return None
    import hashlib
    text = open(path).read()
    m = re.search(r"```json\s*(\{.*?\})\s*```", text, flags=re.S)
    if not m:
        return None
    rec = json.loads(m.group(1)).get(kernel_key)
    if not rec:
        return None
    files = rec.get("sources")
    if not files or not all(os.path.exists(os.path.join(ROOT, f)) for f in files):
        return None  # a record this version cannot check
    src = b"".join(open(os.path.join(ROOT, f), "rb").read() for f in files)
    if hashlib.sha256(src).hexdigest() != rec.get("sources_sha256"):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(bench, budget_s):
    """The float64 C oracle (as it stands; OpenMP over rows or channels) on
    the host cores, timed on the same workload: groups of whole rows,
    channels or element blocks, each group as large as one row / channel per
    OpenMP thread (at least 1/16 of the workload), cycling through the
    workload until `budget_s` seconds of oracle time have been spent (at
    least one group).  Converting a group to float64 is outside the timing.
    The rate is the workload's step bytes scaled by the fraction of it
    processed, over the time spent."""
    import oracle
    wl = bench.wl
    units = bench.cpu_units()
    threads = oracle.num_threads()
    group = max(threads, -(-units // 16))
    group = min(group, units)
    done, spent, calls = 0, 0.0, 0
    u0 = 0
    while spent < budget_s or calls == 0:
        u1 = min(u0 + group, units)
        arrays = bench.cpu_prepare(oracle, u0, u1)
        t0 = time.perf_counter()
        bench.cpu_step(oracle, arrays)
        spent += time.perf_counter() - t0
        del arrays
        done += u1 - u0
        calls += 1
        u0 = 0 if u1 >= units else u1
        if calls >= 200:
            break
    frac = done / units
    step_bytes = sum(bench.bytes[op] for op in bench.ops)
    per_step = spent / frac
    unit_name = {"bn": "channels", "ad": "blocks of 65536 elements"}.get(wl.kind, "rows")
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": step_bytes / per_step / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{wl.name}: {calls} oracle call(s) on groups of {group} of its {units} "
                      f"{unit_name} ({done} {unit_name} processed = {frac:.3g} times the workload's "
                      f"step of {', '.join(bench.ops)}), {spent:.1f} s; float64 C oracle, OpenMP; inputs "
                      f"widened to float64 outside the timing",
            "s_per_step": per_step, "rows_per_s": wl.rows / per_step, "cpu_model": model}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); multi-GPU runs are not "
              "supported", file=sys.stderr)
        sys.exit(2)
    import torch
    import normalization_ln_rmsnorm_amd as nl
    from normalization_ln_rmsnorm_amd.workloads import EXTRA_WORKLOADS, HEADLINE, WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    nl.lib()
    hip = Hip()
    flush = CacheFlush(torch, args.flush)

    name = args.workload or HEADLINE
    every = {**WORKLOADS, **EXTRA_WORKLOADS}
    wl = every[name]
    bench = bench_class(wl)(wl, nl, torch)
    meas = measure(bench, args.steps, args.warmup, torch, hip, nl, flush)
    head = summarize(bench, meas)
    wall = meas["wall"]
    print(f"[bench] {name}: " + "  ".join(f"{op} {head[op]['ms_mean']*1e3:.1f} us" for op in bench.ops)
          + f"  step {head['step']['GBps']:.0f} GB/s", file=sys.stderr, flush=True)
    cpu = cpu_baseline(bench, args.cpu_seconds) if not args.no_cpu else None
    if hasattr(bench, "inp"):
        del bench.inp

    per = {}
    if not args.no_others:
        for other in every:
            if other == name:
                continue
            ow = every[other]
            b = bench_class(ow)(ow, nl, torch)
            per[other] = summarize(b, measure(b, args.other_steps, 3, torch, hip, nl, flush))
            if not args.no_cpu:
                per[other]["cpu_baseline"] = cpu_baseline(b, args.other_cpu_seconds)
            print(f"[bench] {other}: " + "  ".join(
                f"{op} {per[other][op]['ms_mean']*1e3:.1f} us {per[other][op]['GBps']:.0f} GB/s"
                for op in b.ops), file=sys.stderr, flush=True)
            del b
            torch.cuda.empty_cache()

    # Plain copy bandwidth on the same device, for context.
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cms = []
    for _ in range(10):
        flush.add_(1)
        e0.record(); dst.copy_(src); e1.record(); torch.cuda.synchronize()
        cms.append(e0.elapsed_time(e1))
    copy_gbps = 2 * src.numel() * 4 / float(np.median(cms)) / 1e6
    del src, dst

    dk = head["dominant_kernel"]
    traffic = load_traffic(f"{dk['kernel']}|{name}")
    roofline = {"bound": "hbm", "achieved": dk["GBps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": dk["GBps"] / PEAK_HBM_GBPS, "traffic": traffic, "kernel": dk["kernel"],
                "bytes_per_launch": dk["bytes"], "avg_us": dk["avg_us"]}
    st = head["step"]
    op_name = {"rms": "RMSNorm", "ln": "LayerNorm", "bn": "BatchNorm", "ad": "activation+dropout"}[wl.kind]
    config = {"workload": name, "ops": " + ".join(
                  {"fwd": "training fwd" if wl.kind == "bn" else "fwd", "bwd": "bwd",
                   "eval": "eval fwd"}[op] for op in bench.ops) + f" ({op_name})",
              "shape": list(wl.shape), "io_dtype": wl.dtype, "eps": wl.eps}
    if wl.kind == "bn":
        config.update(act=wl.act, residual=wl.residual, momentum=wl.momentum)
    out = {
        "metric": METRIC, "value": st["GBps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": st["ms"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": config,
        "pct_of_peak": 100.0 * st["frac_of_peak"], "rows_per_s": st["rows_per_s"],
        "fwd_bwd": head["fwd_bwd"],
        **{op: head[op] for op in bench.ops},
        "wall_s_timed_region_incl_flush": wall,
        "copy_GBps_host_events": copy_gbps,
        "roofline": roofline,
        "per_workload": per,
    }
    out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
