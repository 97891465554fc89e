"""Host-side pieces of bench.py (no GPU): the algorithmic byte counts, the
traffic-record check and the one-GPU guard."""
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from normalization_ln_rmsnorm_amd.workloads import EXTRA_WORKLOADS, WORKLOADS  # noqa: E402


def test_rowwise_bytes_rms_bf16():
    M, N = 16384, 4096
    b = bench.bytes_rowwise("rms", M, N, 2)
    U = M * N * 2
    # forward: x in, y out, w, rstd out; backward kernel: dy, x in, dx out, w, rstd
    assert b["fwd"] == 2 * U + N * 2 + M * 4
    assert b["bwd_kernel"] == 3 * U + N * 2 + M * 4
    assert b["bwd"] == b["bwd_kernel"] + N * 2  # + dw out


def test_rowwise_bytes_ln_f32():
    M, N = 64, 256
    b = bench.bytes_rowwise("ln", M, N, 4)
    U = M * N * 4
    assert b["fwd"] == 2 * U + 2 * N * 4 + 2 * M * 4
    assert b["bwd"] == 3 * U + N * 4 + 2 * M * 4 + 2 * N * 4


def test_bn_bytes_residual_and_eval():
    wl = WORKLOADS["bn_f32_64x256x56x56"]
    Nb, C, H, W = wl.shape
    U = Nb * C * H * W * 4
    b = bench.bytes_bn(wl, 4)
    assert wl.residual
    assert b["fwd"] == 4 * U + 8 * C * 4          # x twice, res, y
    assert b["bwd"] == 7 * U + 8 * C * 4
    wl4 = WORKLOADS["bn_bf16_256x64x112x112"]
    Nb, C, H, W = wl4.shape
    U4 = Nb * C * H * W * 2
    b4 = bench.bytes_bn(wl4, 2)
    assert not wl4.residual and wl4.eval_after_train
    assert b4["bwd"] == 5 * U4 + 8 * C * 4
    assert b4["eval"] == 2 * U4 + 8 * C * 4


def _records():
    text = open(os.path.join(ROOT, "profiles", "pmc_traffic.md")).read()
    m = re.search(r"```json\s*(\{.*?\})\s*```", text, flags=re.S)
    assert m, "pmc_traffic.md holds no JSON record"
    return json.loads(m.group(1))


def test_traffic_records_resolve():
    """Every record names existing sources and, while they are unchanged,
    yields its byte count; a stale or foreign record yields None, never an
    exception."""
    every = {**WORKLOADS, **EXTRA_WORKLOADS}
    for key, rec in _records().items():
        kernel, wl = key.split("|")
        assert wl in every, key
        got = bench.load_traffic(key)
        assert got is None or (isinstance(got, int) and got > 0), (key, got)
    assert bench.load_traffic("no_such_kernel|no_such_workload") is None


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _host_bench(cls, wl, inp, **attrs):
    """A bench object with host inputs only (no device tensors): enough for
    the CPU-baseline leg."""
    b = object.__new__(cls)
    b.wl, b.inp = wl, inp
    for k, v in attrs.items():
        setattr(b, k, v)
    return b


@pytest.mark.parametrize("name", ["bn_bf16_256x64x112x112", "bn_f32_64x256x56x56", "rms_bf16_16384x4096",
                                  "actdrop_bf16_16384x4096"])
def test_cpu_baseline_on_a_small_variant(name):
    """The oracle timing leg on a shrunken copy of each workload kind: it
    cycles over groups of channels / rows / element blocks, reports the
    threads used and what was sampled."""
    import dataclasses

    import numpy as np

    from normalization_ln_rmsnorm_amd import workloads as W
    wl = {**WORKLOADS, **EXTRA_WORKLOADS}[name]
    if wl.kind == "bn":
        wl = dataclasses.replace(wl, shape=(4, 8, 7, 7))
        b = _host_bench(bench.BnBench, wl, W.gen_bn(wl), ops=["fwd", "bwd"] + (
            ["eval"] if wl.eval_after_train else []), bytes=bench.bytes_bn(wl, bench.ELEM_SIZE[wl.dtype]))
    elif wl.kind == "ad":
        wl = dataclasses.replace(wl, shape=(3, 70000))
        inp = W.gen_act_dropout(wl)

        class _X:  # numel() of the device input
            def numel(self):
                return inp["x"].size
        b = _host_bench(bench.AdBench, wl, inp, ops=["fwd", "bwd"], x=_X(), p=0.1, seed=7,
                        bytes=bench.bytes_act_dropout(wl, 2))
    else:
        wl = dataclasses.replace(wl, shape=(40, 256))
        b = _host_bench(bench.RowBench, wl, W.gen_rowwise(wl), ops=["fwd", "bwd"],
                        bytes=bench.bytes_rowwise(wl.kind, 40, 256, bench.ELEM_SIZE[wl.dtype]))
    r = bench.cpu_baseline(b, 0.05)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["value"] > 0
    assert r["cores"] >= 1 and np.isfinite(r["s_per_step"])
    assert name in r["sample"]
