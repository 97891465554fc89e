"""Build libmi355norm.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Each .hip file is compiled to an object in parallel, then linked into
normalization_ln_rmsnorm_amd/libmi355norm.so.  Packed-FP32 instructions are
disabled for the device code (-packed-fp32-ops).
"""
import os
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build", "mi355norm")
OUT = os.path.join(HERE, "libmi355norm.so")
# (source, object name, extra flags): row_inst.hip and bn_inst.hip are
# compiled once per I/O dtype (and row operation) so the kernels build in
# parallel.
SOURCES = [("api_common.hip", "api_common", []), ("rownorm.hip", "rownorm", []),
           ("batchnorm.hip", "batchnorm", []),
           *[("row_inst.hip", f"row_{io}_{op}", [f"-DMI355NORM_ROW_IO={i}", f"-DMI355NORM_ROW_RMS={r}"])
             for i, io in enumerate(("f32", "bf16", "f16")) for r, op in enumerate(("ln", "rms"))],
           ("act_dropout.hip", "act_dropout", []),
           *[("ad_inst.hip", f"ad_{io}", [f"-DMI355NORM_AD_IO={i}"])
             for i, io in enumerate(("f32", "bf16", "f16"))],
           ("bn_inst.hip", "bn_f32", ["-DMI355NORM_BN_IO=0"]),
           ("bn_inst.hip", "bn_bf16", ["-DMI355NORM_BN_IO=1"]),
           ("bn_inst.hip", "bn_f16", ["-DMI355NORM_BN_IO=2"])]
ARCH = os.environ.get("MI355NORM_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument"]


def build(verbose: bool = False, tuning: bool = False, out: str = None) -> str:
    """Compile and link the library.  tuning=True defines MI355NORM_TUNING,
    which compiles in the environment overrides of the launch plans used by
    tuning sweeps (the regular library has none); such a build goes to
    `out`, never over the regular library."""
    if tuning and not out:
        raise ValueError("a tuning build needs its own output path")
    out = out or OUT
    build_dir = BUILD + ("_tuning" if tuning else "")
    os.makedirs(build_dir, exist_ok=True)
    t0 = time.time()
    procs = []
    objs = []
    for src, name, extra in SOURCES:
        obj = os.path.join(build_dir, name + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, *(["-DMI355NORM_TUNING"] if tuning else []), *extra, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((name, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        log, _ = p.communicate()
        text = "\n".join(l for l in log.decode(errors="replace").splitlines()
                         if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append(src)
            print(text, file=sys.stderr)
        elif verbose and text.strip():
            print(text)
    if failed:
        raise RuntimeError("HIP compile failed: " + ", ".join(failed))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    if verbose:
        print(f"built {out} in {time.time() - t0:.1f}s", flush=True)
    return out


if __name__ == "__main__":
    build(verbose=True)
