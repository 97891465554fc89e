"""C ABI checks that need no GPU: the library loads, exports every function
include/mi355norm.h declares, and rejects bad arguments on the host (the
validation runs before anything touches the HIP runtime)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mi355norm.h")

OK, ENULL, ESHAPE, EDTYPE, EACT, EARG, EWS = 0, -1, -2, -3, -4, -5, -6
F32, BF16, F16 = 0, 1, 2
P = ctypes.c_void_p(4096)  # a non-NULL pointer that validation must reject before use
NULL = None


@pytest.fixture(scope="module")
def lib():
    from normalization_ln_rmsnorm_amd import normlib
    if not os.path.exists(normlib.LIB_PATH):
        from normalization_ln_rmsnorm_amd import build
        build.build()
    return normlib.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["ln_fwd", "ln_bwd", "ln_bwd_workspace_bytes", "rms_fwd", "rms_bwd",
              "rms_bwd_workspace_bytes", "bn_workspace_bytes", "bn_fwd_train", "bn_fwd_eval",
              "bn_bwd", "norm_status_str", "norm_arm_kernel_events", "norm_last_kernel_count",
              "norm_last_kernel_name", "norm_last_main_kernel", "act_dropout_fwd",
              "act_dropout_bwd"]:
        assert n in names, n


def test_every_declared_symbol_is_exported(lib):
    from normalization_ln_rmsnorm_amd import normlib
    out = subprocess.run(["nm", "-D", "--defined-only", normlib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for n in declared_functions():
        assert n in exported, f"{n} declared in mi355norm.h but not exported"
        getattr(lib, n)


def test_status_strings(lib):
    for code in (OK, ENULL, ESHAPE, EDTYPE, EACT, EARG, EWS, -7, 99):
        s = lib.norm_status_str(code)
        assert isinstance(s, bytes) and len(s) > 0


def test_row_errors(lib):
    # dtype, shapes, eps, null pointers
    assert lib.ln_fwd(7, 4, 8, 1e-5, P, NULL, NULL, P, NULL, NULL, NULL) == EDTYPE
    assert lib.ln_fwd(F32, 4, 0, 1e-5, P, NULL, NULL, P, NULL, NULL, NULL) == ESHAPE
    assert lib.ln_fwd(F32, -1, 8, 1e-5, P, NULL, NULL, P, NULL, NULL, NULL) == ESHAPE
    assert lib.ln_fwd(F32, 4, 32769, 1e-5, P, NULL, NULL, P, NULL, NULL, NULL) == ESHAPE
    assert lib.ln_fwd(BF16, 4, 65537, 1e-5, P, NULL, NULL, P, NULL, NULL, NULL) == ESHAPE
    assert lib.ln_fwd(F16, 4, 65537, 1e-5, P, NULL, NULL, P, NULL, NULL, NULL) == ESHAPE
    assert lib.ln_fwd(3, 4, 8, 1e-5, P, NULL, NULL, P, NULL, NULL, NULL) == EDTYPE
    assert lib.rms_bwd_workspace_bytes(F16, 4, 8) == lib.rms_bwd_workspace_bytes(BF16, 4, 8)
    assert lib.ln_fwd(F32, 4, 8, -1.0, P, NULL, NULL, P, NULL, NULL, NULL) == EARG
    assert lib.ln_fwd(F32, 4, 8, float("nan"), P, NULL, NULL, P, NULL, NULL, NULL) == EARG
    assert lib.ln_fwd(F32, 4, 8, 1e-5, NULL, NULL, NULL, P, NULL, NULL, NULL) == ENULL
    assert lib.ln_fwd(F32, 4, 8, 1e-5, P, NULL, NULL, NULL, NULL, NULL, NULL) == ENULL
    assert lib.ln_fwd(F32, 0, 8, 1e-5, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == OK
    assert lib.rms_fwd(F32, 4, 8, 1e-5, NULL, NULL, P, NULL, NULL) == ENULL
    assert lib.rms_fwd(BF16, 4, 8, -2.0, P, NULL, P, NULL, NULL) == EARG
    # backward: missing statistics, workspace
    assert lib.ln_bwd(F32, 4, 8, P, P, NULL, NULL, P, P, NULL, NULL, NULL, 0, NULL) == ENULL
    assert lib.ln_bwd(F32, 4, 8, P, P, NULL, P, NULL, P, NULL, NULL, NULL, 0, NULL) == ENULL
    need = lib.ln_bwd_workspace_bytes(F32, 4, 8)
    assert need >= 4 * 8 * 4
    assert lib.ln_bwd(F32, 4, 8, P, P, NULL, P, P, P, P, NULL, NULL, 0, NULL) == EWS
    assert lib.ln_bwd(F32, 4, 8, P, P, NULL, P, P, P, P, NULL, P, need - 1, NULL) == EWS
    assert lib.rms_bwd(F32, 4, 8, P, P, NULL, NULL, P, NULL, NULL, 0, NULL) == ENULL
    assert lib.rms_bwd(F32, 4, 8, P, P, NULL, P, P, P, NULL, 0, NULL) == EWS
    assert lib.rms_bwd_workspace_bytes(F32, 4, 8) >= 4 * 8 * 4
    assert lib.ln_bwd_workspace_bytes(9, 4, 8) == 0
    assert lib.rms_bwd_workspace_bytes(F32, 4, 0) == 0


def test_bn_errors(lib):
    ws = lib.bn_workspace_bytes(F32, 2, 3, 5)
    assert ws > 0
    args = lambda **k: dict(dict(dt=F32, Nb=2, C=3, HW=5, eps=1e-5, mom=0.1, act=0, ap=0.0, x=P, res=NULL,
                                 w=NULL, b=NULL, rm=NULL, rv=NULL, sm=P, sr=P, y=P, ws=P,
                                 wsb=ws, s=NULL), **k)

    def train(**k):
        a = args(**k)
        return lib.bn_fwd_train(a["dt"], a["Nb"], a["C"], a["HW"], a["eps"], a["mom"], a["act"],
                                a["ap"], a["x"], a["res"], a["w"], a["b"], a["rm"], a["rv"],
                                a["sm"], a["sr"], a["y"], a["ws"], a["wsb"], a["s"])

    assert train(dt=4) == EDTYPE
    assert train(dt=3) == EDTYPE
    assert train(act=15) == EACT
    assert train(act=-1) == EACT
    assert train(act=10, ap=0.0) == EARG    # CELU divides by its alpha
    assert train(act=7, ap=float("nan")) == EARG
    assert train(act=8, ap=float("inf")) == EARG
    assert train(mom=1.5) == EARG
    assert train(mom=-0.1) == EARG
    assert train(eps=-1.0) == EARG
    assert train(Nb=1, HW=1) == EARG        # one value per channel: no unbiased variance
    assert train(Nb=-1) == ESHAPE
    assert train(x=NULL) == ENULL
    assert train(sm=NULL) == ENULL
    assert train(y=NULL) == ENULL
    assert train(ws=NULL) == EWS
    assert train(wsb=ws - 1) == EWS
    assert train(C=0) == OK
    assert lib.bn_fwd_eval(F32, 2, 3, 5, 1e-5, 0, 0.0, P, NULL, NULL, NULL, NULL, P, P, NULL) == ENULL
    assert lib.bn_fwd_eval(F32, 2, 3, 5, 1e-5, 25, 0.0, P, NULL, NULL, NULL, P, P, P, NULL) == EACT
    assert lib.bn_fwd_eval(F32, 2, 3, 5, 1e-5, 10, 0.0, P, NULL, NULL, NULL, P, P, P, NULL) == EARG
    assert lib.bn_fwd_eval(F32, 0, 3, 5, 1e-5, 0, 0.0, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                           NULL) == OK
    # backward: residual without dres, missing saved statistics, workspace
    assert lib.bn_bwd(F32, 2, 3, 5, 0, 0.0, P, P, P, NULL, NULL, P, P, P, NULL, NULL, NULL, P, ws,
                      NULL) == ENULL
    assert lib.bn_bwd(F32, 2, 3, 5, 0, 0.0, P, P, NULL, NULL, NULL, NULL, P, P, NULL, NULL, NULL, P,
                      ws, NULL) == ENULL
    assert lib.bn_bwd(F32, 2, 3, 5, 0, 0.0, P, P, NULL, NULL, NULL, P, P, P, NULL, NULL, NULL, P, 8,
                      NULL) == EWS
    assert lib.bn_bwd(F32, 2, 3, 5, 17, 0.0, P, P, NULL, NULL, NULL, P, P, P, NULL, NULL, NULL, P, ws,
                      NULL) == EACT
    assert lib.bn_bwd(F32, 2, 3, 5, 10, 0.0, P, P, NULL, NULL, NULL, P, P, P, NULL, NULL, NULL, P, ws,
                      NULL) == EARG
    assert lib.bn_workspace_bytes(F32, -1, 3, 5) == 0


def test_workspace_sizes_scale(lib):
    small = lib.bn_workspace_bytes(F32, 64, 256, 3136)
    big = lib.bn_workspace_bytes(BF16, 256, 64, 12544)
    assert 0 < small < 1 << 22 and 0 < big < 1 << 22
    assert lib.rms_bwd_workspace_bytes(BF16, 16384, 4096) <= 64 << 20


def test_timing_hook_bookkeeping_without_gpu(lib):
    """A call that fails validation launches nothing and disarms the hook."""
    ev = (ctypes.c_void_p * 2)(None, None)
    lib.norm_arm_kernel_events(ev, 1)
    assert lib.ln_fwd(F32, 4, 0, 1e-5, P, NULL, NULL, P, NULL, NULL, NULL) == ESHAPE
    assert lib.norm_last_kernel_count() == 0
    assert lib.norm_last_main_kernel() == -1
    assert lib.norm_last_kernel_name(0) == b""
    lib.norm_arm_kernel_events(None, 0)


def test_act_dropout_errors(lib):
    fwd = lambda **k: lib.act_dropout_fwd(*[k.get(n, d) for n, d in (
        ("dt", F32), ("n", 16), ("act", 2), ("ap", 0.0), ("p", 0.1), ("seed", 1), ("off", 0),
        ("x", P), ("y", P), ("s", NULL))])
    assert fwd(dt=3) == EDTYPE
    assert fwd(n=-1) == ESHAPE
    assert fwd(act=15) == EACT
    assert fwd(act=10, ap=0.0) == EARG
    for bad in (-0.1, 1.5, float("nan")):
        assert fwd(p=bad) == EARG
    assert fwd(off=2) == EARG  # the offset must be a multiple of 8
    assert fwd(off=4) == EARG
    assert fwd(off=(1 << 64) - 8) == EARG  # offset + n overflows
    assert fwd(x=NULL) == ENULL
    assert fwd(y=NULL) == ENULL
    assert fwd(n=0, x=NULL, y=NULL) == OK
    assert lib.act_dropout_bwd(F32, 16, 0, 0.0, 0.5, 1, 0, P, NULL, P, NULL) == ENULL
    assert lib.act_dropout_bwd(F32, 16, 0, 0.0, 0.5, 1, 6, P, P, P, NULL) == EARG
    assert lib.act_dropout_bwd(BF16, 0, 0, 0.0, 0.5, 1, 0, NULL, NULL, NULL, NULL) == OK


def test_bn_force_path_hook(lib):
    """The test hook pins the data path; the workspace query follows it, and
    invalid settings are refused without a change."""
    lib.norm_bn_force_path.restype = ctypes.c_int
    lib.norm_bn_force_path.argtypes = [ctypes.c_int]
    auto = lib.bn_workspace_bytes(BF16, 256, 64, 12544)
    assert lib.norm_bn_force_path(1) == 0
    plane = lib.bn_workspace_bytes(BF16, 256, 64, 12544)
    assert lib.norm_bn_force_path(2) == 1
    cols = lib.bn_workspace_bytes(BF16, 256, 64, 12544)
    assert lib.norm_bn_force_path(3) == -1 and lib.norm_bn_force_path(-1) == -1
    assert lib.norm_bn_force_path(0) == 2
    assert auto == plane and cols != plane and cols > 0
    assert lib.bn_workspace_bytes(BF16, 256, 64, 12544) == auto


def test_regular_build_reads_no_environment():
    """The shipped library has no run-time tuning knobs: it does not import
    getenv (tuning sweeps use a separate build with -DMI355NORM_TUNING)."""
    from normalization_ln_rmsnorm_amd import normlib
    out = subprocess.run(["nm", "-D", "--undefined-only", normlib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    imported = set(line.split()[-1].split("@")[0] for line in out.splitlines() if line.strip())
    assert "getenv" not in imported and "secure_getenv" not in imported


def test_noalloc_entry_point_validation(lib):
    """rms_bwd_noalloc checks its arguments like rms_bwd, and refuses a shape
    whose partial rows exceed the static scratch before touching the GPU."""
    f = lib.rms_bwd_noalloc
    assert f(3, 4, 8, P, P, P, P, P, P, NULL) == EDTYPE
    assert f(BF16, 4, 0, P, P, P, P, P, P, NULL) == ESHAPE
    assert f(BF16, 4, 8, NULL, P, P, P, P, P, NULL) == ENULL
    assert f(BF16, 4, 8, P, P, P, NULL, P, P, NULL) == ENULL
    assert f(BF16, 8192, 16384, P, P, P, P, P, P, NULL) == EWS
    assert f(F32, 8192, 32768, P, P, P, P, P, P, NULL) == EWS
    assert f(BF16, 0, 8, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == OK
