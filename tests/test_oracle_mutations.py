"""The oracle's pins catch plausible mistakes (CPU only).

Each mutant is a copy of oracle/norm_oracle.c with one planted mistake: a
dropped term, a wrong sign, divisor or index, a convention flipped (the
biased running variance, eps outside the root, the residual after the
activation, the derivative's side at a kink), a wrong constant of the
random generator or a wrong word / counter layout of the dropout mask.  The
mutant is built with the oracle's own compiler flags and the pin suites
(test_oracle_pins.py, test_oracle_dropout_pins.py) run against it in a
subprocess; at least one pin must fail for every mutant.  The mistakes are
planted only here, in copies on the CPU.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "norm_oracle.c")
PINS = [os.path.join(ROOT, "tests", "test_oracle_pins.py"),
        os.path.join(ROOT, "tests", "test_oracle_dropout_pins.py")]

# (name, text in norm_oracle.c, replacement, occurrences replaced: 0 = all)
MUTANTS = [
    ("ln: unbiased variance", "double var = ss / (double)N;", "double var = ss / (double)(N - 1);", 1),
    ("ln: eps outside the root", "double r = 1.0 / sqrt(var + eps);", "double r = 1.0 / sqrt(var) + eps;", 1),
    ("ln: bias dropped", "y[i * N + j] = xhat * wj + bj;", "y[i * N + j] = xhat * wj;", 1),
    ("ln bwd: mean(g) term dropped", "rstd[i] * (g - c_g - xhat * c_gx)", "rstd[i] * (g - xhat * c_gx)", 1),
    ("ln bwd: sign of the xhat term", "rstd[i] * (g - c_g - xhat * c_gx)", "rstd[i] * (g - c_g + xhat * c_gx)", 1),
    ("ln bwd: db column index", "sb += dy[i * N + j];", "sb += dy[i * N + (N - 1 - j)];", 1),
    ("ln bwd: dw from x, not xhat", "sw += dy[i * N + j] * xhat;", "sw += dy[i * N + j] * x[i * N + j];", 1),
    ("rms: sum of squares, not mean", "double r = 1.0 / sqrt(ss / (double)N + eps);",
     "double r = 1.0 / sqrt(ss + eps);", 1),
    ("rms bwd: one factor of r dropped", "r * (g - xr[j] * r * r * c)", "r * (g - xr[j] * r * c)", 1),
    ("rms bwd: dw without rstd", "s += dy[i * N + j] * x[i * N + j] * rstd[i];",
     "s += dy[i * N + j] * x[i * N + j];", 1),
    ("bn: unbiased normalizing variance", "var_biased[c] = ss / n;", "var_biased[c] = ss / (n - 1.0);", 1),
    ("bn: biased running variance", "momentum * var[c] * n / (n - 1.0);", "momentum * var[c];", 1),
    ("bn: momentum on the old value", "(1.0 - momentum) * running_mean[c] + momentum * mu[c]",
     "momentum * running_mean[c] + (1.0 - momentum) * mu[c]", 1),
    ("bn: residual after the activation",
     "if (res) z += res[idx];\n                y[idx] = orc_act(act, act_p, z);",
     "y[idx] = orc_act(act, act_p, z) + (res ? res[idx] : 0.0);", 1),
    ("bn eval: eps outside the root", "double r = 1.0 / sqrt(running_var[c] + eps);",
     "double r = 1.0 / sqrt(running_var[c]) + eps;", 1),
    ("bn bwd: db term dropped", "(n * dz - sum_dz - xhat * sum_dz_xhat)", "(n * dz - xhat * sum_dz_xhat)", 1),
    ("bn bwd: dres before the activation", "if (dres) dres[idx] = dz;", "if (dres) dres[idx] = dy[idx];", 1),
    ("bn bwd: grad_at ignored", "if (grad_at && !isnan(grad_at[idx])) z = grad_at[idx];\n", "", 0),
    ("bn bwd: grad_at in the sums only", "if (grad_at && !isnan(grad_at[idx])) z = grad_at[idx];\n"
     "                double dz = dy[idx] * orc_act_grad(act, act_p, z);\n                dx[idx]",
     "double dz = dy[idx] * orc_act_grad(act, act_p, z);\n                dx[idx]", 1),
    ("gelu': z phi term dropped", "return Phi + z * phi;", "return Phi;", 1),
    ("relu'(0) = 1", "case ORC_ACT_RELU: return z > 0.0 ? 1.0 : 0.0;",
     "case ORC_ACT_RELU: return z >= 0.0 ? 1.0 : 0.0;", 1),
    ("silu': wrong factor", "return s * (1.0 + z * (1.0 - s));", "return s * (1.0 + z * s);", 1),
    ("mish': sigmoid factor dropped", "return t + z * sigm(z) * (1.0 - t * t);",
     "return t + z * (1.0 - t * t);", 1),
    ("leaky: slope ignored", "case ORC_ACT_LEAKY_RELU: return z > 0.0 ? z : p * z;",
     "case ORC_ACT_LEAKY_RELU: return z > 0.0 ? z : 0.01 * z;", 1),
    ("elu: alpha ignored", "case ORC_ACT_ELU: return z > 0.0 ? z : p * expm1(z);",
     "case ORC_ACT_ELU: return z > 0.0 ? z : expm1(z);", 1),
    ("celu: inner scale dropped", "return z > 0.0 ? z : p * expm1(z / p);", "return z > 0.0 ? z : p * expm1(z);", 1),
    ("selu: alpha dropped", "kSeluScale * (z > 0.0 ? z : kSeluAlpha * expm1(z))",
     "kSeluScale * (z > 0.0 ? z : expm1(z))", 1),
    ("softplus: threshold", "case ORC_ACT_SOFTPLUS: return z > 20.0 ? z : log1p(exp(z));",
     "case ORC_ACT_SOFTPLUS: return z > 2.0 ? z : log1p(exp(z));", 1),
    ("hardswish': kink sides", "return z <= -3.0 ? 0.0 : (z < 3.0 ? z / 3.0 + 0.5 : 1.0);",
     "return z < -3.0 ? 0.0 : (z <= 3.0 ? z / 3.0 + 0.5 : 1.0);", 1),
    ("welford: M2 update", "m2 += delta * (x[i] - mean);", "m2 += delta * delta;", 1),
    ("chan: merge term without / n", "delta * delta * a[0] * b[0] / n", "delta * delta * a[0] * b[0]", 1),
    ("philox: multiplier", "(uint64_t)0xD2511F53u * c0", "(uint64_t)0xD2511F55u * c0", 1),
    ("philox: Weyl key step", "k1 += 0xBB67AE85u;", "k1 += 0x9E3779B9u;", 1),
    ("mask: word order", "const uint32_t word = w[(e % 8) / 2];", "const uint32_t word = w[3 - (e % 8) / 2];", 1),
    ("mask: half order", "(e % 2 == 0) ? (word & 0xFFFFu) : (word >> 16)",
     "(e % 2 == 1) ? (word & 0xFFFFu) : (word >> 16)", 1),
    ("mask: four elements per counter", "const uint64_t blk = e / 8;", "const uint64_t blk = e / 4;", 1),
    ("mask: counter per element", "const uint64_t blk = e / 8;", "const uint64_t blk = e;", 1),
    ("mask: 24-bit threshold", "return (uint32_t)floor(p * 65536.0 + 0.5);",
     "return (uint32_t)floor(p * 16777216.0 + 0.5) >> 8;", 1),
    ("mask: seed high word", "(uint32_t)(seed >> 32)}", "0u}", 1),
    ("dropout: survivors not rescaled", "orc_act(act, act_p, x[i]) / (1.0 - p)", "orc_act(act, act_p, x[i])", 1),
    ("dropout: unmasked backward", "dx[i] = orc_kept(offset + (uint64_t)i, seed, t)", "dx[i] = 1", 1),
]


def _mutate(text, old, new, count):
    n = text.count(old)
    assert n >= 1, f"mutation text not found: {old!r}"
    return text.replace(old, new) if count == 0 else text.replace(old, new, count)


def _run_mutant(args):
    idx, (name, old, new, count), text, tmp = args
    src = os.path.join(tmp, f"mut{idx}.c")
    lib = os.path.join(tmp, f"libmut{idx}.so")
    with open(src, "w") as f:
        f.write(_mutate(text, old, new, count))
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-std=c11",
                    "-D_GNU_SOURCE", "-shared", "-fPIC", f"-I{os.path.dirname(SRC)}", src, "-o", lib,
                    "-lm"], check=True, capture_output=True)
    env = dict(os.environ, NORM_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *PINS], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    return name, r.returncode, r.stdout[-400:]


def test_every_mutant_fails_a_pin():
    text = open(SRC).read()
    for name, old, new, count in MUTANTS:  # every planting applies to the current source
        _mutate(text, old, new, count)
    with tempfile.TemporaryDirectory() as tmp:
        jobs = [(i, m, text, tmp) for i, m in enumerate(MUTANTS)]
        with ThreadPoolExecutor(max_workers=4) as pool:
            results = list(pool.map(_run_mutant, jobs))
    survivors = [(name, tail) for name, rc, tail in results if rc == 0]
    assert not survivors, "mutants that pass every pin: " + "; ".join(n for n, _ in survivors)
    # A mutant must fail a pin, not crash the interpreter.
    crashed = [name for name, rc, _ in results if rc not in (1,)]
    assert not crashed, f"mutants whose pin run did not end in a test failure: {crashed}"


def test_unmutated_oracle_passes_the_pins():
    """Control: the same harness on the unmodified source passes."""
    text = open(SRC).read()
    with tempfile.TemporaryDirectory() as tmp:
        name, rc, tail = _run_mutant((0, ("control", "", "", 1), text, tmp))
    assert rc == 0, tail
