"""Fit of the exponent polynomial used by gelu_fast_rel (norm_device.hpp).

The fp16 GELU forward writes erfc(u) / 2 as t * 2^(-u^2 log2(e) + P(t)),
t = 1 / (1 + u / 2), the functional form of Press et al., Numerical Recipes
(2nd ed., section 6.2).  P(t) = log2(erfcx(u) / t) - 1 (erfcx(u) =
exp(u^2) erfc(u); the -1 is the 1/2) is smooth in t on (0, 1]; this script
fits it with a degree-5 polynomial, weighted least squares on Chebyshev
nodes of t for u in [0, 8] with Lawson's reweighting towards the minimax
fit, then reports the error of the fit and of the float32 GELU built from
it (float32 rounding emulated step by step, z on a dense grid over
[-12, 12]).  Run: python gelu_erfc_fit.py.  A development aid: nothing
imports it.
"""
import numpy as np
from scipy.special import erfc, erfcx

DEG = 5
U_MAX = 8.0


def target(t):
    u = 2.0 * (1.0 / t - 1.0)
    return np.log2(erfcx(u)) - np.log2(t) - 1.0


def fit():
    t_min = 1.0 / (1.0 + U_MAX / 2.0)
    k = np.arange(6000)
    t = t_min + (1.0 - t_min) * (np.cos(np.pi * (k + 0.5) / 6000) + 1.0) / 2.0
    w = np.ones_like(t)
    for _ in range(60):
        a = np.vander(t, DEG + 1) * np.sqrt(w)[:, None]
        c, *_ = np.linalg.lstsq(a, target(t) * np.sqrt(w), rcond=None)
        e = np.abs(np.polyval(c, t) - target(t))
        w = w * (e / e.max() + 1e-3)
        w /= w.sum()
    return c, t_min


def fma32(a, b, c):
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64) + np.asarray(c, np.float64)).astype(np.float32)


def gelu32(z, c):
    c = c.astype(np.float32)
    z = z.astype(np.float32)
    az = np.abs(z)
    t = (np.float32(1.0) / fma32(az, np.float32(0.35355339), np.float32(1.0))).astype(np.float32)
    p = fma32(t, c[0], c[1])
    for ci in c[2:-1]:
        p = fma32(t, p, ci)
    arg = fma32(t, p, fma32(z, (z * np.float32(-0.7213475108)).astype(np.float32), c[-1]))
    h = (t * np.exp2(arg).astype(np.float32)).astype(np.float32)
    return fma32(-az, h, np.maximum(z, np.float32(0.0)))


def main():
    c, t_min = fit()
    tt = np.linspace(t_min, 1.0, 400001)
    err = np.abs(np.polyval(c, tt) - target(tt)).max()
    print("P(t), highest degree first (log2 units):", ", ".join(f"{x:.9e}" for x in c))
    print(f"relative error of erfc on u in [0, {U_MAX}]: {err * np.log(2.0):.2e}")
    z = np.linspace(-12.0, 12.0, 2000001)
    ref = z * 0.5 * erfc(-z / np.sqrt(2.0))
    got = gelu32(z, c).astype(np.float64)
    m = np.abs(ref) > 2.0 ** -24
    rel = (np.abs(got - ref)[m] / np.abs(ref[m])).max()
    print(f"float32 GELU, relative error where |GELU| > 2^-24: {rel:.2e} ({rel / 2.0 ** -10:.4f} fp16 ulp)")


if __name__ == "__main__":
    main()
