"""Fits the polynomial behind the grouped GEMM's GELU epilogue.

GELU(z) = z Phi(z) = max(z, 0) - a Phi(-a) with a = |z|. The kernel evaluates
Phi(-a) as 2^P(a), P a degree-7 polynomial fitted by least squares to
log2 Phi(-a) on 0 <= a <= 6 (a is clamped to 6, where a Phi(-a) < 1e-8).
Run it to print the float32 coefficients and the error of the whole GELU
against the exact one, evaluated the way the kernel does it (float32 FMA
Horner steps, one exp2).
"""
import numpy as np
from scipy.special import log_ndtr, ndtr

A_MAX, DEG = 6.0, 7


def fit():
    a = np.linspace(0.0, A_MAX, 400001)
    u = a / A_MAX
    V = np.vander(u, DEG + 1, increasing=True)
    c_u, *_ = np.linalg.lstsq(V, log_ndtr(-a) / np.log(2.0), rcond=None)
    return (c_u / A_MAX ** np.arange(DEG + 1)).astype(np.float32)


def gelu_like_kernel(co, z):
    z = z.astype(np.float32)
    a = np.minimum(np.abs(z), np.float32(A_MAX))
    p = np.full_like(a, co[-1])
    for c in co[-2::-1]:   # fmaf(p, a, c): one rounding per step
        p = (p.astype(np.float64) * a + np.float64(c)).astype(np.float32)
    q = np.exp2(p.astype(np.float64)).astype(np.float32)
    return (np.maximum(z, 0).astype(np.float64) - a.astype(np.float64) * q).astype(np.float32)


if __name__ == "__main__":
    co = fit()
    print("coefficients c0..c7:", ", ".join(f"{float(c)!r}f" for c in co))
    z = np.linspace(-30, 30, 3000001)
    exact = z * ndtr(z)
    err = np.abs(gelu_like_kernel(co, z) - exact)
    big = np.abs(exact) > 1e-6
    print(f"max abs error {err.max():.2e}; max relative error where |GELU| > 1e-6: "
          f"{(err[big] / np.abs(exact[big])).max():.2e}")
