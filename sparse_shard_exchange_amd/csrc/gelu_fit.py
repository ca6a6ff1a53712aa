"""Derive the constants of the GEMM epilogue's GELU (csrc/gemm.h, gelu()).

GELU(z) = z Phi(z). With h(a) = erfc(a / sqrt 2) / 2 for a = |z| >= 0, this is
z (1 - h) for z >= 0 and z h for z < 0, i.e. max(z, 0) - |z| h(|z|).

h is written as t 2^(P(t) - c a^2) with t = 1 / (1 + p a) and c = log2(e) / 2:
the Gaussian factor exp(-a^2 / 2) is exact in that form, and what is left,
log2(h / t) + c a^2, is a smooth function of t on (0, 1] with a finite limit
at t -> 0 (the asymptotic series of erfc), so a low-degree polynomial P fits
it with a small ABSOLUTE error, which is a RELATIVE error of h, uniformly over
the whole tail (the Chebyshev-style form t exp(-x^2 + poly(t)) of Numerical
Recipes' erfcc; the degree, p and coefficients here are fitted afresh).

The fit is minimax on a dense grid of a in [0, 16] (a linear program), for
degree 4 and the p that minimises the error. It prints the constants and the
maximum relative error of h and of GELU when the formula is evaluated in fp32
the way the kernel does (fused multiply-adds, fp32 reciprocal and exp2),
emulated here with fp32 rounding after every operation.

    python sparse_shard_exchange_amd/csrc/gelu_fit.py
"""
from __future__ import annotations

import numpy as np
from scipy.optimize import linprog
from scipy.special import erfc

C = np.log2(np.e) / 2.0
DEG = 4


def _grid(amax: float = 16.0, n: int = 6000) -> np.ndarray:
    return np.concatenate([np.linspace(0.0, 4.0, n // 2), np.linspace(4.0, amax, n // 2)])


def fit(p: float, deg: int = DEG):
    a = _grid()
    t = 1.0 / (1.0 + p * a)
    h = 0.5 * erfc(a / np.sqrt(2.0))
    f = np.log2(h / t) + C * a * a
    V = np.vander(t, deg + 1)
    m = len(t)
    A = np.block([[V, -np.ones((m, 1))], [-V, -np.ones((m, 1))]])
    b = np.concatenate([f, -f])
    cost = np.zeros(deg + 2)
    cost[-1] = 1.0
    r = linprog(cost, A_ub=A, b_ub=b, bounds=[(None, None)] * (deg + 1) + [(0, None)], method="highs")
    return r.x[-1] * np.log(2.0), r.x[:-1]  # max relative error of h, coefficients (highest first)


def best_fit(deg: int = DEG):
    best = None
    for p in np.linspace(0.15, 0.8, 66):
        e, co = fit(p, deg)
        if best is None or e < best[0]:
            best = (e, p, co)
    e, p, co = best
    for p2 in np.linspace(p - 0.01, p + 0.01, 21):
        e2, co2 = fit(p2, deg)
        if e2 < e:
            e, p, co = e2, p2, co2
    return e, float(np.float32(p)), co


def gelu_f32(z: np.ndarray, p: float, co) -> np.ndarray:
    """The kernel's evaluation order with fp32 rounding after each operation."""
    f = np.float32
    z = z.astype(np.float32)
    a = np.abs(z)
    t = (f(1.0) / (f(p) * a + f(1.0)).astype(np.float32)).astype(np.float32)
    q = np.full_like(z, f(co[0]))
    for c in co[1:]:
        q = (q.astype(np.float64) * t + np.float64(f(c))).astype(np.float32)
    zz = (z * z).astype(np.float32)
    u = (zz.astype(np.float64) * np.float64(f(-C)) + q).astype(np.float32)
    e = np.exp2(u.astype(np.float64)).astype(np.float32)
    h = (t * e).astype(np.float32)
    return ((-a).astype(np.float64) * h + np.maximum(z, f(0.0))).astype(np.float32)


def main():
    e, p, co = best_fit()
    co32 = [float(np.float32(c)) for c in co]
    print(f"p = {p!r}")
    print("coefficients, highest degree first:", [repr(np.float32(c)) for c in co32])
    print(f"max relative error of h on the grid (exact arithmetic): {e:.3e}")
    z = np.concatenate([-np.geomspace(1e-6, 12.0, 200001), np.geomspace(1e-6, 12.0, 200001), [0.0]])
    exact = 0.5 * z * erfc(-z / np.sqrt(2.0))
    got = gelu_f32(z, p, co32).astype(np.float64)
    nz = exact != 0
    rel = np.abs(got[nz] - exact[nz]) / np.abs(exact[nz])
    print(f"max relative error of GELU in emulated fp32 on z in [-12, 12]: {rel.max():.3e}")


if __name__ == "__main__":
    main()
