"""Fit the cubic used by the device function exp2_poly (fa_device.h).

2^x = 2^floor(x) * 2^f with f = x - floor(x) in [0, 1) (Cody-Waite style range reduction; the
power of two is added to the float's exponent field), and 2^f ~ p(f) = 1 + c1 f + c2 f^2 + c3 f^3
with p(0) = 1 exactly, the coefficients chosen to minimise the largest relative error on [0, 1)
(Lecture 21 notes §5.2 names Lawson's algorithm for this fit). Lawson's algorithm: repeated
weighted least squares whose weights are multiplied by the current absolute errors, which
converges to the minimax (equioscillating) solution.

Usage: python -m exact_io_aware_03_amd.fit_exp2   (prints the fp32 coefficients)
"""

from __future__ import annotations

import numpy as np


def fit(degree: int = 3, n: int = 4001, iters: int = 400) -> np.ndarray:
    f = np.linspace(0.0, 1.0, n)
    t = np.exp2(f)
    # relative residual (1 + sum c_k f^k - 2^f) / 2^f, linear in c
    a = np.stack([f ** k / t for k in range(1, degree + 1)], axis=1)
    b = (t - 1.0) / t
    w = np.full(n, 1.0 / n)
    c = None
    for _ in range(iters):
        sw = np.sqrt(w)
        c, *_ = np.linalg.lstsq(a * sw[:, None], b * sw, rcond=None)
        e = np.abs(a @ c - b)
        w = w * e
        w /= w.sum()
    return c


def max_rel_error(c: np.ndarray, n: int = 100001) -> float:
    f = np.linspace(0.0, 1.0, n)
    p = 1.0 + sum(ck * f ** (k + 1) for k, ck in enumerate(c))
    return float(np.max(np.abs(p / np.exp2(f) - 1.0)))


if __name__ == "__main__":
    c = fit()
    c32 = c.astype(np.float32)
    print("coefficients c1, c2, c3 (fp32):", ", ".join(f"{float(x):.9e}f" for x in c32))
    print(f"max relative error on [0, 1): {max_rel_error(c):.3e} (fp64 coefficients), "
          f"{max_rel_error(c32.astype(np.float64)):.3e} (fp32)")
