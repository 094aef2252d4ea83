"""Helpers for the GPU parity tests: upload seeded inputs, compare against the oracle."""

from __future__ import annotations

import sys

import numpy as np

# Tolerances (stated for the five workloads): bf16 outputs max abs 2e-2 and mean abs 2e-3
# against the fp64 oracle, fp32 outputs max abs 1e-5, logsumexp max abs 1e-3.
BF16_MAX, BF16_MEAN, F32_MAX, LSE_MAX = 2e-2, 2e-3, 1e-5, 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype: str):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def to_np(t) -> np.ndarray:
    import torch

    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def bf16_ulp(x) -> np.ndarray:
    """Spacing of bf16 numbers at |x|: 2^(e - 7) for 2^e <= |x| < 2^(e + 1) (8 significant bits)."""
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


U_BF16 = 2.0 ** -8  # bf16 unit roundoff: 8 significant bits, round to nearest even


def bf16_bounds(ref: np.ndarray, terms=None):
    """Per-element max-abs bound and mean-abs bound for a bf16 output whose exact value is ref.

    The stated absolute bounds (2e-2, 2e-3) presume outputs of order one. A bf16 output is the
    RNE rounding of the kernel's fp32 value, which alone moves it by up to half a bf16 spacing
    (2^-6 = 0.0156 for |x| in [4, 8), 2^-5 = 0.031 for |x| in [8, 16)); on top of that the
    method rounds P (and dS in the backward) to bf16 before the products, a relative error of
    at most 2^-8 per term, i.e. at most another half spacing for a sum whose terms do not
    cancel. Without `terms` the bound per element is therefore max(2e-2, one bf16 spacing of
    |ref|), which is 2e-2 for |ref| < 4 and relaxes only above; the mean bound is max(2e-3,
    half the mean spacing), twice the expected effect of the output rounding alone.

    Where the terms of a sum cancel, its rounding error is not tied to |ref|. `terms` are then
    the oracle's first-order sizes T of the rounded terms (oracle.rounding), and each element
    may also be off by u (T + |ref|), u = 2^-8: the method's bf16 rounding of P, of dS and of the
    O that D is formed from, and of the output, added up without cancellation. The mean bound
    may then also be a quarter of the mean of that (measured: at most a tenth)."""
    ulp = bf16_ulp(ref)
    tol, tol_mean = np.maximum(BF16_MAX, ulp), max(BF16_MEAN, 0.5 * float(ulp.mean()))
    if terms is not None:
        first = U_BF16 * (np.asarray(terms, dtype=np.float64) + np.abs(ref))
        tol = np.maximum(tol, first)
        tol_mean = max(tol_mean, 0.25 * float(first.mean()))
    return tol, tol_mean


def check(name: str, got: np.ndarray, ref: np.ndarray, dtype: str, is_lse: bool = False, config: bool = False,
          terms=None):
    """Compare a GPU result (float64 view) with the oracle element by element.

    config=True marks one of the five stated workloads: bf16 outputs must meet the plain
    bounds (max abs 2e-2, mean abs 2e-3). Other cases (small, ragged and edge shapes, where
    GQA sums and short rows make some outputs large) use the format-derived bounds of
    bf16_bounds. Either way, elements with |ref| >= 4 (where half a bf16 spacing is already
    0.0156) and |ref| >= 8 (where it exceeds 2e-2) are counted and their largest error is
    reported in bf16 spacings. `terms` (oracle.rounding's sizes, for outputs that are sums which
    may cancel) widen the bounds of the other cases as bf16_bounds describes."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite GPU values"
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    big = float(np.abs(ref).max())
    msg = f"  {name}: max_abs={mx:.3e} mean_abs={mean:.3e} max|ref|={big:.3f} n={ref.size}"
    if not is_lse and dtype != "f32":
        for lim in (4.0, 8.0):
            sel = np.abs(ref) >= lim
            if sel.any():
                in_ulp = float((err[sel] / bf16_ulp(ref[sel])).max())
                msg += f" | {int(sel.sum())} with |ref|>={lim:g}: max err {float(err[sel].max()):.3e} = {in_ulp:.2f} ulp"
    say(msg)
    if is_lse:
        assert mx <= LSE_MAX, f"{name}: lse max abs {mx}"
    elif dtype == "f32":
        assert mx <= F32_MAX, f"{name}: fp32 max abs {mx}"
    elif config:
        assert mx <= BF16_MAX, f"{name}: bf16 max abs {mx} (max|ref|={big})"
        assert mean <= BF16_MEAN, f"{name}: bf16 mean abs {mean}"
    else:
        tol, tol_mean = bf16_bounds(ref, terms)
        worst = int(np.argmax(err / tol))
        assert err.flat[worst] <= tol.flat[worst], (
            f"{name}: bf16 error {err.flat[worst]:.4e} at |ref|={abs(ref.flat[worst]):.3f} over its bound "
            f"{tol.flat[worst]:.4e}")
        assert mean <= tol_mean, f"{name}: bf16 mean abs {mean} over {tol_mean}"
    return mx, mean
