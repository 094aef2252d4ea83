"""Helpers for the GPU parity tests: upload seeded inputs, compare against the oracle."""

from __future__ import annotations

import sys

import numpy as np

# Tolerances (see the design notes): bf16 outputs max abs 2e-2 and mean abs 2e-3 against the
# fp64 oracle, fp32 outputs max abs 1e-5, logsumexp max abs 1e-3.
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


def check(name: str, got: np.ndarray, ref: np.ndarray, dtype: str, is_lse: bool = False):
    """Compare a GPU result (float64 view) with the oracle element by element."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite GPU values"
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    big = float(np.abs(ref).max())
    say(f"  {name}: max_abs={mx:.3e} mean_abs={mean:.3e} max|ref|={big:.3f} n={ref.size}")
    if is_lse:
        assert mx <= LSE_MAX, f"{name}: lse max abs {mx}"
    elif dtype == "f32":
        assert mx <= F32_MAX, f"{name}: fp32 max abs {mx}"
    else:
        assert mx <= BF16_MAX, f"{name}: bf16 max abs {mx} (max|ref|={big})"
        assert mean <= BF16_MEAN, f"{name}: bf16 mean abs {mean}"
    return mx, mean
