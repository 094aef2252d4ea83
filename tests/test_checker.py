"""The parity checker's bf16 bounds (tests/gpu_util.py) against the bf16 format itself."""

import numpy as np
import pytest

from gpu_util import BF16_MAX, BF16_MEAN, bf16_bounds, bf16_ulp, check


def _bf16_values(n, seed):
    # random positive normal bf16 numbers (as float64) and the next larger bf16 number
    rng = np.random.Generator(np.random.PCG64(seed))
    bits = rng.integers(0x0080, 0x7F7F, size=n, dtype=np.uint32)  # positive, normal, finite
    x = (bits << 16).view(np.float32).astype(np.float64)
    nxt = ((bits + 1) << 16).view(np.float32).astype(np.float64)
    return x, nxt


def test_ulp_is_the_spacing_of_bf16_numbers():
    x, nxt = _bf16_values(20000, 1)
    assert np.array_equal(bf16_ulp(x), nxt - x)
    assert np.array_equal(bf16_ulp(-x), nxt - x)
    assert bf16_ulp(1.0) == 2.0 ** -7 and bf16_ulp(4.73) == 2.0 ** -5 and bf16_ulp(8.0) == 2.0 ** -4


def test_bounds_relax_only_where_half_a_spacing_nears_the_budget():
    ref = np.array([0.0, 0.5, 1.0, 3.99, 4.0, 7.5, 8.0, 12.0])
    tol, _ = bf16_bounds(ref)
    assert np.all(tol[:4] == BF16_MAX)  # |ref| < 4: the stated 2e-2
    assert tol[4] == tol[5] == 2.0 ** -5 and tol[6] == tol[7] == 2.0 ** -4
    # the output rounding alone (half a spacing) always fits the bound, with as much again left
    x, _ = _bf16_values(5000, 2)
    tol, _ = bf16_bounds(x)
    assert np.all(tol >= bf16_ulp(x))
    # mean bound: the stated 2e-3 for outputs of order one
    _, m = bf16_bounds(np.random.Generator(np.random.PCG64(3)).standard_normal(4096) * 0.3)
    assert m == BF16_MEAN


def test_check_plain_bound_for_the_stated_workloads():
    ref = np.random.Generator(np.random.PCG64(4)).standard_normal(4096) * 0.5
    ref[7] = 4.73
    got = ref.copy()
    got[7] += 0.0224  # the error the format and the method allow at |ref| = 4.73 (0.72 spacing)
    check("edge", got, ref, "bf16")  # passes under the format-derived bound
    with pytest.raises(AssertionError):
        check("config", got, ref, "bf16", config=True)  # the stated workloads keep 2e-2
    got[7] = ref[7] + 0.04
    with pytest.raises(AssertionError):
        check("edge", got, ref, "bf16")  # more than one spacing (0.031) fails


def test_terms_widen_the_bound_only_by_their_first_order_size():
    # an output that is a cancelling sum: |ref| = 2 but its rounded terms add up to T = 40, so
    # the method's bf16 rounding may move it by up to 2^-8 (40 + 2) = 0.164
    rng = np.random.Generator(np.random.PCG64(5))
    ref = rng.standard_normal(4096) * 0.5
    terms = np.abs(ref) + 0.1
    ref[11], terms[11] = 2.0, 40.0
    got = ref.copy()
    got[11] += 0.15
    check("cancelling", got, ref, "bf16", terms=terms)  # inside u (T + |ref|)
    with pytest.raises(AssertionError):
        check("cancelling", got, ref, "bf16")  # without the terms: 2e-2 at |ref| = 2
    with pytest.raises(AssertionError):
        check("cancelling", got, ref, "bf16", config=True, terms=terms)  # the stated workloads ignore them
    got[11] = ref[11] + 0.2
    with pytest.raises(AssertionError):
        check("cancelling", got, ref, "bf16", terms=terms)  # past u (T + |ref|)
    got = ref + 0.05 * rng.choice([-1.0, 1.0], size=ref.size)  # a widespread error past 2e-2
    with pytest.raises(AssertionError):
        check("wrong", got, ref, "bf16", terms=terms)
