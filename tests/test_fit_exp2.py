"""The cubic of exp2_poly: the constants in fa_device.h are what fit_exp2.py's Lawson fit gives,
and the fit is minimax (its relative error equioscillates: 4 extrema of equal size, alternating
in sign, with p(0) = 1 fixed)."""

import os
import re

import numpy as np

from exact_io_aware_03_amd import fit_exp2

HERE = os.path.dirname(os.path.abspath(__file__))


def device_coefficients():
    text = open(os.path.join(HERE, "..", "exact_io_aware_03_amd", "csrc", "fa_device.h")).read()
    body = text[text.index("float exp2_poly(float x)"):]
    body = body[:body.index("}")]
    nums = [float(x) for x in re.findall(r"([0-9]\.[0-9]+e[-+][0-9]+)f", body)]
    c3, c2, c1 = nums[:3]  # Horner order in the source
    return np.array([c1, c2, c3])


def test_device_constants_are_the_fit():
    c = fit_exp2.fit().astype(np.float32).astype(np.float64)
    assert np.allclose(device_coefficients(), c, rtol=2e-7, atol=0)


def test_fit_is_minimax():
    c = fit_exp2.fit()
    f = np.linspace(0.0, 1.0, 200001)
    e = (1.0 + c[0] * f + c[1] * f ** 2 + c[2] * f ** 3) / np.exp2(f) - 1.0
    assert e[0] == 0.0  # p(0) = 1
    emax = np.abs(e).max()
    assert emax < 9e-5
    # interior extrema and the end point f = 1 all reach the same magnitude, alternating in sign
    idx = [i for i in range(1, len(f) - 1) if abs(e[i]) >= abs(e[i - 1]) and abs(e[i]) >= abs(e[i + 1])]
    ext = [e[i] for i in idx] + [e[-1]]
    big = [x for x in ext if abs(x) > 0.99 * emax]
    assert len(big) >= 3
    assert all(np.sign(a) != np.sign(b) for a, b in zip(big, big[1:]))
