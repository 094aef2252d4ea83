"""Pins for the dropout oracle (oracle/dropout.py): the Philox4x32-10 known-answer vectors of
the generator's authors, the block mapping checked element by element against single calls,
the keep rate, p = 0 against the attention oracle, exercise 4's identity, and finite
differences of the dropout backward (Lecture 21 notes §2.8, exercise 4)."""

import numpy as np
import pytest

from oracle import attention as ora
from oracle import dropout as odp

RNG = lambda s: np.random.Generator(np.random.PCG64(s))  # noqa: E731


@pytest.mark.parametrize("ctr,key,expect", [
    # known-answer vectors published with the generator (Salmon et al., SC'11, Random123)
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
])
def test_philox_known_answers(ctr, key, expect):
    assert tuple(int(x) for x in odp.philox4x32_10(np.array(ctr), key)) == expect


def test_block_mapping_element_by_element():
    B, Hq, Nq, Nk, p, seed, off = 2, 3, 13, 22, 0.4, 0x1234567890AB, 77
    z = odp.keep_mask(B, Hq, Nq, Nk, p, seed, off)
    t = odp.threshold(p)
    key = (seed & 0xFFFFFFFF, seed >> 32)
    rng = RNG(1)
    for _ in range(200):
        b, h, i, j = rng.integers(B), rng.integers(Hq), rng.integers(Nq), rng.integers(Nk)
        w = odp.philox4x32_10(np.array([j // 4, i // 4, b * Hq + h, off]), key)[i % 4]
        byte = (int(w) >> (8 * (j % 4))) & 0xFF
        assert z[b, h, i, j] == (byte >= t)


def test_keep_rate_and_independence():
    p = 0.3
    t = odp.threshold(p)
    assert t == 76
    z = odp.keep_mask(2, 2, 256, 256, p, 42, 0)
    q = (256 - t) / 256
    n = z.size
    assert abs(z.mean() - q) < 5 * np.sqrt(q * (1 - q) / n)
    z2 = odp.keep_mask(2, 2, 256, 256, p, 42, 1)  # another offset: an independent mask
    assert abs((z != z2).mean() - 2 * q * (1 - q)) < 0.01
    assert odp.keep_mask(1, 1, 8, 8, 0.0, 5, 0).all() and odp.threshold(0.999) == 255
    with pytest.raises(ValueError):
        odp.threshold(1.0)


def _inputs(B, N, Hq, Hkv, d, seed):
    rng = RNG(seed)
    return [rng.standard_normal((B, N, h, d)) for h in (Hq, Hkv, Hkv, Hq)]


def test_p_zero_is_plain_attention():
    q, k, v, do = _inputs(1, 37, 4, 2, 16, 3)
    keep = odp.keep_mask(1, 4, 37, 37, 0.0, 9, 0)
    for causal in (False, True):
        o, l = odp.forward(q, k, v, keep, 0.0, causal, 0.3)
        ro, rl = ora.forward(q, k, v, causal, 0.3)
        assert np.abs(o - ro).max() < 1e-13 and np.abs(l - rl).max() < 1e-13
        g = odp.backward(q, k, v, do, keep, 0.0, causal, 0.3)
        rg = ora.backward(q, k, v, do, causal, 0.3)
        assert max(np.abs(a - b).max() for a, b in zip(g, rg)) < 1e-12


def test_exercise_4_identity_with_dropout():
    q, k, v, do = _inputs(1, 29, 1, 1, 8, 4)
    keep = odp.keep_mask(1, 1, 29, 29, 0.5, 11, 3)
    o, _ = odp.forward(q, k, v, keep, 0.5, True, 0.4)
    r = 256.0 / (256 - odp.threshold(0.5))
    pm = ora.probabilities(q[0, :, 0], k[0, :, 0], 0.4, True)
    dp = (do[0, :, 0] @ v[0, :, 0].T) * keep[0, 0] * r
    assert np.abs((pm * dp).sum(1) - (do[0, :, 0] * o[0, :, 0]).sum(1)).max() < 1e-13


def test_dropout_backward_finite_differences():
    q, k, v, do = _inputs(1, 11, 2, 1, 4, 5)
    keep = odp.keep_mask(1, 2, 11, 11, 0.25, 13, 0)
    for causal in (False, True):
        f = lambda q_, k_, v_: (odp.forward(q_, k_, v_, keep, 0.25, causal, 0.7)[0] * do).sum()  # noqa: E731
        dq, dk, dv = odp.backward(q, k, v, do, keep, 0.25, causal, 0.7)
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            for idx in [(0, 0, 0, 0), (0, 5, 0, 3), (0, 10, x.shape[2] - 1, 1)]:
                e = np.zeros_like(x)
                e[idx] = 1e-6
                args = {"q": [q, k, v], "k": [q, k, v], "v": [q, k, v]}[name]
                pos = [a + e if n == name else a for a, n in zip(args, "qkv")]
                neg = [a - e if n == name else a for a, n in zip(args, "qkv")]
                fd = (f(*pos) - f(*neg)) / 2e-6
                assert abs(fd - g[idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx, fd, g[idx])
