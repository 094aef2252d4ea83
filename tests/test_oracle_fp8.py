"""Pins for the FP8 quantise step of the oracle (oracle/fp8.py), from the definition of the
OCP E4M3 format, the algebra of the Hadamard transform, and the lecture's claim that the
rotation spreads outliers (Lecture 21 notes §4.4, exercise 8)."""

import math

import numpy as np
import pytest

from oracle import fp8

RNG = lambda s: np.random.Generator(np.random.PCG64(s))  # noqa: E731


def test_e4m3_table_spot_values():
    v = fp8.decode_e4m3(np.arange(256, dtype=np.uint8))
    assert v[0x38] == 1.0 and v[0xB8] == -1.0
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0  # largest finite: 1.75 * 2^8
    assert v[0x01] == 2.0 ** -9  # smallest subnormal: 1/8 * 2^-6
    assert v[0x08] == 2.0 ** -6  # smallest normal
    assert v[0x07] == 7 * 2.0 ** -9  # largest subnormal
    assert v[0x30] == 0.5 and v[0x44] == 3.0 and v[0x77] == 240.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isfinite(v).sum() == 254
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and np.signbit(v[0x80])


def test_e4m3_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(fp8.round_e4m3(fp8.decode_e4m3(codes)), codes)


def test_e4m3_ties_to_even_and_nearest():
    pos = np.array([c for c in range(0x7F)], dtype=np.uint8)  # 0x00 .. 0x7E, increasing values
    v = fp8.decode_e4m3(pos)
    assert np.all(np.diff(v) > 0)
    mid = (v[:-1] + v[1:]) / 2
    got = fp8.round_e4m3(mid)
    even = np.where(pos[:-1] % 2 == 0, pos[:-1], pos[1:])  # the code with mantissa LSB 0
    assert np.array_equal(got, even)
    # just off the midpoints: nearest neighbour
    assert np.array_equal(fp8.round_e4m3(mid - (v[1:] - v[:-1]) * 1e-6), pos[:-1])
    assert np.array_equal(fp8.round_e4m3(mid + (v[1:] - v[:-1]) * 1e-6), pos[1:])
    assert np.array_equal(fp8.round_e4m3(-mid), even | 0x80)


def test_e4m3_error_bound_and_monotone():
    x = np.sort(RNG(1).uniform(-448, 448, 20000))
    c = fp8.round_e4m3(x)
    y = fp8.decode_e4m3(c)
    assert np.all(np.diff(y) >= 0)
    a = np.abs(x)
    ulp = np.where(a < 2.0 ** -6, 2.0 ** -9, np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
    assert np.all(np.abs(y - x) <= ulp / 2 + 1e-300)
    with pytest.raises(ValueError):
        fp8.round_e4m3([449.0])


def test_hadamard_and_fast_transform():
    for d in (2, 8, 64, 128):
        h = fp8.hadamard(d)
        assert np.array_equal(h @ h.T, d * np.eye(d))
        x = RNG(d).integers(-50, 50, size=(7, d)).astype(np.float32)
        assert np.array_equal(fp8.fwht_f32(x).astype(np.float64), x.astype(np.float64) @ h)  # exact on integers
        xr = RNG(d + 1).standard_normal((5, d)).astype(np.float32)
        ref = xr.astype(np.float64) @ h
        assert np.abs(fp8.fwht_f32(xr) - ref).max() <= 1e-5 * np.abs(ref).max()


def test_rotation_is_orthogonal_and_cancels_in_scores():
    d = 128
    rng = RNG(5)
    signs = rng.choice([-1.0, 1.0], size=d)
    j = np.diag(signs) @ fp8.hadamard(d) / math.sqrt(d)
    assert np.abs(j @ j.T - np.eye(d)).max() < 1e-14
    q, k = rng.standard_normal((40, d)), rng.standard_normal((50, d))
    assert np.abs((q @ j) @ (k @ j).T - q @ k.T).max() < 1e-12  # (QJ)(KJ)^T = QK^T (exercise 8)
    # the fp32 rotation is the same map up to fp32 rounding
    assert np.abs(fp8.rotate_f32(q, signs) - q @ j).max() < 1e-5


def test_block_quantisation():
    rng = RNG(7)
    x = rng.standard_normal((2, 150, 3, 64)).astype(np.float32)
    x[:, 64:128, 1] = 0.0  # one all-zero block
    codes, scales, deq = fp8.quantize(x)
    assert scales.shape == (2, 3, 3)
    assert np.all(scales[:, 1, 1] == 1.0) and np.all(codes[:, 64:128, 1] == 0)
    vals = fp8.decode_e4m3(codes)
    for b in range(2):
        for h in range(3):
            for i, (r0, r1) in enumerate([(0, 64), (64, 128), (128, 150)]):
                blk = x[b, r0:r1, h].astype(np.float64)
                if not np.any(blk):
                    continue
                amax = np.abs(blk).max()
                assert scales[b, h, i] == np.float32(np.float32(amax) / np.float32(448.0))
                assert np.abs(vals[b, r0:r1, h]).max() == 448.0  # the block's largest value hits 448
                # dequantisation error: half a spacing of E4M3 (relative 2^-4), or 2^-10 * scale
                err = np.abs(deq[b, r0:r1, h] - blk)
                assert np.all(err <= np.maximum(np.abs(blk) * 2.0 ** -4, 2.0 ** -10 * scales[b, h, i]) * (1 + 1e-6))


def test_rotation_spreads_outliers():
    # "normal + 0.1% large values" (§4.4): every rotated coordinate is a +-1-weighted sum of all
    # input coordinates over sqrt(d), so a lone large value is spread and max/RMS drops sharply
    # (the page reports 26.9 -> 5.0 on its data); the RMS itself is unchanged (J is orthogonal)
    rng = RNG(11)
    n, d = 1024, 128
    q = rng.standard_normal((1, n, 1, d)).astype(np.float32)
    q[rng.random(q.shape) < 0.001] *= 30.0
    signs = rng.choice([-1.0, 1.0], size=d)
    rq = fp8.rotate_f32(q, signs).astype(np.float64)
    rms = lambda t: np.sqrt((np.asarray(t, np.float64) ** 2).mean())  # noqa: E731
    assert abs(rms(rq) / rms(q) - 1) < 1e-5
    assert np.abs(q).max() / rms(q) > 3 * np.abs(rq).max() / rms(rq)
