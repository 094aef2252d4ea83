"""FP8 quantise step of the FP8 attention path: random-sign Hadamard rotation of Q and K, one
scale per block of rows, rounding to the OCP E4M3 format.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product library never imports it.

Sources (cited by page and section):
  * "Lecture 21: Optimizing Attention for Modern Hardware (FlashAttention 1-4)", CMU 11-868
    notes -- §4.4 (FP8 and incoherent processing: one scale per block instead of per tensor;
    Q and K both multiplied by the same random orthogonal J, a random-sign Hadamard matrix, so
    (QJ)(KJ)^T = QK^T while outliers are spread over all dimensions; the fast transform costs
    O(d log d)) and exercise 8 (the rotation cancels in QK^T but not in PV, which is why V is
    not rotated).
  * "Flash Attention 3/4 笔记" (KaiSpace), section 4 (FP8 layout conversion and accuracy:
    block quantisation per Br x d block; incoherent processing with M built from a Hadamard
    transform and a random +-1 diagonal).

Readings where the pages are silent (listed in the design notes as well):
  * the format is OCP E4M3 (bias 7, largest finite value 448, no infinities, S.1111.111 is
    NaN), rounding is to nearest with ties to even, and values are clamped to +-448 first;
  * J = diag(signs) H_d / sqrt(d): the signs multiply first, then the (Sylvester, natural
    order) Hadamard transform, then 1/sqrt(d);
  * a block is 64 consecutive rows of one (batch, head); its scale is amax / 448 and its
    values are multiplied by 448 / amax (both fp32, correctly rounded) before rounding, so
    the block's largest magnitude maps to 448 (an all-zero block gets scale 1);
  * the rotation, the scale and the multiplication are done in fp32 in a fixed order (the
    butterfly stages h = 1, 2, 4, ..., d/2 with (a, b) -> (a + b, a - b)), because the code
    is an integer decided by floating point: the GPU makes the same decisions in fp32.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
BLOCK_ROWS = 64


def decode_e4m3(codes) -> np.ndarray:
    """Values (fp64) of OCP E4M3 codes: sign, 4-bit exponent (bias 7), 3-bit mantissa;
    exponent field 0 is subnormal (M * 2^-9); S.1111.111 is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def round_e4m3(x) -> np.ndarray:
    """OCP E4M3 code of each value, rounded to nearest with ties to even. |x| must be <= 448
    (the quantiser clamps first). Subnormal spacing is 2^-9; a normal value 2^e * f, f in
    [1, 2), has spacing 2^(e-3)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("round_e4m3 takes finite values with |x| <= 448")
    neg = np.signbit(x)
    a = np.abs(x)
    # subnormal range (below 2^-6): multiples of 2^-9; M = 8 is the smallest normal, code 0x08
    sub = np.rint(a * 2.0 ** 9)  # np.rint rounds halves to even
    f, E = np.frexp(a)  # a = f * 2^E, f in [0.5, 1)
    e = E - 1  # a = 2^e * (2f), 2f in [1, 2)
    m = np.rint(a * np.exp2(3.0 - e))  # in [8, 16]
    carry = m == 16
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 8, m)
    normal_code = ((e + 7) << 3) + (m.astype(np.int64) - 8)
    code = np.where(a < 2.0 ** -6, sub.astype(np.int64), normal_code)
    code = np.where(a == 0, 0, code)
    return (code | (neg.astype(np.int64) << 7)).astype(np.uint8)


def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix H_d (entries +-1, natural order), fp64; H H^T = d I."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def fwht_f32(x) -> np.ndarray:
    """x @ H_d along the last axis in fp32: butterfly stages h = 1, 2, 4, ..., d/2, each
    replacing the pair (x[i], x[i+h]) (bit h of i clear) with (a + b, a - b)."""
    y = np.array(x, dtype=np.float32)
    d = y.shape[-1]
    h = 1
    while h < d:
        v = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a, b = v[..., 0, :], v[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2).reshape(y.shape)
        h *= 2
    return y


def rotate_f32(x, signs) -> np.ndarray:
    """x J with J = diag(signs) H_d / sqrt(d), in fp32: signs, transform, then one multiply by
    the fp32 value of 1/sqrt(d)."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    s = np.asarray(signs, dtype=np.float32)
    return fwht_f32(x * s) * np.float32(1.0 / np.sqrt(d))


def quantize(x, signs=None, block: int = BLOCK_ROWS):
    """Quantise a BSHD tensor [B, N, H, d] to E4M3 with one scale per (b, h, block of rows).

    Returns (codes uint8 [B, N, H, d], scales fp32 [B, H, ceil(N/block)], dequantised fp64
    [B, N, H, d] = decode(code) * scale). With `signs` (d values of +-1) the rows are rotated
    by J first; the dequantised tensor is then in the rotated basis."""
    x = np.asarray(x, dtype=np.float32)
    B, N, H, d = x.shape
    y = rotate_f32(x, signs) if signs is not None else x.copy()
    nb = (N + block - 1) // block
    scales = np.ones((B, H, nb), dtype=np.float32)
    codes = np.zeros(x.shape, dtype=np.uint8)
    for i in range(nb):
        r0, r1 = i * block, min(N, (i + 1) * block)
        blk = y[:, r0:r1]  # [B, rows, H, d]
        amax = np.abs(blk).max(axis=(1, 3))  # [B, H]
        sc = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        safe = np.where(amax > 0, amax, np.float32(1.0)).astype(np.float32)
        inv = np.where(amax > 0, np.float32(E4M3_MAX) / safe, np.float32(1.0)).astype(np.float32)
        scales[:, :, i] = sc
        q = (blk * inv[:, None, :, None]).astype(np.float32)
        q = np.clip(q, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
        codes[:, r0:r1] = round_e4m3(q)
    rows = np.arange(N) // block
    deq = decode_e4m3(codes) * scales.astype(np.float64)[:, :, rows].transpose(0, 2, 1)[..., None]
    return codes, scales, deq
