"""Attention with dropout on the probabilities, and the counter-based generator its mask comes from.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product library never imports it.

Sources (cited by page and section):
  * "Lecture 21: Optimizing Attention for Modern Hardware (FlashAttention 1-4)", CMU 11-868
    notes -- §2.8 (dropout: keep the seed, not the mask; the mask of block (i, j) depends only
    on (seed, i, j) and forward and backward regenerate it with a counter-based generator such
    as Philox) and exercise 4 (with O = (P * Z / (1 - p)) V the identity
    sum_k P_ik dP_ik = dO_i . O_i still holds, dP taken through the dropout).
  * J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random numbers: as easy as
    1, 2, 3" (SC'11): the Philox4x32-10 generator (multipliers 0xD2511F53, 0xCD9E8D57, Weyl
    key increments 0x9E3779B9, 0xBB67AE85, ten rounds).

Readings where the pages are silent (listed in the design notes as well):
  * dropout acts on the normalised probabilities: O = (P * Z / (1 - p)) V; L stays the
    logsumexp of the scores without dropout;
  * p is used at 1/256 resolution: t = min(255, floor(256 p)), an element is kept when its
    random byte is >= t, and kept values are scaled by 256 / (256 - t);
  * one Philox call covers a 4 x 4 block of (query row, key) positions of one (batch, query
    head): counter = (key // 4, row // 4, b * H_q + h, offset), key = (seed mod 2^32,
    seed // 2^32); output word (row % 4) holds the bytes of keys 4 (key // 4) .. +3, byte
    (key % 4) (little-endian) for the key.
"""

from __future__ import annotations

import numpy as np

from . import attention as att

PHILOX_M = (0xD2511F53, 0xCD9E8D57)
PHILOX_W = (0x9E3779B9, 0xBB67AE85)
MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key) -> np.ndarray:
    """Philox4x32-10 of counters `ctr` (uint [..., 4]) under key (k0, k1): ten rounds of
    (c0, c1, c2, c3) -> (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)), the key
    advancing by the Weyl increments after every round. Returns uint32 [..., 4]."""
    c = np.asarray(ctr, dtype=np.uint64) & MASK32
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0, k1 = np.uint64(key[0]) & MASK32, np.uint64(key[1]) & MASK32
    m0, m1 = np.uint64(PHILOX_M[0]), np.uint64(PHILOX_M[1])
    for _ in range(10):
        p0, p1 = m0 * c0, m1 * c2  # < 2^64: exact in uint64
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & MASK32, (p0 >> np.uint64(32)) ^ c3 ^ k1, p0 & MASK32)
        k0 = (k0 + np.uint64(PHILOX_W[0])) & MASK32
        k1 = (k1 + np.uint64(PHILOX_W[1])) & MASK32
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def threshold(p: float) -> int:
    """Byte threshold t for dropout probability p in [0, 1): keep iff byte >= t."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return min(255, int(np.floor(256.0 * p)))


def keep_mask_head(bh: int, Nq: int, Nk: int, p: float, seed: int, offset: int) -> np.ndarray:
    """Z [Nq, Nk] (bool) of one (batch, query head) with index bh = b * H_q + h."""
    t = threshold(p)
    key = (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    nr, nc = (Nq + 3) // 4, (Nk + 3) // 4
    rg, cg = np.meshgrid(np.arange(nr), np.arange(nc), indexing="ij")
    ctr = np.stack([cg, rg, np.full_like(rg, bh), np.full_like(rg, offset & 0xFFFFFFFF)], axis=-1)
    words = philox4x32_10(ctr, key)  # [nr, nc, 4]: word r = row 4 rg + r
    by = words[..., None].view(np.uint8).reshape(nr, nc, 4, 4)  # [.., row % 4, key % 4], little-endian
    return (by >= t).transpose(0, 2, 1, 3).reshape(nr * 4, nc * 4)[:Nq, :Nk]


def keep_mask(B: int, Hq: int, Nq: int, Nk: int, p: float, seed: int, offset: int) -> np.ndarray:
    """Z [B, Hq, Nq, Nk] (bool): the kept positions, from one Philox call per 4 x 4 block."""
    z = np.zeros((B, Hq, Nq, Nk), dtype=bool)
    for b in range(B):
        for h in range(Hq):
            z[b, h] = keep_mask_head(b * Hq + h, Nq, Nk, p, seed, offset)
    return z


def _heads(B, Hq, Hkv):
    g = Hq // Hkv
    return [(b, h, h // g) for b in range(B) for h in range(Hq)]


def forward(q, k, v, keep, p: float, causal: bool = False, scale: float | None = None):
    """O = (P * Z / (1 - p_t)) V with p_t = t / 256, and L (without dropout), in fp64."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    B, Nq, Hq, d = q.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    r = 256.0 / (256 - threshold(p))
    _, lse = att.forward(q, k, v, causal, scale)
    o = np.zeros_like(q)
    for b, h, g in _heads(B, Hq, k.shape[2]):
        pm = att.probabilities(q[b, :, h], k[b, :, g], scale, causal)
        o[b, :, h] = (pm * keep[b, h] * r) @ v[b, :, g]
    return o, lse


def backward(q, k, v, do, keep, p: float, causal: bool = False, scale: float | None = None):
    """dQ, dK, dV (fp64) of f = sum(O * dO) for the dropout forward above, from the definition:
    with Pd = P * Z r, dV = Pd^T dO, dPd = dO V^T, dP = dPd * Z r, dS = P * (dP - rowsum(P dP)),
    dQ = scale dS K, dK = scale dS^T Q (GQA: dK, dV summed over a group's heads)."""
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    B, Nq, Hq, d = q.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    r = 256.0 / (256 - threshold(p))
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b, h, g in _heads(B, Hq, k.shape[2]):
        pm = att.probabilities(q[b, :, h], k[b, :, g], scale, causal)
        zr = keep[b, h] * r
        dv[b, :, g] += (pm * zr).T @ do[b, :, h]
        dp = (do[b, :, h] @ v[b, :, g].T) * zr
        ds = pm * (dp - (pm * dp).sum(axis=1, keepdims=True))
        dq[b, :, h] = scale * ds @ k[b, :, g]
        dk[b, :, g] += scale * ds.T @ q[b, :, h]
    return dq, dk, dv
