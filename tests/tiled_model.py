"""fp64 CPU model of the tiled schedule the HIP kernels follow (test code, not the oracle).

It reproduces the order of operations of the GPU path -- online softmax over K/V tiles with
whole-tile causal skipping, split-KV partials merged by logsumexp, and the K/V-outer
backward that rebuilds P from the saved logsumexp -- so that the schedule itself can be
checked against the plain definition without a GPU. It shares no code with oracle/.

Sources: Lecture 21 notes (CMU 11-868), §2.2 (online update of m, l and the output),
§2.5 (whole-tile causal skip), §2.6 (recompute backward with D = rowsum(dO * O), K/V-outer
loop with dQ accumulated across blocks), §3.2 (deferred normalisation, only L stored),
§6.1 (Flash-Decoding partials and their merge); exercise 3 (the merge is associative and
commutative).
"""

from __future__ import annotations

import math

import numpy as np


def fwd_tiled(qh, kh, vh, scale, causal, br=128, bc=64, order=None):
    """Online-softmax forward over Q blocks (outer) and K/V tiles (inner), base-2 exponent.

    Returns (O, L) with L the natural-log logsumexp. `order` is the Q-block visiting order
    (longest-first for causal); the result must not depend on it.
    """
    nq, d = qh.shape
    nk = kh.shape[0]
    c = scale / math.log(2.0)  # scores in log2 units: exp(x) = 2^(x / ln 2)
    o = np.zeros((nq, vh.shape[1]))
    lse = np.zeros(nq)
    nblk = -(-nq // br)
    blocks = range(nblk) if order is None else order
    for i in blocks:
        r0, r1 = i * br, min(nq, (i + 1) * br)
        rows = np.arange(r0, r1)
        m = np.full(r1 - r0, -np.inf)
        l = np.zeros(r1 - r0)
        acc = np.zeros((r1 - r0, vh.shape[1]))
        last = min(nk, r1) if causal else nk  # keys past the block's last query are skipped
        for j0 in range(0, last, bc):
            j1 = min(nk, j0 + bc)
            s = c * (qh[r0:r1] @ kh[j0:j1].T)
            if causal and j1 - 1 > r0:  # tile crosses the diagonal: mask in-tile
                s = np.where(np.arange(j0, j1)[None, :] > rows[:, None], -np.inf, s)
            mn = np.maximum(m, s.max(axis=1))
            alpha = np.exp2(m - mn)
            p = np.exp2(s - mn[:, None])
            l = alpha * l + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ vh[j0:j1]
            m = mn
        o[r0:r1] = acc / l[:, None]
        lse[r0:r1] = (m + np.log2(l)) * math.log(2.0)
    return o, lse


def fwd_tiled_lazy(qh, kh, vh, scale, tau, bc=128):
    """Non-causal online softmax in fp32 with conditional rescaling (Lecture 21 notes §5.3):
    the reference max m of a row moves only when a tile's max exceeds it by more than tau
    (base-2 units), so P = 2^(s - m) may reach 2^tau; acc and l are rescaled only then.

    Returns (O, L, rescales) with rescales the number of reference moves per row (the first
    tile's counts as one)."""
    f32 = np.float32
    q, k, v = (np.asarray(t, dtype=f32) for t in (qh, kh, vh))
    nq, nk = q.shape[0], k.shape[0]
    c = f32(scale / math.log(2.0))
    m = np.full(nq, -np.inf, dtype=f32)
    l = np.zeros(nq, dtype=f32)
    acc = np.zeros((nq, v.shape[1]), dtype=f32)
    moves = np.zeros(nq, dtype=np.int64)
    with np.errstate(over="ignore", invalid="ignore"):
        for j0 in range(0, nk, bc):
            j1 = min(nk, j0 + bc)
            s = (q @ k[j0:j1].T) * c
            tmax = s.max(axis=1)
            move = tmax > m + f32(tau)
            mn = np.where(move, tmax, m).astype(f32)
            alpha = np.exp2(m - mn).astype(f32)  # 1 where the reference stays, 0 at the first tile
            p = np.exp2(s - mn[:, None]).astype(f32)
            l = (alpha * l + p.sum(axis=1, dtype=f32)).astype(f32)
            acc = (alpha[:, None] * acc + p @ v[j0:j1]).astype(f32)
            moves += move
            m = mn
        o = acc / l[:, None]
        lse = (m.astype(np.float64) + np.log2(l.astype(np.float64))) * math.log(2.0)
    return o, lse, moves


def decode_partials(q, kh, vh, n, scale, chunk):
    """Split-KV partials (m2, l, o) for one sequence and one kv head; q is [G, d]."""
    c = scale / math.log(2.0)
    parts = []
    for j0 in range(0, n, chunk):
        j1 = min(n, j0 + chunk)
        s = c * (q @ kh[j0:j1].T)
        m = s.max(axis=1)
        p = np.exp2(s - m[:, None])
        parts.append((m, p.sum(axis=1), p @ vh[j0:j1]))
    return parts


def merge(a, b):
    """Merge two partials expressed relative to their own maxima."""
    ma, la, oa = a
    mb, lb, ob = b
    m = np.maximum(ma, mb)
    fa, fb = np.exp2(ma - m), np.exp2(mb - m)
    return m, fa * la + fb * lb, fa[:, None] * oa + fb[:, None] * ob


def finish(part):
    m, l, o = part
    return o / l[:, None], (m + np.log2(l)) * math.log(2.0)


def bwd_tiled(qh, kh, vh, doh, lse, scale, causal, br=64, bc=128):
    """K/V-outer backward: per K/V block, loop over the Q blocks that see it.

    P is rebuilt as exp(scale*S - L); D = rowsum(dO * O) comes from a pre-pass over O.
    dK, dV stay with their block; dQ is accumulated across blocks (atomics on the GPU).
    """
    nq, nk = qh.shape[0], kh.shape[0]
    o, _ = fwd_tiled(qh, kh, vh, scale, causal)
    dd = (doh * o).sum(axis=1)
    dq = np.zeros_like(qh)
    dk = np.zeros_like(kh)
    dv = np.zeros_like(vh)
    for j0 in range(0, nk, bc):
        j1 = min(nk, j0 + bc)
        cols = np.arange(j0, j1)
        first = (j0 // br) * br if causal else 0  # Q blocks entirely above the tile are skipped
        for r0 in range(first, nq, br):
            r1 = min(nq, r0 + br)
            rows = np.arange(r0, r1)
            s = scale * (qh[r0:r1] @ kh[j0:j1].T)
            p = np.exp(s - lse[r0:r1, None])
            if causal:
                p = np.where(cols[None, :] > rows[:, None], 0.0, p)
            dv[j0:j1] += p.T @ doh[r0:r1]
            dp = doh[r0:r1] @ vh[j0:j1].T
            ds = p * (dp - dd[r0:r1, None])
            dk[j0:j1] += scale * (ds.T @ qh[r0:r1])
            dq[r0:r1] += scale * (ds @ kh[j0:j1])
    return dq, dk, dv
