"""fp64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg
may import this module. The product library (exact_io_aware_03_amd) never imports it, and this
module imports nothing from the product: the two share no code.

What it computes is the plain definition, written out in three steps per (batch, head):

    S = scale * Q K^T,   P = softmax(S) row by row (masked entries excluded),   O = P V,
    L = m + ln(sum_j exp(S_ij - m)),  m = max_j S_ij  (the per-row logsumexp).

Sources (cited by page and section):
  * "Lecture 21: Optimizing Attention for Modern Hardware (FlashAttention 1-4)", CMU 11-868
    notes -- §0.4 (notation: S, P, L = m + log l), §1.4 (standard attention as three kernels:
    S, then P, then O), §2.2 (subtracting the row maximum for stability), §2.5 (causal: query
    i sees keys up to i), §2.6 (backward formulas and the identity sum_k P_ik dP_ik = dO_i.O_i),
    §6.1 (decode: one query against the whole cached sequence).
  * "FlashAttention Tiling 策略与在线 Softmax" (ybb.press), §1 (the S, P, O definition).

Readings where the pages are silent (each is listed in the design notes as well):
  * scale multiplies the raw scores before the max and the exp; L is the natural-log
    logsumexp of the scaled scores;
  * causal means key j is visible to query i iff j <= i (top-left aligned, N_q == N_k);
  * GQA: query head h uses kv head h // (H_q // H_kv);
  * the backward is the vector-Jacobian product of f = sum(O * dO); no gradient flows
    through L; dQ and dK carry the scale factor that the lecture omits.

Rows are independent, so each head is processed in row blocks; a block whose rows all mask a
column range simply does not compute it. That changes nothing in the arithmetic that
defines each row.
"""

from __future__ import annotations

import numpy as np

_ROW_BLOCK = 1024


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _visible_cols(row: int, nk: int, causal: bool) -> int:
    """Number of leading keys visible to query `row` (causal: j <= row)."""
    return min(row + 1, nk) if causal else nk


def scores(qh: np.ndarray, kh: np.ndarray, scale: float) -> np.ndarray:
    """Step 1 of the three-step definition: S = scale * Q K^T for one head (fp64)."""
    return scale * (_as64(qh) @ _as64(kh).T)


def softmax_rows(s: np.ndarray, ncols: np.ndarray):
    """Step 2: row softmax of S with row r restricted to its first ncols[r] columns.

    Returns (P, m, L): P has zeros at masked positions, m is the row max over visible
    entries and L = m + ln(sum exp(s - m)) is the row logsumexp.
    """
    s = _as64(s)
    cols = np.arange(s.shape[1])[None, :]
    visible = cols < np.asarray(ncols)[:, None]
    sm = np.where(visible, s, -np.inf)
    m = sm.max(axis=1)
    e = np.where(visible, np.exp(sm - m[:, None]), 0.0)
    l = e.sum(axis=1)
    p = e / l[:, None]
    return p, m, m + np.log(l)


def head_forward(qh, kh, vh, scale: float, causal: bool, rows=None):
    """O and L for one head: qh [Nq, d], kh/vh [Nk, d]. `rows` selects query rows."""
    qh, kh, vh = _as64(qh), _as64(kh), _as64(vh)
    nq, nk = qh.shape[0], kh.shape[0]
    if causal and nq != nk:
        raise ValueError("causal attention needs N_q == N_k")
    rows = np.arange(nq) if rows is None else np.asarray(rows)
    o = np.empty((rows.size, vh.shape[1]))
    lse = np.empty(rows.size)
    for s0 in range(0, rows.size, _ROW_BLOCK):
        r = rows[s0 : s0 + _ROW_BLOCK]
        ncols = np.array([_visible_cols(int(i), nk, causal) for i in r])
        c = int(ncols.max())  # columns past c are masked for every row of this block
        p, _, l_ = softmax_rows(scores(qh[r], kh[:c], scale), ncols)
        o[s0 : s0 + r.size] = p @ vh[:c]  # step 3: O = P V
        lse[s0 : s0 + r.size] = l_
    return o, lse


def forward(q, k, v, causal: bool = False, scale: float | None = None, heads=None, rows=None):
    """Exact attention forward, fp64.

    q [B, Nq, Hq, d]; k, v [B, Nk, Hkv, d]. Returns (O [B, Nq, Hq, d], L [B, Hq, Nq]).
    `heads` (list of (b, h)) and `rows` (query indices) restrict the computation; outputs
    outside the selection are NaN.
    """
    B, Nq, Hq, d = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    o = np.full((B, Nq, Hq, v.shape[3]), np.nan)
    lse = np.full((B, Hq, Nq), np.nan)
    sel = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else heads
    r = np.arange(Nq) if rows is None else np.asarray(rows)
    for b, h in sel:
        ob, lb = head_forward(q[b, :, h], k[b, :, h // G], v[b, :, h // G], scale, causal, r)
        o[b, r, h] = ob
        lse[b, h, r] = lb
    return o, lse


def decode(q, k_cache, v_cache, seqlens, scale: float | None = None, heads=None):
    """Single-query attention against ragged cached sequences, fp64.

    q [B, 1, Hq, d]; caches [B, Nk_max, Hkv, d]; seqlens [B] (>= 1). Sequence b attends its
    first seqlens[b] cached keys, no mask. Returns (O [B, 1, Hq, d], L [B, Hq]).
    """
    B, nq, Hq, d = q.shape
    if nq != 1:
        raise ValueError("decode takes one query per sequence")
    Hkv = k_cache.shape[2]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    o = np.full((B, 1, Hq, v_cache.shape[3]), np.nan)
    lse = np.full((B, Hq), np.nan)
    sel = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else heads
    for b, h in sel:
        n = int(seqlens[b])
        ob, lb = head_forward(q[b, :, h], k_cache[b, :n, h // G], v_cache[b, :n, h // G], scale, False)
        o[b, 0, h] = ob[0]
        lse[b, h] = lb[0]
    return o, lse


def head_backward(qh, kh, vh, doh, scale: float, causal: bool):
    """Gradients of f = sum(O * dO) for one head, from the definition (fp64).

    P is rebuilt from scratch; dV = P^T dO; dP = dO V^T; the softmax Jacobian gives
    dS = P * (dP - D) with D_i = sum_j P_ij dP_ij; then dQ = scale dS K, dK = scale dS^T Q.
    """
    qh, kh, vh, doh = _as64(qh), _as64(kh), _as64(vh), _as64(doh)
    nq, nk = qh.shape[0], kh.shape[0]
    if causal and nq != nk:
        raise ValueError("causal attention needs N_q == N_k")
    dq = np.zeros_like(qh)
    dk = np.zeros_like(kh)
    dv = np.zeros_like(vh)
    for s0 in range(0, nq, _ROW_BLOCK):
        r = np.arange(s0, min(nq, s0 + _ROW_BLOCK))
        ncols = np.array([_visible_cols(int(i), nk, causal) for i in r])
        c = int(ncols.max())
        p, _, _ = softmax_rows(scores(qh[r], kh[:c], scale), ncols)
        dv[:c] += p.T @ doh[r]
        dp = doh[r] @ vh[:c].T
        dd = (p * dp).sum(axis=1)
        ds = p * (dp - dd[:, None])
        dq[r] = scale * (ds @ kh[:c])
        dk[:c] += scale * (ds.T @ qh[r])
    return dq, dk, dv


def backward(q, k, v, do, causal: bool = False, scale: float | None = None, heads=None):
    """dQ, dK, dV (fp64) of f = sum(O * dO). For GQA, dK/dV sum over the query heads of a group.

    `heads` (list of kv-head pairs (b, hkv)) restricts the computation: dQ is filled for the
    query heads of those groups, dK/dV for those kv heads; the rest is NaN.
    """
    B, Nq, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    sel = [(b, g) for b in range(B) for g in range(Hkv)] if heads is None else heads
    for b, g in sel:
        dk[b, :, g] = 0.0
        dv[b, :, g] = 0.0
        for h in range(g * G, (g + 1) * G):
            a, bk, bv = head_backward(q[b, :, h], k[b, :, g], v[b, :, g], do[b, :, h], scale, causal)
            dq[b, :, h] = a
            dk[b, :, g] += bk
            dv[b, :, g] += bv
    return dq, dk, dv


def probabilities(qh, kh, scale: float, causal: bool):
    """The full P matrix of one head (for property checks on small inputs)."""
    nq, nk = qh.shape[0], kh.shape[0]
    ncols = np.array([_visible_cols(i, nk, causal) for i in range(nq)])
    p, _, _ = softmax_rows(scores(qh, kh, scale), ncols)
    return p
