"""First-order size of the rounding that the bf16 method does on purpose.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product library never imports it.

The method reaches the exact result up to rounding (Lecture 21 notes §2.2: only the order of
the sums changes), but on the bf16 path it also rounds some intermediates to bf16 by design
(the readings of the pages that the parity tests follow):
  * the probabilities P are rounded to bf16 before the P V product, the row sum l is taken
    from the unrounded P (Lecture 21 notes §5.2 reports the effect of bf16 P at N = 512);
  * the backward rounds P (for dV) and dS (for dQ and dK) to bf16 before those products
    (§2.6), and forms D = rowsum(dO * O) from the forward's bf16 output O, which the
    identity sum_j P_ij dP_ij = dO_i . O_i (§2.6) allows;
  * every output is rounded to bf16 at the end.

Rounding x to bf16 moves it by at most u |x| with u = 2^-8 (8 significant bits, round to
nearest even). To first order the error of an output element is therefore at most
u (T + |exact|), with T the sum of the magnitudes of the terms whose operands were rounded:

  forward:   T_O[i]   = sum_j Pd_ij |V_j|
  backward:  T_dV[j]  = sum_i Pd_ij |dO_i|
             e_D[i]   = sum_d |dO_id| (|O_id| + T_O[i, d])        (D from the rounded O, whose
                                                              P was rounded as well)
             T_dQ[i]  = scale (sum_j |dS_ij| |K_j| + e_D[i] sum_j P_ij |K_j|)
             T_dK[j]  = scale (sum_i |dS_ij| |Q_i| + sum_i P_ij e_D[i] |Q_i|)

where Pd = P (Z / (1 - p_t) with dropout, Z the keep mask) and, for GQA, T_dK and T_dV sum over
the query heads of a group. Unlike a bound in terms of |exact| alone, T grows with the terms of
a sum that cancels: large softmax scales, few keys with many query rows, dropout's 1 / (1 - p).
The fp32 accumulation adds far less than this and is left to the absolute floor of the checks.
"""

from __future__ import annotations

import numpy as np

from . import attention as att
from . import dropout as odp

U_BF16 = 2.0 ** -8


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


_ROW_BLOCK = 1024


def _blocks(qh, kh, scale, causal):
    """Row blocks of one head: (rows, visible key count c, P [rows, c]) from the oracle's own
    scores and masked softmax, so no N_q x N_k matrix is formed at once."""
    nq, nk = qh.shape[0], kh.shape[0]
    for s0 in range(0, nq, _ROW_BLOCK):
        r = np.arange(s0, min(nq, s0 + _ROW_BLOCK))
        ncols = np.array([min(int(i) + 1, nk) if causal else nk for i in r])
        c = int(ncols.max())
        pm, _, _ = att.softmax_rows(att.scores(qh[r], kh[:c], scale), ncols)
        yield r, c, pm


def _zr(keep, p, b, h, r, c):
    if keep is None:
        return 1.0
    return keep[b, h][r][:, :c] * (256.0 / (256 - odp.threshold(p)))


def forward_terms(q, k, v, causal: bool = False, scale: float | None = None, keep=None, p: float = 0.0):
    """T_O [B, N_q, H_q, d]: sum_j Pd_ij |V_jd| per output element (fp64)."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, Nq, Hq, d = q.shape
    G = Hq // k.shape[2]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    t = np.zeros_like(q)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for r, c, pm in _blocks(q[b, :, h], k[b, :, g], scale, causal):
                t[b, r, h] = (pm * _zr(keep, p, b, h, r, c)) @ np.abs(v[b, :c, g])
    return t


def backward_terms(q, k, v, do, causal: bool = False, scale: float | None = None, keep=None, p: float = 0.0,
                   parts: bool = False):
    """(T_dQ, T_dK, T_dV) in the layouts of Q, K and V (fp64), as in the module docstring.

    parts=True returns them split by the rounding each part comes from, as a dict of
    {"dQ": {...}, "dK": {...}, "dV": {...}} with keys "dS" (dS rounded before the product; for
    dV: "P", P Z rounded), "D_O" (D formed from the rounded output O: |dO| |O| summed over d)
    and "D_P" (D formed from an O whose P was rounded in the forward: |dO| T_O summed over d);
    the totals are the sums of the parts."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, Nq, Hq, d = q.shape
    G = Hq // k.shape[2]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    part = {n: {m: np.zeros_like(x) for m in ms} for n, x, ms in
            (("dQ", q, ("dS", "D_O", "D_P")), ("dK", k, ("dS", "D_O", "D_P")), ("dV", v, ("P",)))}
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for r, c, pm in _blocks(q[b, :, h], k[b, :, g], scale, causal):
                zr = _zr(keep, p, b, h, r, c)
                pd = pm * zr
                vv, dor = v[b, :c, g], do[b, r, h]
                o = pd @ vv
                t_o = pd @ np.abs(vv)
                e_do = (np.abs(dor) * np.abs(o)).sum(axis=1)
                e_dp = (np.abs(dor) * t_o).sum(axis=1)
                dpd = (dor @ vv.T) * zr
                ds = pm * (dpd - (pm * dpd).sum(axis=1, keepdims=True))
                ak, aq = np.abs(k[b, :c, g]), np.abs(q[b, r, h])
                part["dV"]["P"][b, :c, g] += pd.T @ np.abs(dor)
                part["dQ"]["dS"][b, r, h] = scale * (np.abs(ds) @ ak)
                part["dK"]["dS"][b, :c, g] += scale * (np.abs(ds).T @ aq)
                for name, e in (("D_O", e_do), ("D_P", e_dp)):
                    part["dQ"][name][b, r, h] = scale * e[:, None] * (pm @ ak)
                    part["dK"][name][b, :c, g] += scale * ((pm * e[:, None]).T @ aq)
    if parts:
        return part
    return tuple(sum(part[n].values()) for n in ("dQ", "dK", "dV"))
