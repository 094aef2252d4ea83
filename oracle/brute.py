"""Pure-Python per-row brute force for tiny attention inputs.

TEST INFRASTRUCTURE ONLY (see oracle/attention.py for who may import it). It shares no code
with oracle/attention.py: no numpy in the arithmetic, scores by explicit loops, sums with
math.fsum, exponentials with math.exp.

Per query row i (Lecture 21 notes, §0.4 and §1.4; §2.5 for the causal visible set):
    s_j = scale * sum_t q_it k_jt            for visible keys j
    w_j = exp(s_j - max_j s_j)
    O_i = sum_j w_j v_j / sum_j w_j,         L_i = max_j s_j + ln(sum_j w_j)
"""

from __future__ import annotations

import math


def row_attention(qrow, keys, values, scale):
    """One query row against lists of key and value rows (plain Python floats)."""
    s = [scale * math.fsum(a * b for a, b in zip(qrow, kr)) for kr in keys]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    den = math.fsum(w)
    d = len(values[0])
    o = [math.fsum(w[j] * values[j][t] for j in range(len(values))) / den for t in range(d)]
    return o, m + math.log(den)


def attention(q, k, v, causal, scale):
    """q [B][Nq][Hq][d], k/v [B][Nk][Hkv][d] nested lists -> (O nested lists, L [B][Hq][Nq])."""
    B, Nq, Hq = len(q), len(q[0]), len(q[0][0])
    Nk, Hkv = len(k[0]), len(k[0][0])
    G = Hq // Hkv
    O = [[[None] * Hq for _ in range(Nq)] for _ in range(B)]
    L = [[[None] * Nq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(Nq):
                n = (i + 1) if causal else Nk
                keys = [k[b][j][g] for j in range(n)]
                vals = [v[b][j][g] for j in range(n)]
                o, lse = row_attention(q[b][i][h], keys, vals, scale)
                O[b][i][h] = o
                L[b][h][i] = lse
    return O, L
