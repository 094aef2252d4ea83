"""Pins of oracle.rounding: its first-order sizes must bound what the bf16 rounding of the method
actually does.

The check runs the method with its bf16 roundings made explicit (P rounded before P V, the
output O rounded, D formed from that rounded O, P Z and dS rounded before the gradient
products, every output rounded; Lecture 21 notes §2.6 and §5.2), everything else in fp64, and
requires |emulated - exact| <= 2^-8 (T + |exact|) element by element. The inputs include the
regimes where a bound in |exact| alone fails: a large softmax scale, few keys under many query
rows, GQA sums and dropout's 1 / (1 - p). Leaving a term out of T (the D term, say) breaks
it at the larger scales.
"""

import numpy as np
import pytest

import workloads
from oracle import attention as ora
from oracle import dropout as odp
from oracle import rounding as rnd


def _bf16(x):
    return workloads.round_to_bf16(np.asarray(x, dtype=np.float64)).astype(np.float64)


ALL = ("P_fwd", "O", "P_dv", "dS", "out")


def _emulate(q, k, v, do, causal, scale, keep=None, p=0.0, on=ALL):
    """The method's arithmetic with the bf16 roundings named in `on`, fp64 otherwise: "P_fwd" (P
    before P V), "O" (the forward's output, from which D is formed), "P_dv" (P Z before dV),
    "dS" (before dQ and dK) and "out" (the gradients)."""
    rd = lambda x, what: _bf16(x) if what in on else x  # noqa: E731
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    r = 256.0 / (256 - odp.threshold(p)) if keep is not None else 1.0
    o = np.zeros_like(q)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            s = scale * q[b, :, h] @ k[b, :, g].T
            if causal:
                s[np.triu(np.ones((Nq, Nk), bool), 1)] = -np.inf
            m = s.max(axis=1, keepdims=True)
            pt = np.exp(s - m)
            l = pt.sum(axis=1, keepdims=True)
            z = keep[b, h] if keep is not None else np.ones((Nq, Nk), bool)
            o[b, :, h] = rd(r * (rd(np.where(z, pt, 0.0), "P_fwd") @ v[b, :, g]) / l, "O")
            pm = pt / l
            dvv = (do[b, :, h] * o[b, :, h]).sum(axis=1, keepdims=True)  # D from the forward's O
            dp = np.where(z, do[b, :, h] @ v[b, :, g].T, 0.0) * r
            ds = rd(pm * (dp - dvv), "dS")
            dv[b, :, g] += r * (rd(np.where(z, pm, 0.0), "P_dv").T @ do[b, :, h])
            dq[b, :, h] = scale * ds @ k[b, :, g]
            dk[b, :, g] += scale * ds.T @ q[b, :, h]
    return o, rd(dq, "out"), rd(dk, "out"), rd(dv, "out")


def _case(B, Nq, Nk, Hq, Hkv, d, causal, scale, p):
    inp = workloads.make_attention_inputs(B, Nq, Nk, Hq, Hkv, d, seed=6100 + Nq + Nk + d, with_do=True)
    q, k, v, do = (inp[n].astype(np.float64) for n in ("q", "k", "v", "do"))
    keep = odp.keep_mask(B, Hq, Nq, Nk, p, 77, 1) if p > 0 else None
    if keep is None:
        eo, _ = ora.forward(q, k, v, causal, scale)
        exact = ora.backward(q, k, v, do, causal, scale)
    else:
        eo, _ = odp.forward(q, k, v, keep, p, causal, scale)
        exact = odp.backward(q, k, v, do, keep, p, causal, scale)
    return q, k, v, do, keep, eo, exact


CASES = [
    # B, Nq, Nk, Hq, Hkv, d, causal, scale, p
    (1, 64, 64, 2, 1, 32, True, 0.35, 0.0),
    (2, 96, 80, 4, 2, 64, False, 0.2, 0.0),
    (1, 300, 4, 4, 2, 32, False, 1 / np.sqrt(32), 0.0),  # few keys, many query rows, GQA
    (1, 120, 120, 4, 1, 64, True, 0.2, 0.3),
    (2, 70, 90, 2, 2, 32, False, 0.05, 0.3),
]


@pytest.mark.parametrize("B,Nq,Nk,Hq,Hkv,d,causal,scale,p", CASES)
def test_terms_bound_the_methods_rounding(B, Nq, Nk, Hq, Hkv, d, causal, scale, p):
    # all roundings at once against the totals, the output's own rounding included
    q, k, v, do, keep, eo, exact = _case(B, Nq, Nk, Hq, Hkv, d, causal, scale, p)
    got = _emulate(q, k, v, do, causal, scale, keep, p)
    terms = (rnd.forward_terms(q, k, v, causal, scale, keep, p),) + rnd.backward_terms(q, k, v, do, causal, scale, keep, p)
    worst = 0.0
    for name, e, x, t in zip(("O", "dQ", "dK", "dV"), got, (eo,) + tuple(exact), terms):
        err = np.abs(e - x)
        bound = rnd.U_BF16 * (t + np.abs(x)) + 1e-12
        assert np.all(err <= bound), (name, float((err / bound).max()))
        worst = max(worst, float((err / bound).max()))
    assert worst > 0.05  # the roundings are really there and the bound is not vacuous


@pytest.mark.parametrize("B,Nq,Nk,Hq,Hkv,d,causal,scale,p", CASES)
def test_each_part_bounds_its_own_rounding(B, Nq, Nk, Hq, Hkv, d, causal, scale, p):
    # one rounding at a time, against the part of the terms that accounts for it: a part that
    # is too small (a signed sum, a dropped factor) fails here even where another part is large
    q, k, v, do, keep, eo, exact = _case(B, Nq, Nk, Hq, Hkv, d, causal, scale, p)
    part = rnd.backward_terms(q, k, v, do, causal, scale, keep, p, parts=True)
    t_o = rnd.forward_terms(q, k, v, causal, scale, keep, p)
    checks = [
        ("P_fwd", [("O", 0, eo, t_o), ("dQ", 1, exact[0], part["dQ"]["D_P"]), ("dK", 2, exact[1], part["dK"]["D_P"])]),
        ("O", [("dQ", 1, exact[0], part["dQ"]["D_O"]), ("dK", 2, exact[1], part["dK"]["D_O"])]),
        ("dS", [("dQ", 1, exact[0], part["dQ"]["dS"]), ("dK", 2, exact[1], part["dK"]["dS"])]),
        ("P_dv", [("dV", 3, exact[2], part["dV"]["P"])]),
    ]
    for src, outs in checks:
        got = _emulate(q, k, v, do, causal, scale, keep, p, on=(src,))
        worst = 0.0
        for name, i, x, t in outs:
            err = np.abs(got[i] - x)
            bound = rnd.U_BF16 * t * (1 + 1e-9) + 1e-12
            assert np.all(err <= bound), (src, name, float((err / bound).max()))
            worst = max(worst, float((err / bound).max()))
        assert worst > 0.05, (src, worst)


def test_terms_equal_the_result_when_nothing_cancels():
    # with V >= 0 the forward's terms are O itself; with dO >= 0 (no dropout) T_dV is dV
    for causal in (False, True):
        nk = 50 if causal else 40
        inp = workloads.make_attention_inputs(2, 50, nk, 4, 2, 16, seed=6201 + nk, with_do=True)
        q, k = inp["q"].astype(np.float64), inp["k"].astype(np.float64)
        v, do = np.abs(inp["v"].astype(np.float64)), np.abs(inp["do"].astype(np.float64))
        o, _ = ora.forward(q, k, v, causal, 0.3)
        assert np.allclose(rnd.forward_terms(q, k, v, causal, 0.3), o, rtol=1e-13, atol=1e-13)
        _, _, dv = ora.backward(q, k, v, do, causal, 0.3)
        _, _, tv = rnd.backward_terms(q, k, v, do, causal, 0.3)
        assert np.allclose(tv, dv, rtol=1e-13, atol=1e-13)
