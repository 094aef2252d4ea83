"""Pins for the fp64 oracle: checks against facts the pages and the mathematics fix.

Every test here is CPU-only. None of them retypes the oracle's formula: they use
invariants (row sums, shift and permutation invariance), closed forms (uniform weights,
a single key, a dominant key, causal row 0), an independent pure-Python brute force, finite
differences and torch float64 autograd as an outside library routine.
"""

import math

import numpy as np
import pytest

from oracle import attention as ora
from oracle import brute
import workloads


def _rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def _tolist(x):
    return np.asarray(x, dtype=np.float64).tolist()


# ---- P-1: rows of P sum to one ---------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(causal):
    q, k = _rand((37, 16), 1), _rand((37, 16), 2)
    p = ora.probabilities(q, k, 0.25, causal)
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    if causal:
        assert np.all(np.triu(p, 1) == 0.0)


# ---- P-2: invariance of P to shifting a row's scores (needs the max subtraction) -------
@pytest.mark.parametrize("c", [-745.0, -50.0, 50.0, 760.0])
def test_shift_invariance(c):
    s = _rand((9, 13), 3) * 4.0
    ncols = np.array([13, 5, 1, 13, 7, 13, 2, 13, 13])
    p0, m0, l0 = ora.softmax_rows(s, ncols)
    p1, m1, l1 = ora.softmax_rows(s + c, ncols)
    assert np.all(np.isfinite(p1))
    # s + c itself rounds to ulp(|c|)/2, so the bound grows with the shift
    tol = 4 * np.spacing(abs(c) + 16.0)
    np.testing.assert_allclose(p1, p0, rtol=0, atol=tol)
    np.testing.assert_allclose(l1 - c, l0, rtol=0, atol=tol)


# ---- P-3: causal row 0 is exactly V[0] -------------------------------------------------
def test_causal_row0_is_v0():
    inp = workloads.make_attention_inputs(2, 33, 33, 4, 2, 16, seed=11)
    o, lse = ora.forward(inp["q"], inp["k"], inp["v"], causal=True, scale=0.3)
    for b in range(2):
        for h in range(4):
            g = h // 2
            assert np.array_equal(o[b, 0, h], inp["v"][b, 0, g].astype(np.float64))
            want = 0.3 * float(np.dot(inp["q"][b, 0, h].astype(np.float64), inp["k"][b, 0, g].astype(np.float64)))
            assert abs(lse[b, h, 0] - want) < 1e-13


# ---- P-4: joint permutation of K/V rows leaves a non-causal result unchanged -----------
def test_kv_permutation_invariance():
    inp = workloads.make_attention_inputs(1, 20, 29, 2, 1, 8, seed=12)
    perm = np.random.Generator(np.random.PCG64(5)).permutation(29)
    o0, l0 = ora.forward(inp["q"], inp["k"], inp["v"], False, 0.4)
    o1, l1 = ora.forward(inp["q"], inp["k"][:, perm], inp["v"][:, perm], False, 0.4)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l1, l0, rtol=0, atol=1e-14)


# ---- P-5: numpy oracle vs an independent pure-Python brute force -----------------------
@pytest.mark.parametrize(
    "B,Nq,Nk,Hq,Hkv,d,causal",
    [(1, 7, 7, 1, 1, 4, False), (2, 9, 9, 2, 1, 8, True), (1, 5, 13, 4, 2, 3, False), (1, 16, 16, 2, 2, 8, True)],
)
def test_oracle_matches_brute_force(B, Nq, Nk, Hq, Hkv, d, causal):
    inp = workloads.make_attention_inputs(B, Nq, Nk, Hq, Hkv, d, seed=100 + Nq + d)
    scale = 1.0 / math.sqrt(d)
    o, lse = ora.forward(inp["q"], inp["k"], inp["v"], causal, scale)
    ob, lb = brute.attention(_tolist(inp["q"]), _tolist(inp["k"]), _tolist(inp["v"]), causal, scale)
    np.testing.assert_allclose(o, np.array(ob), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, np.array(lb), rtol=0, atol=1e-13)


def test_decode_matches_brute_force_and_ignores_padding():
    inp = workloads.make_decode_inputs(3, 4, 2, 12, 8, seed=7, lengths=[1, 12, 5])
    k, v = inp["k"].copy(), inp["v"].copy()
    for b, n in enumerate(inp["seqlens"]):
        k[b, n:] = np.nan  # padding must never be read
        v[b, n:] = np.nan
    o, lse = ora.decode(inp["q"], k, v, inp["seqlens"], 0.5)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    for b, n in enumerate(inp["seqlens"]):
        ob, lb = brute.attention(
            _tolist(inp["q"][b : b + 1]), _tolist(inp["k"][b : b + 1, :n]), _tolist(inp["v"][b : b + 1, :n]), False, 0.5
        )
        np.testing.assert_allclose(o[b : b + 1], np.array(ob), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[b], np.array(lb)[0, :, 0], rtol=0, atol=1e-13)
    # a single cached key: O = V_0 and L = its score
    assert np.array_equal(o[0, 0, 0], inp["v"][0, 0, 0].astype(np.float64))


# ---- P-6: closed forms -----------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_zero_scores_give_uniform_average(causal):
    inp = workloads.make_attention_inputs(1, 24, 24, 2, 2, 8, seed=21)
    o, lse = ora.forward(inp["q"], inp["k"], inp["v"], causal, scale=0.0)
    v = inp["v"].astype(np.float64)
    for i in range(24):
        n = i + 1 if causal else 24
        np.testing.assert_allclose(o[0, i], v[0, :n].mean(axis=0), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[0, :, i], math.log(n), rtol=0, atol=1e-14)


def test_single_key():
    inp = workloads.make_attention_inputs(1, 6, 1, 3, 1, 5, seed=22)
    o, lse = ora.forward(inp["q"], inp["k"], inp["v"], False, 0.7)
    for h in range(3):
        np.testing.assert_array_equal(o[0, :, h], np.broadcast_to(inp["v"][0, 0, 0], (6, 5)))
        np.testing.assert_allclose(lse[0, h], 0.7 * inp["q"][0, :, h].astype(np.float64) @ inp["k"][0, 0, 0], atol=1e-13)


def test_dominant_key_selects_its_value():
    d, nk = 16, 12
    k = np.eye(nk, d)[None, :, None, :]  # orthonormal keys
    v = _rand((1, nk, 1, d), 9)
    q = np.zeros((1, nk, 1, d))
    for j in range(nk):
        q[0, j, 0] = 80.0 * k[0, j, 0]  # query j aligned with key j only
    o, _ = ora.forward(q, k, v, False, 1.0)
    np.testing.assert_allclose(o[0, :, 0], v[0, :, 0], rtol=0, atol=1e-12)


# ---- P-8: backward D identity: sum_j P_ij dP_ij = dO_i . O_i ---------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_backward_d_identity(causal):
    q, k, v, do = _rand((40, 8), 31), _rand((40, 8), 32), _rand((40, 8), 33), _rand((40, 8), 34)
    p = ora.probabilities(q, k, 0.35, causal)
    o, _ = ora.head_forward(q, k, v, 0.35, causal)
    dp = do @ v.T
    np.testing.assert_allclose((p * dp).sum(axis=1), (do * o).sum(axis=1), rtol=0, atol=1e-13)


# ---- P-9: backward vs finite differences and vs torch float64 autograd -----------------
def _f(q, k, v, do, causal, scale):
    o, _ = ora.forward(q, k, v, causal, scale)
    return float((o * do).sum())


@pytest.mark.parametrize("causal,Hq,Hkv", [(False, 2, 1), (True, 2, 2), (True, 4, 2)])
def test_backward_finite_differences(causal, Hq, Hkv):
    B, N, d = 1, 6, 3
    g = np.random.Generator(np.random.PCG64(40 + Hq))
    q = g.standard_normal((B, N, Hq, d))
    k = g.standard_normal((B, N, Hkv, d))
    v = g.standard_normal((B, N, Hkv, d))
    do = g.standard_normal((B, N, Hq, d))
    scale = 0.6
    dq, dk, dv = ora.backward(q, k, v, do, causal, scale)
    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = _f(args["q"], args["k"], args["v"], do, causal, scale)
            args[name] = xm
            fmn = _f(args["q"], args["k"], args["v"], do, causal, scale)
            fd[idx] = (fp - fmn) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=0, atol=2e-8, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd(causal):
    torch = pytest.importorskip("torch")
    B, N, Hq, Hkv, d = 2, 33, 4, 2, 16
    inp = workloads.make_attention_inputs(B, N, N, Hq, Hkv, d, seed=44, with_do=True)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = ora.backward(inp["q"], inp["k"], inp["v"], inp["do"], causal, scale)
    t = {n: torch.tensor(inp[n], dtype=torch.float64, requires_grad=(n != "do")) for n in ("q", "k", "v", "do")}
    qh = t["q"].permute(0, 2, 1, 3)
    kh = t["k"].permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    vh = t["v"].permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    s = scale * torch.matmul(qh, kh.transpose(-1, -2).contiguous())
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), vh).permute(0, 2, 1, 3)
    (o * t["do"]).sum().backward()
    np.testing.assert_allclose(dq, t["q"].grad.numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk, t["k"].grad.numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv, t["v"].grad.numpy(), rtol=0, atol=1e-13)
    # the forward against torch too (an outside library routine for softmax)
    of, _ = ora.forward(inp["q"], inp["k"], inp["v"], causal, scale)
    np.testing.assert_allclose(of, o.detach().numpy(), rtol=0, atol=1e-13)


# ---- selections: sampled rows/heads equal the full computation -------------------------
def test_row_and_head_selection_matches_full():
    inp = workloads.make_attention_inputs(2, 50, 50, 4, 2, 8, seed=55)
    o, lse = ora.forward(inp["q"], inp["k"], inp["v"], True, 0.3)
    rows = np.array([0, 7, 31, 49])
    o2, l2 = ora.forward(inp["q"], inp["k"], inp["v"], True, 0.3, heads=[(1, 3)], rows=rows)
    np.testing.assert_array_equal(o2[1, rows, 3], o[1, rows, 3])
    np.testing.assert_array_equal(l2[1, 3, rows], lse[1, 3, rows])
    assert np.isnan(o2[0]).all()


# ---- input recipe ----------------------------------------------------------------------
def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.0078125 + 2 ** -9, 1.01171875, -3.14159, 65504.0], dtype=np.float32)
    r = workloads.round_to_bf16(x.copy())
    # reference by exhaustive nearest search over the two bf16 neighbours
    for xi, ri in zip(x, r):
        u = int(np.float32(xi).view(np.uint32))
        lo = np.uint32(u & 0xFFFF0000).view(np.float32)
        hi = np.uint32((u & 0xFFFF0000) + 0x10000).view(np.float32)
        dlo, dhi = abs(float(xi) - float(lo)), abs(float(xi) - float(hi))
        if dlo < dhi:
            want = lo
        elif dhi < dlo:
            want = hi
        else:
            want = lo if ((u >> 16) & 1) == 0 else hi
        assert ri == want


def test_workload_generators_are_seeded():
    a = workloads.make_attention_inputs(1, 8, 8, 2, 1, 4, seed=3, outlier_frac=0.5, outlier_scale=20.0)
    b = workloads.make_attention_inputs(1, 8, 8, 2, 1, 4, seed=3, outlier_frac=0.5, outlier_scale=20.0)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n])
    assert np.abs(a["k"]).max() > 6.0  # outliers present
    d = workloads.make_decode_inputs(16, 4, 2, 8192, 8, seed=4)
    assert d["seqlens"].min() >= 1024 and d["seqlens"].max() <= 8192
    for bi, n in enumerate(d["seqlens"]):
        assert not d["k"][bi, n:].any() and d["k"][bi, n - 1].any()
