"""GPU parity of dropout (fa_fwd_dropout / fa_bwd_dropout through the C ABI): the regenerated
keep mask bit for bit against the oracle's Philox, and outputs and gradients against the fp64
dropout oracle (Lecture 21 notes §2.8, exercise 4)."""

import math

import numpy as np
import pytest

import workloads
from gpu_util import check, say, to_dev, to_np
from oracle import dropout as odp

pytestmark = pytest.mark.gpu


def _fa():
    import exact_io_aware_03_amd as fa

    return fa


def test_mask_bit_for_bit():
    # V = identity (key j -> unit vector j) turns O into P * Z * r: its nonzero pattern is Z
    import torch

    fa = _fa()
    B, N, Hq, Hkv, d, p, seed, off = 2, 128, 4, 2, 128, 0.375, 0x9E3779B97F4A7C15, 5
    inp = workloads.make_attention_inputs(B, N, N, Hq, Hkv, d, seed=1701)
    v = np.zeros((B, N, Hkv, d), dtype=np.float32)
    for j in range(N):
        v[:, j, :, j] = 1.0
    for causal in (False, True):
        say(f"dropout mask causal={causal}")
        o, _ = fa.forward_dropout(to_dev(inp["q"], "bf16"), to_dev(inp["k"], "bf16"), to_dev(v, "bf16"), p, seed, off,
                                  causal=causal, scale=0.05)
        torch.cuda.synchronize()
        o = to_np(o)  # [B, N, Hq, d]; column j of row i is P_ij Z_ij r
        z = odp.keep_mask(B, Hq, N, N, p, seed, off)
        vis = np.tril(np.ones((N, N), bool)) if causal else np.ones((N, N), bool)
        for b in range(B):
            for h in range(Hq):
                got = o[b, :, h, :N] != 0
                assert np.array_equal(got & vis, z[b, h] & vis)
                assert not np.any(got & ~vis)


SMALL = [
    # B, Nq, Nk, Hq, Hkv, d, causal, p
    (1, 128, 128, 1, 1, 128, False, 0.25),
    (2, 300, 300, 2, 2, 128, True, 0.25),
    (2, 300, 300, 4, 2, 128, False, 0.25),  # GQA
    (2, 300, 300, 4, 2, 128, True, 0.5),    # GQA with the mask: the causal K/V-outer path with dropout
    (1, 77, 333, 4, 1, 64, False, 0.125),
    (1, 257, 257, 2, 2, 64, True, 0.25),
]


@pytest.mark.parametrize("B,Nq,Nk,Hq,Hkv,d,causal,p", SMALL)
def test_dropout_forward_and_backward(B, Nq, Nk, Hq, Hkv, d, causal, p):
    import torch

    fa = _fa()
    seed, off = 1234567, 3
    say(f"dropout B={B} Nq={Nq} Nk={Nk} Hq={Hq} Hkv={Hkv} d={d} causal={causal} p={p}")
    inp = workloads.make_attention_inputs(B, Nq, Nk, Hq, Hkv, d, seed=1800 + Nq + Nk + d, with_do=True)
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = fa.forward_dropout(q, k, v, p, seed, off, causal=causal, scale=scale)
    keep = odp.keep_mask(B, Hq, Nq, Nk, p, seed, off)
    ro, rl = odp.forward(inp["q"], inp["k"], inp["v"], keep, p, causal, scale)
    check("O", to_np(o), ro, "bf16")
    check("L", to_np(lse), rl, "bf16", is_lse=True)
    if Nq != Nk and causal:
        return
    dq, dk, dv = fa.backward_dropout(q, k, v, o, do, lse, p, seed, off, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv = odp.backward(inp["q"], inp["k"], inp["v"], inp["do"], keep, p, causal, scale)
    check("dQ", to_np(dq), rq, "bf16")
    check("dK", to_np(dk), rk, "bf16")
    check("dV", to_np(dv), rv, "bf16")


def test_zero_probability_is_the_plain_path():
    import torch

    fa = _fa()
    inp = workloads.make_attention_inputs(1, 200, 200, 2, 1, 128, seed=1901, with_do=True)
    q, k, v, do = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    o0, l0 = fa.forward(q, k, v, causal=True)
    o1, l1 = fa.forward_dropout(q, k, v, 0.001, 7, 0, causal=True)  # below 1/256: no dropout
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_dropout_training_shape_sampled_heads():
    import torch

    fa = _fa()
    w = workloads.WORKLOADS["fwd_bf16_b16h16n2048d128"]
    p, seed, off = 0.125, 0xC0FFEE, 11
    say(f"dropout training shape p={p}")
    inp = workloads.make_attention_inputs(w.B, w.Nq, w.Nk, w.Hq, w.Hkv, w.d, seed=w.seed, with_do=True)
    q, k, v, do = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = fa.forward_dropout(q, k, v, p, seed, off, causal=True, scale=w.scale)
    dq, dk, dv = fa.backward_dropout(q, k, v, o, do, lse, p, seed, off, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    o, dq, dk, dv = to_np(o), to_np(dq), to_np(dk), to_np(dv)
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    for b, h in [heads[i] for i in workloads.sample_indices(len(heads), 2, 81)]:
        sl = lambda t: t[b:b + 1, :, h:h + 1]  # noqa: E731
        keep = odp.keep_mask_head(b * w.Hq + h, w.Nq, w.Nk, p, seed, off)[None, None]
        ro, _ = odp.forward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), keep, p, True, w.scale)
        rq, rk, rv = odp.backward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["do"]), keep, p, True, w.scale)
        check(f"O[b={b},h={h}]", sl(o), ro, "bf16", config=True)
        check(f"dQ[b={b},h={h}]", sl(dq), rq, "bf16", config=True)
        check(f"dK[b={b},h={h}]", sl(dk), rk, "bf16", config=True)
        check(f"dV[b={b},h={h}]", sl(dv), rv, "bf16", config=True)
