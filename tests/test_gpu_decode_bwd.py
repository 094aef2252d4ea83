"""GPU parity of decode (fa_decode) and backward (fa_bwd) through the C ABI vs the fp64 oracle."""

import math

import numpy as np
import pytest

import workloads
from gpu_util import check, say, to_dev, to_np
from oracle import attention as ora

pytestmark = pytest.mark.gpu


def _fa():
    import exact_io_aware_03_amd as fa

    return fa


def run_decode(inp, scale):
    import torch

    fa = _fa()
    q, k, v = (to_dev(inp[n], "bf16") for n in ("q", "k", "v"))
    lens = torch.from_numpy(inp["seqlens"]).cuda()
    o, lse = fa.decode(q, k, v, lens, scale=scale)
    torch.cuda.synchronize()
    return to_np(o), to_np(lse)


@pytest.mark.parametrize(
    "B,Hq,Hkv,Nk_max,d,lengths",
    [
        (4, 8, 2, 1100, 128, [1, 255, 256, 1100]),
        (3, 32, 8, 8192, 128, [8192, 257, 4097]),
        (2, 8, 8, 600, 64, [600, 3]),
        (2, 16, 2, 700, 128, [513, 64]),   # 8 query heads per kv head
        (2, 16, 1, 300, 64, [300, 129]),   # 16 query heads per kv head
    ],
)
def test_decode_small(B, Hq, Hkv, Nk_max, d, lengths):
    say(f"decode B={B} Hq={Hq} Hkv={Hkv} Nk_max={Nk_max} d={d} lens={lengths}")
    inp = workloads.make_decode_inputs(B, Hq, Hkv, Nk_max, d, seed=500 + Nk_max, lengths=lengths)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_decode(inp, scale)
    ro, rl = ora.decode(inp["q"], inp["k"], inp["v"], inp["seqlens"], scale)
    check("O", o, ro, "bf16")
    check("L", lse, rl, "bf16", is_lse=True)


def test_decode_config():
    w = workloads.WORKLOADS["decode_bf16_b64hq32hkv8d128"]
    say(f"decode config {w.name}")
    inp = workloads.make_workload_inputs(w)
    o, lse = run_decode(inp, w.scale)
    ro, rl = ora.decode(inp["q"], inp["k"], inp["v"], inp["seqlens"], w.scale)
    check("O", o, ro, "bf16")
    check("L", lse, rl, "bf16", is_lse=True)


def run_fwd_bwd(inp, causal, scale):
    import torch

    fa = _fa()
    q, k, v, do = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return to_np(dq), to_np(dk), to_np(dv)


@pytest.mark.parametrize(
    "B,N,Hq,Hkv,d,causal",
    [
        (1, 128, 1, 1, 128, False),
        (1, 128, 1, 1, 128, True),
        (2, 300, 2, 2, 128, True),   # ragged
        (1, 200, 4, 2, 64, False),   # GQA, d = 64
        (1, 257, 4, 1, 128, True),   # GQA 4:1, ragged
        (1, 64, 2, 2, 64, True),
    ],
)
def test_bwd_small(B, N, Hq, Hkv, d, causal):
    say(f"bwd B={B} N={N} Hq={Hq} Hkv={Hkv} d={d} causal={causal}")
    inp = workloads.make_attention_inputs(B, N, N, Hq, Hkv, d, seed=900 + N + d, with_do=True)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = run_fwd_bwd(inp, causal, scale)
    rq, rk, rv = ora.backward(inp["q"], inp["k"], inp["v"], inp["do"], causal, scale)
    check("dQ", dq, rq, "bf16")
    check("dK", dk, rk, "bf16")
    check("dV", dv, rv, "bf16")


def test_bwd_config():
    w = workloads.WORKLOADS["bwd_bf16_causal_b8h16n4096d128"]
    say(f"bwd config {w.name}")
    inp = workloads.make_workload_inputs(w)
    dq, dk, dv = run_fwd_bwd(inp, True, w.scale)
    pairs = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    sel = [pairs[i] for i in workloads.sample_indices(len(pairs), 3, 51)]
    say(f"  oracle gradients on heads {sel}")
    rq, rk, rv = ora.backward(inp["q"], inp["k"], inp["v"], inp["do"], True, w.scale, heads=sel)
    for b, g in sel:
        check(f"dQ[b={b},h={g}]", dq[b, :, g], rq[b, :, g], "bf16")
        check(f"dK[b={b},h={g}]", dk[b, :, g], rk[b, :, g], "bf16")
        check(f"dV[b={b},h={g}]", dv[b, :, g], rv[b, :, g], "bf16")
