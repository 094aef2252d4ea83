"""GPU checks of the FMA-unit exponential (fa_exp2_poly, fa_fwd_poly_exp2) through the C ABI.

Pins from "Lecture 21: Optimizing Attention for Modern Hardware" (CMU 11-868) §5.2: a cubic
2^f with p(0) = 1 after Cody-Waite reduction, once P is rounded to bf16, equals the bf16
rounding of the exact exponential for about 99% of values and differs by one bf16 spacing for
the rest; inside attention with bf16 P its error is the same as with the exact exponential
(3.1e-3 for both at N = 512 on the lecture's data). The references are exact 2^x in fp64 and the
fp64 oracle.
"""

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


def bf16_round(x64):
    """Round fp64 values to the nearest bf16 (ties to even), via the nearest fp32."""
    f = np.asarray(x64, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def gpu_exp2_poly(x):
    import torch

    fa = _fa()
    xt = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    yt = torch.empty_like(xt)
    fa.fa_exp2_poly(xt, yt)
    torch.cuda.synchronize()
    return yt.cpu().numpy().astype(np.float64)


def test_exp2_poly_elementwise():
    # the range scores take after the max is subtracted, up to 2^8 above it (conditional rescaling)
    x = np.linspace(-30.0, 8.0, 1 << 20, dtype=np.float32)
    y = gpu_exp2_poly(x)
    exact = np.exp2(x.astype(np.float64))
    rel = np.abs(y / exact - 1.0)
    say(f"  exp2_poly max relative error {rel.max():.3e}")
    assert rel.max() <= 8.6e-5 + 2e-7  # the fit's minimax error plus fp32 evaluation rounding
    yb, eb = bf16_round(y), bf16_round(exact)
    same = float(np.mean(yb == eb))
    spacing = np.exp2(np.floor(np.log2(eb)) - 7)
    steps = np.abs(yb - eb) / spacing
    say(f"  after bf16 rounding: {100 * same:.2f}% identical, max {steps.max():.0f} spacing")
    # the lecture prints the share rounded to a whole percent (99%): it must round to 99
    assert same >= 0.985
    assert steps.max() <= 1.0
    # below -127 (masked scores are -inf) the result is exactly zero
    z = gpu_exp2_poly(np.array([-np.inf, -1e30, -200.0, -127.0], dtype=np.float32))
    assert np.all(z == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_poly_exp2_error_equals_exact_exp_at_n512(causal):
    # the lecture's comparison at N = 512: with bf16 P the polynomial's error disappears in P's
    # rounding, so the poly forward is as close to exact attention as the v_exp_f32 forward
    import torch

    fa = _fa()
    inp = workloads.make_attention_inputs(1, 512, 512, 4, 4, 128, seed=2512 + causal)
    q, k, v = (to_dev(inp[n], "bf16") for n in ("q", "k", "v"))
    ro, rl = ora.forward(inp["q"], inp["k"], inp["v"], causal, 1.0 / math.sqrt(128))
    errs = {}
    for name, fn in (("exact", fa.fa_fwd), ("poly", fa.fa_fwd_poly_exp2)):
        o = torch.empty_like(q)
        lse = torch.empty(1, 4, 512, dtype=torch.float32, device="cuda")
        fn(q, k, v, o, lse, causal, 1.0 / math.sqrt(128))
        torch.cuda.synchronize()
        errs[name] = float(np.abs(to_np(o) - ro).max())
        check(f"O ({name})", to_np(o), ro, "bf16")
        check(f"L ({name})", to_np(lse), rl, "bf16", is_lse=True)
    say(f"  max |O - O_exact|: v_exp_f32 {errs['exact']:.3e}, polynomial {errs['poly']:.3e}")
    assert errs["poly"] <= 1.25 * errs["exact"] + 1e-3


@pytest.mark.parametrize("B,Nq,Nk,Hq,Hkv,d,causal", [
    (2, 300, 300, 4, 2, 128, True),   # ragged, GQA
    (1, 77, 333, 4, 1, 128, False),   # N_q != N_k
    (2, 257, 257, 2, 2, 64, True),
    (1, 1, 1, 1, 1, 64, False),
])
def test_fwd_poly_exp2_small(B, Nq, Nk, Hq, Hkv, d, causal):
    import torch

    fa = _fa()
    say(f"fwd poly B={B} Nq={Nq} Nk={Nk} Hq={Hq} Hkv={Hkv} d={d} causal={causal}")
    inp = workloads.make_attention_inputs(B, Nq, Nk, Hq, Hkv, d, seed=2600 + Nq + Nk + d)
    q, k, v = (to_dev(inp[n], "bf16") for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, Nq, dtype=torch.float32, device="cuda")
    fa.fa_fwd_poly_exp2(q, k, v, o, lse, causal, 1.0 / math.sqrt(d))
    torch.cuda.synchronize()
    ro, rl = ora.forward(inp["q"], inp["k"], inp["v"], causal, 1.0 / math.sqrt(d))
    check("O", to_np(o), ro, "bf16")
    check("L", to_np(lse), rl, "bf16", is_lse=True)
