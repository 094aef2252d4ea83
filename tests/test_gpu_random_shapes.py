"""GPU parity on seeded random shapes inside the supported envelope, every entry point against
the fp64 oracle.

Each case draws B, the query and kv heads (GQA groups of 1, 2 or 4), d, the mask, the lengths
(ragged, N_q != N_k without the mask; some cases with few keys under many query rows or few rows
over many keys), the softmax scale (1/sqrt(d), 0.05 or 0.2), a dropout
probability and a decode batch with ragged cache lengths. Larger scales, few keys under many
query rows and dropout make the outputs cancelling sums of large terms, where the method's bf16
rounding of P and dS is not tied to |exact|; the bf16 bounds therefore include the oracle's
first-order size of that rounding (oracle.rounding; Lecture 21 notes §2.6, §5.2). The fp32
forward keeps its 1e-5 bound, the persistent forward must equal fa_fwd bit for bit, and the
backward workspaces must be zero after every call.
"""

import math

import numpy as np
import pytest

import workloads
from gpu_util import check, say, to_dev, to_np
from oracle import attention as ora
from oracle import dropout as odp
from oracle import rounding as rnd

pytestmark = pytest.mark.gpu


def _fa():
    import exact_io_aware_03_amd as fa

    return fa


def _draw(i):
    """Case i: mode 0-1 any shape (causal or not), 2 few keys under many query rows, 3 few query
    rows over many keys (both without the mask)."""
    rng = np.random.default_rng([20261202, i])
    mode = int(rng.integers(0, 4))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4]))
    d = int(rng.choice([64, 128]))
    causal = mode < 2 and bool(rng.integers(0, 2))
    B = int(rng.integers(1, 4))
    if mode == 2:
        Nq, Nk = int(rng.integers(100, 513)), int(rng.integers(1, 17))
    elif mode == 3:
        Nq, Nk = int(rng.integers(1, 17)), int(rng.integers(100, 513))
    else:
        Nq = int(rng.integers(1, 513))
        Nk = Nq if causal else int(rng.integers(1, 513))
    return dict(mode=mode, B=B, Nq=Nq, Nk=Nk, Hq=Hkv * G, Hkv=Hkv, d=d, causal=causal,
                scale=float(rng.choice([1 / math.sqrt(d), 1 / math.sqrt(d), 0.05, 0.2])),
                seed=int(rng.integers(1, 1 << 30)), p=float(rng.choice([0.1, 0.3])),
                dseed=int(rng.integers(0, 1 << 62)), off=int(rng.integers(0, 100)),
                Bd=int(rng.integers(1, 25)), Nmax=int(rng.integers(1, 2500)), lseed=int(rng.integers(1, 1 << 30)))


@pytest.mark.parametrize("i", range(16))
def test_random_shape(i):
    import torch

    fa = _fa()
    c = _draw(i)
    B, Nq, Nk, Hq, Hkv, d, causal, scale = (c[n] for n in ("B", "Nq", "Nk", "Hq", "Hkv", "d", "causal", "scale"))
    say(f"random shape {i}: {c}")
    inp = workloads.make_attention_inputs(B, Nq, Nk, Hq, Hkv, d, seed=c["seed"], with_do=True)
    q, k, v, do = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    args = (inp["q"], inp["k"], inp["v"])

    # forward: bf16, persistent (bit for bit), polynomial exp2, fp32
    ro, rl = ora.forward(*args, causal, scale)
    t_o = rnd.forward_terms(*args, causal, scale)
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    check("O", to_np(o), ro, "bf16", terms=t_o)
    check("L", to_np(lse), rl, "bf16", is_lse=True)
    ws = torch.zeros(fa.fa_fwd_persistent_workspace_size(), dtype=torch.uint8, device="cuda")
    o2, l2 = torch.empty_like(o), torch.empty_like(lse)
    fa.fa_fwd_persistent(q, k, v, o2, l2, ws, causal, scale)
    o3, l3 = torch.empty_like(o), torch.empty_like(lse)
    fa.fa_fwd_poly_exp2(q, k, v, o3, l3, causal, scale)
    torch.cuda.synchronize()
    assert torch.equal(o2, o) and torch.equal(l2, lse) and int(ws.count_nonzero()) == 0
    check("O (poly exp2)", to_np(o3), ro, "bf16", terms=t_o)
    check("L (poly exp2)", to_np(l3), rl, "bf16", is_lse=True)
    of, lf = fa.forward(*(to_dev(x, "f32") for x in args), causal=causal, scale=scale)
    torch.cuda.synchronize()
    check("O (fp32)", to_np(of), ro, "f32")
    check("L (fp32)", to_np(lf), rl, "f32", is_lse=True)

    # backward: both paths (the single pass takes d = 128)
    ref = ora.backward(*args, inp["do"], causal, scale)
    terms = rnd.backward_terms(*args, inp["do"], causal, scale)
    nz = 256 + 4 * 64 * d * B * Hq * -(-Nq // 64)
    for single in (False, True) if d == 128 else (False,):
        wsb = torch.zeros(fa.fa_bwd_workspace_size(B, Hq, Nq, d), dtype=torch.uint8, device="cuda")
        g = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
        (fa.fa_bwd_single_pass if single else fa.fa_bwd)(q, k, v, o, do, lse, *g, wsb, causal, scale)
        torch.cuda.synchronize()
        assert int(wsb[:nz].count_nonzero()) == 0
        for n, x, r, t in zip(("dQ", "dK", "dV"), g, ref, terms):
            check(f"{n}{' (single pass)' if single else ''}", to_np(x), r, "bf16", terms=t)

    # dropout, forward and backward
    p, dseed, off = c["p"], c["dseed"], c["off"]
    keep = odp.keep_mask(B, Hq, Nq, Nk, p, dseed, off)
    od, ld = fa.forward_dropout(q, k, v, p, dseed, off, causal=causal, scale=scale)
    rod, rld = odp.forward(*args, keep, p, causal, scale)
    check("O (dropout)", to_np(od), rod, "bf16", terms=rnd.forward_terms(*args, causal, scale, keep, p))
    check("L (dropout)", to_np(ld), rld, "bf16", is_lse=True)
    gd = fa.backward_dropout(q, k, v, od, do, ld, p, dseed, off, causal=causal, scale=scale)
    torch.cuda.synchronize()
    refd = odp.backward(*args, inp["do"], keep, p, causal, scale)
    termsd = rnd.backward_terms(*args, inp["do"], causal, scale, keep, p)
    for n, x, r, t in zip(("dQ", "dK", "dV"), gd, refd, termsd):
        check(f"{n} (dropout)", to_np(x), r, "bf16", terms=t)

    # decode: ragged cache lengths, the same heads and head dimension
    lens = np.random.default_rng(c["lseed"]).integers(1, c["Nmax"] + 1, size=c["Bd"])
    say(f"  decode B={c['Bd']} Nk_max={c['Nmax']} lengths {int(lens.min())}..{int(lens.max())}")
    di = workloads.make_decode_inputs(c["Bd"], Hq, Hkv, c["Nmax"], d, seed=c["lseed"], lengths=lens)
    qd, kd, vd = (to_dev(di[n], "bf16") for n in ("q", "k", "v"))
    odc, ldc = fa.decode(qd, kd, vd, torch.from_numpy(di["seqlens"]).cuda(), scale=scale)
    torch.cuda.synchronize()
    rdo, rdl = ora.decode(di["q"], di["k"], di["v"], di["seqlens"], scale)
    t_dec = np.concatenate([rnd.forward_terms(di["q"][b:b + 1], di["k"][b:b + 1, :n], di["v"][b:b + 1, :n], False, scale)
                            for b, n in enumerate(di["seqlens"])])
    check("O (decode)", to_np(odc), rdo, "bf16", terms=t_dec)
    check("L (decode)", to_np(ldc), rdl, "bf16", is_lse=True)
