"""GPU parity of the persistent forward (fa_fwd_persistent through the C ABI): the fp64
oracle on small shapes, and bit-for-bit identity with fa_fwd everywhere, since every task is
computed by the same code in the same order; the workspace counters are zero after every call
(Lecture 21 notes §4.5)."""

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


_WS = {}


def _workspace():
    # one zero-filled workspace for the whole module: every call must leave it zero
    import torch

    if "ws" not in _WS:
        _WS["ws"] = torch.zeros(_fa().fa_fwd_persistent_workspace_size(), dtype=torch.uint8, device="cuda")
    return _WS["ws"]


def run_both(inp, causal, scale):
    import torch

    fa = _fa()
    q, k, v = (to_dev(inp[n], "bf16") for n in ("q", "k", "v"))
    B, Nq, Hq, _ = q.shape
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    l1 = torch.empty((B, Hq, Nq), dtype=torch.float32, device="cuda")
    l2 = torch.empty_like(l1)
    fa.fa_fwd(q, k, v, o1, l1, causal, scale)
    ws = _workspace()
    fa.fa_fwd_persistent(q, k, v, o2, l2, ws, causal, scale)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0, "the counters must be zero after the call"
    o1, o2, l1, l2 = to_np(o1), to_np(o2), to_np(l1), to_np(l2)
    say(f"  identical to fa_fwd: O {np.array_equal(o1, o2)}, L {np.array_equal(l1, l2)}")
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    return o2, l2


CASES = [
    # B, Nq, Nk, Hq, Hkv, d, causal
    (1, 128, 128, 1, 1, 128, False),   # one task: a single workgroup
    (2, 300, 300, 4, 2, 128, True),    # ragged rows, GQA
    (1, 77, 333, 4, 1, 128, False),    # N_q != N_k, ragged both ways
    (2, 257, 257, 2, 2, 64, True),
    (1, 5, 1000, 2, 1, 64, False),
    (4, 700, 451, 32, 8, 128, False),  # 384 tasks: more than the compute units, taken from the queues
    (3, 1100, 1100, 24, 8, 128, True),  # 360 causal tasks of 1..5 row blocks
    (3, 300, 192, 64, 64, 64, False),
]


@pytest.mark.parametrize("B,Nq,Nk,Hq,Hkv,d,causal", CASES)
def test_persistent_small(B, Nq, Nk, Hq, Hkv, d, causal):
    say(f"fwd persistent B={B} Nq={Nq} Nk={Nk} Hq={Hq} Hkv={Hkv} d={d} causal={causal}")
    inp = workloads.make_attention_inputs(B, Nq, Nk, Hq, Hkv, d, seed=3000 + Nq + Nk + d)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_both(inp, causal, scale)
    heads = [(b, h) for b in range(B) for h in range(Hq)][:8]  # the first 8 (batch, head) pairs
    ro, rl = ora.forward(inp["q"], inp["k"], inp["v"], causal, scale, heads=heads)
    for b, h in heads:
        check(f"O[b={b},h={h}]", o[b, :, h], ro[b, :, h], "bf16")
        check(f"L[b={b},h={h}]", lse[b, h], rl[b, h], "bf16", is_lse=True)


@pytest.mark.parametrize("name,causal", [("fwd_bf16_b16h16n2048d128", False), ("fwd_bf16_b16h16n2048d128", True),
                                         ("fwd_bf16_causal_h32n16384d128", True)])
def test_persistent_full_sizes(name, causal):
    w = workloads.WORKLOADS[name]
    say(f"fwd persistent {name} causal={causal}")
    inp = workloads.make_workload_inputs(w)
    o, lse = run_both(inp, causal, w.scale)
    rows = np.unique(np.concatenate([[0, 1, w.Nq - 1], workloads.sample_indices(w.Nq, 6, 41)]))
    say(f"  oracle on {rows.size} rows of every head")
    ro, rl = ora.forward(inp["q"], inp["k"], inp["v"], causal, w.scale, rows=rows)
    check("O[rows]", o[:, rows], ro[:, rows], "bf16", config=True)
    check("L[rows]", lse[:, :, rows], rl[:, :, rows], "bf16", is_lse=True)


def test_persistent_two_streams_two_workspaces():
    # two calls in flight at once on two streams, each with its own workspace: the queues of
    # one call never hand out the other's tasks, and both results equal fa_fwd's
    import torch

    fa = _fa()
    cases = [workloads.make_attention_inputs(4, 1000, 1000, 16, 4, 128, seed=3101),
             workloads.make_attention_inputs(2, 1500, 1500, 8, 8, 64, seed=3102)]
    dev = [tuple(to_dev(inp[n], "bf16") for n in ("q", "k", "v")) for inp in cases]
    outs, refs = [], []
    for (q, k, v), causal in zip(dev, (True, False)):
        B, Nq, Hq, _ = q.shape
        o1 = torch.empty_like(q)
        l1 = torch.empty((B, Hq, Nq), dtype=torch.float32, device="cuda")
        fa.fa_fwd(q, k, v, o1, l1, causal, None)
        refs.append((o1, l1))
        outs.append((torch.empty_like(q), torch.empty_like(l1)))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [torch.zeros(fa.fa_fwd_persistent_workspace_size(), dtype=torch.uint8, device="cuda") for _ in range(2)]
    for rep in range(3):
        for i, ((q, k, v), causal) in enumerate(zip(dev, (True, False))):
            with torch.cuda.stream(streams[i]):
                fa.fa_fwd_persistent(q, k, v, outs[i][0], outs[i][1], wss[i], causal, None, stream=streams[i])
        torch.cuda.synchronize()
        for i in range(2):
            assert int(wss[i].count_nonzero()) == 0
            assert torch.equal(outs[i][0], refs[i][0]) and torch.equal(outs[i][1], refs[i][1]), (rep, i)
        say(f"  two streams, repeat {rep}: both identical to fa_fwd")
