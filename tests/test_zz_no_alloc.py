"""fa_decode_noalloc (the decode that allocates nothing: its scratch is a static per-GPU array
in the library) through the C ABI against fa_decode with a workspace, on calls in a row: the
second smaller than the first, so it finds the first call's contents in the array, and a third
larger than the second, whose arrival counters cover more of the array than the second's did
and must still start at zero (they lie where no call writes partials)."""

import math

import numpy as np
import pytest

import workloads
from gpu_util import check, say, to_dev, to_np
from oracle import attention as ora

pytestmark = pytest.mark.gpu


def _pair(fa, inp, scale):
    import torch

    q, k, v = (to_dev(inp[n], "bf16") for n in ("q", "k", "v"))
    lens = torch.from_numpy(inp["seqlens"]).cuda()
    B, _, Hq, d = q.shape
    ws = torch.zeros(fa.fa_decode_workspace_size(B, Hq, k.shape[1], d), dtype=torch.uint8, device="cuda")
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    l1 = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    l2 = torch.empty_like(l1)
    fa.fa_decode(q, k, v, lens, o1, l1, ws, scale)
    fa.fa_decode_noalloc(q, k, v, lens, o2, l2, scale)
    torch.cuda.synchronize()
    return (to_np(o1), to_np(l1)), (to_np(o2), to_np(l2))


def test_decode_noalloc_matches_decode_twice():
    import exact_io_aware_03_amd as fa

    w = workloads.WORKLOADS["decode_bf16_b64hq32hkv8d128"]
    big = workloads.make_workload_inputs(w)
    small = workloads.make_decode_inputs(3, 8, 2, 700, 128, seed=9, lengths=[1, 300, 700])
    medium = workloads.make_decode_inputs(16, 16, 4, 2048, 128, seed=11, len_range=(1, 2048))
    cases = (("decode workload", big, w.scale), ("small GQA 4:1", small, 1 / math.sqrt(128)),
             ("medium GQA 4:1, more counters than the small call", medium, 1 / math.sqrt(128)))
    for name, inp, scale in cases:
        say(f"noalloc {name}: B={inp['q'].shape[0]} Hq={inp['q'].shape[2]} Hkv={inp['k'].shape[2]}")
        (o1, l1), (o2, l2) = _pair(fa, inp, scale)
        say(f"  identical to fa_decode: O {np.array_equal(o1, o2)}, L {np.array_equal(l1, l2)}")
        check("O noalloc vs fa_decode", o2, o1, "bf16")
        check("L noalloc vs fa_decode", l2, l1, "bf16", is_lse=True)
        if inp["q"].shape[0] <= 16:
            ro, rl = ora.decode(inp["q"], inp["k"], inp["v"], inp["seqlens"], scale)
            check("O noalloc vs oracle", o2, ro, "bf16")
            check("L noalloc vs oracle", l2, rl, "bf16", is_lse=True)


def test_decode_noalloc_under_graph_capture():
    # the callers it is for: a HIP graph holds one call and replays it; every replay, with eager
    # work between (another shape's call through the same scratch array, fills, syncs), gives
    # the eager call's result bit for bit
    import torch

    import exact_io_aware_03_amd as fa

    inp = workloads.make_decode_inputs(16, 16, 4, 2048, 128, seed=12, len_range=(1, 2048))
    other = workloads.make_decode_inputs(5, 8, 8, 900, 64, seed=13, len_range=(1, 900))
    scale = 1 / math.sqrt(128)
    q, k, v = (to_dev(inp[n], "bf16") for n in ("q", "k", "v"))
    lens = torch.from_numpy(inp["seqlens"]).cuda()
    q2, k2, v2 = (to_dev(other[n], "bf16") for n in ("q", "k", "v"))
    lens2 = torch.from_numpy(other["seqlens"]).cuda()
    B, _, Hq, _ = q.shape
    o_ref = torch.empty_like(q)
    l_ref = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    fa.fa_decode_noalloc(q, k, v, lens, o_ref, l_ref, scale)  # eager; also finds the scratch address
    o2 = torch.empty_like(q2)
    l2 = torch.empty((q2.shape[0], q2.shape[2]), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    o, l = torch.empty_like(o_ref), torch.empty_like(l_ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fa.fa_decode_noalloc(q, k, v, lens, o, l, scale)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fa.fa_decode_noalloc(q, k, v, lens, o, l, scale)
    torch.cuda.synchronize()
    for rep in range(4):
        o.zero_()
        l.zero_()
        fa.fa_decode_noalloc(q2, k2, v2, lens2, o2, l2, 1 / math.sqrt(64))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        same = torch.equal(o, o_ref) and torch.equal(l, l_ref)
        say(f"  graph replay {rep}: identical to the eager call: {same}")
        assert same
    ro, rl = ora.decode(inp["q"], inp["k"], inp["v"], inp["seqlens"], scale)
    check("O graph replay vs oracle", to_np(o), ro, "bf16")
    check("L graph replay vs oracle", to_np(l), rl, "bf16", is_lse=True)
