"""GPU parity of decode (fa_decode) and backward (fa_bwd) through the C ABI vs the fp64 oracle."""

import math
import time

import numpy as np
import pytest

import workloads
from gpu_util import check, say, to_dev, to_np
from oracle import attention as ora
from oracle import rounding as rnd

pytestmark = pytest.mark.gpu


def _fa():
    import exact_io_aware_03_amd as fa

    return fa


def run_decode(inp, scale):
    import torch

    fa = _fa()
    q, k, v = (to_dev(inp[n], "bf16") for n in ("q", "k", "v"))
    lens = torch.from_numpy(inp["seqlens"]).cuda()
    B, _, Hq, d = q.shape
    # partial area all 0xFF (NaN as fp32): a read of a partial the kernels never wrote shows; the
    # arrival counters at the start of the workspace are zero, as the contract asks
    ws = torch.full((fa.fa_decode_workspace_size(B, Hq, k.shape[1], d),), 255, dtype=torch.uint8, device="cuda")
    n_cnt = (B * Hq * 4 + 255) // 256 * 256
    ws[:n_cnt] = 0
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    fa.fa_decode(q, k, v, lens, o, lse, ws, scale)
    torch.cuda.synchronize()
    # every call leaves the counters zero
    assert int(ws[:n_cnt].count_nonzero()) == 0
    return to_np(o), to_np(lse)


@pytest.mark.parametrize(
    "B,Hq,Hkv,Nk_max,d,lengths",
    [
        (4, 8, 2, 1100, 128, [1, 255, 256, 1100]),
        (3, 32, 8, 8192, 128, [8192, 257, 4097]),
        (2, 8, 8, 600, 64, [600, 3]),
        (2, 16, 2, 700, 128, [513, 64]),   # 8 query heads per kv head
        (2, 16, 1, 300, 64, [300, 129]),   # 16 query heads per kv head
        # the persistent split of the block list: more sequences than one wave scans at once,
        # more workers than blocks (empty workers), one sequence over many workers, kv heads
        # that leave spare waves (3), several kv heads per wave (16), several workers per
        # workgroup (1 kv head), a one-key cache
        (100, 8, 8, 200, 128, [int(x) for x in np.random.default_rng(7).integers(1, 201, size=100)]),
        (1, 8, 8, 8192, 128, [8192]),
        (2, 6, 3, 500, 128, [500, 77]),
        (2, 32, 16, 300, 64, [300, 190]),
        (3, 4, 1, 1000, 128, [1000, 1, 640]),
        (1, 2, 2, 1, 64, [1]),
        # workgroups whose waves step through the blocks together: 8 query heads per kv head
        # (4 waves, 2 kv heads each), 16 per kv head (4 waves, one kv head each)
        (2, 64, 8, 400, 128, [400, 130]),
        (2, 64, 4, 300, 64, [300, 65]),
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


def test_decode_reuses_its_workspace():
    # two calls on one workspace, the second with other lengths: the counters the first call
    # leaves (zero) serve the second, and both results match the oracle
    import torch

    fa = _fa()
    B, Hq, Hkv, Nk_max, d = 6, 16, 4, 3000, 128
    ws = torch.zeros(fa.fa_decode_workspace_size(B, Hq, Nk_max, d), dtype=torch.uint8, device="cuda")
    for lengths, seed in (([3000, 1, 2999, 64, 1500, 700], 801), ([5, 3000, 3000, 129, 1, 2048], 802)):
        inp = workloads.make_decode_inputs(B, Hq, Hkv, Nk_max, d, seed=seed, lengths=lengths)
        q, k, v = (to_dev(inp[n], "bf16") for n in ("q", "k", "v"))
        lens = torch.from_numpy(inp["seqlens"]).cuda()
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        fa.fa_decode(q, k, v, lens, o, lse, ws, 1 / math.sqrt(d))
        torch.cuda.synchronize()
        ro, rl = ora.decode(inp["q"], inp["k"], inp["v"], inp["seqlens"], 1 / math.sqrt(d))
        check("O", to_np(o), ro, "bf16")
        check("L", to_np(lse), rl, "bf16", is_lse=True)


def test_decode_config():
    w = workloads.WORKLOADS["decode_bf16_b64hq32hkv8d128"]
    say(f"decode config {w.name}")
    inp = workloads.make_workload_inputs(w)
    o, lse = run_decode(inp, w.scale)
    ro, rl = ora.decode(inp["q"], inp["k"], inp["v"], inp["seqlens"], w.scale)
    check("O", o, ro, "bf16", config=True)
    check("L", lse, rl, "bf16", is_lse=True)


def bwd_zeroed_bytes(B, Hq, Nq, d):
    """Bytes at the start of the fa_bwd workspace that are zero between calls: the task-pool
    counters and the tagged fp32 partial sums of dQ."""
    return 256 + 4 * 64 * d * B * Hq * -(-Nq // 64)


def run_fwd_bwd(inp, causal, scale, ws=None, single_pass=False):
    import torch

    fa = _fa()
    bwd = fa.fa_bwd_single_pass if single_pass else fa.fa_bwd
    q, k, v, do = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    B, Nq, Hq, d = q.shape
    nc = bwd_zeroed_bytes(B, Hq, Nq, d)
    if ws is None:
        # D all 0xFF (NaN as fp32): a row of D the kernels read before writing would show; the
        # counters and partial sums start at zero, as the contract asks
        ws = torch.full((fa.fa_bwd_workspace_size(B, Hq, Nq, d),), 255, dtype=torch.uint8, device="cuda")
        ws[:nc] = 0
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bwd(q, k, v, o, do, lse, dq, dk, dv, ws, causal, scale)
    torch.cuda.synchronize()
    # every call leaves the counters and partial sums zero (a bounded wait that ran out would
    # leave its count here)
    assert int(torch.count_nonzero(ws[:nc])) == 0
    return to_np(dq), to_np(dk), to_np(dv)


def single_pass_supported(Nk, d, causal):
    """Shapes fa_bwd_single_pass takes: d = 128 and at most 255 key blocks of 128 (8-bit adder
    tags), with or without the mask."""
    n_tc = -(-Nk // 128)
    return d == 128 and n_tc <= 255


@pytest.mark.parametrize(
    "B,Nq,Nk,Hq,Hkv,d,causal,seed",
    [
        (1, 128, 128, 1, 1, 128, False, None),
        (1, 128, 128, 1, 1, 128, True, None),
        (2, 300, 300, 2, 2, 128, True, None),   # ragged
        (1, 200, 200, 4, 2, 64, False, None),   # GQA, d = 64
        (1, 257, 257, 4, 1, 128, True, None),   # GQA 4:1, ragged
        # the same shape at the inputs where the plain 2e-2 bound first failed (dV 0.0224 at
        # |ref| = 4.73): the dK/dV of a kv head sum four query heads and reach |ref| 7.5
        (1, 257, 257, 4, 1, 128, True, 1542),
        (1, 64, 64, 2, 2, 64, True, None),
        (1, 100, 333, 2, 1, 128, False, None),  # N_q != N_k, both ragged
        (1, 520, 70, 2, 1, 64, False, None),    # more query rows than keys
        (1, 1, 1, 1, 1, 128, False, None),      # one query, one key: dS = 0, dV = dO
        (1, 256, 2048, 4, 2, 128, False, None),  # 16 key blocks, fewer query blocks than key blocks
        (1, 64, 2100, 2, 1, 128, False, None),  # 17 key blocks without the mask, more than half an XCD
        (1, 64, 32769, 1, 1, 128, False, None),  # 257 key blocks: past the single pass's 8-bit tags
        (1, 1100, 1100, 2, 1, 128, True, None),  # causal GQA, 9 key blocks, ragged
    ],
)
@pytest.mark.parametrize("single_pass", [False, True])
def test_bwd_small(B, Nq, Nk, Hq, Hkv, d, causal, seed, single_pass):
    if seed is None:
        seed = 900 + Nq + d if Nq == Nk else 950 + Nq + 3 * Nk + d
    say(f"bwd B={B} Nq={Nq} Nk={Nk} Hq={Hq} Hkv={Hkv} d={d} causal={causal} seed={seed} single_pass={single_pass}")
    inp = workloads.make_attention_inputs(B, Nq, Nk, Hq, Hkv, d, seed=seed, with_do=True)
    scale = 1.0 / math.sqrt(d)
    if single_pass and not single_pass_supported(Nk, d, causal):
        fa = _fa()
        with pytest.raises(fa.FAError) as e:
            run_fwd_bwd(inp, causal, scale, single_pass=True)
        assert e.value.code == -2  # FA_ERR_UNSUPPORTED, before any device work
        return
    dq, dk, dv = run_fwd_bwd(inp, causal, scale, single_pass=single_pass)
    rq, rk, rv = ora.backward(inp["q"], inp["k"], inp["v"], inp["do"], causal, scale)
    check("dQ", dq, rq, "bf16")
    check("dK", dk, rk, "bf16")
    check("dV", dv, rv, "bf16")


@pytest.mark.parametrize("single_pass", [False, True])
def test_bwd_255_key_blocks(single_pass):
    # the largest key-block count the single pass takes (Nk = 32640, 8-bit adder tags): every
    # block of dQ gets 255 adders, without the mask; the two-kernel path on the same inputs
    B, Nq, Nk, Hq, Hkv, d = 1, 100, 32640, 2, 1, 128
    say(f"bwd 255 key blocks B={B} Nq={Nq} Nk={Nk} Hq={Hq} Hkv={Hkv} single_pass={single_pass}")
    inp = workloads.make_attention_inputs(B, Nq, Nk, Hq, Hkv, d, seed=5301, with_do=True)
    # with 32640 keys every P is about 3e-5 and the gradients are small next to the 2e-2 floor;
    # dO times 64 (exact in bf16) brings them to order one
    inp["do"] = inp["do"] * 64.0
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = run_fwd_bwd(inp, False, scale, single_pass=single_pass)
    args = (inp["q"], inp["k"], inp["v"], inp["do"], False, scale)
    for n, g, r, t in zip(("dQ", "dK", "dV"), (dq, dk, dv), ora.backward(*args), rnd.backward_terms(*args)):
        check(n, g, r, "bf16", terms=t)


@pytest.mark.parametrize("single_pass", [False, True])
def test_bwd_long_causal(single_pass):
    # one long causal head: 256 query blocks, 128 key blocks (the single pass's longest task
    # walks 256 blocks; its shortest two)
    B, N, Hq, Hkv, d = 1, 16384, 1, 1, 128
    say(f"bwd long causal N={N} single_pass={single_pass}")
    inp = workloads.make_attention_inputs(B, N, N, Hq, Hkv, d, seed=5302, with_do=True)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = run_fwd_bwd(inp, True, scale, single_pass=single_pass)
    say("  oracle gradients and rounding terms")
    args = (inp["q"], inp["k"], inp["v"], inp["do"], True, scale)
    for n, g, r, t in zip(("dQ", "dK", "dV"), (dq, dk, dv), ora.backward(*args), rnd.backward_terms(*args)):
        check(n, g, r, "bf16", terms=t)


@pytest.mark.parametrize("single_pass", [False, True])
def test_bwd_config(single_pass):
    w = workloads.WORKLOADS["bwd_bf16_causal_b8h16n4096d128"]
    say(f"bwd config {w.name} single_pass={single_pass}")
    inp = workloads.make_workload_inputs(w)
    dq, dk, dv = run_fwd_bwd(inp, True, w.scale, single_pass=single_pass)
    pairs = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    sel = [pairs[i] for i in workloads.sample_indices(len(pairs), 3, 51)]
    say(f"  oracle gradients on heads {sel}")
    rq, rk, rv = ora.backward(inp["q"], inp["k"], inp["v"], inp["do"], True, w.scale, heads=sel)
    for b, g in sel:
        check(f"dQ[b={b},h={g}]", dq[b, :, g], rq[b, :, g], "bf16", config=True)
        check(f"dK[b={b},h={g}]", dk[b, :, g], rk[b, :, g], "bf16", config=True)
        check(f"dV[b={b},h={g}]", dv[b, :, g], rv[b, :, g], "bf16", config=True)


@pytest.mark.parametrize("single_pass", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_training_shape(causal, single_pass):
    # the shape and launch configuration the benchmark step times, on sampled heads
    w = workloads.WORKLOADS["fwd_bf16_b16h16n2048d128"]
    say(f"bwd training shape {w.name} causal={causal} single_pass={single_pass}")
    inp = workloads.make_attention_inputs(w.B, w.Nq, w.Nk, w.Hq, w.Hkv, w.d, seed=w.seed, with_do=True)
    dq, dk, dv = run_fwd_bwd(inp, causal, w.scale, single_pass=single_pass)
    pairs = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    sel = [pairs[i] for i in workloads.sample_indices(len(pairs), 3, 61 + causal)]
    say(f"  oracle gradients on heads {sel}")
    rq, rk, rv = ora.backward(inp["q"], inp["k"], inp["v"], inp["do"], causal, w.scale, heads=sel)
    for b, g in sel:
        check(f"dQ[b={b},h={g}]", dq[b, :, g], rq[b, :, g], "bf16", config=True)
        check(f"dK[b={b},h={g}]", dk[b, :, g], rk[b, :, g], "bf16", config=True)
        check(f"dV[b={b},h={g}]", dv[b, :, g], rv[b, :, g], "bf16", config=True)


@pytest.mark.parametrize("single_pass", [False, True])
def test_bwd_reuses_its_workspace(single_pass):
    # three calls on one workspace (same B, Hq, Nq; other kv heads, mask and inputs): the counters
    # and partial sums each call leaves must be the zeros the next one starts from, and the
    # results match a call on a fresh workspace bit for bit
    import torch

    fa = _fa()
    ws = torch.zeros(fa.fa_bwd_workspace_size(2, 4, 700, 128), dtype=torch.uint8, device="cuda")
    for (Hkv, causal, seed) in ((2, True, 77), (4, False, 78), (1, True, 79)):
        say(f"bwd workspace reuse B=2 N=700 Hq=4 Hkv={Hkv} causal={causal} single_pass={single_pass}")
        inp = workloads.make_attention_inputs(2, 700, 700, 4, Hkv, 128, seed=seed, with_do=True)
        got = run_fwd_bwd(inp, causal, 0.09, ws=ws, single_pass=single_pass)
        ref = run_fwd_bwd(inp, causal, 0.09, single_pass=single_pass)
        for a, b in zip(got, ref):
            assert np.array_equal(a, b)


@pytest.mark.parametrize("single_pass", [False, True])
def test_bwd_and_fwd_are_reproducible(single_pass):
    # no atomics and a fixed summation order: two calls give bit-identical results
    import torch

    fa = _fa()
    inp = workloads.make_attention_inputs(2, 700, 700, 4, 2, 128, seed=4242, with_do=True)
    q, k, v, do = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    B, Nq, Hq, d = q.shape
    runs = []
    for _ in range(2):
        o, lse = fa.forward(q, k, v, causal=True, scale=0.1)
        ws = torch.zeros(fa.fa_bwd_workspace_size(B, Hq, Nq, d), dtype=torch.uint8, device="cuda")
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        (fa.fa_bwd_single_pass if single_pass else fa.fa_bwd)(q, k, v, o, do, lse, dq, dk, dv, ws, True, 0.1)
        torch.cuda.synchronize()
        runs.append([t.clone() for t in (o, lse, dq, dk, dv)])
    for a, b in zip(*runs):
        assert torch.equal(a, b)


def test_single_pass_two_streams_two_workspaces():
    # two single-pass calls in flight at once on two streams (one per mask, 16 key blocks per
    # head), each with its own workspace: a task only waits for tasks of its own call taken before
    # it, so neither call needs all of its workgroups resident, and both results are bit-identical
    # to the same call run alone
    import torch

    fa = _fa()
    cases = [(workloads.make_attention_inputs(2, 2048, 2048, 8, 4, 128, seed=5101, with_do=True), False),
             (workloads.make_attention_inputs(2, 2048, 2048, 8, 8, 128, seed=5102, with_do=True), True)]
    dev, refs, outs, wss = [], [], [], []
    for inp, causal in cases:
        q, k, v, do = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
        o, lse = fa.forward(q, k, v, causal=causal, scale=0.09)
        B, Nq, Hq, d = q.shape
        ws = torch.zeros(fa.fa_bwd_workspace_size(B, Hq, Nq, d), dtype=torch.uint8, device="cuda")
        r = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
        fa.fa_bwd_single_pass(q, k, v, o, do, lse, *r, ws, causal, 0.09)
        dev.append((q, k, v, o, do, lse, causal))
        refs.append(r)
        outs.append([torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)])
        wss.append((ws, bwd_zeroed_bytes(B, Hq, Nq, d)))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for i, (q, k, v, o, do, lse, causal) in enumerate(dev):
            with torch.cuda.stream(streams[i]):
                fa.fa_bwd_single_pass(q, k, v, o, do, lse, *outs[i], wss[i][0], causal, 0.09, stream=streams[i])
        torch.cuda.synchronize()
        for i in range(2):
            ws, nc = wss[i]
            assert int(torch.count_nonzero(ws[:nc])) == 0, (rep, i)
            for a, b in zip(outs[i], refs[i]):
                assert torch.equal(a, b), (rep, i)
        say(f"  two streams, repeat {rep}: both identical to the calls run alone")


@pytest.mark.parametrize("causal", [False, True])
def test_single_pass_bounded_wait_reports_a_broken_workspace(causal):
    # A workspace whose task-pool counters do not start at zero breaks the call's contract: every
    # pool skips its first task, so some blocks never get their first adder and the adders after
    # it wait for a tag that never comes. Each such wait ends after 0.2 s, the wave stops waiting
    # for the rest of the launch, the kernel still finishes, the event is counted in the word the
    # kernel never clears, and the last workgroup still resets the pool counters. A call on a
    # zeroed workspace afterwards is exact again (bit-identical to a clean run).
    import torch

    fa = _fa()
    inp = workloads.make_attention_inputs(1, 512, 512, 16, 16, 128, seed=5201, with_do=True)
    q, k, v, do = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal=causal, scale=0.09)
    B, Nq, Hq, d = q.shape
    nc = bwd_zeroed_bytes(B, Hq, Nq, d)
    ws = torch.zeros(fa.fa_bwd_workspace_size(B, Hq, Nq, d), dtype=torch.uint8, device="cuda")
    ref = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    fa.fa_bwd_single_pass(q, k, v, o, do, lse, *ref, ws, causal, 0.09)
    torch.cuda.synchronize()
    ctr = ws[:64].view(torch.int32)
    assert int(torch.count_nonzero(ws[:nc])) == 0
    ctr[:8] = 1  # the eight task-pool counters
    out = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    t0 = time.perf_counter()
    fa.fa_bwd_single_pass(q, k, v, o, do, lse, *out, ws, causal, 0.09)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    c = ctr.tolist()
    say(f"  broken workspace: call returned after {dt:.2f} s, waits that ran out: {c[15]}, counters {c[:9]}")
    assert c[15] > 0
    assert c[:9] == [0] * 9
    ws.zero_()
    fa.fa_bwd_single_pass(q, k, v, o, do, lse, *out, ws, causal, 0.09)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws[:nc])) == 0
    for a, b in zip(out, ref):
        assert torch.equal(a, b)
