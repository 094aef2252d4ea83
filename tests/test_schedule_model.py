"""A model of fa_bwd_single_pass's schedule, checked on the CPU.

The kernel's rules restated (per-XCD pools of (kv head, key block) tasks taken in order; the
visiting order of query blocks; each key block's rank among a block's adders; tags that a
reader waits for and a writer sets once its step is done) and run under random interleavings
of the workgroups of each XCD: every block's ranks are 0 .. count-1 once each, the last adder is
marked, all tags return to zero, and the run never reaches a state where no workgroup can move
(no deadlock) -- with 32 workgroups per XCD and with as few as one, with and without the mask.
The adders of a block are key blocks 0 .. Tc-1 without the mask and 0 .. floor(i/2) with it
(Lecture 21 notes §2.6: key block j sees query rows from 128 j on; 64-row query blocks).
"""

import random

import pytest

BQ, BK = 64, 128


def task_steps(causal, G, n_tr, n_tc, j):
    """(g, i, rank, last) for each step of key block j's task, as the kernel walks them."""
    qb_first = (j * BK) // BQ if causal else 0
    n_steps = G * (n_tr - qb_first)

    def make(sa, sb):
        if causal:
            g, i = sa, sb
            cnt = min(n_tc, (BQ * i + BQ - 1) // BK + 1)
            return (g, i, cnt - 1 - j, j == 0)
        # without the mask every key block walks the G * Tr blocks in the same order
        return (sb // n_tr, sb % n_tr, n_tc - 1 - j, j == 0)

    # causal: query blocks from the last one down, the G heads at each block
    sa, sb = 0, (n_tr - 1 if causal else 0)
    out = []
    for _ in range(n_steps):
        out.append(make(sa, sb))
        if causal:
            sa += 1
            if sa == G:
                sa, sb = 0, sb - 1
            continue
        sb += 1
    return out


def run(B, Hkv, G, Nq, Nk, causal, per_xcd=32, n_pools=8, seed=0):
    n_tr, n_tc, heads = -(-Nq // BQ), -(-Nk // BK), B * Hkv
    adders = {}
    for bh in range(heads):
        for j in range(n_tc):
            for (g, i, rank, last) in task_steps(causal, G, n_tr, n_tc, j):
                adders.setdefault((bh, g, i), []).append((rank, last))
    assert len(adders) == heads * G * n_tr
    for (bh, g, i), lst in adders.items():
        assert sorted(r for r, _ in lst) == list(range(len(lst)))
        assert [r for r, last in lst if last] == [len(lst) - 1]
        assert len(lst) == (min(n_tc, i // 2 + 1) if causal else n_tc)
    rng = random.Random(seed)
    pools = [[(h, n_tc - 1 - jj) for h in range(p, heads, n_pools) for jj in range(n_tc)]
             for p in range(n_pools)]
    grab, tag = [0] * n_pools, {}
    wgs = [{"pool": p, "task": None} for p in range(n_pools) for _ in range(per_xcd)]
    active = list(range(len(wgs)))

    def can_move(w):
        if w["task"] is None:
            return True
        g, i, rank, _ = w["steps"][w["st"]]
        return tag.get((w["task"][0], g, i), 0) == rank

    while active:
        k = rng.choice(active)
        w = wgs[k]
        if w["task"] is None:
            p = w["pool"]
            if grab[p] == len(pools[p]):
                active.remove(k)
                continue
            w["task"], grab[p] = pools[p][grab[p]], grab[p] + 1
            w["steps"], w["st"] = task_steps(causal, G, n_tr, n_tc, w["task"][1]), 0
            continue
        if not can_move(w):
            assert any(can_move(wgs[x]) for x in active), "no workgroup can move"
            continue
        g, i, rank, last = w["steps"][w["st"]]
        tag[(w["task"][0], g, i)] = 0 if last else rank + 1
        w["st"] += 1
        if w["st"] == len(w["steps"]):
            w["task"] = None
    assert all(v == 0 for v in tag.values())


@pytest.mark.parametrize("B,Hkv,G,Nq,Nk,causal", [
    (1, 1, 1, 2048, 2048, False), (2, 2, 2, 2048, 2048, False), (1, 2, 2, 256, 2048, False),
    (1, 1, 1, 1024, 2048, False), (1, 1, 2, 100, 333, False), (2, 4, 3, 333, 2000, False),
    (1, 1, 1, 64, 2048, False), (1, 1, 1, 1, 1, False),
    (2, 2, 1, 300, 300, True), (1, 1, 4, 1000, 1000, True), (3, 5, 1, 4096, 4096, True),
])
def test_schedule(B, Hkv, G, Nq, Nk, causal):
    run(B, Hkv, G, Nq, Nk, causal, seed=B + Nq)


@pytest.mark.parametrize("B,Hkv,G,Nq,Nk", [(2, 2, 1, 300, 300), (1, 1, 4, 1000, 1000)])
def test_causal_needs_no_coresidency(B, Hkv, G, Nq, Nk):
    run(B, Hkv, G, Nq, Nk, True, per_xcd=1, seed=3)


@pytest.mark.parametrize("G,N", [(1, 2048), (4, 1000), (3, 333)])
def test_causal_blocks_reached_at_the_same_offset(G, N):
    # every key block reaches query block (g, i) the same number of steps after its start, so the
    # adders of a block arrive in the order their tasks were taken (largest j first) and follow
    # one another closely
    n_tr, n_tc = -(-N // BQ), -(-N // BK)
    for j in range(n_tc):
        for s, (g, i, rank, _) in enumerate(task_steps(True, G, n_tr, n_tc, j)):
            assert s == (n_tr - 1 - i) * G + g
            assert rank == min(n_tc, i // 2 + 1) - 1 - j


@pytest.mark.parametrize("B,Hkv,G,Nq,Nk", [(1, 1, 1, 2048, 2048), (2, 2, 2, 300, 4000), (1, 1, 1, 64, 2100), (3, 2, 3, 333, 2000)])
@pytest.mark.parametrize("per_xcd", [1, 5, 32])
def test_noncausal_any_residency(B, Hkv, G, Nq, Nk, per_xcd):
    run(B, Hkv, G, Nq, Nk, False, per_xcd=per_xcd, seed=per_xcd + Nk)
