"""A model of fa_fwd_persistent's task queues, checked on the CPU.

The kernel's rules restated (Lecture 21 notes §4.5): one workgroup per compute unit; queue q
lists the one-shot grid's workgroups q, q + P, q + 2P, ... (P queues, one per XCD, or one);
a workgroup takes the next index of its own XCD's queue and, once that queue is empty, of the
next queues in turn, leaving when all P are empty; each workgroup then adds one to the leaver
count, and the one that brings it to the grid size sets every counter back to zero. Run under
random interleavings of the workgroups' queue operations: every task is taken exactly once,
in each queue's order, and the counters end at zero, for grids smaller and larger than the
task count and for a slow XCD whose queue the others drain.
"""

import random

import pytest

MAX_POOLS = 8


def run(n_tasks, n_cu, seed, slow_xcd=None):
    rng = random.Random(seed)
    P = MAX_POOLS if n_cu % MAX_POOLS == 0 else 1
    grid = min(n_cu, n_tasks)
    ctr = [0] * (MAX_POOLS + 1)
    taken, taker = [], {}
    # workgroup g runs on XCD g % 8 (the hardware's round-robin placement)
    state = [{"home": (g % 8) % P, "tried": 0, "left": False} for g in range(grid)]
    per_queue = [[] for _ in range(P)]
    live = list(range(grid))
    while live:
        # a slow XCD's workgroups move a tenth as often
        weights = [0.1 if slow_xcd is not None and g % 8 == slow_xcd else 1.0 for g in live]
        g = rng.choices(live, weights)[0]
        st = state[g]
        if st["tried"] < P:  # one queue operation: take from the current queue or move on
            q = (st["home"] + st["tried"]) % P
            i = ctr[q]
            ctr[q] += 1
            if i < (n_tasks - q + P - 1) // P:
                wg = q + P * i
                taken.append(wg)
                taker[wg] = g
                per_queue[q].append(wg)
            else:
                st["tried"] += 1
        else:  # all queues empty: leave
            fin = ctr[MAX_POOLS]
            ctr[MAX_POOLS] += 1
            if fin == grid - 1:
                ctr = [0] * (MAX_POOLS + 1)
            live.remove(g)
    return taken, per_queue, ctr, P, taker


@pytest.mark.parametrize("n_tasks,n_cu", [(2048, 256), (4096, 256), (1, 256), (7, 256), (300, 256),
                                          (1000, 96), (513, 250), (2048, 8)])
@pytest.mark.parametrize("seed", [1, 2])
def test_every_task_once_and_counters_back_to_zero(n_tasks, n_cu, seed):
    taken, per_queue, ctr, P, _ = run(n_tasks, n_cu, seed)
    assert sorted(taken) == list(range(n_tasks))
    for q, lst in enumerate(per_queue):
        assert lst == list(range(q, n_tasks, P))  # each queue hands out its workgroups in order
    assert ctr == [0] * (MAX_POOLS + 1)


def test_other_xcds_drain_a_slow_xcds_queue():
    taken, per_queue, ctr, P, taker = run(4096, 256, seed=3, slow_xcd=5)
    assert sorted(taken) == list(range(4096)) and ctr == [0] * (MAX_POOLS + 1)
    assert P == 8 and per_queue[5] == list(range(5, 4096, 8))
    helped = sum(1 for wg in per_queue[5] if taker[wg] % 8 != 5)
    assert helped > len(per_queue[5]) // 4  # most of the slow XCD's queue goes to the others
