"""GPU parity of the forward (fa_fwd through the C ABI) against the fp64 oracle."""

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


def run_fwd(inp, causal, scale, dtype):
    fa = _fa()
    q, k, v = (to_dev(inp[n], dtype) for n in ("q", "k", "v"))
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    import torch

    torch.cuda.synchronize()
    return to_np(o), to_np(lse)


SMALL = [
    # B, Nq, Nk, Hq, Hkv, d, causal, dtype
    (1, 128, 128, 1, 1, 128, False, "bf16"),
    (1, 128, 128, 1, 1, 128, True, "bf16"),
    (2, 300, 300, 4, 2, 128, True, "bf16"),    # ragged: not a multiple of the 128-row block
    (1, 77, 333, 4, 1, 128, False, "bf16"),    # N_q != N_k, G = 4, ragged both ways
    (2, 257, 257, 2, 2, 64, True, "bf16"),
    (1, 129, 65, 8, 2, 64, False, "bf16"),
    (1, 1, 1, 1, 1, 128, False, "bf16"),       # a single key and query
    (1, 5, 1000, 2, 1, 64, False, "bf16"),
    # more (batch, head, row block) tasks than compute units: ragged rows and keys with GQA, and
    # the minimum of three key tiles at d = 64
    (4, 700, 451, 32, 8, 128, False, "bf16"),
    (3, 300, 192, 64, 64, 64, False, "bf16"),
    (1, 256, 256, 1, 1, 64, False, "f32"),
    (2, 200, 200, 4, 2, 64, True, "f32"),
    (1, 70, 190, 2, 1, 128, False, "f32"),
]


@pytest.mark.parametrize("B,Nq,Nk,Hq,Hkv,d,causal,dtype", SMALL)
def test_fwd_small(B, Nq, Nk, Hq, Hkv, d, causal, dtype):
    say(f"fwd small B={B} Nq={Nq} Nk={Nk} Hq={Hq} Hkv={Hkv} d={d} causal={causal} {dtype}")
    inp = workloads.make_attention_inputs(B, Nq, Nk, Hq, Hkv, d, seed=1000 + Nq + Nk + d, dtype=dtype)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_fwd(inp, causal, scale, dtype)
    ro, rl = ora.forward(inp["q"], inp["k"], inp["v"], causal, scale)
    check("O", o, ro, dtype)
    check("L", lse, rl, dtype, is_lse=True)


def test_fwd_f32_single_head_config():
    w = workloads.WORKLOADS["fwd_f32_256x64"]
    say(f"fwd config {w.name}")
    inp = workloads.make_workload_inputs(w)
    o, lse = run_fwd(inp, False, w.scale, "f32")
    ro, rl = ora.forward(inp["q"], inp["k"], inp["v"], False, w.scale)
    check("O", o, ro, "f32")
    check("L", lse, rl, "f32", is_lse=True)


def test_causal_row0_is_v0_bf16():
    inp = workloads.make_attention_inputs(2, 384, 384, 4, 2, 128, seed=77)
    o, _ = run_fwd(inp, True, 1 / math.sqrt(128), "bf16")
    v = inp["v"].astype(np.float64)
    for h in range(4):
        # P = [1] in row 0, so the bf16 output reproduces V[0] exactly
        np.testing.assert_array_equal(o[:, 0, h], v[:, 0, h // 2])


def test_kv_permutation_invariance_gpu():
    inp = workloads.make_attention_inputs(1, 200, 300, 2, 2, 128, seed=78)
    perm = np.random.Generator(np.random.PCG64(3)).permutation(300)
    o0, l0 = run_fwd(inp, False, 0.1, "bf16")
    inp2 = dict(inp, k=inp["k"][:, perm], v=inp["v"][:, perm])
    o1, l1 = run_fwd(inp2, False, 0.1, "bf16")
    assert np.abs(o1 - o0).max() <= 2e-2 and np.abs(l1 - l0).max() <= 1e-4


def test_large_scores_no_overflow():
    # scores of a few hundred: exp must see only differences from the running max
    inp = workloads.make_attention_inputs(1, 130, 130, 1, 1, 64, seed=79)
    inp["q"] = workloads.round_to_bf16(inp["q"] * 8.0)
    o, lse = run_fwd(inp, True, 1.0, "bf16")
    ro, rl = ora.forward(inp["q"], inp["k"], inp["v"], True, 1.0)
    assert np.all(np.isfinite(o))
    check("O", o, ro, "bf16")
    assert np.abs(lse - rl).max() <= 1e-3 * max(1.0, np.abs(rl).max() / 64)


@pytest.mark.parametrize("causal", [False, True])
def test_rising_scores_move_the_reference(causal):
    # scores rising by ~60 (base 2) along the keys: the conditional rescale (threshold 8) fires
    # several times per row, in the masked diagonal tiles too
    rng = np.random.Generator(np.random.PCG64(86))
    B, N, H, d = 1, 1024, 2, 128
    q = rng.standard_normal((B, N, H, d))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    ramp = np.linspace(0.0, 60.0 * math.log(2.0), N)
    k = ramp[None, :, None, None] * q[:, :1] + 0.05 * rng.standard_normal((B, N, H, d))
    v = rng.standard_normal((B, N, H, d))
    inp = {n: workloads.round_to_bf16(x.astype(np.float32)) for n, x in (("q", q), ("k", k), ("v", v))}
    o, lse = run_fwd(inp, causal, 1.0, "bf16")
    ro, rl = ora.forward(inp["q"], inp["k"], inp["v"], causal, 1.0)
    check("O", o, ro, "bf16")
    check("L", lse, rl, "bf16", is_lse=True)


def _sampled_config(w, causal, n_heads, n_rows, seed):
    say(f"fwd config {w.name} causal={causal}")
    inp = workloads.make_workload_inputs(w)
    o, lse = run_fwd(inp, causal, w.scale, w.dtype)
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    pick = workloads.sample_indices(len(heads), n_heads, seed)
    sel = [heads[i] for i in pick]
    say(f"  oracle on {len(sel)} full heads")
    ro, rl = ora.forward(inp["q"], inp["k"], inp["v"], causal, w.scale, heads=sel)
    for b, h in sel:
        check(f"O[b={b},h={h}]", o[b, :, h], ro[b, :, h], w.dtype, config=True)
        check(f"L[b={b},h={h}]", lse[b, h], rl[b, h], w.dtype, is_lse=True)
    rows = np.unique(np.concatenate([[0, 1, w.Nq - 1], workloads.sample_indices(w.Nq, n_rows, seed + 1)]))
    say(f"  oracle on {rows.size} rows of every head")
    ro, rl = ora.forward(inp["q"], inp["k"], inp["v"], causal, w.scale, rows=rows)
    check("O[rows]", o[:, rows], ro[:, rows], w.dtype, config=True)
    check("L[rows]", lse[:, :, rows], rl[:, :, rows], w.dtype, is_lse=True)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_training_shape(causal):
    _sampled_config(workloads.WORKLOADS["fwd_bf16_b16h16n2048d128"], causal, n_heads=6, n_rows=12, seed=21)


def test_fwd_long_context_causal():
    _sampled_config(workloads.WORKLOADS["fwd_bf16_causal_h32n16384d128"], True, n_heads=2, n_rows=8, seed=31)
