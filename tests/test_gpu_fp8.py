"""GPU parity of the FP8 path through the C ABI: the quantise step bit-exact against the
oracle's, and the FP8 forward against the fp64 oracle run on the dequantised (rotated) Q and K
and the bf16 V (Lecture 21 notes §4.4 and exercise 8)."""

import math

import numpy as np
import pytest

import workloads
from gpu_util import check, say, to_dev, to_np
from oracle import attention as ora
from oracle import fp8 as ofp8

pytestmark = pytest.mark.gpu


def _fa():
    import exact_io_aware_03_amd as fa

    return fa


def _signs(d, seed):
    return np.random.Generator(np.random.PCG64(seed)).choice([-1.0, 1.0], size=d).astype(np.float32)


def gpu_quantize(x, signs):
    import torch

    fa = _fa()
    xs = to_dev(x, "bf16")
    sg = None if signs is None else torch.from_numpy(signs).cuda()
    x8, sc = fa.quantize_fp8(xs, sg)
    torch.cuda.synchronize()
    return x8.cpu().numpy(), sc.cpu().numpy()


@pytest.mark.parametrize("shape,rotate,outliers", [
    ((2, 200, 3, 128), True, 0.0),
    ((2, 200, 3, 128), False, 0.0),
    ((1, 64, 2, 64), True, 0.0),
    ((1, 130, 4, 128), True, 0.01),   # element-wise outliers x20
    ((1, 1, 1, 128), True, 0.0),      # a single row
])
def test_quantize_matches_oracle_bit_for_bit(shape, rotate, outliers):
    B, N, H, d = shape
    say(f"quantize {shape} rotate={rotate} outliers={outliers}")
    rng = np.random.Generator(np.random.PCG64(300 + N + d))
    x = rng.standard_normal(shape).astype(np.float32)
    if outliers:
        x[rng.random(shape) < outliers] *= 20.0
    x = workloads.round_to_bf16(x)
    signs = _signs(d, 7) if rotate else None
    codes, scales = gpu_quantize(x, signs)
    rc, rs, _ = ofp8.quantize(x, signs)
    assert np.array_equal(scales, rs)
    diff = np.argwhere(codes != rc)
    assert diff.size == 0, f"{len(diff)} codes differ, first at {diff[:3].tolist()}"


def run_fwd_fp8(q8, qs, k8, ks, v, causal, scale):
    import torch

    fa = _fa()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    o, lse = fa.forward_fp8(t(q8), t(k8), to_dev(v, "bf16"), t(qs), t(ks), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return to_np(o), to_np(lse)


@pytest.mark.parametrize("B,Nq,Nk,Hq,Hkv,causal,d", [
    (1, 256, 256, 1, 1, False, 128),
    (1, 256, 256, 1, 1, True, 128),
    (2, 300, 300, 4, 2, True, 128),   # ragged, GQA
    (1, 77, 333, 4, 1, False, 128),   # N_q != N_k
    (1, 1, 1, 1, 1, False, 128),
    # d = 64: 64-byte E4M3 rows, the K tile padded to one load per wave
    (1, 256, 256, 2, 1, False, 64),
    (2, 300, 300, 4, 2, True, 64),    # ragged, GQA
    (1, 77, 333, 4, 1, False, 64),
    (1, 1, 1, 1, 1, False, 64),
])
def test_fwd_fp8_small(B, Nq, Nk, Hq, Hkv, causal, d):
    say(f"fwd fp8 B={B} Nq={Nq} Nk={Nk} Hq={Hq} Hkv={Hkv} causal={causal} d={d}")
    inp = workloads.make_attention_inputs(B, Nq, Nk, Hq, Hkv, d, seed=1500 + Nq + Nk + (0 if d == 128 else 64))
    signs = _signs(d, 8)
    q8, qs, qd = ofp8.quantize(inp["q"], signs)
    k8, ks, kd = ofp8.quantize(inp["k"], signs)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_fwd_fp8(q8, qs, k8, ks, inp["v"], causal, scale)
    ro, rl = ora.forward(qd, kd, inp["v"], causal, scale)
    check("O", o, ro, "bf16")
    check("L", lse, rl, "bf16", is_lse=True)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp8_training_shape(causal):
    # the shape the benchmark times, quantised on the GPU (bit-identical to the oracle's codes)
    import torch

    fa = _fa()
    w = workloads.WORKLOADS["fwd_bf16_b16h16n2048d128"]
    say(f"fwd fp8 training shape causal={causal}")
    inp = workloads.make_workload_inputs(w)
    signs = _signs(w.d, 9)
    sg = torch.from_numpy(signs).cuda()
    q8, qs = fa.quantize_fp8(to_dev(inp["q"], "bf16"), sg)
    k8, ks = fa.quantize_fp8(to_dev(inp["k"], "bf16"), sg)
    o, lse = fa.forward_fp8(q8, k8, to_dev(inp["v"], "bf16"), qs, ks, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    o, lse = to_np(o), to_np(lse)
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    sel = [heads[i] for i in workloads.sample_indices(len(heads), 3, 71 + causal)]
    bsel = sorted({b for b, _ in sel})
    say(f"  oracle quantise of batches {bsel}, attention on heads {sel}")
    _, rqs, qd = ofp8.quantize(inp["q"][bsel], signs)
    _, rks, kd = ofp8.quantize(inp["k"][bsel], signs)
    assert np.array_equal(qs.cpu().numpy()[bsel], rqs) and np.array_equal(ks.cpu().numpy()[bsel], rks)
    for b, h in sel:
        bi = bsel.index(b)
        ro, rl = ora.forward(qd[bi:bi + 1, :, h:h + 1], kd[bi:bi + 1, :, h:h + 1], inp["v"][b:b + 1, :, h:h + 1],
                             causal, w.scale)
        check(f"O[b={b},h={h}]", o[b:b + 1, :, h:h + 1], ro, "bf16", config=True)
        check(f"L[b={b},h={h}]", lse[b:b + 1, h:h + 1], rl, "bf16", is_lse=True)


def test_fp8_error_against_unquantised_attention():
    # how far FP8 Q/K move the result from exact attention on the bf16 inputs, with and without
    # the rotation, on K with element-wise outliers (x20 on 1%, as in the long-context
    # workload), reported; the magnitudes of §4.4's experiment are pinned on the oracle
    # quantiser on the CPU
    d, n = 128, 1024
    inp = workloads.make_attention_inputs(1, n, n, 4, 4, d, seed=1601, outlier_frac=0.01, outlier_scale=20.0)
    scale = 1.0 / math.sqrt(d)
    ro, _ = ora.forward(inp["q"], inp["k"], inp["v"], True, scale)
    errs = {}
    for rotate in (False, True):
        signs = _signs(d, 10) if rotate else None
        q8, qs, _ = ofp8.quantize(inp["q"], signs)
        k8, ks, _ = ofp8.quantize(inp["k"], signs)
        o, _ = run_fwd_fp8(q8, qs, k8, ks, inp["v"], True, scale)
        e = np.abs(o - ro)
        errs[rotate] = (float(e.max()), float(np.sqrt((e ** 2).mean())))
    say(f"  FP8 vs exact: no rotation max/rms {errs[False]}, rotation {errs[True]}; "
        f"RMS ratio {errs[False][1] / errs[True][1]:.2f}")
