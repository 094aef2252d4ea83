"""Benchmark of the exact-attention hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]

A step is one training pass of the hot path on the training-shape workload (B=16, H=16,
N=2048, d=128, bf16): fa_fwd then fa_bwd (recomputing P from the saved L), without and with the
causal mask. `value` is the step's algorithmic TFLOP/s: 4*N_q*N_k*d per head for a forward and
10*N_q*N_k*d for a backward (five products, the recomputation of S included) over the visible
pairs (N(N+1)/2 with the causal mask). The ragged GQA decode is an inference path of its own
and is reported in `results` in HBM GB/s, as are the long-context causal forward and the
causal backward of the backward workload. Every kernel time comes from HIP events on the stream
the library launches on. The fp64 CPU oracle is timed on a bounded sample of the training-shape
forward (`cpu_baseline`). Inputs are the seeded synthetic tensors of workloads.py, resident in
device memory before any timed region. One JSON line on stdout.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "attn fwd/bwd TFLOPS & % bf16 MFMA peak (d=128); decode HBM GB/s"
PEAK_BF16_TFLOPS = 2516.6  # 256 CUs x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense fp8 MFMA
# the FP8 path runs Q K^T (half the FLOPs) on fp8 MFMA and P V on bf16 MFMA
PEAK_FP8_QK_TFLOPS = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fwd_flops(B, H, Nq, Nk, d, causal):
    if causal:
        return 4.0 * B * H * d * Nq * (Nq + 1) / 2
    return 4.0 * B * H * Nq * Nk * d


def bwd_flops(B, H, N, d, causal):
    # five matmuls (S recomputed, dV, dP, dK, dQ) over the visible pairs
    pairs = N * (N + 1) / 2 if causal else N * N
    return 10.0 * B * H * d * pairs


def decode_bytes(w, lens):
    kv = 2 * w.Hkv * w.d * 2 * int(np.sum(lens.astype(np.int64)))
    return kv + w.B * w.Hq * w.d * 2 * 2 + w.B * w.Hq * 4  # + Q read, O write, L write


def dev(x, dtype="bf16"):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def time_launches(fn, reps, warmup):
    """Per-launch durations (ms) with HIP events on the current stream (the launch stream)."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def csrc_sha256():
    import hashlib
    import glob

    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "exact_io_aware_03_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(call):
    """HBM bytes per call of `call` from the committed FETCH_SIZE/WRITE_SIZE summary, or None when
    the kernel sources changed since those counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_counters.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("csrc_sha256") != csrc_sha256() or call not in rec.get("calls", {}):
        return None
    return int(rec["calls"][call]["traffic_bytes"])


def cpu_baseline(w, budget_s=12.0):
    """The fp64 oracle, as it stands, on whole heads of the workload until ~budget_s elapse."""
    from oracle import attention as ora

    try:
        from threadpoolctl import threadpool_info

        cores = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = 1
    inp = workloads.make_attention_inputs(1, w.Nq, w.Nk, 4, 4, w.d, seed=w.seed, dtype=w.dtype)
    flops, heads, t0 = 0.0, 0, time.perf_counter()
    while True:
        h = heads % 4
        ora.forward(inp["q"], inp["k"], inp["v"], False, w.scale, heads=[(0, h)])
        heads += 1
        flops += fwd_flops(1, 1, w.Nq, w.Nk, w.d, False)
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
        "sample": f"{heads} whole heads (N_q=N_k={w.Nq}, d={w.d}, no mask) of the training-shape forward, "
                  f"fp64 numpy, {dt:.1f} s",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="only the training-shape forward step")
    ap.add_argument("--reps", type=int, default=10, help="timed launches per extra workload")
    ap.add_argument("--calib", action="store_true",
                    help="first run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (--gpus {args.gpus} refused)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_io_aware_03_amd as fa

    fa.lib()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    if args.calib:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")  # 1 GiB read, 1 GiB written
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- the step: training-shape forward + backward, without and with the causal mask ----
    w = workloads.WORKLOADS["fwd_bf16_b16h16n2048d128"]
    log(f"[bench] generating {w.name} (+ dO from the same seeded stream)")
    inp = workloads.make_attention_inputs(w.B, w.Nq, w.Nk, w.Hq, w.Hkv, w.d, w.seed, w.dtype, with_do=True)
    q, k, v, do = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["do"])
    del inp
    o = {m: torch.empty_like(q) for m in (False, True)}
    lse = {m: torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda") for m in (False, True)}
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_workspace_size(w.B, w.Hq, w.Nq, w.d), dtype=torch.uint8, device="cuda")

    def fwd(m):
        fa.fa_fwd(q, k, v, o[m], lse[m], causal=m, scale=w.scale)

    def bwd(m):
        fa.fa_bwd(q, k, v, o[m], do, lse[m], dq, dk, dv, ws, causal=m, scale=w.scale)

    def step():
        for m in (False, True):
            fwd(m)
            bwd(m)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ff = {m: fwd_flops(w.B, w.Hq, w.Nq, w.Nk, w.d, m) for m in (False, True)}
    bf = {m: bwd_flops(w.B, w.Hq, w.Nq, w.d, m) for m in (False, True)}
    step_flops = sum(ff.values()) + sum(bf.values())
    value = step_flops * args.steps / dt / 1e12
    log(f"[bench] step: {dt / args.steps * 1e3:.3f} ms, {value:.1f} TFLOP/s")

    # ---- per-call times of the step's parts, HIP events on the launch stream ----
    results = {}
    part_ms = {}
    for m in (False, True):
        tag = "causal" if m else "nc"
        f_ms = float(np.mean(time_launches(lambda: fwd(m), args.reps * 2, 3)))
        b_ms = float(np.mean(time_launches(lambda: bwd(m), args.reps, 2)))
        part_ms[("fwd", m)], part_ms[("bwd", m)] = f_ms, b_ms
        for kind, ms, fl in (("fwd", f_ms, ff[m]), ("bwd", b_ms, bf[m])):
            tf = fl / (ms * 1e-3) / 1e12
            results[f"{kind}_{tag}_b16h16n2048d128"] = {"ms": round(ms, 4), "tflops": round(tf, 2),
                                                        "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    # the dominant part of the step: the call with the largest share of the step's time
    dom = max(part_ms, key=part_ms.get)
    dom_ms = part_ms[dom]
    dom_flops = (ff if dom[0] == "fwd" else bf)[dom[1]]
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    dom_call = "%s %s" % ("fa_fwd" if dom[0] == "fwd" else "fa_bwd", "causal" if dom[1] else "non-causal")
    dom_name = {"fwd": "fwd_bf16_kernel<128,%s>" % ("true" if dom[1] else "false"),
                "bwd": "fa_bwd %s (bwd_dq_kernel<128> + bwd_main_kernel<128>)" % ("causal" if dom[1] else "non-causal")}[dom[0]]
    del q, k, v, do, o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()

    if not args.no_extra:
        # long-context causal forward
        w3 = workloads.WORKLOADS["fwd_bf16_causal_h32n16384d128"]
        log(f"[bench] {w3.name}")
        inp = workloads.make_workload_inputs(w3)
        q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
        del inp
        o = torch.empty_like(q)
        lse = torch.empty((w3.B, w3.Hq, w3.Nq), dtype=torch.float32, device="cuda")
        ms = float(np.mean(time_launches(lambda: fa.fa_fwd(q, k, v, o, lse, causal=True, scale=w3.scale),
                                         args.reps, 2)))
        tf = fwd_flops(w3.B, w3.Hq, w3.Nq, w3.Nk, w3.d, True) / (ms * 1e-3) / 1e12
        results["fwd_causal_h32n16384d128"] = {"ms": round(ms, 4), "tflops": round(tf, 2),
                                               "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        del q, k, v, o, lse
        torch.cuda.empty_cache()

        # decode (HBM bound)
        w4 = workloads.WORKLOADS["decode_bf16_b64hq32hkv8d128"]
        log(f"[bench] {w4.name}")
        inp = workloads.make_workload_inputs(w4)
        q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
        lens = torch.from_numpy(inp["seqlens"]).cuda()
        nbytes = decode_bytes(w4, inp["seqlens"])
        del inp
        # three copies of the cache (3 x 2 GiB), used in turn, so no timed call finds the
        # previous call's rows in the 256 MB last-level cache
        caches = [(k, v)] + [(k.clone(), v.clone()) for _ in range(2)]
        o = torch.empty_like(q)
        lse = torch.empty((w4.B, w4.Hq), dtype=torch.float32, device="cuda")
        ws = torch.empty(fa.fa_decode_workspace_size(w4.B, w4.Hq, w4.Nk, w4.d), dtype=torch.uint8, device="cuda")
        turn = [0]

        def decode_call():
            kc, vc = caches[turn[0] % 3]
            turn[0] += 1
            fa.fa_decode(q, kc, vc, lens, o, lse, ws, scale=w4.scale)

        ms = float(np.mean(time_launches(decode_call, args.reps * 2, 3)))
        gbs = nbytes / (ms * 1e-3) / 1e9
        results["decode_b64hq32hkv8d128"] = {"ms": round(ms, 4), "gbs": round(gbs, 1),
                                             "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "bytes": nbytes}
        del q, k, v, o, lse, ws, lens, caches
        torch.cuda.empty_cache()

        # causal backward (dQ kernel + dK/dV kernel), forward untimed
        w5 = workloads.WORKLOADS["bwd_bf16_causal_b8h16n4096d128"]
        log(f"[bench] {w5.name}")
        inp = workloads.make_workload_inputs(w5)
        q, k, v, do = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["do"])
        del inp
        o, lse = fa.forward(q, k, v, causal=True, scale=w5.scale)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(fa.fa_bwd_workspace_size(w5.B, w5.Hq, w5.Nq, w5.d), dtype=torch.uint8, device="cuda")
        ms = float(np.mean(time_launches(
            lambda: fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, causal=True, scale=w5.scale), args.reps, 2)))
        tf = bwd_flops(w5.B, w5.Hq, w5.Nq, w5.d, True) / (ms * 1e-3) / 1e12
        results["bwd_causal_b8h16n4096d128"] = {"ms": round(ms, 4), "tflops": round(tf, 2),
                                                "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                                                "tflops_8n2d_convention": round(0.8 * tf, 2)}
        del q, k, v, do, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()

        # FP8 forward on the training shape: Q and K quantised to E4M3 beforehand (as the kernel
        # producing them would hand them over), so the timed call is the attention alone; the
        # quantise pass is timed on its own (HBM bound: 2 bytes read, 1 written per value)
        log("[bench] fwd_fp8_b16h16n2048d128")
        inp = workloads.make_attention_inputs(w.B, w.Nq, w.Nk, w.Hq, w.Hkv, w.d, w.seed, w.dtype)
        q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
        del inp
        signs = np.random.Generator(np.random.PCG64(9)).choice([-1.0, 1.0], size=w.d).astype(np.float32)
        signs = torch.from_numpy(signs).cuda()
        q8, qs = fa.quantize_fp8(q, signs)
        k8, ks = fa.quantize_fp8(k, signs)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda")
        for m in (False, True):
            ms = float(np.mean(time_launches(
                lambda: fa.fa_fwd_fp8(q8, k8, v, qs, ks, o, lse, causal=m, scale=w.scale), args.reps * 2, 3)))
            tf = ff[m] / (ms * 1e-3) / 1e12
            results["fwd_fp8_%s_b16h16n2048d128" % ("causal" if m else "nc")] = {
                "ms": round(ms, 4), "tflops": round(tf, 2), "peak": round(PEAK_FP8_QK_TFLOPS, 1),
                "frac_peak": round(tf / PEAK_FP8_QK_TFLOPS, 4)}
        ms = float(np.mean(time_launches(lambda: fa.fa_quantize_fp8(q, signs, q8, qs), args.reps, 2)))
        qbytes = q.numel() * 3 + qs.numel() * 4
        results["quantize_fp8_b16h16n2048d128"] = {"ms": round(ms, 4), "gbs": round(qbytes / (ms * 1e-3) / 1e9, 1),
                                                   "frac_hbm": round(qbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        del q, k, v, q8, k8, qs, ks, o, lse, signs
        torch.cuda.empty_cache()

        # dropout on P (p = 0.1) on the training shape without the mask: forward and backward
        # regenerate the keep mask from (seed, offset); FLOPs counted as without dropout
        log("[bench] dropout_b16h16n2048d128")
        inp = workloads.make_attention_inputs(w.B, w.Nq, w.Nk, w.Hq, w.Hkv, w.d, w.seed, w.dtype, with_do=True)
        q, k, v, do = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["do"])
        del inp
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda")
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(fa.fa_bwd_workspace_size(w.B, w.Hq, w.Nq, w.d), dtype=torch.uint8, device="cuda")
        pd, seed = 0.1, 0x5EED
        f_ms = float(np.mean(time_launches(
            lambda: fa.fa_fwd_dropout(q, k, v, o, lse, pd, seed, 0, scale=w.scale), args.reps * 2, 3)))
        b_ms = float(np.mean(time_launches(
            lambda: fa.fa_bwd_dropout(q, k, v, o, do, lse, dq, dk, dv, ws, pd, seed, 0, scale=w.scale), args.reps, 2)))
        for kind, ms, fl in (("fwd", f_ms, ff[False]), ("bwd", b_ms, bf[False])):
            tf = fl / (ms * 1e-3) / 1e12
            results[f"{kind}_dropout0.1_nc_b16h16n2048d128"] = {"ms": round(ms, 4), "tflops": round(tf, 2),
                                                               "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        del q, k, v, do, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.Hq, "N": w.Nq, "d": w.d,
                   "masks": ["none", "causal"], "step": "fa_fwd + fa_bwd, without and with the causal mask"},
        "roofline": {"kernel": dom_name, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(dom_call)},
        "results": results,
    }
    if not args.no_cpu:
        log("[bench] cpu baseline (fp64 oracle)")
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
