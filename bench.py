"""Benchmark of the exact-attention hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]

A step is one training pass of the hot path on the training-shape workload (B=16, H=16,
N=2048, d=128, bf16): fa_fwd then fa_bwd (recomputing P from the saved L), without and with the
causal mask. `value` is the step's algorithmic TFLOP/s: 4*N_q*N_k*d per head for a forward and
10*N_q*N_k*d for a backward (five products, the recomputation of S included) over the visible
pairs (N(N+1)/2 with the causal mask). The ragged GQA decode is an inference path of its own
and is reported in `results` in HBM GB/s, as are the long-context causal forward and the
causal backward of the backward workload, and the single-head fp32 forward (against the fp32
matrix peak). Every kernel time comes from HIP events on the stream the library launches on:
per part, 10 untimed launches then 50 timed ones, reported as median, minimum and mean (the
roofline uses the mean launch duration). The fp64 CPU oracle is timed on a bounded sample of the
training-shape forward (`cpu_baseline`), and on a bounded sample of each of the five workloads
beside the GPU figures (`cpu_baseline.per_workload`). Inputs are the seeded synthetic tensors of
workloads.py, resident in device memory before any timed region. After the timed parts the
step runs back to back for about 3 s while `amd-smi metric` samples the XCD clocks and the
socket power (`gpu_state`; null where the tool is missing or fails). One JSON line on stdout.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import shutil
import subprocess
import sys
import threading
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
PEAK_F32_TFLOPS = 157.3  # MI355X fp32 matrix (and vector) peak


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


def time_launches(fn, reps=50, warmup=10):
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


def stats(ms_list):
    """median / min / mean of per-launch durations (ms)."""
    a = np.asarray(ms_list, dtype=np.float64)
    return {"ms": round(float(np.median(a)), 4), "ms_min": round(float(a.min()), 4),
            "ms_mean": round(float(a.mean()), 4), "launches": int(a.size)}


def rate_entry(ms_list, work, kind):
    """Result entry for one part: times, and the rate at the median (TFLOP/s or GB/s)."""
    st = stats(ms_list)
    if kind == "hbm":
        gbs = work / (st["ms"] * 1e-3) / 1e9
        st.update(gbs=round(gbs, 1), frac_hbm=round(gbs / PEAK_HBM_GBS, 4))
    else:
        peak = {"bf16": PEAK_BF16_TFLOPS, "f32": PEAK_F32_TFLOPS, "fp8qk": PEAK_FP8_QK_TFLOPS}[kind]
        tf = work / (st["ms"] * 1e-3) / 1e12
        st.update(tflops=round(tf, 2), frac_peak=round(tf / peak, 4))
        if kind != "bf16":
            st["peak"] = round(peak, 1)
    return st


def _smi_sample():
    """One `amd-smi metric` reading of GPU 0: the gfx clock of each XCD (MHz) and the socket
    power (W); None if the tool is missing or its output is not what is expected."""
    exe = shutil.which("amd-smi")
    if exe is None:
        return None
    try:
        r = subprocess.run([exe, "metric", "-g", "0", "-c", "-p", "--json"], capture_output=True, text=True,
                           timeout=30)
    except (OSError, subprocess.TimeoutExpired):
        return None
    i = r.stdout.find("{")
    if r.returncode != 0 or i < 0:
        return None
    try:
        g = json.loads(r.stdout[i:])["gpu_data"][0]
        clk = [float(v["clk"]["value"]) for name, v in g["clock"].items()
               if name.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
        pw = g["power"]["socket_power"]
        power = float(pw["value"]) if isinstance(pw, dict) else None
    except (ValueError, KeyError, IndexError, TypeError):
        return None
    return {"gfx_mhz": clk, "power_w": power} if clk else None


def gpu_state(step, seconds=3.0):
    """Clock and power while the step runs back to back: a thread takes amd-smi readings (child
    processes) until the load ends; only readings that finished under load count."""
    import torch

    samples, stop = [], threading.Event()

    def sampler():
        time.sleep(0.5)  # the clocks settle under the load first
        while not stop.is_set():
            s = _smi_sample()
            if s is None:
                return
            if not stop.is_set():
                samples.append(s)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(4):
            step()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=40)
    if not samples:
        return None
    clk = [c for s in samples for c in s["gfx_mhz"]]
    pw = [s["power_w"] for s in samples if s["power_w"] is not None]
    return {"source": "amd-smi metric -c -p", "load": "the bench step back to back for %.0f s" % seconds,
            "samples": len(samples), "gfx_mhz_median": float(np.median(clk)), "gfx_mhz_min": min(clk),
            "gfx_mhz_max": max(clk), "socket_power_w_median": float(np.median(pw)) if pw else None}


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


def _host_threads():
    """Threads the oracle's BLAS pool runs with, set to the cores this process may use."""
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info, threadpool_limits

        threadpool_limits(limits=cores)
        used = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        used = cores
    return cores, int(used)


def cpu_baseline(w, budget_s=12.0):
    """The fp64 oracle, as it stands, on whole heads of the training-shape forward until about
    budget_s elapse (the headline baseline), then on a bounded sample of each of the five
    workloads (rates in the workload's own unit, beside the GPU figures)."""
    from oracle import attention as ora

    cores, threads = _host_threads()
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
    del inp
    return {
        "value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "host_cores": cores,
        "sample": f"{heads} whole heads (N_q=N_k={w.Nq}, d={w.d}, no mask) of the training-shape forward, "
                  f"fp64 numpy, {dt:.1f} s, BLAS pool of {threads} threads",
    }


def oracle_per_workload():
    """Oracle rate on a bounded sample of each workload: (sample text, seconds, rate, unit,
    estimated seconds for the whole workload). Samples: the fp32 forward whole; one head of the
    training-shape forward with and without the mask; 512 rows of one head of the long-context
    forward; 8 of the 64 decode sequences; the backward of one head of the backward workload."""
    from oracle import attention as ora

    out = {}
    warm = workloads.make_attention_inputs(1, 256, 256, 1, 1, 128, seed=0)
    ora.forward(warm["q"], warm["k"], warm["v"], False, 0.1)  # BLAS pool start-up, untimed

    def put(name, sample, dt, work, full_work, unit):
        scale = 1e12 if unit == "TFLOP/s" else 1e9
        out[name] = {"sample": sample, "s": round(dt, 3), "rate": round(work / dt / scale, 6), "unit": unit,
                     "est_full_s": round(dt * full_work / work, 1)}

    w1 = workloads.WORKLOADS["fwd_f32_256x64"]
    inp = workloads.make_workload_inputs(w1)
    t0 = time.perf_counter()
    ora.forward(inp["q"], inp["k"], inp["v"], False, w1.scale)
    fl = fwd_flops(1, 1, w1.Nq, w1.Nk, w1.d, False)
    put("fwd_f32_256x64", "whole", time.perf_counter() - t0, fl, fl, "TFLOP/s")

    w2 = workloads.WORKLOADS["fwd_bf16_b16h16n2048d128"]
    inp = workloads.make_attention_inputs(1, w2.Nq, w2.Nk, 1, 1, w2.d, seed=w2.seed)
    for m in (False, True):
        t0 = time.perf_counter()
        ora.forward(inp["q"], inp["k"], inp["v"], m, w2.scale)
        fl = fwd_flops(1, 1, w2.Nq, w2.Nk, w2.d, m)
        put("fwd_%s_b16h16n2048d128" % ("causal" if m else "nc"), "one head", time.perf_counter() - t0, fl,
            fl * w2.B * w2.Hq, "TFLOP/s")

    w3 = workloads.WORKLOADS["fwd_bf16_causal_h32n16384d128"]
    inp = workloads.make_attention_inputs(1, w3.Nq, w3.Nk, 1, 1, w3.d, seed=w3.seed,
                                          outlier_frac=w3.outlier_frac, outlier_scale=w3.outlier_scale)
    rows = np.arange(w3.Nq - 512, w3.Nq)  # the 512 longest rows
    t0 = time.perf_counter()
    ora.forward(inp["q"], inp["k"], inp["v"], True, w3.scale, rows=rows)
    fl = 4.0 * w3.d * float(np.sum(rows + 1))
    put("fwd_causal_h32n16384d128", "the last 512 rows of one head", time.perf_counter() - t0, fl,
        fwd_flops(1, w3.Hq, w3.Nq, w3.Nk, w3.d, True), "TFLOP/s")

    w4 = workloads.WORKLOADS["decode_bf16_b64hq32hkv8d128"]
    lens = np.random.Generator(np.random.PCG64([w4.seed, 1])).integers(
        w4.len_range[0], w4.len_range[1], endpoint=True, size=w4.B).astype(np.int32)
    sub = lens[:8]
    inp = workloads.make_decode_inputs(8, w4.Hq, w4.Hkv, int(sub.max()), w4.d, seed=w4.seed, lengths=sub)
    t0 = time.perf_counter()
    ora.decode(inp["q"], inp["k"], inp["v"], inp["seqlens"], w4.scale)
    by = 2 * w4.Hkv * w4.d * 2 * float(np.sum(sub)) + 8 * w4.Hq * (w4.d * 4 + 4)
    put("decode_b64hq32hkv8d128", "8 of the 64 sequences", time.perf_counter() - t0, by, decode_bytes(w4, lens),
        "GB/s")

    w5 = workloads.WORKLOADS["bwd_bf16_causal_b8h16n4096d128"]
    inp = workloads.make_attention_inputs(1, w5.Nq, w5.Nk, 1, 1, w5.d, seed=w5.seed, with_do=True)
    t0 = time.perf_counter()
    ora.backward(inp["q"], inp["k"], inp["v"], inp["do"], True, w5.scale)
    fl = bwd_flops(1, 1, w5.Nq, w5.d, True)
    put("bwd_causal_b8h16n4096d128", "one head", time.perf_counter() - t0, fl, fl * w5.B * w5.Hq, "TFLOP/s")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="only the training-shape forward step")
    ap.add_argument("--reps", type=int, default=50, help="timed launches per part (after 10 untimed)")
    ap.add_argument("--no-smi", action="store_true", help="skip the amd-smi clock and power sampling")
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
    reps = args.reps

    # ---- the step: training-shape forward + backward, without and with the causal mask ----
    w = workloads.WORKLOADS["fwd_bf16_b16h16n2048d128"]
    log(f"[bench] generating {w.name} (+ dO from the same seeded stream)")
    inp = workloads.make_attention_inputs(w.B, w.Nq, w.Nk, w.Hq, w.Hkv, w.d, w.seed, w.dtype, with_do=True)
    q, k, v, do = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["do"])
    del inp
    o = {m: torch.empty_like(q) for m in (False, True)}
    lse = {m: torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda") for m in (False, True)}
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.zeros(fa.fa_bwd_workspace_size(w.B, w.Hq, w.Nq, w.d), dtype=torch.uint8, device="cuda")

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
    part = {}
    for m in (False, True):
        tag = "causal" if m else "nc"
        for kind, fn, fl in (("fwd", fwd, ff[m]), ("bwd", bwd, bf[m])):
            t = time_launches(lambda: fn(m), reps)
            part[(kind, m)] = float(np.mean(t))
            results[f"{kind}_{tag}_b16h16n2048d128"] = rate_entry(t, fl, "bf16")
    # the dominant part of the step: the call with the largest share of the step's time; its
    # roofline figure uses the mean launch duration
    dom = max(part, key=part.get)
    dom_ms = part[dom]
    dom_flops = (ff if dom[0] == "fwd" else bf)[dom[1]]
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    dom_call = "%s %s" % ("fa_fwd" if dom[0] == "fwd" else "fa_bwd", "causal" if dom[1] else "non-causal")
    dom_name = {"fwd": "fwd_bf16_kernel<128,%s>" % ("true" if dom[1] else "false"),
                "bwd": "fa_bwd %s (%s)" % ("causal" if dom[1] else "non-causal", BWD_KERNELS)}[dom[0]]
    state = None if args.no_smi else gpu_state(step)
    del q, k, v, do, o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()

    if not args.no_extra:
        extra_parts(fa, w, ff, bf, results, reps)

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
        "gpu_state": state,
        "build": fa.build_info(),
    }
    if not args.no_cpu:
        log("[bench] cpu baseline (fp64 oracle)")
        line["cpu_baseline"] = cpu_baseline(w)
        if not args.no_extra:
            log("[bench] oracle per workload (bounded samples)")
            per = oracle_per_workload()
            for name, rec in per.items():
                gpu = results.get(name)
                if gpu is not None:
                    rec["gpu_ms"] = gpu["ms"]
                    rec["gpu_speedup_est"] = round(rec["est_full_s"] * 1e3 / gpu["ms"], 1)
            line["cpu_baseline"]["per_workload"] = per
    print(json.dumps(line), flush=True)


BWD_KERNELS = "bwd_dq_kernel<128> + bwd_main_kernel<128>"


def extra_parts(fa, w, ff, bf, results, reps):
    """The other workloads (long-context forward, decode, backward workload, fp32 forward) and
    the next-row paths (FP8 forward, dropout), each timed per launch."""
    import torch

    # single-head fp32 forward (latency-bound; reported against the fp32 peak)
    w1 = workloads.WORKLOADS["fwd_f32_256x64"]
    log(f"[bench] {w1.name}")
    inp = workloads.make_workload_inputs(w1)
    q, k, v = dev(inp["q"], "f32"), dev(inp["k"], "f32"), dev(inp["v"], "f32")
    o = torch.empty_like(q)
    lse = torch.empty((1, 1, w1.Nq), dtype=torch.float32, device="cuda")
    t = time_launches(lambda: fa.fa_fwd(q, k, v, o, lse, causal=False, scale=w1.scale), reps)
    results["fwd_f32_256x64"] = rate_entry(t, fwd_flops(1, 1, w1.Nq, w1.Nk, w1.d, False), "f32")
    del q, k, v, o, lse

    # long-context causal forward
    w3 = workloads.WORKLOADS["fwd_bf16_causal_h32n16384d128"]
    log(f"[bench] {w3.name}")
    inp = workloads.make_workload_inputs(w3)
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    del inp
    o = torch.empty_like(q)
    lse = torch.empty((w3.B, w3.Hq, w3.Nq), dtype=torch.float32, device="cuda")
    t = time_launches(lambda: fa.fa_fwd(q, k, v, o, lse, causal=True, scale=w3.scale), reps)
    results["fwd_causal_h32n16384d128"] = rate_entry(t, fwd_flops(w3.B, w3.Hq, w3.Nq, w3.Nk, w3.d, True), "bf16")
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
    # three copies of the cache (3 x 2 GiB), used in turn, so no timed call finds the previous
    # call's rows in the 256 MB last-level cache
    caches = [(k, v)] + [(k.clone(), v.clone()) for _ in range(2)]
    o = torch.empty_like(q)
    lse = torch.empty((w4.B, w4.Hq), dtype=torch.float32, device="cuda")
    ws = torch.zeros(fa.fa_decode_workspace_size(w4.B, w4.Hq, w4.Nk, w4.d), dtype=torch.uint8, device="cuda")
    turn = [0]

    def decode_call():
        kc, vc = caches[turn[0] % 3]
        turn[0] += 1
        fa.fa_decode(q, kc, vc, lens, o, lse, ws, scale=w4.scale)

    results["decode_b64hq32hkv8d128"] = dict(rate_entry(time_launches(decode_call, reps), nbytes, "hbm"),
                                             bytes=nbytes)
    del q, k, v, o, lse, ws, lens, caches
    torch.cuda.empty_cache()

    # causal backward of the backward workload, forward untimed
    w5 = workloads.WORKLOADS["bwd_bf16_causal_b8h16n4096d128"]
    log(f"[bench] {w5.name}")
    inp = workloads.make_workload_inputs(w5)
    q, k, v, do = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["do"])
    del inp
    o, lse = fa.forward(q, k, v, causal=True, scale=w5.scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.zeros(fa.fa_bwd_workspace_size(w5.B, w5.Hq, w5.Nq, w5.d), dtype=torch.uint8, device="cuda")
    t = time_launches(lambda: fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, causal=True, scale=w5.scale), reps)
    e = rate_entry(t, bwd_flops(w5.B, w5.Hq, w5.Nq, w5.d, True), "bf16")
    e["tflops_8n2d_convention"] = round(0.8 * e["tflops"], 2)
    results["bwd_causal_b8h16n4096d128"] = e
    # the single-pass backward (dQ summed across key blocks in the workspace) on the same call
    t = time_launches(lambda: fa.fa_bwd_single_pass(q, k, v, o, do, lse, dq, dk, dv, ws, causal=True,
                                                    scale=w5.scale), reps)
    results["bwd_single_pass_causal_b8h16n4096d128"] = rate_entry(t, bwd_flops(w5.B, w5.Hq, w5.Nq, w5.d, True), "bf16")
    del q, k, v, do, o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()

    # the single-pass backward on the training shape, both masks
    log("[bench] bwd_single_pass_b16h16n2048d128")
    inp = workloads.make_attention_inputs(w.B, w.Nq, w.Nk, w.Hq, w.Hkv, w.d, w.seed, w.dtype, with_do=True)
    q, k, v, do = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["do"])
    del inp
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.zeros(fa.fa_bwd_workspace_size(w.B, w.Hq, w.Nq, w.d), dtype=torch.uint8, device="cuda")
    for m in (False, True):
        o, lse = fa.forward(q, k, v, causal=m, scale=w.scale)
        t = time_launches(lambda: fa.fa_bwd_single_pass(q, k, v, o, do, lse, dq, dk, dv, ws, causal=m,
                                                        scale=w.scale), reps)
        results[f"bwd_single_pass_{'causal' if m else 'nc'}_b16h16n2048d128"] = rate_entry(t, bf[m], "bf16")
    del q, k, v, do, o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()

    # the forward with a quarter of the exponentials from the FMA-unit polynomial (training shape)
    log("[bench] fwd_poly_exp2_b16h16n2048d128")
    inp = workloads.make_attention_inputs(w.B, w.Nq, w.Nk, w.Hq, w.Hkv, w.d, w.seed, w.dtype)
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    del inp
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda")
    for m in (False, True):
        t = time_launches(lambda: fa.fa_fwd_poly_exp2(q, k, v, o, lse, causal=m, scale=w.scale), reps)
        results[f"fwd_poly_exp2_{'causal' if m else 'nc'}_b16h16n2048d128"] = rate_entry(t, ff[m], "bf16")
    # the persistent forward (per-XCD task queues) on the same inputs
    log("[bench] fwd_persistent_b16h16n2048d128")
    pws = torch.zeros(fa.fa_fwd_persistent_workspace_size(), dtype=torch.uint8, device="cuda")
    for m in (False, True):
        t = time_launches(lambda: fa.fa_fwd_persistent(q, k, v, o, lse, pws, causal=m, scale=w.scale), reps)
        results[f"fwd_persistent_{'causal' if m else 'nc'}_b16h16n2048d128"] = rate_entry(t, ff[m], "bf16")
    del q, k, v, o, lse, pws
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
        t = time_launches(lambda: fa.fa_fwd_fp8(q8, k8, v, qs, ks, o, lse, causal=m, scale=w.scale), reps)
        results["fwd_fp8_%s_b16h16n2048d128" % ("causal" if m else "nc")] = rate_entry(t, ff[m], "fp8qk")
    t = time_launches(lambda: fa.fa_quantize_fp8(q, signs, q8, qs), reps)
    results["quantize_fp8_b16h16n2048d128"] = rate_entry(t, q.numel() * 3 + qs.numel() * 4, "hbm")
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
    ws = torch.zeros(fa.fa_bwd_workspace_size(w.B, w.Hq, w.Nq, w.d), dtype=torch.uint8, device="cuda")
    pd, seed = 0.1, 0x5EED
    t = time_launches(lambda: fa.fa_fwd_dropout(q, k, v, o, lse, pd, seed, 0, scale=w.scale), reps)
    results["fwd_dropout0.1_nc_b16h16n2048d128"] = rate_entry(t, ff[False], "bf16")
    t = time_launches(lambda: fa.fa_bwd_dropout(q, k, v, o, do, lse, dq, dk, dv, ws, pd, seed, 0, scale=w.scale), reps)
    results["bwd_dropout0.1_nc_b16h16n2048d128"] = rate_entry(t, bf[False], "bf16")
    del q, k, v, do, o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
