"""The library's calls under HIP graph capture.

No call allocates, synchronises with the host or clears memory with a memset (the counters that
the persistent kernels and the decode merge use are reset by the last workgroup to leave), so a
whole pass can be captured into one graph and replayed. One graph holds every main entry point
with caller-allocated outputs and workspaces: the bf16 and fp32 forward, the persistent and the
polynomial-exp forward, both backward paths, the dropout forward and backward, the FP8
quantise and forward, and decode. It is replayed several times with eager work in between
(other calls, fills, synchronisations) and every replay must equal the eager calls bit for bit,
the workspaces back to zero.
"""

import math

import numpy as np
import pytest

import workloads
from gpu_util import check, say, to_dev, to_np
from oracle import attention as ora

pytestmark = pytest.mark.gpu


def test_every_entry_point_in_one_replayed_graph():
    import torch

    import exact_io_aware_03_amd as fa

    B, N, Hq, Hkv, d, causal = 2, 700, 4, 2, 128, True
    scale = 1.0 / math.sqrt(d)
    inp = workloads.make_attention_inputs(B, N, N, Hq, Hkv, d, seed=5401, with_do=True)
    q, k, v, do = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    qf, kf, vf = (to_dev(inp[n], "f32") for n in ("q", "k", "v"))
    dec = workloads.make_decode_inputs(6, Hq, Hkv, 900, d, seed=5402, len_range=(1, 900))
    qd, kd, vd = (to_dev(dec[n], "bf16") for n in ("q", "k", "v"))
    lens = torch.from_numpy(dec["seqlens"]).cuda()
    signs = torch.from_numpy(np.random.Generator(np.random.PCG64(5403)).choice([-1.0, 1.0], size=d)
                             .astype(np.float32)).cuda()
    p, seed, off = 0.2, 0x5EED5EED12345, 9
    nsb = (N + 63) // 64

    def buffers():
        f32 = dict(dtype=torch.float32, device="cuda")
        bufs = {
            "o": torch.empty_like(q), "l": torch.empty((B, Hq, N), **f32),
            "of": torch.empty_like(qf), "lf": torch.empty((B, Hq, N), **f32),
            "op": torch.empty_like(q), "lp": torch.empty((B, Hq, N), **f32),
            "oy": torch.empty_like(q), "ly": torch.empty((B, Hq, N), **f32),
            "dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
            "dq1": torch.empty_like(q), "dk1": torch.empty_like(k), "dv1": torch.empty_like(v),
            "od": torch.empty_like(q), "ld": torch.empty((B, Hq, N), **f32),
            "dqd": torch.empty_like(q), "dkd": torch.empty_like(k), "dvd": torch.empty_like(v),
            "q8": torch.empty(q.shape, dtype=torch.uint8, device="cuda"), "qs": torch.empty((B, Hq, nsb), **f32),
            "k8": torch.empty(k.shape, dtype=torch.uint8, device="cuda"), "ks": torch.empty((B, Hkv, nsb), **f32),
            "o8": torch.empty_like(q), "l8": torch.empty((B, Hq, N), **f32),
            "odc": torch.empty_like(qd), "ldc": torch.empty((qd.shape[0], Hq), **f32),
        }
        ws = {
            "bwd": torch.zeros(fa.fa_bwd_workspace_size(B, Hq, N, d), dtype=torch.uint8, device="cuda"),
            "bwd1": torch.zeros(fa.fa_bwd_workspace_size(B, Hq, N, d), dtype=torch.uint8, device="cuda"),
            "bwdd": torch.zeros(fa.fa_bwd_workspace_size(B, Hq, N, d), dtype=torch.uint8, device="cuda"),
            "pers": torch.zeros(fa.fa_fwd_persistent_workspace_size(), dtype=torch.uint8, device="cuda"),
            "dec": torch.zeros(fa.fa_decode_workspace_size(qd.shape[0], Hq, kd.shape[1], d), dtype=torch.uint8,
                               device="cuda"),
        }
        return bufs, ws

    def run_all(b, w):
        fa.fa_fwd(q, k, v, b["o"], b["l"], causal, scale)
        fa.fa_fwd(qf, kf, vf, b["of"], b["lf"], causal, scale)
        fa.fa_fwd_persistent(q, k, v, b["op"], b["lp"], w["pers"], causal, scale)
        fa.fa_fwd_poly_exp2(q, k, v, b["oy"], b["ly"], causal, scale)
        fa.fa_bwd(q, k, v, b["o"], do, b["l"], b["dq"], b["dk"], b["dv"], w["bwd"], causal, scale)
        fa.fa_bwd_single_pass(q, k, v, b["o"], do, b["l"], b["dq1"], b["dk1"], b["dv1"], w["bwd1"], causal, scale)
        fa.fa_fwd_dropout(q, k, v, b["od"], b["ld"], p, seed, off, causal, scale)
        fa.fa_bwd_dropout(q, k, v, b["od"], do, b["ld"], b["dqd"], b["dkd"], b["dvd"], w["bwdd"], p, seed, off,
                          causal, scale)
        fa.fa_quantize_fp8(q, signs, b["q8"], b["qs"])
        fa.fa_quantize_fp8(k, signs, b["k8"], b["ks"])
        fa.fa_fwd_fp8(b["q8"], b["k8"], v, b["qs"], b["ks"], b["o8"], b["l8"], causal, scale)
        fa.fa_decode(qd, kd, vd, lens, b["odc"], b["ldc"], w["dec"], scale)

    ref, wref = buffers()
    run_all(ref, wref)
    torch.cuda.synchronize()
    out, wout = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_all(out, wout)  # warm-up on the stream that captures
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_all(out, wout)
    torch.cuda.synchronize()
    other = workloads.make_attention_inputs(1, 300, 300, 2, 2, 64, seed=5404)
    oq, ok_, ov = (to_dev(other[n], "bf16") for n in ("q", "k", "v"))
    for rep in range(3):
        for t in out.values():
            t.fill_(7)
        fa.forward(oq, ok_, ov, causal=True)  # eager work on the same device between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        bad = [n for n in ref if not torch.equal(out[n], ref[n])]
        say(f"  graph replay {rep}: outputs differing from the eager calls: {bad}")
        assert not bad
        nz = 256 + 4 * 64 * d * B * Hq * -(-N // 64)
        for name in ("bwd", "bwd1", "bwdd"):
            assert int(wout[name][:nz].count_nonzero()) == 0, name
        assert int(wout["pers"].count_nonzero()) == 0
        assert int(wout["dec"][:(qd.shape[0] * Hq * 4 + 255) // 256 * 256].count_nonzero()) == 0
    # the replayed results are the library's: the forward against the oracle
    ro, rl = ora.forward(inp["q"], inp["k"], inp["v"], causal, scale)
    check("O (graph replay)", to_np(out["o"]), ro, "bf16")
    check("L (graph replay)", to_np(out["l"]), rl, "bf16", is_lse=True)
