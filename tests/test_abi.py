"""The C-ABI library loads, exports every function include/fa.h declares, and validates its
arguments on the host (no GPU needed: every call here fails validation before any HIP call).
The planner helpers are pinned to the numbers printed in the lecture notes."""

import ctypes
import json
import os
import re

import pytest

import exact_io_aware_03_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLD = json.load(open(os.path.join(ROOT, "tests", "golden", "lecture21_pins.json")))["pins"]

INVALID, UNSUPPORTED, WORKSPACE = -1, -2, -4
P = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: validation rejects the call first
MIS = ctypes.c_void_p(0x10008)  # misaligned


def declared_functions():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    L = fa.lib()
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(fa.EXPORTED)
    assert L.fa_version() == 1


def fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=1, Nq=8, Nk=8, d=64, causal=0, scale=0.125, dtype=1)
    a.update(kw)
    return fa.lib().fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"],
                           a["d"], a["causal"], a["scale"], a["dtype"], None)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(q=None), INVALID), (dict(lse=None), INVALID), (dict(o=MIS), INVALID),
        (dict(B=0), INVALID), (dict(Nk=0), INVALID), (dict(Hq=3, Hkv=2), INVALID),
        (dict(scale=0.0), INVALID), (dict(scale=-1.0), INVALID), (dict(scale=float("nan")), INVALID),
        (dict(scale=float("inf")), INVALID),
        (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED), (dict(dtype=7), UNSUPPORTED),
        (dict(causal=1, Nq=8, Nk=9), UNSUPPORTED),
        # one batch of Q/O or K/V must stay below 2 GiB (32-bit buffer offsets)
        (dict(Nq=1 << 20, Hq=8, Hkv=8, d=128), UNSUPPORTED), (dict(Nk=1 << 23, Hq=1, Hkv=1, d=128), UNSUPPORTED),
    ],
)
def test_fwd_validation(kw, code):
    assert fwd(**kw) == code


def fwd_persistent(ws=P, ws_bytes=256, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=1, Nq=8, Nk=8, d=64, causal=0, scale=0.125, dtype=1)
    a.update(kw)
    return fa.lib().fa_fwd_persistent(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Nq"],
                                      a["Nk"], a["d"], a["causal"], a["scale"], a["dtype"], ws, ws_bytes, None)


def test_fwd_persistent_validation():
    # 16 int counters (8 queues, the leaver count, padding), one 256-byte block
    assert fa.fa_fwd_persistent_workspace_size() == 256
    # bf16 only and the workspace, then the forward's own checks, all before any HIP call
    assert fwd_persistent(q=None) == INVALID
    assert fwd_persistent(d=96) == UNSUPPORTED
    assert fwd_persistent(causal=1, Nk=9) == UNSUPPORTED
    assert fwd_persistent(dtype=0) == UNSUPPORTED
    assert fwd_persistent(ws=None) == WORKSPACE
    assert fwd_persistent(ws_bytes=255) == WORKSPACE
    assert fwd_persistent(ws=MIS) == WORKSPACE


def bwd(ws=P, ws_bytes=None, **kw):
    a = dict(B=1, Hq=2, Hkv=1, Nq=8, Nk=8, d=64, causal=0, scale=0.125, dtype=1)
    a.update(kw)
    need = fa.fa_bwd_workspace_size(a["B"], a["Hq"], a["Nq"], a["d"])
    ws_bytes = need if ws_bytes is None else ws_bytes
    ptrs = [kw.pop(n, P) for n in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv")]
    return fa.lib().fa_bwd(*ptrs, a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["causal"], a["scale"],
                           a["dtype"], ws, ws_bytes, None)


def bwd_single(ws=P, ws_bytes=None, **kw):
    a = dict(B=1, Hq=2, Hkv=1, Nq=8, Nk=8, d=128, causal=0, scale=0.125, dtype=1)
    a.update(kw)
    need = fa.fa_bwd_workspace_size(a["B"], a["Hq"], a["Nq"], a["d"])
    ws_bytes = need if ws_bytes is None else ws_bytes
    return fa.lib().fa_bwd_single_pass(P, P, P, P, P, P, P, P, P, a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"],
                                       a["causal"], a["scale"], a["dtype"], ws, ws_bytes, None)


def test_bwd_single_pass_validation():
    # shapes the single pass does not take are refused before any device work
    assert bwd_single(d=64) == UNSUPPORTED
    assert bwd_single(dtype=0) == UNSUPPORTED
    assert bwd_single(Nk=32641) == UNSUPPORTED              # 256 key blocks without the mask
    assert bwd_single(Nq=32641, Nk=32641, causal=1, Hq=1) == UNSUPPORTED  # 256 key blocks with it
    assert bwd_single(ws=None) == WORKSPACE
    assert bwd_single(ws_bytes=fa.fa_bwd_workspace_size(1, 2, 8, 128) - 1) == WORKSPACE
    assert bwd_single(Hq=3, Hkv=2) == INVALID
    # the workspace: 256 bytes of pool counters, the fp32 partial sums (64 rows x d per query head
    # and 64-row block), then D padded to 256 bytes
    pad = lambda n: -(-n // 256) * 256
    for (B, Hq, Nq, d) in ((1, 2, 8, 128), (16, 16, 2048, 128), (2, 3, 100, 64)):
        assert fa.fa_bwd_workspace_size(B, Hq, Nq, d) == 256 + 4 * 64 * d * B * Hq * -(-Nq // 64) + pad(4 * B * Hq * Nq)


def test_bwd_validation():
    need = fa.fa_bwd_workspace_size(1, 2, 8, 64)
    assert need >= 2 * 8 * 4  # D = rowsum(dO * O), fp32 per (head, row)
    assert bwd(dtype=0) == UNSUPPORTED  # fp32 backward is not provided
    assert bwd(ws=None) == WORKSPACE
    assert bwd(ws_bytes=need - 1) == WORKSPACE
    assert bwd(Hq=2, Hkv=3) == INVALID
    assert bwd(causal=1, Nk=9) == UNSUPPORTED
    assert bwd(d=32) == UNSUPPORTED
    assert bwd(Nq=1 << 20, Nk=8, Hq=8, Hkv=8, d=128) == UNSUPPORTED  # 2 GiB per batch of Q
    assert bwd(Nk=1 << 23, Hq=1, Hkv=1, d=128) == UNSUPPORTED  # 2 GiB per batch of K
    assert fa.lib().fa_bwd(None, P, P, P, P, P, P, P, P, 1, 2, 1, 8, 8, 64, 0, 0.1, 1, P, need, None) == INVALID


def dec(ws=P, ws_bytes=None, **kw):
    a = dict(B=2, Hq=8, Hkv=2, Nq=1, Nk=300, d=128, scale=0.1, dtype=1)
    a.update(kw)
    need = fa.fa_decode_workspace_size(a["B"], a["Hq"], a["Nk"], a["d"])
    ws_bytes = need if ws_bytes is None else ws_bytes
    return fa.lib().fa_decode(P, P, P, kw.get("seqlens", P), P, P, a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"],
                              a["d"], a["scale"], a["dtype"], ws, ws_bytes, None)


def test_decode_validation():
    assert dec(Nq=2) == INVALID
    assert dec(seqlens=None) == INVALID
    assert dec(seqlens=ctypes.c_void_p(0x10002)) == INVALID  # int32 lengths not 4-byte aligned
    assert dec(dtype=0) == UNSUPPORTED
    assert dec(Hq=64, Hkv=2) == UNSUPPORTED  # more than 16 query heads per kv head
    assert dec(ws=None) == WORKSPACE
    assert dec(ws_bytes=16) == WORKSPACE
    # partials for ceil(300/256) = 2 splits of 2*8 query heads, d + 2 floats each
    assert fa.fa_decode_workspace_size(2, 8, 300, 128) >= 2 * 8 * 2 * (128 + 2) * 4


def dec_noalloc(**kw):
    a = dict(B=2, Hq=8, Hkv=2, Nq=1, Nk=300, d=128, scale=0.1, dtype=1)
    a.update(kw)
    return fa.lib().fa_decode_noalloc(P, P, P, kw.get("seqlens", P), P, P, a["B"], a["Hq"], a["Hkv"], a["Nq"],
                                      a["Nk"], a["d"], a["scale"], a["dtype"], None)


def test_decode_noalloc_validation_and_scratch_limit():
    # the same argument checks as fa_decode, then the static scratch limit, all before any HIP call:
    # the counters take a fixed 512 KiB at the start of the 32 MiB array, and the partials,
    # (256 + B) * Hq * (d + 2) * 4 bytes, must fit in the rest
    assert dec_noalloc(Nq=2) == INVALID
    assert dec_noalloc(seqlens=None) == INVALID
    assert dec_noalloc(dtype=0) == UNSUPPORTED
    assert dec_noalloc(Hq=64, Hkv=2) == UNSUPPORTED
    SCRATCH = -5
    assert dec_noalloc(B=2000, Hq=32, Hkv=8) == SCRATCH  # (2256 * 32 * 130 * 4) B > 32 MiB
    assert dec_noalloc(B=64, Hq=256, Hkv=16) == SCRATCH  # (320 * 256 * 130 * 4) B > 32 MiB
    # partials of B = 1740, Hq = 32, d = 128 take 31.67 MiB: they would fit beside counters sized
    # for this shape (0.21 MiB), but not beside the fixed 512 KiB counter region
    part = lambda B: -(-(256 + B) * 32 * 128 * 4 // 256) * 256 + -(-(256 + B) * 32 * 8 // 256) * 256
    assert part(1740) + 4 * 1740 * 32 <= 32 << 20 < part(1740) + (512 << 10)
    assert dec_noalloc(B=1740, Hq=32, Hkv=8) == SCRATCH
    assert b"static" in fa.lib().fa_strerror(SCRATCH)


def test_strerror_names_every_code():
    for c in (0, -1, -2, -3, -4, -5):
        assert fa.lib().fa_strerror(c)
    assert b"unknown" in fa.lib().fa_strerror(5)


# ---- planner helpers pinned to the lecture's printed numbers --------------------------------

def test_wave_efficiency_pin():
    pin = GOLD["wave_efficiency_256_blocks"]
    assert round(fa.wave_efficiency(256, 108), 2) == pin["sms_108"]
    assert round(fa.wave_efficiency(256, 132), 2) == pin["sms_132"]


def test_split_heuristic_pins():
    p = GOLD["decode_splits_b1_h32_sms132"]
    assert round(fa.wave_efficiency(p["blocks"], p["sms"]), 2) == p["no_split_util"]
    assert fa.plan_splits(p["blocks"], p["sms"], 0.85) == p["splits"]
    assert round(fa.wave_efficiency(p["blocks"] * p["splits"], p["sms"]), 2) == p["split_util"]
    p = GOLD["decode_splits_b2_hkv8_sms132"]
    assert round(fa.wave_efficiency(p["blocks"], p["sms"]), 2) == p["no_split_util"]
    assert fa.plan_splits(p["blocks"], p["sms"], 0.85) == p["splits"]


def test_lpt_pins():
    p = GOLD["lpt_toy"]
    ms, loads = fa.schedule_makespan(p["tasks"], p["workers"], longest_first=False)
    assert loads == p["natural_loads"] and ms == max(p["natural_loads"])
    ms, loads = fa.schedule_makespan(p["tasks"], p["workers"], longest_first=True)
    assert loads == p["lpt_loads"] and ms == max(p["lpt_loads"])
    assert fa.lpt_makespan(p["tasks"], p["workers"]) == (max(p["lpt_loads"]), p["lpt_loads"])
    p = GOLD["lpt_exercise10"]
    assert fa.lpt_makespan(p["tasks"], p["workers"])[0] == p["lpt_makespan"]
    assert fa.schedule_makespan(p["tasks"], p["workers"], False)[0] == p["natural_makespan"]
    assert fa.schedule_makespan(p["tasks"], p["workers"], True)[0] == p["lpt_makespan"]
    assert -(-sum(p["tasks"]) // p["workers"]) == p["lower_bound"]
    # a load past INT_MAX is refused rather than wrapped
    assert fa.schedule_makespan([2**31 - 1, 1], 1, False)[0] == -1


def test_build_info_names_the_target():
    info = fa.build_info()
    assert "gfx950" in info and "sched=" in info


def test_plan_splits_rejects_bad_fractions():
    assert fa.plan_splits(32, 132, 0.0) == -1 and fa.plan_splits(32, 132, 1.5) == -1
    assert fa.plan_splits(32, 132, 1.0) >= 1


def test_causal_tile_count_pin():
    p = GOLD["causal_tiles_n1024_block64"]
    assert fa.causal_tiles(1024, 64, 64) == p["computed"]
    # the forward's own tiling: 128-row query blocks, 64-key tiles
    T = 2048 // 64
    assert fa.causal_tiles(2048, 128, 64) == sum(2 * i + 2 for i in range(2048 // 128)) <= T * T


def test_decode_workspace_size():
    # int32 arrival counters (B * Hq), then fp32 partials (o, then m and l) for 2048 + B splits of
    # every query head, each part padded to 256 bytes
    def pad(x):
        return (x + 255) // 256 * 256

    for B, Hq, d in [(64, 32, 128), (1, 1, 64), (3, 5, 128)]:
        slots = (2048 + B) * Hq
        assert fa.lib().fa_decode_workspace_size(B, Hq, 8192, d) == pad(B * Hq * 4) + pad(slots * d * 4) + pad(slots * 8)
    assert fa.lib().fa_decode_workspace_size(0, 32, 8192, 128) == 0


def test_fp8_validation_and_scale_count():
    L = fa.lib()
    assert L.fa_fp8_scale_count(2, 130, 3) == 2 * 3 * 3
    assert L.fa_fp8_scale_count(0, 130, 3) == 0
    q = lambda **kw: L.fa_quantize_fp8(kw.get("x", P), kw.get("signs", None), kw.get("x8", P), kw.get("sc", P),  # noqa: E731
                                       kw.get("B", 1), kw.get("N", 8), kw.get("H", 1), kw.get("d", 128), None)
    assert q(x=None) == INVALID and q(sc=None) == INVALID and q(x8=MIS) == INVALID and q(signs=MIS) == INVALID
    assert q(N=0) == INVALID and q(d=96) == UNSUPPORTED

    def f(**kw):
        a = dict(q8=P, k8=P, v=P, qs=P, ks=P, o=P, lse=P, B=1, Hq=2, Hkv=1, Nq=8, Nk=8, d=128, causal=0, scale=0.1)
        a.update(kw)
        return L.fa_fwd_fp8(a["q8"], a["k8"], a["v"], a["qs"], a["ks"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                            a["Nq"], a["Nk"], a["d"], a["causal"], a["scale"], None)
    assert f(qs=None) == INVALID and f(ks=None) == INVALID and f(k8=None) == INVALID
    assert f(d=96) == UNSUPPORTED  # d in {64, 128}
    assert f(causal=1, Nk=9) == UNSUPPORTED and f(Hq=3, Hkv=2) == INVALID and f(scale=0.0) == INVALID


def test_dropout_validation():
    L = fa.lib()

    def f(**kw):
        a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=1, Nq=8, Nk=8, d=64, causal=0, scale=0.125, p=0.1,
                 seed=1, off=0)
        a.update(kw)
        return L.fa_fwd_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"],
                                a["d"], a["causal"], a["scale"], a["p"], a["seed"], a["off"], None)
    assert f(p=1.0) == INVALID and f(p=-0.01) == INVALID and f(p=float("nan")) == INVALID
    assert f(q=None) == INVALID and f(d=96) == UNSUPPORTED and f(causal=1, Nk=9) == UNSUPPORTED

    def b(ws=P, ws_bytes=None, **kw):
        a = dict(B=1, Hq=2, Hkv=1, Nq=8, Nk=8, d=64, causal=0, scale=0.125, p=0.1)
        a.update(kw)
        need = fa.fa_bwd_workspace_size(a["B"], a["Hq"], a["Nq"], a["d"])
        return L.fa_bwd_dropout(P, P, P, P, P, P, P, P, P, a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"],
                                a["causal"], a["scale"], a["p"], 5, 0, ws, need if ws_bytes is None else ws_bytes, None)
    assert b(p=1.5) == INVALID and b(ws=None) == WORKSPACE and b(d=32) == UNSUPPORTED and b(Hq=3, Hkv=2) == INVALID
