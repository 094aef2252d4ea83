"""Seeded synthetic inputs for exact attention, shared by the tests, the bench and smoke().

This module only draws random numbers and lays them out; it holds none of the attention
arithmetic, so the fp64 oracle and the HIP path can both consume its arrays without sharing
any of the method's code.

Recipe (the source pages measure on models and datasets that are not available; these iid
tensors stand in for them at the shapes of the five workloads):

* generator: ``numpy.random.Generator(PCG64(seed))``, ``standard_normal(dtype=float32)``;
* draw order: Q, K, V, then dO (backward only), then the outlier mask (long-context only);
  decode draws Q, then the valid cache rows of K sequence by sequence, then those of V, and
  takes the lengths from a child stream ``PCG64([seed, 1])``;
* bf16 workloads draw in fp32 and round each value to the nearest bf16 (ties to even); the
  arrays returned are fp32 holding exactly those bf16 values, so an upcast to fp64 gives the
  oracle the very numbers the GPU reads;
* long-context workload: a per-element Bernoulli(0.01) mask over K, masked entries x20,
  applied in fp32 before rounding ("1% of K entries" read element-wise);
* decode: per-sequence KV lengths uniform on [1024, 8192] inclusive; the cache is padded to
  N_k_max rows and rows at or past a sequence's length are zero (never read).

Layouts: Q, O, dO are [B, N_q, H_q, d]; K, V are [B, N_k, H_kv, d]; d is innermost.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class Workload:
    """One named workload: shapes, dtype, mask mode and seed."""

    name: str
    kind: str  # "fwd", "decode" or "bwd"
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    dtype: str
    causal: tuple = (False,)
    seed: int = 0
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    len_range: tuple = ()
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


WORKLOADS = {
    # single-head fp32 forward, small enough for a pure-Python check
    "fwd_f32_256x64": Workload("fwd_f32_256x64", "fwd", 1, 1, 1, 256, 256, 64, F32, (False,), seed=1),
    # training-shape forward, run both with and without the causal mask
    "fwd_bf16_b16h16n2048d128": Workload(
        "fwd_bf16_b16h16n2048d128", "fwd", 16, 16, 16, 2048, 2048, 128, BF16, (False, True), seed=2
    ),
    # long-context causal forward with element-wise K outliers
    "fwd_bf16_causal_h32n16384d128": Workload(
        "fwd_bf16_causal_h32n16384d128", "fwd", 1, 32, 32, 16384, 16384, 128, BF16, (True,), seed=3,
        outlier_frac=0.01, outlier_scale=20.0,
    ),
    # single-query decode, GQA 32/8, ragged KV lengths
    "decode_bf16_b64hq32hkv8d128": Workload(
        "decode_bf16_b64hq32hkv8d128", "decode", 64, 32, 8, 1, 8192, 128, BF16, (False,), seed=4,
        len_range=(1024, 8192),
    ),
    # causal backward
    "bwd_bf16_causal_b8h16n4096d128": Workload(
        "bwd_bf16_causal_b8h16n4096d128", "bwd", 8, 16, 16, 4096, 4096, 128, BF16, (True,), seed=5
    ),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32 holding bf16 values.

    Works in place on chunks to bound memory for multi-GiB tensors. NaN/Inf are not expected.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    u = flat.view(np.uint32)
    step = 1 << 24
    for s in range(0, u.size, step):
        c = u[s : s + step]
        bias = ((c >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
        c += bias
        c &= np.uint32(0xFFFF0000)
    return x


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of fp32 values that are already bf16-representable (for raw upload)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def make_attention_inputs(
    B: int, Nq: int, Nk: int, Hq: int, Hkv: int, d: int, seed: int, dtype: str = BF16,
    with_do: bool = False, outlier_frac: float = 0.0, outlier_scale: float = 1.0,
):
    """Q, K, V (and dO) for forward/backward workloads, fp32 arrays in BSHD layout."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _normal(rng, (B, Nq, Hq, d))
    k = _normal(rng, (B, Nk, Hkv, d))
    v = _normal(rng, (B, Nk, Hkv, d))
    out = {"q": q, "k": k, "v": v}
    if with_do:
        out["do"] = _normal(rng, (B, Nq, Hq, d))
    if outlier_frac > 0.0:
        # Bernoulli mask drawn after the tensors, in chunks of uniform draws.
        flat = k.reshape(-1)
        step = 1 << 24
        for s in range(0, flat.size, step):
            m = rng.random(size=min(step, flat.size - s), dtype=np.float32) < np.float32(outlier_frac)
            flat[s : s + step][m] *= np.float32(outlier_scale)
    if dtype == BF16:
        for key in out:
            out[key] = round_to_bf16(out[key])
    return out


def make_decode_inputs(
    B: int, Hq: int, Hkv: int, Nk_max: int, d: int, seed: int, len_range=(1024, 8192),
    dtype: str = BF16, lengths=None,
):
    """Decode inputs: q [B,1,Hq,d]; padded caches [B,Nk_max,Hkv,d]; int32 lengths [B].

    Each sequence's valid rows are drawn in batch order from one stream; rows past a
    sequence's length stay zero. ``lengths`` overrides the drawn lengths (edge-case tests).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _normal(rng, (B, 1, Hq, d))
    if lengths is None:
        # lengths are drawn from a child stream so the tensor draws above stay in the
        # documented order regardless of how many cache rows are valid
        lrng = np.random.Generator(np.random.PCG64([seed, 1]))
        lengths = lrng.integers(len_range[0], len_range[1], endpoint=True, size=B).astype(np.int32)
    lengths = np.asarray(lengths, dtype=np.int32)
    assert lengths.shape == (B,) and lengths.min() >= 1 and lengths.max() <= Nk_max
    kc = np.zeros((B, Nk_max, Hkv, d), dtype=np.float32)
    vc = np.zeros((B, Nk_max, Hkv, d), dtype=np.float32)
    rnd = round_to_bf16 if dtype == BF16 else (lambda x: x)
    for b in range(B):
        n = int(lengths[b])
        kc[b, :n] = rnd(_normal(rng, (n, Hkv, d)))
    for b in range(B):
        n = int(lengths[b])
        vc[b, :n] = rnd(_normal(rng, (n, Hkv, d)))
    if dtype == BF16:
        q = round_to_bf16(q)
    return {"q": q, "k": kc, "v": vc, "seqlens": lengths}


def make_workload_inputs(w: Workload):
    """Inputs for a named workload (full size)."""
    if w.kind == "decode":
        return make_decode_inputs(w.B, w.Hq, w.Hkv, w.Nk, w.d, w.seed, w.len_range, w.dtype)
    return make_attention_inputs(
        w.B, w.Nq, w.Nk, w.Hq, w.Hkv, w.d, w.seed, w.dtype, with_do=(w.kind == "bwd"),
        outlier_frac=w.outlier_frac, outlier_scale=w.outlier_scale,
    )


def sample_indices(n: int, k: int, seed: int) -> np.ndarray:
    """k distinct sorted indices in [0, n) from a seeded stream (for sampled checks)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    k = min(k, n)
    return np.sort(rng.choice(n, size=k, replace=False))
