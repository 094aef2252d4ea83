"""Python binding of libfa, the gfx950 exact-attention library (see include/fa.h).

The functions named like the C entry points (fa_fwd, fa_bwd, fa_decode) marshal torch device
tensors into pointers, sizes and the current HIP stream and raise on a non-zero status; all
computation happens in libfa's kernels. forward/backward/decode are conveniences that also
allocate the outputs with torch. There is no fallback: if libfa.so is missing or fails to
load, importing the binding's functions raises.
"""

from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# FA_LIB_VARIANT=<name> loads libfa_<name>.so, a build with another compiler scheduling strategy
# (python -m exact_io_aware_03_amd.build --sched-strategy <name>); the default build is libfa.so
_VARIANT = os.environ.get("FA_LIB_VARIANT", "")
LIB_PATH = os.path.join(_HERE, f"libfa_{_VARIANT}.so" if _VARIANT else "libfa.so")

FA_F32 = 0
FA_BF16 = 1
_STATUS = {0: "FA_OK", -1: "FA_ERR_INVALID_ARG", -2: "FA_ERR_UNSUPPORTED", -3: "FA_ERR_HIP", -4: "FA_ERR_WORKSPACE",
           -5: "FA_ERR_SCRATCH"}

EXPORTED = (
    "fa_fwd", "fa_bwd", "fa_bwd_workspace_size", "fa_decode", "fa_decode_workspace_size", "fa_strerror",
    "fa_version", "fa_wave_efficiency", "fa_plan_splits", "fa_schedule_makespan", "fa_causal_tiles",
    "fa_fp8_scale_count", "fa_quantize_fp8", "fa_fwd_fp8", "fa_fwd_dropout", "fa_bwd_dropout",
    "fa_lpt_makespan", "fa_build_info", "fa_decode_noalloc", "fa_bwd_single_pass", "fa_fwd_poly_exp2",
    "fa_exp2_poly", "fa_fwd_persistent", "fa_fwd_persistent_workspace_size",
)

_lib = None


class FAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_STATUS.get(code, code)}: {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libfa.so (built in-tree by exact_io_aware_03_amd.build); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} not built; run `python -m exact_io_aware_03_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
    L.fa_fwd.restype = i
    L.fa_bwd_workspace_size.argtypes = [i, i, i, i]
    L.fa_bwd_workspace_size.restype = sz
    L.fa_bwd.argtypes = [vp] * 9 + [i] * 7 + [f, i, vp, sz, vp]
    L.fa_bwd.restype = i
    L.fa_bwd_single_pass.argtypes = [vp] * 9 + [i] * 7 + [f, i, vp, sz, vp]
    L.fa_bwd_single_pass.restype = i
    L.fa_fwd_persistent_workspace_size.argtypes = []
    L.fa_fwd_persistent_workspace_size.restype = sz
    L.fa_fwd_persistent.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp, sz, vp]
    L.fa_fwd_persistent.restype = i
    L.fa_fwd_poly_exp2.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
    L.fa_fwd_poly_exp2.restype = i
    L.fa_exp2_poly.argtypes = [vp, vp, ctypes.c_long, vp]
    L.fa_exp2_poly.restype = i
    L.fa_decode_workspace_size.argtypes = [i, i, i, i]
    L.fa_decode_workspace_size.restype = sz
    L.fa_decode.argtypes = [vp] * 6 + [i] * 6 + [f, i, vp, sz, vp]
    L.fa_decode.restype = i
    L.fa_decode_noalloc.argtypes = [vp] * 6 + [i] * 6 + [f, i, vp]
    L.fa_decode_noalloc.restype = i
    L.fa_strerror.argtypes = [i]
    L.fa_strerror.restype = ctypes.c_char_p
    L.fa_version.restype = i
    L.fa_wave_efficiency.argtypes = [i, i]
    L.fa_wave_efficiency.restype = ctypes.c_double
    L.fa_plan_splits.argtypes = [i, i, f]
    L.fa_plan_splits.restype = i
    L.fa_schedule_makespan.argtypes = [ctypes.POINTER(i), i, i, i, ctypes.POINTER(i)]
    L.fa_schedule_makespan.restype = i
    L.fa_lpt_makespan.argtypes = [ctypes.POINTER(i), i, i, ctypes.POINTER(i)]
    L.fa_lpt_makespan.restype = i
    L.fa_build_info.restype = ctypes.c_char_p
    L.fa_causal_tiles.argtypes = [i, i, i]
    L.fa_causal_tiles.restype = ctypes.c_long
    L.fa_fp8_scale_count.argtypes = [i, i, i]
    L.fa_fp8_scale_count.restype = sz
    L.fa_quantize_fp8.argtypes = [vp] * 4 + [i] * 4 + [vp]
    L.fa_quantize_fp8.restype = i
    L.fa_fwd_fp8.argtypes = [vp] * 7 + [i] * 7 + [f, vp]
    L.fa_fwd_fp8.restype = i
    u64, u32 = ctypes.c_ulonglong, ctypes.c_uint
    L.fa_fwd_dropout.argtypes = [vp] * 5 + [i] * 7 + [f, f, u64, u32, vp]
    L.fa_fwd_dropout.restype = i
    L.fa_bwd_dropout.argtypes = [vp] * 9 + [i] * 7 + [f, f, u64, u32, vp, sz, vp]
    L.fa_bwd_dropout.restype = i
    _lib = L
    return L


def _check(code: int):
    if code != 0:
        raise FAError(code, lib().fa_strerror(code).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need_contig(*ts):
    for t in ts:
        if t is not None and (not t.is_contiguous() or not t.is_cuda):
            raise ValueError("tensors must be contiguous device tensors")


# ---- entry points with the C names (caller provides the outputs) ---------------------------

def fa_fwd(q, k, v, o, lse, causal: bool = False, scale: float | None = None, stream=None) -> None:
    """O and lse for q [B,Nq,Hq,d], k/v [B,Nk,Hkv,d] (see include/fa.h)."""
    _need_contig(q, k, v, o, lse)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(lib().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d, int(causal),
                        scale, _dtype_code(q), _stream(stream)))


def fa_fwd_persistent_workspace_size() -> int:
    return int(lib().fa_fwd_persistent_workspace_size())


def fa_fwd_persistent(q, k, v, o, lse, workspace, causal: bool = False, scale: float | None = None,
                      stream=None) -> None:
    """fa_fwd (bf16) from the persistent kernel with per-XCD task queues; `workspace` is a
    zero-initialised device buffer of fa_fwd_persistent_workspace_size() bytes."""
    _need_contig(q, k, v, o, lse, workspace)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(lib().fa_fwd_persistent(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
                                   int(causal), scale, _dtype_code(q), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))


def fa_fwd_poly_exp2(q, k, v, o, lse, causal: bool = False, scale: float | None = None, stream=None) -> None:
    """fa_fwd (bf16) with a quarter of the exponentials from the FMA-unit polynomial."""
    _need_contig(q, k, v, o, lse)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(lib().fa_fwd_poly_exp2(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d, int(causal),
                                  scale, _stream(stream)))


def fa_exp2_poly(x, y, stream=None) -> None:
    """y = 2^x from the FMA-unit polynomial, fp32 device tensors of equal size."""
    _need_contig(x, y)
    if x.numel() != y.numel():
        raise ValueError("x and y differ in size")
    _check(lib().fa_exp2_poly(_ptr(x), _ptr(y), x.numel(), _stream(stream)))


def _bwd_call(fn, q, k, v, o, dout, lse, dq, dk, dv, workspace, causal, scale, stream) -> None:
    _need_contig(q, k, v, o, dout, lse, dq, dk, dv, workspace)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
              B, Hq, Hkv, Nq, Nk, d, int(causal), scale, _dtype_code(q), _ptr(workspace), ws_bytes, _stream(stream)))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, causal: bool = False, scale: float | None = None,
           stream=None) -> None:
    _bwd_call(lib().fa_bwd, q, k, v, o, dout, lse, dq, dk, dv, workspace, causal, scale, stream)


def fa_bwd_single_pass(q, k, v, o, dout, lse, dq, dk, dv, workspace, causal: bool = False,
                       scale: float | None = None, stream=None) -> None:
    _bwd_call(lib().fa_bwd_single_pass, q, k, v, o, dout, lse, dq, dk, dv, workspace, causal, scale, stream)


def fa_decode(q, k_cache, v_cache, seqlens, o, lse, workspace, scale: float | None = None, stream=None) -> None:
    _need_contig(q, k_cache, v_cache, seqlens, o, lse, workspace)
    B, Nq, Hq, d = q.shape
    Nk_max, Hkv = k_cache.shape[1], k_cache.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().fa_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(o), _ptr(lse), B, Hq, Hkv,
                           Nq, Nk_max, d, scale, _dtype_code(q), _ptr(workspace), ws_bytes, _stream(stream)))


def fa_decode_noalloc(q, k_cache, v_cache, seqlens, o, lse, scale: float | None = None, stream=None) -> None:
    """fa_decode with its scratch in the library's static per-GPU array (allocates nothing)."""
    _need_contig(q, k_cache, v_cache, seqlens, o, lse)
    B, Nq, Hq, d = q.shape
    Nk_max, Hkv = k_cache.shape[1], k_cache.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(lib().fa_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(o), _ptr(lse), B, Hq,
                                   Hkv, Nq, Nk_max, d, scale, _dtype_code(q), _stream(stream)))


def fa_quantize_fp8(x, signs, x8, scales, stream=None) -> None:
    """E4M3 codes and per-64-row block scales of a bf16 [B,N,H,d] tensor, rotated by
    diag(signs) H_d / sqrt(d) first when `signs` (d fp32 values of +-1) is given."""
    _need_contig(x, signs, x8, scales)
    B, N, H, d = x.shape
    _check(lib().fa_quantize_fp8(_ptr(x), _ptr(signs), _ptr(x8), _ptr(scales), B, N, H, d, _stream(stream)))


def fa_fwd_fp8(q8, k8, v, q_scale, k_scale, o, lse, causal: bool = False, scale: float | None = None,
               stream=None) -> None:
    """O and lse from E4M3 q8/k8 (with their block scales) and bf16 v (see include/fa.h)."""
    _need_contig(q8, k8, v, q_scale, k_scale, o, lse)
    B, Nq, Hq, d = q8.shape
    Nk, Hkv = k8.shape[1], k8.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(lib().fa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v), _ptr(q_scale), _ptr(k_scale), _ptr(o), _ptr(lse), B, Hq,
                            Hkv, Nq, Nk, d, int(causal), scale, _stream(stream)))


def fa_fwd_dropout(q, k, v, o, lse, p: float, seed: int, offset: int = 0, causal: bool = False,
                   scale: float | None = None, stream=None) -> None:
    """The forward with dropout probability p on P (bf16; see include/fa.h)."""
    _need_contig(q, k, v, o, lse)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(lib().fa_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d, int(causal),
                                scale, p, seed, offset, _stream(stream)))


def fa_bwd_dropout(q, k, v, o, dout, lse, dq, dk, dv, workspace, p: float, seed: int, offset: int = 0,
                   causal: bool = False, scale: float | None = None, stream=None) -> None:
    _need_contig(q, k, v, o, dout, lse, dq, dk, dv, workspace)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().fa_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                                _ptr(dv), B, Hq, Hkv, Nq, Nk, d, int(causal), scale, p, seed, offset,
                                _ptr(workspace), ws_bytes, _stream(stream)))


def fa_bwd_workspace_size(B: int, Hq: int, Nq: int, d: int) -> int:
    return int(lib().fa_bwd_workspace_size(B, Hq, Nq, d))


def fa_decode_workspace_size(B: int, Hq: int, Nk_max: int, d: int) -> int:
    return int(lib().fa_decode_workspace_size(B, Hq, Nk_max, d))


# ---- allocating conveniences ---------------------------------------------------------------

def forward(q, k, v, causal: bool = False, scale: float | None = None, stream=None):
    import torch

    B, Nq, Hq, _ = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, o, lse, causal, scale, stream)
    return o, lse


def backward(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None, stream=None):
    import torch

    B, Nq, Hq, d = q.shape
    ws = torch.zeros(fa_bwd_workspace_size(B, Hq, Nq, d), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, causal, scale, stream)
    return dq, dk, dv


def decode(q, k_cache, v_cache, seqlens, scale: float | None = None, stream=None):
    import torch

    B, _, Hq, d = q.shape
    # zero-filled: the arrival counters at its start must be zero before a first use
    ws = torch.zeros(fa_decode_workspace_size(B, Hq, k_cache.shape[1], d), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    fa_decode(q, k_cache, v_cache, seqlens, o, lse, ws, scale, stream)
    return o, lse


def forward_dropout(q, k, v, p: float, seed: int, offset: int = 0, causal: bool = False,
                    scale: float | None = None, stream=None):
    import torch

    B, Nq, Hq, _ = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    fa_fwd_dropout(q, k, v, o, lse, p, seed, offset, causal, scale, stream)
    return o, lse


def backward_dropout(q, k, v, o, dout, lse, p: float, seed: int, offset: int = 0, causal: bool = False,
                     scale: float | None = None, stream=None):
    import torch

    B, Nq, Hq, d = q.shape
    ws = torch.zeros(fa_bwd_workspace_size(B, Hq, Nq, d), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa_bwd_dropout(q, k, v, o, dout, lse, dq, dk, dv, ws, p, seed, offset, causal, scale, stream)
    return dq, dk, dv


def quantize_fp8(x, signs=None, stream=None):
    """(codes uint8 [B,N,H,d], scales fp32 [B,H,ceil(N/64)]) of a bf16 tensor."""
    import torch

    B, N, H, _ = x.shape
    x8 = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scales = torch.empty((B, H, (N + 63) // 64), dtype=torch.float32, device=x.device)
    fa_quantize_fp8(x, signs, x8, scales, stream)
    return x8, scales


def forward_fp8(q8, k8, v, q_scale, k_scale, causal: bool = False, scale: float | None = None, stream=None):
    import torch

    B, Nq, Hq, d = q8.shape
    o = torch.empty((B, Nq, Hq, d), dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q8.device)
    fa_fwd_fp8(q8, k8, v, q_scale, k_scale, o, lse, causal, scale, stream)
    return o, lse


# ---- planner helpers -----------------------------------------------------------------------

def wave_efficiency(n_blocks: int, n_cus: int) -> float:
    return float(lib().fa_wave_efficiency(n_blocks, n_cus))


def plan_splits(n_blocks: int, n_cus: int, frac: float = 0.85) -> int:
    return int(lib().fa_plan_splits(n_blocks, n_cus, frac))


def schedule_makespan(tasks, workers: int, longest_first: bool):
    n = len(tasks)
    arr = (ctypes.c_int * max(n, 1))(*tasks)
    loads = (ctypes.c_int * workers)()
    ms = lib().fa_schedule_makespan(arr, n, workers, int(longest_first), loads)
    return ms, list(loads)


def lpt_makespan(tasks, workers: int):
    n = len(tasks)
    arr = (ctypes.c_int * max(n, 1))(*tasks)
    loads = (ctypes.c_int * workers)()
    ms = lib().fa_lpt_makespan(arr, n, workers, loads)
    return ms, list(loads)


def build_info() -> str:
    return lib().fa_build_info().decode()


def causal_tiles(n: int, br: int, bc: int) -> int:
    return int(lib().fa_causal_tiles(n, br, bc))


