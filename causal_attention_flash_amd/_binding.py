"""ctypes binding of libcausal_attn.so (include/attn.h), with the same entry-point names.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch provides device memory and the current
stream.  There is no fallback: if the library is not built, loading fails
with an error that says so.
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcausal_attn.so")

ATTN_F32 = 0
ATTN_BF16 = 1
ATTN_F16 = 2

STATUS_NAMES = {
    0: "ATTN_OK",
    1: "ATTN_ERR_NULL",
    2: "ATTN_ERR_SHAPE",
    3: "ATTN_ERR_UNSUPPORTED",
    4: "ATTN_ERR_ALIGNMENT",
    5: "ATTN_ERR_WORKSPACE",
    6: "ATTN_ERR_HIP",
    7: "ATTN_ERR_ALIAS",
    8: "ATTN_ERR_SCRATCH",
}

# Every symbol include/attn.h declares, with its ctypes signature.
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_F = ctypes.c_float
_INT = ctypes.c_int
_SZ = ctypes.c_size_t
SIGNATURES = {
    "attn_fwd": (_INT, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _F, _INT, _INT, _P]),
    "attn_fwd_gqa": (_INT, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _F, _INT, _INT, _P]),
    "attn_fwd_fp8qk": (_INT, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _F, _F, _F, _INT, _INT, _P]),
    "attn_bwd_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64, _INT]),
    "attn_bwd_gqa_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I64, _INT]),
    "attn_bwd": (_INT, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _I64, _I64, _I64, _I64, _F, _INT, _INT, _P]),
    "attn_bwd_gqa": (_INT, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _I64, _I64, _I64, _I64, _I64, _F, _INT, _INT,
                            _P]),
    "attn_bwd_noalloc": (_INT, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _F, _INT, _INT, _P]),
    "attn_bwd_atomic_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64, _INT]),
    "attn_bwd_atomic": (_INT, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _I64, _I64, _I64, _I64, _F, _INT, _INT,
                               _P]),
    "attn_bwd_preprocess": (_INT, [_P, _P, _P, _I64, _I64, _I64, _I64, _INT, _P]),
    "attn_bwd_dkdv": (_INT, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _F, _INT, _INT, _P]),
    "attn_bwd_dq": (_INT, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _F, _INT, _INT, _P]),
    "attn_bwd_dq_delta": (_INT, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _F, _INT, _INT, _P]),
    "attn_decode_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I64, _INT]),
    "attn_decode": (_INT, [_P, _P, _P, _P, _P, _P, _P, _SZ, _I64, _I64, _I64, _I64, _I64, _F, _INT, _P]),
    "attn_clock_sample": (_INT, [_P, _I64, _P]),
    "attn_status_string": (ctypes.c_char_p, [_INT]),
}

_lib = None


class AttnError(RuntimeError):
    """A non-OK status from the C ABI."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {status_string(status)}")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and return the library; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m causal_attention_flash_amd.build` "
            "(hipcc, gfx950). There is no fallback implementation.")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


# ------------------------------------------------------------- raw C entry points
# Plain integers for pointers and sizes; `stream` is a hipStream_t as an int
# (0 = default stream).  Each returns the attn_status integer.

def c_attn_fwd(q, k, v, o, lse, B, H, S, D, scale, causal, dtype, stream=0) -> int:
    return load_library().attn_fwd(q, k, v, o, lse, B, H, S, D, scale, causal, dtype, stream)


def c_attn_fwd_gqa(q, k, v, o, lse, B, H, H_kv, S, D, scale, causal, dtype, stream=0) -> int:
    return load_library().attn_fwd_gqa(q, k, v, o, lse, B, H, H_kv, S, D, scale, causal, dtype, stream)


def c_attn_fwd_fp8qk(q, k, v, o, lse, B, H, H_kv, S, D, scale, q_descale, k_descale, causal, dtype,
                     stream=0) -> int:
    return load_library().attn_fwd_fp8qk(q, k, v, o, lse, B, H, H_kv, S, D, scale, q_descale, k_descale, causal,
                                         dtype, stream)


def c_attn_bwd_workspace_bytes(B, H, S, D, dtype) -> int:
    return load_library().attn_bwd_workspace_bytes(B, H, S, D, dtype)


def c_attn_bwd_gqa_workspace_bytes(B, H, H_kv, S, D, dtype) -> int:
    return load_library().attn_bwd_gqa_workspace_bytes(B, H, H_kv, S, D, dtype)


def c_attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, ws_bytes, B, H, S, D, scale, causal, dtype, stream=0) -> int:
    return load_library().attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, ws_bytes, B, H, S, D, scale, causal,
                                   dtype, stream)


def c_attn_bwd_gqa(q, k, v, o, do, lse, dq, dk, dv, ws, ws_bytes, B, H, H_kv, S, D, scale, causal, dtype,
                   stream=0) -> int:
    return load_library().attn_bwd_gqa(q, k, v, o, do, lse, dq, dk, dv, ws, ws_bytes, B, H, H_kv, S, D, scale, causal,
                                       dtype, stream)


def c_attn_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, B, H, S, D, scale, causal, dtype, stream=0) -> int:
    return load_library().attn_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, B, H, S, D, scale, causal, dtype,
                                           stream)


def c_attn_bwd_atomic_workspace_bytes(B, H, S, D, dtype) -> int:
    return load_library().attn_bwd_atomic_workspace_bytes(B, H, S, D, dtype)


def c_attn_bwd_atomic(q, k, v, o, do, lse, dq, dk, dv, ws, ws_bytes, B, H, S, D, scale, causal, dtype,
                      stream=0) -> int:
    return load_library().attn_bwd_atomic(q, k, v, o, do, lse, dq, dk, dv, ws, ws_bytes, B, H, S, D, scale, causal,
                                          dtype, stream)


def c_attn_clock_sample(out, n, stream=0) -> int:
    return load_library().attn_clock_sample(out, n, stream)


def c_attn_bwd_preprocess(o, do, delta, B, H, S, D, dtype, stream=0) -> int:
    return load_library().attn_bwd_preprocess(o, do, delta, B, H, S, D, dtype, stream)


def c_attn_bwd_dkdv(q, k, v, do, lse, delta, dk, dv, B, H, S, D, scale, causal, dtype, stream=0) -> int:
    return load_library().attn_bwd_dkdv(q, k, v, do, lse, delta, dk, dv, B, H, S, D, scale, causal, dtype, stream)


def c_attn_bwd_dq(q, k, v, do, lse, delta, dq, B, H, S, D, scale, causal, dtype, stream=0) -> int:
    return load_library().attn_bwd_dq(q, k, v, do, lse, delta, dq, B, H, S, D, scale, causal, dtype, stream)


def c_attn_bwd_dq_delta(q, k, v, o, do, lse, delta, dq, B, H, S, D, scale, causal, dtype, stream=0) -> int:
    return load_library().attn_bwd_dq_delta(q, k, v, o, do, lse, delta, dq, B, H, S, D, scale, causal, dtype, stream)


def c_attn_decode_workspace_bytes(B, H, H_kv, L, D, dtype) -> int:
    return load_library().attn_decode_workspace_bytes(B, H, H_kv, L, D, dtype)


def c_attn_decode(q, k, v, kv_lens, o, lse, ws, ws_bytes, B, H, H_kv, L, D, scale, dtype, stream=0) -> int:
    return load_library().attn_decode(q, k, v, kv_lens, o, lse, ws, ws_bytes, B, H, H_kv, L, D, scale, dtype, stream)


# ------------------------------------------------------------- torch-tensor wrappers

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float16:
        return ATTN_F16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise ValueError(f"unsupported dtype {t.dtype}: use torch.bfloat16, torch.float16 or torch.float32")


def _check_tensors(names_and_tensors, shape, dtype, device):
    for name, t in names_and_tensors:
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")
        if t.dtype != dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _stream(device) -> int:
    return _torch().cuda.current_stream(device).cuda_stream


def _scale(scale, D):
    return 1.0 / math.sqrt(D) if scale is None else float(scale)


def _call(fn, where, *args):
    st = fn(*args)
    if st != 0:
        raise AttnError(st, where)


def attn_fwd(q, k, v, scale=None, causal=True):
    """O, LSE = attn_fwd(Q, K, V): [B,H,S,D] tensors (bf16, fp16 or fp32) on one GPU."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, S, D]")
    B, H, S, D = q.shape
    _check_tensors((("q", q), ("k", k), ("v", v)), q.shape, q.dtype, q.device)
    dt = _dtype_code(q)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    _call(c_attn_fwd, "attn_fwd", q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
          B, H, S, D, _scale(scale, D), int(bool(causal)), dt, _stream(q.device))
    return o, lse


def attn_bwd(q, k, v, o, do, lse, scale=None, causal=True):
    """dQ, dK, dV = attn_bwd(Q, K, V, O, dO, LSE) with O, LSE from attn_fwd."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, S, D]")
    B, H, S, D = q.shape
    _check_tensors((("q", q), ("k", k), ("v", v), ("o", o), ("do", do)), q.shape, q.dtype, q.device)
    _check_tensors((("lse", lse),), (B, H, S), torch.float32, q.device)
    dt = _dtype_code(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    nws = c_attn_bwd_workspace_bytes(B, H, S, D, dt)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=q.device)
    _call(c_attn_bwd, "attn_bwd", q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
          lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws.numel(),
          B, H, S, D, _scale(scale, D), int(bool(causal)), dt, _stream(q.device))
    return dq, dk, dv


def attn_bwd_atomic(q, k, v, o, do, lse, scale=None, causal=True):
    """dQ, dK, dV = attn_bwd_atomic(...): as attn_bwd, with dQ accumulated by fp32
    atomic adds in the dK/dV pass (D = 64, bf16 or fp16; dQ not bitwise reproducible)."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, S, D]")
    B, H, S, D = q.shape
    _check_tensors((("q", q), ("k", k), ("v", v), ("o", o), ("do", do)), q.shape, q.dtype, q.device)
    _check_tensors((("lse", lse),), (B, H, S), torch.float32, q.device)
    dt = _dtype_code(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    nws = c_attn_bwd_atomic_workspace_bytes(B, H, S, D, dt)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=q.device)
    _call(c_attn_bwd_atomic, "attn_bwd_atomic", q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
          do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws.numel(),
          B, H, S, D, _scale(scale, D), int(bool(causal)), dt, _stream(q.device))
    return dq, dk, dv


def _kv_heads(q, k):
    """H_kv from K's shape [B, H_kv, S, D] next to Q's [B, H, S, D]."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, H, S, D] and [B, H_kv, S, D]")
    B, H, S, D = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, S, D) or Hkv < 1 or H % Hkv != 0:
        raise ValueError(f"k has shape {tuple(k.shape)}; expected [B, H_kv, S, D] with H_kv dividing H = {H}")
    return Hkv


def attn_fwd_gqa(q, k, v, scale=None, causal=True):
    """O, LSE = attn_fwd_gqa(Q, K, V): Q [B,H,S,D]; K, V [B,H_kv,S,D] (grouped heads)."""
    torch = _torch()
    Hkv = _kv_heads(q, k)
    B, H, S, D = q.shape
    _check_tensors((("q", q),), q.shape, q.dtype, q.device)
    _check_tensors((("k", k), ("v", v)), k.shape, q.dtype, q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    _call(c_attn_fwd_gqa, "attn_fwd_gqa", q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
          B, H, Hkv, S, D, _scale(scale, D), int(bool(causal)), _dtype_code(q), _stream(q.device))
    return o, lse


def attn_fwd_fp8qk(q8, k8, v, q_descale, k_descale, scale=None, causal=True):
    """O, LSE = attn_fwd_fp8qk(Q8, K8, V, q_descale, k_descale): Q8 [B,H,S,D] and K8
    [B,H_kv,S,D] hold OCP E4M3 codes (torch.uint8 or torch.float8_e4m3fn) whose
    values are code * descale; V [B,H_kv,S,D] is bf16 or fp16 and sets O's type."""
    torch = _torch()
    fp8 = getattr(torch, "float8_e4m3fn", None)
    for name, t in (("q8", q8), ("k8", k8)):
        if t.dtype not in (torch.uint8, fp8):
            raise ValueError(f"{name} must hold E4M3 codes (torch.uint8 or torch.float8_e4m3fn), not {t.dtype}")
    Hkv = _kv_heads(q8, k8)
    B, H, S, D = q8.shape
    _check_tensors((("q8", q8),), q8.shape, q8.dtype, q8.device)
    _check_tensors((("k8", k8),), k8.shape, k8.dtype, q8.device)
    _check_tensors((("v", v),), k8.shape, v.dtype, q8.device)
    dt = _dtype_code(v)
    o = torch.empty((B, H, S, D), dtype=v.dtype, device=q8.device)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q8.device)
    _call(c_attn_fwd_fp8qk, "attn_fwd_fp8qk", q8.data_ptr(), k8.data_ptr(), v.data_ptr(), o.data_ptr(),
          lse.data_ptr(), B, H, Hkv, S, D, _scale(scale, D), float(q_descale), float(k_descale),
          int(bool(causal)), dt, _stream(q8.device))
    return o, lse


def attn_bwd_gqa(q, k, v, o, do, lse, scale=None, causal=True):
    """dQ, dK, dV = attn_bwd_gqa(Q, K, V, O, dO, LSE); dK, dV are [B,H_kv,S,D]."""
    torch = _torch()
    Hkv = _kv_heads(q, k)
    B, H, S, D = q.shape
    _check_tensors((("q", q), ("o", o), ("do", do)), q.shape, q.dtype, q.device)
    _check_tensors((("k", k), ("v", v)), k.shape, q.dtype, q.device)
    _check_tensors((("lse", lse),), (B, H, S), torch.float32, q.device)
    dt = _dtype_code(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)
    nws = c_attn_bwd_gqa_workspace_bytes(B, H, Hkv, S, D, dt)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=q.device)
    _call(c_attn_bwd_gqa, "attn_bwd_gqa", q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
          lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws.numel(),
          B, H, Hkv, S, D, _scale(scale, D), int(bool(causal)), dt, _stream(q.device))
    return dq, dk, dv


def attn_bwd_preprocess(o, do):
    """delta = rowsum(dO * O) in fp32, [B, H, S]."""
    torch = _torch()
    B, H, S, D = o.shape
    _check_tensors((("o", o), ("do", do)), o.shape, o.dtype, o.device)
    delta = torch.empty((B, H, S), dtype=torch.float32, device=o.device)
    _call(c_attn_bwd_preprocess, "attn_bwd_preprocess", o.data_ptr(), do.data_ptr(), delta.data_ptr(),
          B, H, S, D, _dtype_code(o), _stream(o.device))
    return delta


def attn_bwd_dkdv(q, k, v, do, lse, delta, scale=None, causal=True, out=None):
    """dK, dV from the dK/dV pass alone (delta from attn_bwd_preprocess)."""
    torch = _torch()
    B, H, S, D = q.shape
    _check_tensors((("q", q), ("k", k), ("v", v), ("do", do)), q.shape, q.dtype, q.device)
    _check_tensors((("lse", lse), ("delta", delta)), (B, H, S), torch.float32, q.device)
    dk, dv = out if out is not None else (torch.empty_like(q), torch.empty_like(q))
    _call(c_attn_bwd_dkdv, "attn_bwd_dkdv", q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
          lse.data_ptr(), delta.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, S, D, _scale(scale, D),
          int(bool(causal)), _dtype_code(q), _stream(q.device))
    return dk, dv


def attn_bwd_dq(q, k, v, do, lse, delta, scale=None, causal=True, out=None):
    """dQ from the dQ pass alone (delta from attn_bwd_preprocess)."""
    torch = _torch()
    B, H, S, D = q.shape
    _check_tensors((("q", q), ("k", k), ("v", v), ("do", do)), q.shape, q.dtype, q.device)
    _check_tensors((("lse", lse), ("delta", delta)), (B, H, S), torch.float32, q.device)
    dq = out if out is not None else torch.empty_like(q)
    _call(c_attn_bwd_dq, "attn_bwd_dq", q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(),
          delta.data_ptr(), dq.data_ptr(), B, H, S, D, _scale(scale, D), int(bool(causal)), _dtype_code(q),
          _stream(q.device))
    return dq


def attn_bwd_dq_delta(q, k, v, o, do, lse, scale=None, causal=True, out=None, delta_out=None):
    """dQ pass that also forms delta = rowsum(dO o O); returns (dQ, delta)."""
    torch = _torch()
    B, H, S, D = q.shape
    _check_tensors((("q", q), ("k", k), ("v", v), ("o", o), ("do", do)), q.shape, q.dtype, q.device)
    _check_tensors((("lse", lse),), (B, H, S), torch.float32, q.device)
    dq = out if out is not None else torch.empty_like(q)
    delta = delta_out if delta_out is not None else torch.empty(B, H, S, dtype=torch.float32, device=q.device)
    _call(c_attn_bwd_dq_delta, "attn_bwd_dq_delta", q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
          do.data_ptr(), lse.data_ptr(), delta.data_ptr(), dq.data_ptr(), B, H, S, D, _scale(scale, D),
          int(bool(causal)), _dtype_code(q), _stream(q.device))
    return dq, delta


def attn_decode(q, k_cache, v_cache, kv_lens=None, scale=None):
    """O, LSE = attn_decode(q [B,H,D], k_cache, v_cache [B,H_kv,L,D], kv_lens int32 [B] or None).

    One new query row per (batch entry, query head) against its cache; sequence b
    uses its first kv_lens[b] cache rows (all L when kv_lens is None).
    """
    torch = _torch()
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B, H, D] and the caches [B, H_kv, L, D]")
    B, H, D = q.shape
    Hkv, L = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Hkv, L, D) or Hkv < 1 or H % Hkv != 0:
        raise ValueError(f"k_cache has shape {tuple(k_cache.shape)}; expected [B, H_kv, L, D] with H_kv dividing {H}")
    _check_tensors((("q", q),), q.shape, q.dtype, q.device)
    _check_tensors((("k_cache", k_cache), ("v_cache", v_cache)), k_cache.shape, q.dtype, q.device)
    lens_ptr = 0
    if kv_lens is not None:
        _check_tensors((("kv_lens", kv_lens),), (B,), torch.int32, q.device)
        lens_ptr = kv_lens.data_ptr()
    dt = _dtype_code(q)
    o = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    nws = c_attn_decode_workspace_bytes(B, H, Hkv, L, D, dt)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=q.device)
    _call(c_attn_decode, "attn_decode", q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), lens_ptr, o.data_ptr(),
          lse.data_ptr(), ws.data_ptr(), ws.numel(), B, H, Hkv, L, D, _scale(scale, D), dt, _stream(q.device))
    return o, lse
