"""ctypes binding of libfa.so: argument marshalling only.

Every step of the attention computation runs in the HIP kernels of libfa.so.
PyTorch provides device memory and the current stream.  If the library is not
built (``python -m io_aware_tiled_10_amd.build``) every call raises; there is no
fallback.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_BF16, FA_F32 = 0, 1
_DT = {torch.bfloat16: FA_BF16, torch.float32: FA_F32}

c_i64x3 = ctypes.c_int64 * 3
c_i64x2 = ctypes.c_int64 * 2


class FwdArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("kv_lens", ctypes.c_void_p),
        ("q_stride", c_i64x3), ("k_stride", c_i64x3), ("v_stride", c_i64x3), ("o_stride", c_i64x3),
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("Nq", ctypes.c_int32), ("Nk", ctypes.c_int32), ("D", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float), ("causal", ctypes.c_int32),
    ]


class BwdArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("dout", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("kv_lens", ctypes.c_void_p),
        ("q_stride", c_i64x3), ("k_stride", c_i64x3), ("v_stride", c_i64x3), ("o_stride", c_i64x3),
        ("do_stride", c_i64x3), ("dq_stride", c_i64x3), ("dk_stride", c_i64x3),
        ("dv_stride", c_i64x3),
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("Nq", ctypes.c_int32), ("Nk", ctypes.c_int32), ("D", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("causal", ctypes.c_int32),
    ]


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p), ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("q_stride", c_i64x2), ("k_stride", c_i64x3), ("v_stride", c_i64x3), ("o_stride", c_i64x2),
        ("Bs", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
        ("cache_len", ctypes.c_int32), ("max_len", ctypes.c_int32), ("split_len", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32), ("scale", ctypes.c_float),
    ]


EXPORTED = ["fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_decode", "fa_decode_workspace_bytes",
            "fa_status_str", "fa_device_supported", "fa_version"]

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libfa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m io_aware_tiled_10_amd.build` (no fallback exists)")
        h = ctypes.CDLL(_LIB_PATH)
        h.fa_fwd.argtypes = [ctypes.POINTER(FwdArgs), ctypes.c_void_p]
        h.fa_fwd.restype = ctypes.c_int
        h.fa_bwd.argtypes = [ctypes.POINTER(BwdArgs), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        h.fa_bwd.restype = ctypes.c_int
        h.fa_bwd_workspace_bytes.argtypes = [ctypes.POINTER(BwdArgs)]
        h.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
        h.fa_decode.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.c_void_p, ctypes.c_size_t,
                                ctypes.c_void_p]
        h.fa_decode.restype = ctypes.c_int
        h.fa_decode_workspace_bytes.argtypes = [ctypes.POINTER(DecodeArgs)]
        h.fa_decode_workspace_bytes.restype = ctypes.c_size_t
        h.fa_status_str.argtypes = [ctypes.c_int]
        h.fa_status_str.restype = ctypes.c_char_p
        h.fa_device_supported.argtypes = [ctypes.c_int]
        h.fa_device_supported.restype = ctypes.c_int
        h.fa_version.argtypes = []
        h.fa_version.restype = ctypes.c_int
        _lib = h
    return _lib


class FaError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(lib().fa_status_str(status).decode())


def _check(status: int) -> None:
    if status != 0:
        raise FaError(status)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _s3(t: torch.Tensor):
    if t.stride(-1) != 1:
        raise ValueError("the last (head) dimension must be contiguous")
    return c_i64x3(*t.stride()[:3])


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _scale(scale: Optional[float], d: int) -> float:
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


# ----------------------------------------------------------------------------------
# forward
# ----------------------------------------------------------------------------------

def fwd_args(q, k, v, o, lse, causal, scale, kv_lens) -> FwdArgs:
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    return FwdArgs(
        q=_ptr(q), k=_ptr(k), v=_ptr(v), o=_ptr(o), lse=_ptr(lse), kv_lens=_ptr(kv_lens),
        q_stride=_s3(q), k_stride=_s3(k), v_stride=_s3(v), o_stride=_s3(o),
        B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, D=D,
        in_dtype=_DT[q.dtype], out_dtype=_DT[o.dtype], scale=_scale(scale, D), causal=int(bool(causal)))


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
        scale: Optional[float] = None, kv_lens: Optional[torch.Tensor] = None,
        out_dtype: Optional[torch.dtype] = None, with_lse: bool = True,
        out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None
        ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """O = softmax(scale Q K^T) V and LSE via ``fa_fwd``; q [B,Hq,Nq,D], k/v [B,Hkv,Nk,D]."""
    B, Hq, Nq, D = q.shape
    o = out if out is not None else torch.empty((B, Hq, Nq, D), dtype=out_dtype or q.dtype,
                                                device=q.device)
    lse = lse_out if lse_out is not None else (
        torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if with_lse else None)
    a = fwd_args(q, k, v, o, lse, causal, scale, kv_lens)
    _check(lib().fa_fwd(ctypes.byref(a), _stream(q.device)))
    return o, lse


# ----------------------------------------------------------------------------------
# backward
# ----------------------------------------------------------------------------------

def bwd_args(q, k, v, o, do, lse, dq, dk, dv, causal, scale, kv_lens) -> BwdArgs:
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    return BwdArgs(
        q=_ptr(q), k=_ptr(k), v=_ptr(v), o=_ptr(o), dout=_ptr(do), lse=_ptr(lse),
        dq=_ptr(dq), dk=_ptr(dk), dv=_ptr(dv), kv_lens=_ptr(kv_lens),
        q_stride=_s3(q), k_stride=_s3(k), v_stride=_s3(v), o_stride=_s3(o), do_stride=_s3(do),
        dq_stride=_s3(dq), dk_stride=_s3(dk), dv_stride=_s3(dv),
        B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, D=D, dtype=_DT[q.dtype], scale=_scale(scale, D),
        causal=int(bool(causal)))


def bwd(q, k, v, o, do, lse, causal: bool = False, scale: Optional[float] = None,
        kv_lens: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
        grads: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None):
    """dQ, dK, dV via ``fa_bwd`` (bf16 in and out, fp32 accumulation)."""
    dq, dk, dv = grads if grads is not None else (torch.empty_like(q), torch.empty_like(k),
                                                  torch.empty_like(v))
    a = bwd_args(q, k, v, o, do, lse, dq, dk, dv, causal, scale, kv_lens)
    need = lib().fa_bwd_workspace_bytes(ctypes.byref(a))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().fa_bwd(ctypes.byref(a), _ptr(workspace), workspace.numel(), _stream(q.device)))
    return dq, dk, dv


def bwd_workspace_bytes(q, k, v, causal=False, scale=None) -> int:
    a = bwd_args(q, k, v, q, q, None, q, k, v, causal, scale, None)
    return lib().fa_bwd_workspace_bytes(ctypes.byref(a))


# ----------------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------------

def decode_args(q, k_cache, v_cache, seq_lens, o, lse, max_len, split_len, scale) -> DecodeArgs:
    Bs, Hq, D = q.shape
    Hkv, cache_len = k_cache.shape[1], k_cache.shape[2]
    if q.stride(-1) != 1 or o.stride(-1) != 1:
        raise ValueError("the last (head) dimension must be contiguous")
    return DecodeArgs(
        q=_ptr(q), k_cache=_ptr(k_cache), v_cache=_ptr(v_cache), seq_lens=_ptr(seq_lens),
        o=_ptr(o), lse=_ptr(lse),
        q_stride=c_i64x2(*q.stride()[:2]), k_stride=_s3(k_cache), v_stride=_s3(v_cache),
        o_stride=c_i64x2(*o.stride()[:2]),
        Bs=Bs, Hq=Hq, Hkv=Hkv, D=D, cache_len=cache_len, max_len=int(max_len),
        split_len=int(split_len), in_dtype=_DT[q.dtype], out_dtype=_DT[o.dtype],
        scale=_scale(scale, D))


def decode(q, k_cache, v_cache, seq_lens, max_len: Optional[int] = None, split_len: int = 2048,
           scale: Optional[float] = None, out_dtype: Optional[torch.dtype] = None,
           with_lse: bool = True, workspace: Optional[torch.Tensor] = None,
           out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None):
    """Split-KV decode via ``fa_decode``; q [Bs,Hq,D], caches [Bs,Hkv,Lcap,D], seq_lens int32."""
    Bs, Hq, D = q.shape
    if max_len is None:
        max_len = k_cache.shape[2]
    o = out if out is not None else torch.empty((Bs, Hq, D), dtype=out_dtype or q.dtype,
                                                device=q.device)
    lse = lse_out if lse_out is not None else (
        torch.empty((Bs, Hq), dtype=torch.float32, device=q.device) if with_lse else None)
    a = decode_args(q, k_cache, v_cache, seq_lens, o, lse, max_len, split_len, scale)
    need = lib().fa_decode_workspace_bytes(ctypes.byref(a))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().fa_decode(ctypes.byref(a), _ptr(workspace), workspace.numel(), _stream(q.device)))
    return o, lse


def device_supported(device: int = 0) -> bool:
    return bool(lib().fa_device_supported(device))
