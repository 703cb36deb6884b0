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


class FwdVarlenArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
        ("q_stride", c_i64x2), ("k_stride", c_i64x2), ("v_stride", c_i64x2), ("o_stride", c_i64x2),
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
        ("total_q", ctypes.c_int32), ("total_k", ctypes.c_int32), ("max_seqlen_q", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float), ("causal", ctypes.c_int32),
    ]


class DecodePagedArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("q_stride", c_i64x2), ("k_stride", c_i64x3), ("v_stride", c_i64x3), ("o_stride", c_i64x2),
        ("table_stride", ctypes.c_int64),
        ("Bs", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
        ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32), ("max_len", ctypes.c_int32),
        ("split_len", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


class QuantizeArgs(ctypes.Structure):
    _fields_ = [
        ("x", ctypes.c_void_p), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
        ("x_stride", c_i64x3), ("codes_stride", c_i64x3),
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32), ("D", ctypes.c_int32),
        ("block", ctypes.c_int32),
    ]


class FwdFp8Args(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("q_scales", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("kv_lens", ctypes.c_void_p),
        ("q_stride", c_i64x3), ("k_stride", c_i64x3), ("v_stride", c_i64x3), ("o_stride", c_i64x3),
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("Nq", ctypes.c_int32), ("Nk", ctypes.c_int32), ("D", ctypes.c_int32),
        ("block", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float), ("causal", ctypes.c_int32),
    ]


EXPORTED = ["fa_fwd", "fa_fwd_dropout", "fa_fwd_varlen", "fa_fwd_fp8", "fa_quantize_fp8", "fa_bwd",
            "fa_bwd_dropout", "fa_bwd_workspace_bytes",
            "fa_decode", "fa_decode_workspace_bytes", "fa_decode_noalloc",
            "fa_decode_paged", "fa_decode_paged_workspace_bytes",
            "fa_status_str", "fa_device_supported", "fa_version"]

_lib = None


def _open(path: str) -> ctypes.CDLL:
    """Load one build of the library and declare the C signatures of its calls."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m io_aware_tiled_10_amd.build` (no fallback exists)")
    h = ctypes.CDLL(path)
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
    h.fa_decode_noalloc.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.c_void_p]
    h.fa_decode_noalloc.restype = ctypes.c_int
    h.fa_fwd_varlen.argtypes = [ctypes.POINTER(FwdVarlenArgs), ctypes.c_void_p]
    h.fa_fwd_varlen.restype = ctypes.c_int
    h.fa_decode_paged.argtypes = [ctypes.POINTER(DecodePagedArgs), ctypes.c_void_p,
                                  ctypes.c_size_t, ctypes.c_void_p]
    h.fa_decode_paged.restype = ctypes.c_int
    h.fa_decode_paged_workspace_bytes.argtypes = [ctypes.POINTER(DecodePagedArgs)]
    h.fa_decode_paged_workspace_bytes.restype = ctypes.c_size_t
    h.fa_fwd_dropout.argtypes = [ctypes.POINTER(FwdArgs), ctypes.c_float, ctypes.c_uint64, ctypes.c_void_p]
    h.fa_fwd_dropout.restype = ctypes.c_int
    h.fa_bwd_dropout.argtypes = [ctypes.POINTER(BwdArgs), ctypes.c_float, ctypes.c_uint64, ctypes.c_void_p,
                                 ctypes.c_size_t, ctypes.c_void_p]
    h.fa_bwd_dropout.restype = ctypes.c_int
    h.fa_quantize_fp8.argtypes = [ctypes.POINTER(QuantizeArgs), ctypes.c_void_p]
    h.fa_quantize_fp8.restype = ctypes.c_int
    h.fa_fwd_fp8.argtypes = [ctypes.POINTER(FwdFp8Args), ctypes.c_void_p]
    h.fa_fwd_fp8.restype = ctypes.c_int
    h.fa_status_str.argtypes = [ctypes.c_int]
    h.fa_status_str.restype = ctypes.c_char_p
    h.fa_device_supported.argtypes = [ctypes.c_int]
    h.fa_device_supported.restype = ctypes.c_int
    h.fa_version.argtypes = []
    h.fa_version.restype = ctypes.c_int
    return h


def lib() -> ctypes.CDLL:
    """The loaded library: libfa.so beside this file, or the build named by the
    FA_LIBRARY environment variable (a sanitizer or debug build of the same sources).
    Raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _open(os.environ.get("FA_LIBRARY") or _LIB_PATH)
    return _lib


def use_library(path: Optional[str]) -> Optional[ctypes.CDLL]:
    """Route every later call to the build at ``path`` (None: the default build);
    returns the handle in use before.  For tests that compare two builds."""
    global _lib
    prev = _lib
    _lib = None if path is None else _open(path)
    return prev


def restore_library(handle: Optional[ctypes.CDLL]) -> None:
    """Undo ``use_library`` with the handle it returned."""
    global _lib
    _lib = handle


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
# argument checks: the C ABI takes raw pointers and trusts the element types, the
# contiguity of LSE / length / offset arrays and the sizes of caller-supplied outputs;
# these checks turn a mismatch into a ValueError before any library call
# ----------------------------------------------------------------------------------

def _need(cond: bool, msg) -> None:
    """Raise ValueError(msg) unless cond; msg may be a callable that builds the message,
    so that a message with formatted values costs nothing when the check passes."""
    if not cond:
        raise ValueError(msg() if callable(msg) else msg)


def _same_device(ref: torch.Tensor, **named) -> None:
    for name, t in named.items():
        if t is not None:
            _need(t.device == ref.device, lambda: f"{name} is on {t.device}, expected {ref.device}")


def _on_gpu(ref: torch.Tensor) -> None:
    _need(ref.device.type == "cuda", lambda: f"tensors must be on a GPU device, got {ref.device}")


def _check_dtype(t: torch.Tensor, name: str, dtypes) -> None:
    _need(t.dtype in dtypes, lambda: f"{name} has dtype {t.dtype}, expected one of {list(dtypes)}")


def _check_shape(t: torch.Tensor, name: str, shape) -> None:
    _need(tuple(t.shape) == tuple(shape),
          lambda: f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_int32_vec(t: Optional[torch.Tensor], name: str, n: int, ref: torch.Tensor) -> None:
    if t is None:
        return
    _check_dtype(t, name, (torch.int32,))
    _need(t.dim() == 1 and t.numel() == n,
          lambda: f"{name} must be a 1-D tensor of {n} elements, got shape {tuple(t.shape)}")
    _need(t.is_contiguous(), lambda: f"{name} must be contiguous")
    _same_device(ref, **{name: t})


def _check_f32_contig(t: Optional[torch.Tensor], name: str, shape, ref: torch.Tensor) -> None:
    if t is None:
        return
    _check_dtype(t, name, (torch.float32,))
    _check_shape(t, name, shape)
    _need(t.is_contiguous(), lambda: f"{name} must be contiguous")
    _same_device(ref, **{name: t})


def _check_out(t: torch.Tensor, name: str, shape, dtypes, ref: torch.Tensor) -> None:
    _check_dtype(t, name, dtypes)
    _check_shape(t, name, shape)
    _same_device(ref, **{name: t})


def _check_inputs(dtypes, ref_name: str, ref: torch.Tensor, ndim: int, **named) -> None:
    """Every named tensor: ``ndim`` dimensions, ref's dtype (one of ``dtypes``), ref's device."""
    _need(ref.dim() == ndim, lambda: f"{ref_name} must have {ndim} dimensions, got {ref.dim()}")
    _check_dtype(ref, ref_name, dtypes)
    for name, t in named.items():
        _need(t.dim() == ndim, lambda: f"{name} must have {ndim} dimensions, got {t.dim()}")
        _need(t.dtype == ref.dtype, lambda: f"{name} has dtype {t.dtype}, {ref_name} has {ref.dtype}")
    _same_device(ref, **named)


def _workspace_bytes(ws: torch.Tensor, ref: torch.Tensor) -> int:
    _need(ws.is_contiguous(), "workspace must be contiguous")
    _same_device(ref, workspace=ws)
    return ws.numel() * ws.element_size()


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
    _check_fwd_inputs(q, k, v, kv_lens)
    B, Hq, Nq, D = q.shape
    o = out if out is not None else torch.empty((B, Hq, Nq, D), dtype=out_dtype or q.dtype,
                                                device=q.device)
    lse = lse_out if lse_out is not None else (
        torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if with_lse else None)
    _check_fwd_outputs(q, o, lse)
    _on_gpu(q)
    a = fwd_args(q, k, v, o, lse, causal, scale, kv_lens)
    _check(lib().fa_fwd(ctypes.byref(a), _stream(q.device)))
    return o, lse


def _check_fwd_inputs(q, k, v, kv_lens) -> None:
    _check_inputs(_DT, "q", q, 4, k=k, v=v)
    _need(k.shape == v.shape, lambda: f"k {tuple(k.shape)} and v {tuple(v.shape)} differ in shape")
    _need(k.shape[0] == q.shape[0] and k.shape[3] == q.shape[3],
          lambda: f"k/v {tuple(k.shape)} do not match q {tuple(q.shape)} in batch or head dim")
    _check_int32_vec(kv_lens, "kv_lens", q.shape[0], q)


def _check_fwd_outputs(q, o, lse) -> None:
    B, Hq, Nq, D = q.shape
    _check_out(o, "out", (B, Hq, Nq, D), _DT, q)
    _check_f32_contig(lse, "lse_out", (B, Hq, Nq), q)


def _s2(t: torch.Tensor):
    if t.stride(-1) != 1:
        raise ValueError("the last (head) dimension must be contiguous")
    return c_i64x2(*t.stride()[:2])


def fwd_varlen_args(q, k, v, o, lse, cu_q, cu_k, max_seqlen_q, causal, scale) -> FwdVarlenArgs:
    Tq, Hq, D = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    return FwdVarlenArgs(
        q=_ptr(q), k=_ptr(k), v=_ptr(v), o=_ptr(o), lse=_ptr(lse),
        cu_seqlens_q=_ptr(cu_q), cu_seqlens_k=_ptr(cu_k),
        q_stride=_s2(q), k_stride=_s2(k), v_stride=_s2(v), o_stride=_s2(o),
        B=cu_q.numel() - 1, Hq=Hq, Hkv=Hkv, D=D, total_q=Tq, total_k=Tk,
        max_seqlen_q=int(max_seqlen_q), in_dtype=_DT[q.dtype], out_dtype=_DT[o.dtype],
        scale=_scale(scale, D), causal=int(bool(causal)))


def fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
               cu_seqlens_k: torch.Tensor, max_seqlen_q: int, causal: bool = False,
               scale: Optional[float] = None, out_dtype: Optional[torch.dtype] = None,
               with_lse: bool = True, out: Optional[torch.Tensor] = None,
               lse_out: Optional[torch.Tensor] = None):
    """Packed variable-length forward via ``fa_fwd_varlen``.

    q [Tq, Hq, D], k/v [Tk, Hkv, D], cu_seqlens_* int32 [B+1] on the device; returns
    O [Tq, Hq, D] and LSE [Hq, Tq].
    """
    _check_inputs(_DT, "q", q, 3, k=k, v=v)
    _need(k.shape == v.shape and k.shape[2] == q.shape[2], "k/v must share a shape and q's head dim")
    _need(cu_seqlens_q.dim() == 1 and cu_seqlens_q.numel() >= 1, "cu_seqlens_q must be 1-D with B + 1 entries")
    nb = cu_seqlens_q.numel()
    _check_int32_vec(cu_seqlens_q, "cu_seqlens_q", nb, q)
    _check_int32_vec(cu_seqlens_k, "cu_seqlens_k", nb, q)
    Tq, Hq, D = q.shape
    o = out if out is not None else torch.empty((Tq, Hq, D), dtype=out_dtype or q.dtype,
                                                device=q.device)
    lse = lse_out if lse_out is not None else (
        torch.empty((Hq, Tq), dtype=torch.float32, device=q.device) if with_lse else None)
    _check_out(o, "out", (Tq, Hq, D), _DT, q)
    _check_f32_contig(lse, "lse_out", (Hq, Tq), q)
    _on_gpu(q)
    a = fwd_varlen_args(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, causal, scale)
    _check(lib().fa_fwd_varlen(ctypes.byref(a), _stream(q.device)))
    return o, lse


FP8_BLOCK = 64


def quantize_fp8(x: torch.Tensor, out: Optional[torch.Tensor] = None,
                 scales_out: Optional[torch.Tensor] = None):
    """Two-pass E4M3 block quantisation via ``fa_quantize_fp8``.

    x [B, H, N, D] bf16 -> (codes uint8 [B, H, N, D], steps fp32 [B, H, ceil(N / 64)]).
    """
    _check_inputs((torch.bfloat16,), "x", x, 4)
    B, H, N, D = x.shape
    codes = out if out is not None else torch.empty((B, H, N, D), dtype=torch.uint8, device=x.device)
    nb = (N + FP8_BLOCK - 1) // FP8_BLOCK
    sc = scales_out if scales_out is not None else torch.empty((B, H, nb), dtype=torch.float32, device=x.device)
    _check_out(codes, "out", (B, H, N, D), (torch.uint8,), x)
    _check_f32_contig(sc, "scales_out", (B, H, nb), x)
    _on_gpu(x)
    a = QuantizeArgs(x=_ptr(x), codes=_ptr(codes), scales=_ptr(sc), x_stride=_s3(x), codes_stride=_s3(codes),
                     B=B, H=H, N=N, D=D, block=FP8_BLOCK)
    _check(lib().fa_quantize_fp8(ctypes.byref(a), _stream(x.device)))
    return codes, sc


def fwd_fp8(q8: torch.Tensor, q_scales: torch.Tensor, k8: torch.Tensor, k_scales: torch.Tensor,
            v: torch.Tensor, causal: bool = False, scale: Optional[float] = None,
            kv_lens: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.bfloat16,
            with_lse: bool = True, out: Optional[torch.Tensor] = None,
            lse_out: Optional[torch.Tensor] = None):
    """Forward with E4M3 Q and K (codes + per-64-row steps) via ``fa_fwd_fp8``."""
    _check_inputs((torch.uint8,), "q8", q8, 4, k8=k8)
    _check_inputs((torch.bfloat16,), "v", v, 4)
    _same_device(q8, v=v)
    B, Hq, Nq, D = q8.shape
    Hkv, Nk = k8.shape[1], k8.shape[2]
    _check_shape(v, "v", (B, Hkv, Nk, D))
    nbq, nbk = (Nq + FP8_BLOCK - 1) // FP8_BLOCK, (Nk + FP8_BLOCK - 1) // FP8_BLOCK
    _check_f32_contig(q_scales, "q_scales", (B, Hq, nbq), q8)
    _check_f32_contig(k_scales, "k_scales", (B, Hkv, nbk), q8)
    _check_int32_vec(kv_lens, "kv_lens", B, q8)
    o = out if out is not None else torch.empty((B, Hq, Nq, D), dtype=out_dtype, device=q8.device)
    lse = lse_out if lse_out is not None else (
        torch.empty((B, Hq, Nq), dtype=torch.float32, device=q8.device) if with_lse else None)
    _check_fwd_outputs(q8, o, lse)
    _on_gpu(q8)
    a = FwdFp8Args(q=_ptr(q8), k=_ptr(k8), v=_ptr(v), q_scales=_ptr(q_scales), k_scales=_ptr(k_scales),
                   o=_ptr(o), lse=_ptr(lse), kv_lens=_ptr(kv_lens),
                   q_stride=_s3(q8), k_stride=_s3(k8), v_stride=_s3(v), o_stride=_s3(o),
                   B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, D=D, block=FP8_BLOCK, out_dtype=_DT[o.dtype],
                   scale=_scale(scale, D), causal=int(bool(causal)))
    _check(lib().fa_fwd_fp8(ctypes.byref(a), _stream(q8.device)))
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
    _check_bwd_inputs(q, k, v, o, do, lse, kv_lens)
    dq, dk, dv = grads if grads is not None else (torch.empty_like(q), torch.empty_like(k),
                                                  torch.empty_like(v))
    for name, g, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_out(g, name, ref.shape, (ref.dtype,), q)
    if workspace is not None:
        _workspace_bytes(workspace, q)
    _on_gpu(q)
    a = bwd_args(q, k, v, o, do, lse, dq, dk, dv, causal, scale, kv_lens)
    need = lib().fa_bwd_workspace_bytes(ctypes.byref(a))
    if workspace is None or _workspace_bytes(workspace, q) < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().fa_bwd(ctypes.byref(a), _ptr(workspace), _workspace_bytes(workspace, q), _stream(q.device)))
    return dq, dk, dv


def fwd_dropout(q, k, v, p_drop: float, seed: int, causal: bool = False, scale: Optional[float] = None,
                kv_lens: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                with_lse: bool = True, out: Optional[torch.Tensor] = None,
                lse_out: Optional[torch.Tensor] = None):
    """Forward with dropout on P via ``fa_fwd_dropout`` (mask from Philox4x32-10 and ``seed``)."""
    _check_fwd_inputs(q, k, v, kv_lens)
    B, Hq, Nq, D = q.shape
    o = out if out is not None else torch.empty((B, Hq, Nq, D), dtype=out_dtype or q.dtype, device=q.device)
    lse = lse_out if lse_out is not None else (
        torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if with_lse else None)
    _check_fwd_outputs(q, o, lse)
    _on_gpu(q)
    a = fwd_args(q, k, v, o, lse, causal, scale, kv_lens)
    _check(lib().fa_fwd_dropout(ctypes.byref(a), float(p_drop), int(seed), _stream(q.device)))
    return o, lse


def bwd_dropout(q, k, v, o, do, lse, p_drop: float, seed: int, causal: bool = False,
                scale: Optional[float] = None, kv_lens: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None,
                grads: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None):
    """Backward of ``fwd_dropout`` (same p_drop and seed) via ``fa_bwd_dropout``."""
    _check_bwd_inputs(q, k, v, o, do, lse, kv_lens)
    dq, dk, dv = grads if grads is not None else (torch.empty_like(q), torch.empty_like(k),
                                                  torch.empty_like(v))
    for name, g, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_out(g, name, ref.shape, (ref.dtype,), q)
    if workspace is not None:
        _workspace_bytes(workspace, q)
    _on_gpu(q)
    a = bwd_args(q, k, v, o, do, lse, dq, dk, dv, causal, scale, kv_lens)
    need = lib().fa_bwd_workspace_bytes(ctypes.byref(a))
    if workspace is None or _workspace_bytes(workspace, q) < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().fa_bwd_dropout(ctypes.byref(a), float(p_drop), int(seed), _ptr(workspace),
                                _workspace_bytes(workspace, q), _stream(q.device)))
    return dq, dk, dv


def _check_bwd_inputs(q, k, v, o, do, lse, kv_lens) -> None:
    _check_inputs((torch.bfloat16,), "q", q, 4, k=k, v=v, o=o, do=do)
    _need(k.shape == v.shape, lambda: f"k {tuple(k.shape)} and v {tuple(v.shape)} differ in shape")
    _need(k.shape[0] == q.shape[0] and k.shape[3] == q.shape[3],
          lambda: f"k/v {tuple(k.shape)} do not match q {tuple(q.shape)} in batch or head dim")
    _check_shape(o, "o", q.shape)
    _check_shape(do, "do", q.shape)
    _need(lse is not None, "lse (the forward's log-sum-exp) is required")
    _check_f32_contig(lse, "lse", q.shape[:3], q)
    _check_int32_vec(kv_lens, "kv_lens", q.shape[0], q)


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
    _check_decode_inputs(q, k_cache, v_cache, seq_lens)
    Bs, Hq, D = q.shape
    if max_len is None:
        max_len = k_cache.shape[2]
    o = out if out is not None else torch.empty((Bs, Hq, D), dtype=out_dtype or q.dtype,
                                                device=q.device)
    lse = lse_out if lse_out is not None else (
        torch.empty((Bs, Hq), dtype=torch.float32, device=q.device) if with_lse else None)
    _check_decode_outputs(q, o, lse)
    if workspace is not None:
        _workspace_bytes(workspace, q)
    _on_gpu(q)
    a = decode_args(q, k_cache, v_cache, seq_lens, o, lse, max_len, split_len, scale)
    need = lib().fa_decode_workspace_bytes(ctypes.byref(a))
    if workspace is None or _workspace_bytes(workspace, q) < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().fa_decode(ctypes.byref(a), _ptr(workspace), _workspace_bytes(workspace, q), _stream(q.device)))
    return o, lse


# largest workspace fa_decode_noalloc takes from its static per-device array
DECODE_NOALLOC_MAX_WORKSPACE_BYTES = 32 << 20


def decode_noalloc(q, k_cache, v_cache, seq_lens, out: torch.Tensor, lse_out: Optional[torch.Tensor] = None,
                   max_len: Optional[int] = None, split_len: int = 2048, scale: Optional[float] = None):
    """Split-KV decode via ``fa_decode_noalloc``: the library takes the chunk partials
    from its static per-device array, so this call allocates nothing (the caller passes
    ``out`` and, if wanted, ``lse_out``).  Calls that overlap on one GPU race."""
    _check_decode_inputs(q, k_cache, v_cache, seq_lens)
    if max_len is None:
        max_len = k_cache.shape[2]
    _check_decode_outputs(q, out, lse_out)
    _on_gpu(q)
    a = decode_args(q, k_cache, v_cache, seq_lens, out, lse_out, max_len, split_len, scale)
    _check(lib().fa_decode_noalloc(ctypes.byref(a), _stream(q.device)))
    return out, lse_out


def _check_decode_inputs(q, k_cache, v_cache, seq_lens) -> None:
    _check_inputs((torch.bfloat16,), "q", q, 3)
    _check_inputs((torch.bfloat16,), "k_cache", k_cache, 4, v_cache=v_cache)
    _same_device(q, k_cache=k_cache)
    _need(k_cache.shape == v_cache.shape, "k_cache and v_cache differ in shape")
    _need(k_cache.shape[0] == q.shape[0] and k_cache.shape[3] == q.shape[2],
          lambda: f"caches {tuple(k_cache.shape)} do not match q {tuple(q.shape)} in sequences or head dim")
    _need(seq_lens is not None, "seq_lens is required")
    _check_int32_vec(seq_lens, "seq_lens", q.shape[0], q)


def _check_decode_outputs(q, o, lse) -> None:
    Bs, Hq, D = q.shape
    _check_out(o, "out", (Bs, Hq, D), _DT, q)
    _check_f32_contig(lse, "lse_out", (Bs, Hq), q)


def decode_paged_args(q, k_pages, v_pages, block_table, seq_lens, o, lse, page_size, max_len,
                      split_len, scale) -> DecodePagedArgs:
    Bs, Hq, D = q.shape
    if q.stride(-1) != 1 or o.stride(-1) != 1 or block_table.stride(-1) != 1:
        raise ValueError("the last dimension must be contiguous")
    return DecodePagedArgs(
        q=_ptr(q), k_pages=_ptr(k_pages), v_pages=_ptr(v_pages), block_table=_ptr(block_table),
        seq_lens=_ptr(seq_lens), o=_ptr(o), lse=_ptr(lse),
        q_stride=c_i64x2(*q.stride()[:2]), k_stride=_s3(k_pages), v_stride=_s3(v_pages),
        o_stride=c_i64x2(*o.stride()[:2]), table_stride=block_table.stride(0),
        Bs=Bs, Hq=Hq, Hkv=k_pages.shape[1], D=D, num_pages=k_pages.shape[0],
        page_size=int(page_size), max_pages_per_seq=block_table.shape[1], max_len=int(max_len),
        split_len=int(split_len), in_dtype=_DT[q.dtype], out_dtype=_DT[o.dtype],
        scale=_scale(scale, D))


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, max_len: int, split_len: int = 2048,
                 scale: Optional[float] = None, out_dtype: Optional[torch.dtype] = None,
                 with_lse: bool = True, workspace: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None):
    """Split-KV decode over a paged cache via ``fa_decode_paged``.

    q [Bs, Hq, D]; k_pages / v_pages indexed [page, head, row, D] through their strides
    (a [P, page, Hkv, D] pool passes ``pool.transpose(1, 2)``); block_table int32 [Bs, W];
    the page size is ``k_pages.shape[2]``.
    """
    _check_inputs((torch.bfloat16,), "q", q, 3)
    _check_inputs((torch.bfloat16,), "k_pages", k_pages, 4, v_pages=v_pages)
    _same_device(q, k_pages=k_pages)
    _need(k_pages.shape == v_pages.shape, "k_pages and v_pages differ in shape")
    _need(k_pages.shape[3] == q.shape[2], "the pools' head dim differs from q's")
    _check_dtype(block_table, "block_table", (torch.int32,))
    _need(block_table.dim() == 2 and block_table.shape[0] == q.shape[0],
          lambda: f"block_table must be [Bs, W] with Bs = {q.shape[0]}, got {tuple(block_table.shape)}")
    _same_device(q, block_table=block_table)
    _check_int32_vec(seq_lens, "seq_lens", q.shape[0], q)
    Bs, Hq, D = q.shape
    o = out if out is not None else torch.empty((Bs, Hq, D), dtype=out_dtype or q.dtype,
                                                device=q.device)
    lse = lse_out if lse_out is not None else (
        torch.empty((Bs, Hq), dtype=torch.float32, device=q.device) if with_lse else None)
    _check_decode_outputs(q, o, lse)
    if workspace is not None:
        _workspace_bytes(workspace, q)
    _on_gpu(q)
    a = decode_paged_args(q, k_pages, v_pages, block_table, seq_lens, o, lse, k_pages.shape[2],
                          max_len, split_len, scale)
    need = lib().fa_decode_paged_workspace_bytes(ctypes.byref(a))
    if workspace is None or _workspace_bytes(workspace, q) < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().fa_decode_paged(ctypes.byref(a), _ptr(workspace), _workspace_bytes(workspace, q),
                                 _stream(q.device)))
    return o, lse


def device_supported(device: int = 0) -> bool:
    return bool(lib().fa_device_supported(device))
