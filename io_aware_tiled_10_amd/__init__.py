"""Exact IO-aware attention for MI355X (gfx950): forward, recompute backward and
split-KV decode (contiguous or paged KV cache), a packed variable-length
forward, an FP8 (E4M3) Q K^T forward and dropout on P, as hand-written HIP kernels behind the C ABI in include/fa.h.

Python-side this package only marshals arguments (``binding``) and draws seeded
synthetic inputs (``inputs``).
"""

from .binding import (FaError, bwd, bwd_dropout, decode, decode_noalloc, decode_paged,  # noqa: F401
                      device_supported,
                      fwd, fwd_dropout, fwd_fp8, fwd_varlen, lib, quantize_fp8)

__all__ = ["fwd", "fwd_dropout", "fwd_varlen", "fwd_fp8", "quantize_fp8", "bwd", "bwd_dropout", "decode", "decode_noalloc",
           "decode_paged", "device_supported", "lib", "FaError"]
