"""Exact IO-aware attention for MI355X (gfx950): forward, recompute backward and
split-KV decode (contiguous or paged KV cache), a packed variable-length
forward and an FP8 (E4M3) Q K^T forward, as hand-written HIP kernels behind the C ABI in include/fa.h.

Python-side this package only marshals arguments (``binding``) and draws seeded
synthetic inputs (``inputs``).
"""

from .binding import (FaError, bwd, decode, decode_paged, device_supported, fwd,  # noqa: F401
                      fwd_fp8, fwd_varlen, lib, quantize_fp8)

__all__ = ["fwd", "fwd_varlen", "fwd_fp8", "quantize_fp8", "bwd", "decode", "decode_paged",
           "device_supported", "lib", "FaError"]
