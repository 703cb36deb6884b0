"""Exact IO-aware attention for MI355X (gfx950): forward, recompute backward and
split-KV decode, as hand-written HIP kernels behind the C ABI in include/fa.h.

Python-side this package only marshals arguments (``binding``) and draws seeded
synthetic inputs (``inputs``).
"""

from .binding import FaError, bwd, decode, device_supported, fwd, lib  # noqa: F401

__all__ = ["fwd", "bwd", "decode", "device_supported", "lib", "FaError"]
