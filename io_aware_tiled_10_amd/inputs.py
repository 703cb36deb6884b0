"""Seeded synthetic inputs for the attention workloads (numpy only).

This module holds no attention arithmetic.  It draws i.i.d. N(0, 1) values with
numpy's PCG64 generator and rounds them to bf16 (round to nearest, ties to
even) where a workload is bf16, so that the HIP library and the fp64 oracle are
handed exactly the same numbers.

Recipe (stated once more in the design doc):

* forward / backward: ``rng = default_rng(seed)``; draw q, k, v (then dO for
  the backward) in that order, each ``rng.standard_normal(shape, float32)`` in
  contiguous [B, H, N, D];
* decode: ``rng = default_rng(seed)``; draw the lengths
  ``rng.integers(lo, hi, endpoint=True, size=Bs)`` first, then q [Bs, Hq, D];
  the cached keys and values of sequence s come from their own generator
  ``default_rng([seed, 1, s])`` (k then v, each [Hkv, L_s, D]) so that a single
  sequence can be regenerated without drawing the whole cache.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

BF16_NAN_BITS = 0x7FC0


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Inputs are finite draws, so the NaN/Inf special cases are not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 value (returned as fp32)."""
    return (bf16_bits(x).astype(np.uint32) << 16).view(np.float32)


def _draw(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    return bf16_round(x) if dtype == "bf16" else x


@dataclass
class AttnInputs:
    """Host copies (fp32 arrays holding exactly the values given to the GPU)."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: Optional[np.ndarray] = None
    dtype: str = "bf16"


def attention_inputs(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, D: int,
                     dtype: str = "bf16", seed: int = 0,
                     with_grad: bool = False) -> AttnInputs:
    rng = np.random.default_rng(seed)
    q = _draw(rng, (B, Hq, Nq, D), dtype)
    k = _draw(rng, (B, Hkv, Nk, D), dtype)
    v = _draw(rng, (B, Hkv, Nk, D), dtype)
    do = _draw(rng, (B, Hq, Nq, D), dtype) if with_grad else None
    return AttnInputs(q, k, v, do, dtype)


@dataclass
class DecodeInputs:
    seq_lens: np.ndarray  # int64 [Bs]
    q: np.ndarray         # fp32 [Bs, Hq, D] (bf16-valued)
    Hkv: int
    D: int
    seed: int

    def kv(self, s: int):
        """Valid cached keys and values of sequence s: two [Hkv, L_s, D] arrays."""
        rng = np.random.default_rng([self.seed, 1, s])
        L = int(self.seq_lens[s])
        k = bf16_round(rng.standard_normal((self.Hkv, L, self.D), dtype=np.float32))
        v = bf16_round(rng.standard_normal((self.Hkv, L, self.D), dtype=np.float32))
        return k, v

    def kv_bits(self, s: int):
        """Same draws as :meth:`kv`, as bf16 bit patterns (uint16)."""
        rng = np.random.default_rng([self.seed, 1, s])
        L = int(self.seq_lens[s])
        k = bf16_bits(rng.standard_normal((self.Hkv, L, self.D), dtype=np.float32))
        v = bf16_bits(rng.standard_normal((self.Hkv, L, self.D), dtype=np.float32))
        return k, v

    def dense_cache(self, lmax: Optional[int] = None, pad_value: float = np.nan):
        """Padded [Bs, Hkv, Lmax, D] caches with ``pad_value`` beyond each length."""
        bs = len(self.seq_lens)
        lmax = int(self.seq_lens.max()) if lmax is None else lmax
        kc = np.full((bs, self.Hkv, lmax, self.D), pad_value, dtype=np.float32)
        vc = np.full_like(kc, pad_value)
        for s in range(bs):
            L = int(self.seq_lens[s])
            kc[s, :, :L], vc[s, :, :L] = self.kv(s)
        return kc, vc


def decode_inputs(Bs: int, Hq: int, Hkv: int, D: int, len_lo: int, len_hi: int,
                  seed: int = 0) -> DecodeInputs:
    rng = np.random.default_rng(seed)
    lens = rng.integers(len_lo, len_hi, endpoint=True, size=Bs).astype(np.int64)
    q = bf16_round(rng.standard_normal((Bs, Hq, D), dtype=np.float32))
    return DecodeInputs(lens, q, Hkv, D, seed)
