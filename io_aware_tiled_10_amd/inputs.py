"""Seeded synthetic inputs for the attention workloads.

This module holds no attention arithmetic.  It draws i.i.d. N(0, 1) values with
numpy's PCG64 generator and rounds them to bf16 (round to nearest, ties to
even) where a workload is bf16, so that the HIP library and the fp64 oracle are
handed exactly the same numbers.

Recipe:

* forward / backward: ``rng = default_rng(seed)``; draw q, k, v (then dO for
  the backward) in that order, each ``rng.standard_normal(shape, float32)`` in
  contiguous [B, H, N, D];
* decode: ``rng = default_rng(seed)``; draw the lengths
  ``rng.integers(lo, hi, endpoint=True, size=Bs)`` first, then q [Bs, Hq, D];
  the cached keys and values of sequence s come from their own generator
  ``default_rng([seed, 1, s])`` (k then v, each [Hkv, L_s, D]) so that a single
  sequence can be regenerated without drawing the whole cache;
* packed variable-length batches: lengths ``default_rng([seed, 7]).integers(lo,
  hi, endpoint=True)``; q, k, v drawn from ``default_rng([seed, 5])`` in that
  order as [total rows, H, D];
* paged caches: the decode cache's pages are placed in the order of
  ``default_rng([seed, 9])`` (numpy pools) or ``default_rng([seed, 11])`` (torch
  pools) permutations of the page pool; unused rows hold NaN.
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


def ragged_lengths(B: int, lo: int, hi: int, seed: int = 0) -> np.ndarray:
    """B sequence lengths drawn uniformly from [lo, hi] (int64)."""
    return np.random.default_rng([seed, 7]).integers(lo, hi, endpoint=True, size=B).astype(np.int64)


def offsets(lens) -> np.ndarray:
    """Prefix offsets [0, l0, l0 + l1, ...] of a packed batch (int32)."""
    return np.concatenate([[0], np.cumsum(np.asarray(lens, dtype=np.int64))]).astype(np.int32)


@dataclass
class VarlenInputs:
    """A packed batch: q [Tq, Hq, D], k and v [Tk, Hkv, D], offsets cu_q, cu_k [B + 1]."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    cu_q: np.ndarray
    cu_k: np.ndarray


def varlen_inputs(lens_q, lens_k, Hq: int, Hkv: int, D: int, dtype: str = "bf16",
                  seed: int = 0) -> VarlenInputs:
    rng = np.random.default_rng([seed, 5])
    cu_q, cu_k = offsets(lens_q), offsets(lens_k)
    q = _draw(rng, (int(cu_q[-1]), Hq, D), dtype)
    k = _draw(rng, (int(cu_k[-1]), Hkv, D), dtype)
    v = _draw(rng, (int(cu_k[-1]), Hkv, D), dtype)
    return VarlenInputs(q, k, v, cu_q, cu_k)


@dataclass
class PagedCache:
    """KV cache scattered over physical pages in a random order.

    k_pages, v_pages [P, Hkv, page_size, D]; block_table [Bs, W] int32, entry j of
    row s naming the page that holds positions j*page_size .. of sequence s, and -1
    past the sequence.  Rows of a page past its sequence's length hold ``pad_value``.
    """
    k_pages: np.ndarray
    v_pages: np.ndarray
    block_table: np.ndarray
    page_size: int


def paged_cache(dec: DecodeInputs, page_size: int, seed: int = 0, spare_pages: int = 0,
                pad_value: float = np.nan) -> PagedCache:
    lens = [int(x) for x in dec.seq_lens]
    npg = [(L + page_size - 1) // page_size for L in lens]
    total = sum(npg) + spare_pages
    perm = np.random.default_rng([seed, 9]).permutation(total).astype(np.int32)
    kp = np.full((total, dec.Hkv, page_size, dec.D), pad_value, dtype=np.float32)
    vp = np.full_like(kp, pad_value)
    table = np.full((len(lens), max(npg + [1])), -1, dtype=np.int32)
    nxt = 0
    for s, L in enumerate(lens):
        k, v = dec.kv(s)
        for j in range(npg[s]):
            page = perm[nxt]
            nxt += 1
            table[s, j] = page
            n = min(page_size, L - j * page_size)
            kp[page, :, :n] = k[:, j * page_size:j * page_size + n]
            vp[page, :, :n] = v[:, j * page_size:j * page_size + n]
    return PagedCache(kp, vp, table, page_size)


def paged_pools_torch(kc, vc, lens, page_size: int, seed: int = 0, spare: int = 0,
                      row_major_heads: bool = False):
    """Scatter dense [Bs, Hkv, Lmax, D] caches (torch, any device) into page pools.

    Pages are placed in a seeded random order.  Returns (k_pages, v_pages, block_table):
    pools indexed [page, head, row, D] -- contiguous, or with ``row_major_heads`` views
    of [page, row, head, D] storage -- whose rows past a sequence's length, and whose
    spare pages, hold NaN; table entries (int32) past a sequence hold -1.
    """
    import torch

    dev = kc.device
    bs, hkv, lmax, d = kc.shape
    npg = [(int(L) + page_size - 1) // page_size for L in lens]
    total = sum(npg) + spare
    perm = torch.from_numpy(np.random.default_rng([seed, 11]).permutation(total)).to(dev)
    table = torch.full((bs, max(npg + [1])), -1, dtype=torch.int32, device=dev)
    s_idx = torch.from_numpy(np.repeat(np.arange(bs), npg)).to(dev)
    j_idx = torch.from_numpy(np.concatenate([np.arange(n) for n in npg] + [np.zeros(0, np.int64)])).to(dev)
    used = perm[:len(s_idx)]
    pos = j_idx[:, None] * page_size + torch.arange(page_size, device=dev)[None, :]
    lens_t = torch.tensor([int(L) for L in lens], dtype=torch.long, device=dev)
    inside = pos < lens_t[s_idx][:, None]
    pos = pos.clamp(max=lmax - 1)
    if len(s_idx):
        table[s_idx, j_idx] = used.to(torch.int32)
    pools = []
    for c in (kc, vc):
        pool = torch.full((total, page_size, hkv, d), float("nan"), dtype=c.dtype, device=dev)
        cr = c.permute(0, 2, 1, 3)
        for p0 in range(0, len(s_idx), 4096):  # bounded temporaries
            sl = slice(p0, p0 + 4096)
            rows = cr[s_idx[sl][:, None], pos[sl]]  # [pages, page_size, Hkv, D]
            rows[~inside[sl]] = float("nan")
            pool[used[sl]] = rows
        pools.append(pool.transpose(1, 2) if row_major_heads else pool.transpose(1, 2).contiguous())
    return pools[0], pools[1], table
