"""Dropout on the attention probabilities, with a counter-based generator.

TEST INFRASTRUCTURE ONLY, like the rest of this package: imported by the test suite,
the package smoke check and the benchmark's ``cpu_baseline`` leg, never by the HIP
library, with which it shares no code.

The self-test page (section C) asks how dropout is carried out inside FlashAttention
without storing a mask; the pages give no recipe.  Readings taken:

* Dropout acts on P = softmax(S) after normalisation: O = (P * Z / keep) V, where Z is
  a 0/1 mask and keep the keep probability; the log-sum-exp is that of the undropped
  scores.  The backward uses the same Z: dV = (P * Z / keep)^T dO, dP = (dO V^T) * Z /
  keep, D_i = rowsum(dO * O), dS = P * (dP - D_i), dQ and dK as without dropout.
* The mask is regenerated, never stored: a counter-based generator, Philox4x32 with 10
  rounds (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3",
  SC 2011), maps a (counter, key) pair to four 32-bit words.
* Element (b, h, i, j) takes byte 4 a + e of the Philox output for counter
  (2 (j // 32) + h2, i, h, b) and key (seed_lo, seed_hi), where h2 = (j // 4) % 2,
  a = (j // 8) % 4, e = j % 4; byte n is bits 8 (n % 4) .. of word n // 4.  (Each group
  of 16 bytes covers the keys 32 c + 4 h2 + 8 a + e of one query: the keys one lane of
  the forward kernel holds.)
* The dropout probability is taken in steps of 1/256: with t = round(256 p) the element
  is kept iff its byte is >= t, so keep = (256 - t) / 256 exactly, and kept values are
  multiplied by 256 / (256 - t).
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .attention import _f64, _kv_len_of, _softmax_rows, visible_mask

M0, M1 = 0xD2511F53, 0xCD9E8D57      # Philox4x32 round multipliers
W0, W1 = 0x9E3779B9, 0xBB67AE85      # Weyl increments of the key
MASK32 = 0xFFFFFFFF


def philox4x32_10(ctr, key):
    """Philox4x32-10 of counters ctr [..., 4] and keys key [..., 2] (uint32 arrays)."""
    c = [np.asarray(ctr[..., n], dtype=np.uint64) for n in range(4)]
    k0 = np.asarray(key[..., 0], dtype=np.uint64)
    k1 = np.asarray(key[..., 1], dtype=np.uint64)
    for _ in range(10):
        p0 = np.uint64(M0) * c[0]
        p1 = np.uint64(M1) * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK32)
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
        k0 = (k0 + np.uint64(W0)) & np.uint64(MASK32)
        k1 = (k1 + np.uint64(W1)) & np.uint64(MASK32)
    return np.stack([x.astype(np.uint32) for x in c], axis=-1)


def threshold(p_drop: float) -> int:
    """Byte threshold t = round(256 p), 0 <= t <= 255."""
    t = int(np.floor(p_drop * 256.0 + 0.5))
    return min(max(t, 0), 255)


def keep_scale(p_drop: float) -> float:
    t = threshold(p_drop)
    return 256.0 / (256 - t)


def mask_bytes(b: int, h: int, rows, nk: int, seed: int) -> np.ndarray:
    """The generator's byte for every (i, j), i in ``rows``, j < nk: uint8 [R, nk]."""
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(nk, dtype=np.int64)
    I, J = np.meshgrid(rows, j, indexing="ij")
    ctr = np.stack([2 * (J // 32) + (J // 4) % 2, I, np.full_like(I, h), np.full_like(I, b)], axis=-1)
    key = np.broadcast_to(np.array([seed & MASK32, (seed >> 32) & MASK32], dtype=np.uint64), I.shape + (2,))
    words = philox4x32_10(ctr.astype(np.uint64), key)
    n = 4 * ((J // 8) % 4) + J % 4
    w = np.take_along_axis(words, (n // 4)[..., None], axis=-1)[..., 0]
    return ((w >> (8 * (n % 4)).astype(np.uint32)) & 0xFF).astype(np.uint8)


def keep_mask(b: int, h: int, rows, nk: int, seed: int, p_drop: float) -> np.ndarray:
    return mask_bytes(b, h, rows, nk, seed) >= threshold(p_drop)


def attn_fwd_dropout(q, k, v, p_drop: float, seed: int, scale: Optional[float] = None,
                     causal: bool = False, kv_lens=None, bh0=(0, 0)):
    """O = (P * Z * keep_scale) V and the undropped LSE, by the plain definition.

    ``bh0`` = (b0, h0) places the given tensors inside a larger batch: element
    (b, h, i, j) of them takes the mask of (b0 + b, h0 + h, i, j), so a slice of
    batch entries and query heads can be checked on its own."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    b_, hq_, nq, d = q.shape
    _, hkv, nk, _ = k.shape
    g = hq_ // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    ks = keep_scale(p_drop)
    o = np.zeros((b_, hq_, nq, d))
    lse = np.full((b_, hq_, nq), -np.inf)
    rows = np.arange(nq)
    for b in range(b_):
        lk = _kv_len_of(kv_lens, b, nk)
        for h in range(hq_):
            kh, vh = k[b, h // g, :lk], v[b, h // g, :lk]
            p, l_ = _softmax_rows(scale * (q[b, h] @ kh.T), visible_mask(rows, nq, lk, lk, causal))
            z = keep_mask(bh0[0] + b, bh0[1] + h, rows, lk, seed, p_drop)
            o[b, h] = (p * z * ks) @ vh
            lse[b, h] = l_
    return o, lse


def attn_bwd_dropout(q, k, v, do, p_drop: float, seed: int, scale: Optional[float] = None,
                     causal: bool = False, kv_lens=None, bh0=(0, 0)):
    """Gradients of L = sum(dO * O) for the dropout forward above (``bh0`` as there).
    Returns (dq, dk, dv, o, lse) in float64."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    b_, hq_, nq, d = q.shape
    _, hkv, nk, _ = k.shape
    g = hq_ // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    ks = keep_scale(p_drop)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    o = np.zeros_like(q)
    lse = np.full((b_, hq_, nq), -np.inf)
    rows = np.arange(nq)
    for b in range(b_):
        lk = _kv_len_of(kv_lens, b, nk)
        for h in range(hq_):
            kh, vh = k[b, h // g, :lk], v[b, h // g, :lk]
            p, l_ = _softmax_rows(scale * (q[b, h] @ kh.T), visible_mask(rows, nq, lk, lk, causal))
            zs = keep_mask(bh0[0] + b, bh0[1] + h, rows, lk, seed, p_drop) * ks
            pd = p * zs
            oh = pd @ vh
            dv[b, h // g, :lk] += pd.T @ do[b, h]
            dp = (do[b, h] @ vh.T) * zs
            di = np.sum(do[b, h] * oh, axis=-1)
            ds = p * (dp - di[:, None])
            dq[b, h] = scale * (ds @ kh)
            dk[b, h // g, :lk] += scale * (ds.T @ q[b, h])
            o[b, h] = oh
            lse[b, h] = l_
    return dq, dk, dv, o, lse
