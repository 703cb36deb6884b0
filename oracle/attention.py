"""Plain fp64 CPU oracle for exact scaled dot-product attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's ``cpu_baseline`` leg may import this module.  It shares no code with
the HIP library and is never a fallback for it.

Every function materialises the full score matrix S and probability matrix P,
as the plain definition of attention does; nothing here is tiled, fused or
reordered beyond that definition.  Query rows may be processed in independent
chunks only to bound host memory (each row of S depends on its own query alone).

Sources (the four web pages the method is described on):

* "二十四：Flash Attention自测题" (book.bogosort.top, LLM tutorial L24), the
  self-test list: section A (the attention formula and the [B,H,N,D] shapes),
  section C (causal mask, padding / variable length, where 1/sqrt(d) applies),
  section D (which small statistics the backward keeps; the dV, dP, dS, dQ, dK
  relations), section F (MHA / MQA / GQA head counts, KV-cache decode).
* "flash attention呢" (agentalpha.top interview answer), 标准答 part 1 (tiling
  and online softmax), part 2 (recompute in the backward) and 高频追问 2
  (split-KV decode merged with the online-softmax update).
* "Flash Attention V2/V3 optimisation" article (aiqz.cc), section V2算法优化
  (online-softmax equations for m, l and the output accumulator, and the single
  division by l at the end) and the Python demo section (row-wise blocks of K/V,
  the same [batch, heads, seq, d] layout).
* Study card airsota.com/?p=1562, section 三 (safe softmax; the online update
  m_new = max(m, max_j z_j), l_new = e^(m - m_new) l + sum_j e^(z_j - m_new);
  the two-block derivation) and section 四 (deferred normalisation, recompute
  from the saved m and l, GQA).

Readings taken where the pages are silent:

* The log-sum-exp saved for the backward is LSE = m + ln(l), natural log, in the
  units of the scaled scores.
* Causal masking is aligned bottom-right: key j is visible to query i iff
  j <= i + (Lk - Nq), where Lk is the number of valid keys of that batch entry.
* Keys at positions >= kv_len do not exist; their memory never influences a
  result.
* GQA groups are contiguous: query head hq reads KV head hq // (Hq // Hkv).
* A query row with no visible key has O = 0 and LSE = -inf; its gradients are 0.
* Packed variable-length batches: sequence b owns query rows cu_q[b]..cu_q[b+1]
  and key rows cu_k[b]..cu_k[b+1] of the packed tensors and sees only its own
  keys; the causal alignment is per sequence.  LSE is laid out [Hq, total rows].
* Paged KV cache: cached position t of sequence s is row t % page_size of the
  physical page block_table[s][t // page_size].

All arithmetic is float64.  Inputs given in bf16 / fp32 are upcast exactly.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "visible_mask",
    "attn_fwd",
    "attn_bwd",
    "attn_bwd_dq_rows",
    "attn_bwd_dkdv_rows",
    "attn_decode",
    "attn_fwd_varlen",
    "attn_decode_paged",
    "online_softmax_attention",
    "decode_split_partials",
    "merge_partials",
    "materialised_score_bytes",
]

# Upper bound on the number of fp64 score elements held at once (256 MiB).
_CHUNK_ELEMS = 1 << 25


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _kv_len_of(kv_lens: Optional[Sequence[int]], b: int, nk: int) -> int:
    if kv_lens is None:
        return nk
    return int(min(max(int(kv_lens[b]), 0), nk))


def visible_mask(rows: np.ndarray, nq: int, nk: int, lk: int, causal: bool) -> np.ndarray:
    """Boolean [len(rows), nk] mask of the (query, key) pairs that exist.

    Keys at j >= lk are padding (self-test page, section C, padding and
    variable length).  With ``causal`` the mask is lower-triangular, aligned so
    that the last query row sees the last valid key (self-test page, section C,
    causal mask; bottom-right reading).
    """
    j = np.arange(nk)[None, :]
    vis = j < lk
    if causal:
        i = np.asarray(rows)[:, None]
        vis = vis & (j <= i + (lk - nq))
    return vis


def _softmax_rows(s: np.ndarray, vis: np.ndarray):
    """Safe softmax of each row of ``s`` over the visible entries.

    Subtracts the row maximum before exponentiating (study card, section 三,
    safe softmax).  Returns (P, LSE); a row with no visible entry (its maximum is
    -inf) gets P = 0 and LSE = -inf.  Every other row follows IEEE arithmetic, so a
    NaN among its visible scores makes its P and LSE NaN.
    """
    if s.shape[-1] == 0:  # no key exists at all
        return np.zeros(s.shape), np.full(s.shape[:-1], -np.inf)
    s = np.where(vis, s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    with np.errstate(invalid="ignore"):
        e = np.exp(s - m_safe)  # exp(-inf) = 0 on masked entries
    l = np.sum(e, axis=-1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(empty, 0.0, e / np.where(empty, 1.0, l))
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    return p, lse[..., 0]


def attn_fwd(q, k, v, scale: Optional[float] = None, causal: bool = False,
             kv_lens: Optional[Sequence[int]] = None,
             rows: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """O = softmax(scale * Q K^T) V and the per-row LSE, by the plain definition.

    Shapes: q [B, Hq, Nq, D]; k, v [B, Hkv, Nk, D]; Hq % Hkv == 0.  Returns
    O [B, Hq, R, D] and LSE [B, Hq, R] in float64, where R = Nq, or len(rows)
    when only the query rows in ``rows`` (absolute indices) are wanted.

    Follows the formula of the self-test page, section A, and the V2/V3
    article's IO section: materialise S = scale * Q K^T, take the row-wise
    softmax P, and form O = P V.  The scale defaults to 1/sqrt(D) (self-test
    page section C; study card section 二).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    b_, hq_, nq, d = q.shape
    _, hkv, nk, _ = k.shape
    assert hq_ % hkv == 0, "Hq must be a multiple of Hkv"
    g = hq_ // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.arange(nq) if rows is None else np.asarray(rows, dtype=np.int64)
    r = len(rows)
    o = np.zeros((b_, hq_, r, d))
    lse = np.full((b_, hq_, r), -np.inf)
    step = max(1, _CHUNK_ELEMS // max(nk, 1))
    for b in range(b_):
        lk = _kv_len_of(kv_lens, b, nk)
        for h in range(hq_):
            # keys at positions >= lk do not exist: never touch their memory
            kh, vh = k[b, h // g, :lk], v[b, h // g, :lk]
            for c0 in range(0, r, step):
                rr = rows[c0:c0 + step]
                s = scale * (q[b, h, rr] @ kh.T)
                p, l_ = _softmax_rows(s, visible_mask(rr, nq, lk, lk, causal))
                o[b, h, c0:c0 + step] = p @ vh
                lse[b, h, c0:c0 + step] = l_
    return o, lse


def attn_bwd(q, k, v, do, scale: Optional[float] = None, causal: bool = False,
             kv_lens: Optional[Sequence[int]] = None):
    """Gradients of L = sum(dO * O) with respect to Q, K and V.

    The chain rule through O = P V, P = softmax(S), S = scale * Q K^T; the
    self-test page (section D) asks for these relations without writing them
    out, so they are stated here:

        dV   = P^T dO
        dP   = dO V^T
        Di   = sum_d dO_id O_id          (equals sum_j P_ij dP_ij)
        dS   = P * (dP - Di)
        dQ   = scale * dS K
        dK   = scale * dS^T Q

    GQA: each KV head's gradient is the sum over the query heads that read it.
    Unlike the GPU backward, this keeps the full P from its own forward (it is
    the materialising baseline, not a recompute).

    Returns (dq, dk, dv, o, lse, delta) in float64.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    b_, hq_, nq, d = q.shape
    _, hkv, nk, _ = k.shape
    g = hq_ // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    o = np.zeros_like(q)
    lse = np.full((b_, hq_, nq), -np.inf)
    delta = np.zeros((b_, hq_, nq))
    rows_all = np.arange(nq)
    step = max(1, _CHUNK_ELEMS // max(nk, 1))
    for b in range(b_):
        lk = _kv_len_of(kv_lens, b, nk)
        for h in range(hq_):
            kh, vh = k[b, h // g, :lk], v[b, h // g, :lk]
            for c0 in range(0, nq, step):
                rr = rows_all[c0:c0 + step]
                s = scale * (q[b, h, rr] @ kh.T)
                p, l_ = _softmax_rows(s, visible_mask(rr, nq, lk, lk, causal))
                oh = p @ vh
                doh = do[b, h, rr]
                dv[b, h // g, :lk] += p.T @ doh
                dp = doh @ vh.T
                di = np.sum(doh * oh, axis=-1)
                ds = p * (dp - di[:, None])
                dq[b, h, rr] = scale * (ds @ kh)
                dk[b, h // g, :lk] += scale * (ds.T @ q[b, h, rr])
                o[b, h, rr] = oh
                lse[b, h, rr] = l_
                delta[b, h, rr] = di
    return dq, dk, dv, o, lse, delta


def attn_bwd_dq_rows(q, k, v, do, rows: Sequence[int], scale: Optional[float] = None,
                     causal: bool = False, kv_lens: Optional[Sequence[int]] = None) -> np.ndarray:
    """dQ of the query rows in ``rows`` only, by the relations of ``attn_bwd``.

    A row's dQ needs its own rows of S, P, O and dP and nothing from the other
    query rows, so sampled rows of a large problem are computed exactly without
    the rest.  Returns dq [B, Hq, len(rows), D] in float64.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    b_, hq_, nq, d = q.shape
    _, hkv, nk, _ = k.shape
    g = hq_ // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rr = np.asarray(rows, dtype=np.int64)
    dq = np.zeros((b_, hq_, len(rr), d))
    for b in range(b_):
        lk = _kv_len_of(kv_lens, b, nk)
        for h in range(hq_):
            kh, vh = k[b, h // g, :lk], v[b, h // g, :lk]
            s = scale * (q[b, h, rr] @ kh.T)
            p, _ = _softmax_rows(s, visible_mask(rr, nq, lk, lk, causal))
            doh = do[b, h, rr]
            di = np.sum(doh * (p @ vh), axis=-1)
            ds = p * (doh @ vh.T - di[:, None])
            dq[b, h] = scale * (ds @ kh)
    return dq


def attn_bwd_dkdv_rows(q, k, v, do, key_rows: Sequence[int], scale: Optional[float] = None,
                       causal: bool = False, kv_lens: Optional[Sequence[int]] = None):
    """dK and dV of the key rows in ``key_rows`` only, by the relations of ``attn_bwd``.

    Key j's gradients are sums over the query rows i that see it, over every query
    head of its GQA group:

        dV_j = sum_i P_ij dO_i,      dK_j = scale * sum_i dS_ij Q_i,
        dS_ij = P_ij (dP_ij - D_i),  dP_ij = dO_i . V_j,  D_i = rowsum(dO_i * O_i).

    P_ij and D_i depend on the whole row i (its normaliser and its O_i), so every
    query row that sees at least one sampled key is formed in full, exactly as in
    ``attn_bwd``; only the sampled key columns are accumulated.  Rows that see none of
    the sampled keys contribute nothing and are skipped.  Keys at or past kv_len do
    not exist and get zero gradients.  Returns dk, dv [B, Hkv, len(key_rows), D] in
    float64.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    b_, hq_, nq, d = q.shape
    _, hkv, nk, _ = k.shape
    g = hq_ // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    kr = np.asarray(key_rows, dtype=np.int64)
    dk = np.zeros((b_, hkv, len(kr), d))
    dv = np.zeros((b_, hkv, len(kr), d))
    rows_all = np.arange(nq)
    step = max(1, _CHUNK_ELEMS // max(nk, 1))
    for b in range(b_):
        lk = _kv_len_of(kv_lens, b, nk)
        sel = kr < lk                      # sampled keys that exist
        if not sel.any():
            continue
        ks = kr[sel]
        for h in range(hq_):
            kh, vh = k[b, h // g, :lk], v[b, h // g, :lk]
            for c0 in range(0, nq, step):
                rr = rows_all[c0:c0 + step]
                vis = visible_mask(rr, nq, lk, lk, causal)
                if not vis[:, ks].any():   # no row of the chunk sees a sampled key
                    continue
                s = scale * (q[b, h, rr] @ kh.T)
                p, _ = _softmax_rows(s, vis)
                doh = do[b, h, rr]
                di = np.sum(doh * (p @ vh), axis=-1)
                pj = p[:, ks]
                dsj = pj * (doh @ vh[ks].T - di[:, None])
                dv[b, h // g, sel] += pj.T @ doh
                dk[b, h // g, sel] += scale * (dsj.T @ q[b, h, rr])
    return dk, dv


def attn_decode(q, k_cache, v_cache, seq_lens: Sequence[int],
                scale: Optional[float] = None, seqs: Optional[Sequence[int]] = None):
    """One-token decode over a variable-length KV cache, by the plain definition.

    q [Bs, Hq, D]; k_cache, v_cache [Bs, Hkv, Lmax, D]; seq_lens [Bs].  The new
    token sees every valid cached key (keys >= seq_lens[s] do not exist).  No
    split: the split-and-merge form is checked separately against this.
    Returns O [S, Hq, D], LSE [S, Hq] for the sequences in ``seqs`` (all by
    default).  Self-test page section F (KV-cache decode); interview answer,
    追问 2.
    """
    q = _f64(q)
    bs, hq_, d = q.shape
    hkv = k_cache.shape[1]
    g = hq_ // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    seqs = list(range(bs)) if seqs is None else list(seqs)
    o = np.zeros((len(seqs), hq_, d))
    lse = np.full((len(seqs), hq_), -np.inf)
    for n, s_ in enumerate(seqs):
        ls = int(seq_lens[s_])
        if ls <= 0:
            continue
        for h in range(hq_):
            kh = _f64(k_cache[s_, h // g, :ls])
            vh = _f64(v_cache[s_, h // g, :ls])
            sc = scale * (kh @ q[s_, h])
            p, l_ = _softmax_rows(sc[None, :], np.ones((1, ls), dtype=bool))
            o[n, h] = (p @ vh)[0]
            lse[n, h] = l_[0]
    return o, lse


def attn_fwd_varlen(q, k, v, cu_q: Sequence[int], cu_k: Sequence[int],
                    scale: Optional[float] = None, causal: bool = False
                    ) -> Tuple[np.ndarray, np.ndarray]:
    """Attention over a packed batch of variable-length sequences (no padding).

    q [Tq, Hq, D]; k, v [Tk, Hkv, D]; cu_q, cu_k [B+1] non-decreasing offsets
    (cu[0] = 0, cu[B] = T).  Sequence b attends with its own rows only; each
    sequence is the plain forward of ``attn_fwd`` on its slice (self-test page,
    section C: padding and variable-length sequences).  Returns O [Tq, Hq, D] and
    LSE [Hq, Tq].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    tq, hq_, d = q.shape
    o = np.zeros((tq, hq_, d))
    lse = np.full((hq_, tq), -np.inf)
    for b in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        if q1 <= q0:
            continue
        qb = q[q0:q1].transpose(1, 0, 2)[None]
        kb = k[k0:k1].transpose(1, 0, 2)[None]
        vb = v[k0:k1].transpose(1, 0, 2)[None]
        ob, lb = attn_fwd(qb, kb, vb, scale, causal)
        o[q0:q1] = ob[0].transpose(1, 0, 2)
        lse[:, q0:q1] = lb[0]
    return o, lse


def attn_decode_paged(q, k_pages, v_pages, block_table, seq_lens: Sequence[int],
                      scale: Optional[float] = None, seqs: Optional[Sequence[int]] = None):
    """One-token decode over a paged KV cache.

    k_pages, v_pages [P, Hkv, page_size, D]; block_table [Bs, W] page ids.  The
    cached keys of sequence s are gathered in position order -- position t is
    row t % page_size of page block_table[s][t // page_size] -- and the plain
    decode of ``attn_decode`` is taken over them (self-test page, section F, why a
    paged KV cache still needs its own decode path; interview answer, 追问 2, the
    blocked computation reading paged KV blocks directly).
    """
    k_pages, v_pages = np.asarray(k_pages), np.asarray(v_pages)
    q = _f64(q)
    ps = k_pages.shape[2]
    bs, hq_, d = q.shape
    hkv = k_pages.shape[1]
    seqs = list(range(bs)) if seqs is None else list(seqs)
    o = np.zeros((len(seqs), hq_, d))
    lse = np.full((len(seqs), hq_), -np.inf)
    for n_, s_ in enumerate(seqs):
        ls = max(int(seq_lens[s_]), 0)
        kd = np.zeros((1, hkv, ls, d))
        vd = np.zeros((1, hkv, ls, d))
        for j in range((ls + ps - 1) // ps):  # positions j*ps .. of page block_table[s][j]
            page = int(block_table[s_][j])
            n = min(ps, ls - j * ps)
            kd[0, :, j * ps:j * ps + n] = k_pages[page, :, :n]
            vd[0, :, j * ps:j * ps + n] = v_pages[page, :, :n]
        o_s, l_s = attn_decode(q[s_:s_ + 1], kd, vd, [ls], scale)
        o[n_], lse[n_] = o_s[0], l_s[0]
    return o, lse


def online_softmax_attention(q, k, v, scale: float, block_edges: Sequence[int],
                             vis: Optional[np.ndarray] = None):
    """The tiled forward recurrence for one head, in fp64, block by block.

    q [Nq, D], k, v [Nk, D]; ``block_edges`` are the key-block boundaries
    (0 = e0 < e1 < ... = Nk, any sizes).  Per block, following the online
    softmax of the V2/V3 article (section V2算法优化) and the study card
    (section 三), with the l update read as the sum over the block (the article's
    printed l update drops the block sum; the study card and the article's demo
    keep it):

        m_new = max(m, rowmax S_blk)
        alpha = exp(m - m_new)
        l     = alpha * l + rowsum exp(S_blk - m_new)
        acc   = alpha * acc + exp(S_blk - m_new) V_blk

    and after the last block O = acc / l once, LSE = m + ln l.  A row whose
    running maximum is still -inf (nothing visible yet) keeps alpha = 0 and adds
    nothing.  Used only to pin the one-shot oracle (the two must agree).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    nq, d = q.shape
    nk = k.shape[0]
    if vis is None:
        vis = np.ones((nq, nk), dtype=bool)
    m = np.full(nq, -np.inf)
    l = np.zeros(nq)
    acc = np.zeros((nq, d))
    for b0, b1 in zip(block_edges[:-1], block_edges[1:]):
        s = scale * (q @ k[b0:b1].T)
        s = np.where(vis[:, b0:b1], s, -np.inf)
        m_new = np.maximum(m, np.max(s, axis=1)) if b1 > b0 else m
        ref = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.exp(m - ref)          # 0 while m is -inf
        pb = np.exp(s - ref[:, None])    # 0 on masked entries
        l = alpha * l + pb.sum(axis=1)
        acc = alpha[:, None] * acc + pb @ v[b0:b1]
        m = m_new
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where(l[:, None] > 0, acc / np.where(l > 0, l, 1.0)[:, None], 0.0)
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def decode_split_partials(q, k, v, scale: float, split_len: int):
    """Split-KV partials for one (sequence, head): q [D], k, v [L, D].

    Chunk c covers keys [c*split_len, min((c+1)*split_len, L)).  Each chunk's
    attention is computed by the plain definition, giving (O_c, LSE_c) as if the
    chunk were the whole sequence (interview answer, 追问 2: each chunk is
    attended independently, then merged).  Returns O [C, D], LSE [C].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    L = k.shape[0]
    n = (L + split_len - 1) // split_len
    o = np.zeros((n, q.shape[0]))
    lse = np.full(n, -np.inf)
    for c in range(n):
        kk = k[c * split_len:min((c + 1) * split_len, L)]
        vv = v[c * split_len:min((c + 1) * split_len, L)]
        s = scale * (kk @ q)
        p, l_ = _softmax_rows(s[None, :], np.ones((1, len(kk)), dtype=bool))
        o[c] = (p @ vv)[0]
        lse[c] = l_[0]
    return o, lse


def merge_partials(o_parts, lse_parts):
    """Merge per-chunk (O_c, LSE_c) into the whole-sequence (O, LSE).

    M = max_c LSE_c, w_c = exp(LSE_c - M), O = sum_c w_c O_c / sum_c w_c,
    LSE = M + ln sum_c w_c: the online-softmax update applied once per chunk,
    each chunk's normalised output weighted by its share of the total exponent
    sum (study card section 三, two-block derivation; interview answer 追问 2).
    With no chunk (or all LSE_c = -inf) the result is O = 0, LSE = -inf.
    """
    o_parts, lse_parts = _f64(o_parts), _f64(lse_parts)
    if lse_parts.size == 0 or not np.isfinite(np.max(lse_parts)):
        return np.zeros(o_parts.shape[1:]), -np.inf
    mx = np.max(lse_parts)
    w = np.exp(lse_parts - mx)
    tot = np.sum(w)
    return (w[:, None] * o_parts).sum(axis=0) / tot, mx + math.log(tot)


def materialised_score_bytes(n: int, itemsize: int, heads: int = 1) -> int:
    """Bytes of one materialised N x N score matrix per head (standard attention).

    The study card's section 三 sizes it for L = 8192 in fp16 (64 Mi elements,
    128 MiB per head).
    """
    return n * n * itemsize * heads
