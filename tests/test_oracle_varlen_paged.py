"""Pins of the oracle's packed variable-length forward and paged-cache decode.

Both are checked against scalar brute force written from the definitions (pure
Python loops, math.fsum), on tiny inputs that include empty sequences, rows with
no visible key, GQA and ragged page tails; planted mistakes in copies of the
oracle functions must be caught by the same brute force.
"""

import math

import numpy as np
import pytest

import oracle
from io_aware_tiled_10_amd import inputs


def brute_varlen(q, k, v, cu_q, cu_k, scale, causal):
    tq, hq, d = q.shape
    g = hq // k.shape[1]
    o = np.zeros((tq, hq, d))
    lse = np.full((hq, tq), -math.inf)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        nq, nk = q1 - q0, k1 - k0
        for h in range(hq):
            for i in range(nq):
                keys = [j for j in range(nk) if (not causal) or j <= i + nk - nq]
                if not keys:
                    continue
                s = {j: scale * math.fsum(float(q[q0 + i, h, t]) * float(k[k0 + j, h // g, t])
                                          for t in range(d)) for j in keys}
                m = max(s.values())
                e = {j: math.exp(s[j] - m) for j in keys}
                l = math.fsum(e.values())
                for t in range(d):
                    o[q0 + i, h, t] = math.fsum(e[j] * float(v[k0 + j, h // g, t]) for j in keys) / l
                lse[h, q0 + i] = m + math.log(l)
    return o, lse


def brute_paged(q, k_pages, v_pages, table, lens, scale):
    bs, hq, d = q.shape
    g = hq // k_pages.shape[1]
    ps = k_pages.shape[2]
    o = np.zeros((bs, hq, d))
    lse = np.full((bs, hq), -math.inf)
    for s in range(bs):
        L = int(lens[s])
        if L == 0:
            continue
        for h in range(hq):
            rows = [(int(table[s][t // ps]), t % ps) for t in range(L)]
            sc = [scale * math.fsum(float(q[s, h, c]) * float(k_pages[pg, h // g, r, c]) for c in range(d))
                  for pg, r in rows]
            m = max(sc)
            e = [math.exp(x - m) for x in sc]
            l = math.fsum(e)
            for c in range(d):
                o[s, h, c] = math.fsum(e[n] * float(v_pages[pg, h // g, r, c]) for n, (pg, r) in enumerate(rows)) / l
            lse[s, h] = m + math.log(l)
    return o, lse


VARLEN = [
    # lens_q, lens_k, Hq, Hkv, D, causal
    ([3, 5, 1], [3, 5, 1], 2, 2, 4, True),
    ([3, 5, 1], [6, 2, 4], 4, 2, 4, False),
    ([4, 0, 6, 2], [2, 3, 6, 0], 2, 1, 3, True),   # empty q, empty k, Nq > Nk
    ([1, 7], [9, 7], 3, 1, 5, True),
]


@pytest.mark.parametrize("case", VARLEN)
def test_varlen_matches_scalar_brute_force(case):
    lq, lk, hq, hkv, d, causal = case
    x = inputs.varlen_inputs(lq, lk, hq, hkv, d, "fp32", seed=1)
    scale = 0.7
    o, lse = oracle.attn_fwd_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, scale, causal)
    ob, lb = brute_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, scale, causal)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-12)


def test_varlen_sequences_do_not_see_each_other():
    x = inputs.varlen_inputs([5, 4, 6], [5, 4, 6], 2, 1, 8, "fp32", seed=2)
    o1, l1 = oracle.attn_fwd_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, None, False)
    k2, v2 = x.k.copy(), x.v.copy()
    k2[5:9] += 3.0
    v2[5:9] -= 1.0
    o2, l2 = oracle.attn_fwd_varlen(x.q, k2, v2, x.cu_q, x.cu_k, None, False)
    for r in (slice(0, 5), slice(9, 15)):
        assert np.array_equal(o1[r], o2[r]) and np.array_equal(l1[:, r], l2[:, r])
    assert not np.allclose(o1[5:9], o2[5:9])


def test_varlen_single_sequence_is_the_padded_forward():
    x = inputs.varlen_inputs([7], [9], 4, 2, 8, "fp32", seed=3)
    o, lse = oracle.attn_fwd_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, None, True)
    # the same data in [B, H, N, D] with trailing padding keys masked by kv_lens
    kpad = np.concatenate([x.k, np.full((3, 2, 8), np.nan, np.float32)])
    vpad = np.concatenate([x.v, np.full((3, 2, 8), np.nan, np.float32)])
    od, ld = oracle.attn_fwd(x.q.transpose(1, 0, 2)[None], kpad.transpose(1, 0, 2)[None],
                             vpad.transpose(1, 0, 2)[None], None, True, [9])
    np.testing.assert_array_equal(o, od[0].transpose(1, 0, 2))
    np.testing.assert_array_equal(lse, ld[0])


PAGED = [
    # Bs, Hq, Hkv, D, len_lo, len_hi, page
    (3, 2, 1, 4, 1, 9, 4),
    (4, 4, 2, 3, 5, 12, 3),
    (2, 2, 2, 5, 8, 8, 8),    # lengths exactly one page
]


@pytest.mark.parametrize("case", PAGED)
def test_paged_decode_matches_scalar_brute_force(case):
    bs, hq, hkv, d, lo, hi, ps = case
    dec = inputs.decode_inputs(bs, hq, hkv, d, lo, hi, seed=4)
    pc = inputs.paged_cache(dec, ps, seed=5, spare_pages=3)
    o, lse = oracle.attn_decode_paged(dec.q, pc.k_pages, pc.v_pages, pc.block_table, dec.seq_lens, 0.5)
    ob, lb = brute_paged(dec.q, pc.k_pages, pc.v_pages, pc.block_table, dec.seq_lens, 0.5)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-12)


def test_paged_decode_equals_contiguous_decode_and_ignores_page_order():
    dec = inputs.decode_inputs(3, 4, 2, 8, 1, 40, seed=6)
    kc, vc = dec.dense_cache()
    od, ld = oracle.attn_decode(dec.q, kc, vc, dec.seq_lens)
    for seed, ps in ((0, 16), (1, 16), (2, 5)):
        pc = inputs.paged_cache(dec, ps, seed=seed, spare_pages=seed)
        o, lse = oracle.attn_decode_paged(dec.q, pc.k_pages, pc.v_pages, pc.block_table, dec.seq_lens)
        np.testing.assert_array_equal(o, od)
        np.testing.assert_array_equal(lse, ld)


# ---- planted mistakes (copies of the oracle functions with one error each)

def _mut_varlen_global_causal(q, k, v, cu_q, cu_k, scale, causal):
    # causal alignment taken on the packed index instead of within each sequence
    tq, hq, d = q.shape
    qb, kb, vb = q.transpose(1, 0, 2)[None], k.transpose(1, 0, 2)[None], v.transpose(1, 0, 2)[None]
    o = np.zeros((tq, hq, d))
    lse = np.full((hq, tq), -np.inf)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if q1 <= q0:
            continue
        ob, lb = oracle.attn_fwd(qb[:, :, :q1], kb[:, :, :k1], vb[:, :, :k1], scale, causal)
        o[q0:q1] = ob[0, :, q0:q1].transpose(1, 0, 2)
        lse[:, q0:q1] = lb[0, :, q0:q1]
    return o, lse


def _mut_paged_row_index(q, k_pages, v_pages, table, lens, scale):
    # page row taken as t // page_size instead of t % page_size
    ps = k_pages.shape[2]
    kd = np.zeros((q.shape[0], k_pages.shape[1], max(lens), k_pages.shape[3]))
    vd = np.zeros_like(kd)
    for s in range(q.shape[0]):
        for t in range(int(lens[s])):
            kd[s, :, t] = k_pages[int(table[s][t // ps]), :, min(t // ps, ps - 1)]
            vd[s, :, t] = v_pages[int(table[s][t // ps]), :, min(t // ps, ps - 1)]
    return oracle.attn_decode(q, kd, vd, lens, scale)


def test_planted_varlen_mistake_is_caught():
    x = inputs.varlen_inputs([3, 5, 1], [3, 5, 1], 2, 2, 4, "fp32", seed=1)
    ob, _ = brute_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, 0.7, True)
    om, _ = _mut_varlen_global_causal(x.q, x.k, x.v, x.cu_q, x.cu_k, 0.7, True)
    assert np.abs(om - ob).max() > 1e-3


def test_planted_paged_mistake_is_caught():
    dec = inputs.decode_inputs(3, 2, 1, 4, 5, 9, seed=4)
    pc = inputs.paged_cache(dec, 4, seed=5, pad_value=0.0)
    ob, _ = brute_paged(dec.q, pc.k_pages, pc.v_pages, pc.block_table, dec.seq_lens, 0.5)
    om, _ = _mut_paged_row_index(dec.q, pc.k_pages, pc.v_pages, pc.block_table, dec.seq_lens, 0.5)
    assert np.abs(om - ob).max() > 1e-3
