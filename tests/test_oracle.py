"""Pins of the fp64 oracle against facts that do not depend on the oracle.

Each test pins the oracle to something other than itself: a scalar brute force
written with Python loops and math.fsum, hand-derived closed forms, invariants
of softmax, the online recurrence of the pages run block by block, and central
finite differences for the backward.  A plausible mistake in the oracle (a
dropped term, a wrong sign or index, a transposed operand, a wrong mask
alignment, a wrong GQA mapping) fails at least one of them; the mutation tests
at the end plant such mistakes in copies of the oracle to show it.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention as ora

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


# --------------------------------------------------------------------------
# scalar brute force (textbook definition, no numpy linear algebra)
# --------------------------------------------------------------------------

def brute_fwd(q, k, v, scale, causal, kv_lens=None):
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    o = np.zeros((B, Hq, Nq, D))
    lse = np.full((B, Hq, Nq), -math.inf)
    for b in range(B):
        lk = Nk if kv_lens is None else min(int(kv_lens[b]), Nk)
        for h in range(Hq):
            g = h // G
            for i in range(Nq):
                keys = [j for j in range(lk) if (not causal) or j <= i + lk - Nq]
                if not keys:
                    continue
                s = {j: scale * math.fsum(float(q[b, h, i, t]) * float(k[b, g, j, t]) for t in range(D))
                     for j in keys}
                m = max(s.values())
                e = {j: math.exp(s[j] - m) for j in keys}
                l = math.fsum(e.values())
                for t in range(D):
                    o[b, h, i, t] = math.fsum(e[j] * float(v[b, g, j, t]) for j in keys) / l
                lse[b, h, i] = m + math.log(l)
    return o, lse


def _rand(rng, *shape):
    return rng.standard_normal(shape)


TINY_CASES = [
    # B, Hq, Hkv, Nq, Nk, D, causal, kv_lens
    (1, 1, 1, 5, 5, 3, False, None),
    (1, 1, 1, 5, 5, 3, True, None),
    (2, 4, 2, 3, 6, 4, False, None),
    (2, 4, 2, 3, 6, 4, True, None),
    (1, 3, 1, 6, 4, 2, True, None),        # Nq > Nk: first rows see nothing
    (2, 2, 1, 4, 6, 3, False, [6, 2]),
    (2, 2, 2, 4, 6, 3, True, [5, 3]),
    (1, 2, 2, 1, 5, 4, True, None),        # one-token decode shape
]


@pytest.mark.parametrize("case", TINY_CASES)
def test_forward_matches_scalar_brute_force(case):
    B, Hq, Hkv, Nq, Nk, D, causal, kv_lens = case
    rng = np.random.default_rng(1234)
    q, k, v = _rand(rng, B, Hq, Nq, D), _rand(rng, B, Hkv, Nk, D), _rand(rng, B, Hkv, Nk, D)
    scale = 0.7
    o, lse = oracle.attn_fwd(q, k, v, scale, causal, kv_lens)
    ob, lseb = brute_fwd(q, k, v, scale, causal, kv_lens)
    assert np.array_equal(np.isinf(lse), np.isinf(lseb))
    fin = np.isfinite(lseb)
    np.testing.assert_allclose(lse[fin], lseb[fin], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(o, ob, rtol=1e-13, atol=1e-14)


def test_row_subset_matches_full():
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 1, 2, 9, 4), _rand(rng, 1, 1, 12, 4), _rand(rng, 1, 1, 12, 4)
    o, lse = oracle.attn_fwd(q, k, v, 0.5, True)
    rows = [0, 4, 8]
    o2, lse2 = oracle.attn_fwd(q, k, v, 0.5, True, rows=rows)
    np.testing.assert_array_equal(o2, o[:, :, rows])
    np.testing.assert_array_equal(lse2, lse[:, :, rows])


# --------------------------------------------------------------------------
# worked examples with closed-form answers (tests/golden)
# --------------------------------------------------------------------------

def _ev(expr):
    env = {"ln2": math.log(2), "ln3": math.log(3), "log": math.log, "exp": math.exp}
    return float(eval(expr, {"__builtins__": {}}, env))


def _arr(nested):
    if isinstance(nested, str):
        return _ev(nested)
    return [_arr(x) for x in nested]


@pytest.mark.parametrize("idx", range(3))
def test_golden_worked_examples(idx):
    case = json.load(open(GOLDEN))["cases"][idx]
    q = np.array(_arr(case["q"]))[None]   # [1, Hq, Nq, D]
    k = np.array(_arr(case["k"]))[None, None] if np.array(_arr(case["k"])).ndim == 2 else np.array(_arr(case["k"]))[None]
    v = np.array(_arr(case["v"]))[None, None] if np.array(_arr(case["v"])).ndim == 2 else np.array(_arr(case["v"]))[None]
    o, lse = oracle.attn_fwd(q, k, v, case["scale"], case["causal"])
    np.testing.assert_allclose(o[0], np.array(_arr(case["o"])), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0], np.array(_arr(case["lse"])), rtol=0, atol=1e-14)


def test_golden_two_block_online_update():
    g = json.load(open(GOLDEN))["two_block_online_update"]
    x = np.array(g["scores"])
    # the scores as S = q k^T with q = 1 and k_j = x_j (D = 1, scale = 1)
    q = np.ones((1, 1))
    k = x[:, None]
    v = np.eye(len(x))
    o, lse = ora.online_softmax_attention(q, k, v, 1.0, [0, g["split"], len(x)])
    m, l = _ev(g["m"]), _ev(g["l"])
    assert abs(lse[0] - (m + math.log(l))) < 1e-15
    np.testing.assert_allclose(o[0], np.exp(x - m) / l, rtol=1e-15, atol=1e-16)


def test_golden_materialised_score_bytes():
    g = json.load(open(GOLDEN))["materialised_scores"]
    assert oracle.materialised_score_bytes(g["n"], g["itemsize"]) == g["bytes"] == 128 * 2**20


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_identity_values_give_rows_of_P_that_sum_to_one(causal):
    # With V = I (D = Nk) the output row is the probability row itself.
    rng = np.random.default_rng(5)
    n = 7
    q, k = _rand(rng, 1, 1, n, n), _rand(rng, 1, 1, n, n)
    v = np.eye(n)[None, None]
    o, _ = oracle.attn_fwd(q, k, v, 0.4, causal)
    p = o[0, 0]
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    if causal:
        assert np.all(np.triu(p, 1) == 0)


@pytest.mark.parametrize("causal", [False, True])
def test_shift_invariance(causal):
    # K -> K + 1 w^T adds scale * q_i . w to every score of row i: O unchanged,
    # LSE_i shifted by exactly that amount (study card section 四 ①).
    rng = np.random.default_rng(6)
    q, k, v = _rand(rng, 2, 2, 6, 5), _rand(rng, 2, 1, 8, 5), _rand(rng, 2, 1, 8, 5)
    w = _rand(rng, 5)
    scale = 0.8
    o1, l1 = oracle.attn_fwd(q, k, v, scale, causal)
    o2, l2 = oracle.attn_fwd(q, k + w, v, scale, causal)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1 + scale * (q @ w), rtol=1e-12, atol=1e-12)


def test_constant_values_give_that_value():
    rng = np.random.default_rng(7)
    q, k = _rand(rng, 1, 3, 5, 4), _rand(rng, 1, 3, 9, 4)
    c = _rand(rng, 4)
    v = np.broadcast_to(c, (1, 3, 9, 4)).copy()
    for causal in (False, True):
        o, lse = oracle.attn_fwd(q, k, v, 0.5, causal)
        np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=1e-13, atol=1e-14)
        _, lse2 = oracle.attn_fwd(q, k, 2 * v + 1, 0.5, causal)
        np.testing.assert_array_equal(lse, lse2)


def test_zero_queries_give_uniform_weights():
    rng = np.random.default_rng(8)
    n, d = 6, 3
    k, v = _rand(rng, 1, 1, n, d), _rand(rng, 1, 1, n, d)
    q = np.zeros((1, 1, n, d))
    o, lse = oracle.attn_fwd(q, k, v, 1.0, False)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0].mean(0), (n, d)), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(n), atol=1e-14)
    o, lse = oracle.attn_fwd(q, k, v, 1.0, True)
    prefix = np.cumsum(v[0, 0], axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(o[0, 0], prefix, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, n + 1)), atol=1e-14)


def test_causal_row_zero_and_single_key():
    rng = np.random.default_rng(9)
    q, k, v = _rand(rng, 1, 1, 4, 3), _rand(rng, 1, 1, 4, 3), _rand(rng, 1, 1, 4, 3)
    o, lse = oracle.attn_fwd(q, k, v, 0.3, True)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 0], atol=1e-15)
    assert abs(lse[0, 0, 0] - 0.3 * q[0, 0, 0] @ k[0, 0, 0]) < 1e-15
    o, lse = oracle.attn_fwd(q, k[:, :, :1], v[:, :, :1], 0.3, False)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0, 0], (4, 3)), atol=1e-15)


def test_fully_masked_rows_are_zero_with_neg_inf_lse():
    rng = np.random.default_rng(10)
    q, k, v = _rand(rng, 2, 1, 3, 2), _rand(rng, 2, 1, 4, 2), _rand(rng, 2, 1, 4, 2)
    o, lse = oracle.attn_fwd(q, k, v, 1.0, False, kv_lens=[0, 4])
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(lse[1]))


def test_padding_memory_never_influences_result():
    rng = np.random.default_rng(11)
    q, k, v = _rand(rng, 1, 2, 4, 3), _rand(rng, 1, 1, 7, 3), _rand(rng, 1, 1, 7, 3)
    o1, l1 = oracle.attn_fwd(q, k, v, 0.6, True, kv_lens=[5])
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 5:] = np.nan
    v2[:, :, 5:] = np.nan
    o2, l2 = oracle.attn_fwd(q, k2, v2, 0.6, True, kv_lens=[5])
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    o3, l3 = oracle.attn_fwd(q, k[:, :, :5], v[:, :, :5], 0.6, True)
    np.testing.assert_allclose(o1, o3, rtol=1e-14, atol=1e-15)


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(12)
    B, Hq, Hkv, N, D = 2, 6, 2, 5, 3
    q, k, v = _rand(rng, B, Hq, N, D), _rand(rng, B, Hkv, N, D), _rand(rng, B, Hkv, N, D)
    G = Hq // Hkv
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    for causal in (False, True):
        o1, l1 = oracle.attn_fwd(q, k, v, 0.5, causal)
        o2, l2 = oracle.attn_fwd(q, kr, vr, 0.5, causal)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


# --------------------------------------------------------------------------
# online recurrence == one-shot (V2/V3 article, V2 section; study card 三)
# --------------------------------------------------------------------------

def _edges(rng, n):
    cuts = sorted(set(rng.integers(1, n, size=rng.integers(0, n)).tolist()))
    return [0] + cuts + [n]


@pytest.mark.parametrize("seed", range(6))
def test_online_recurrence_equals_one_shot(seed):
    rng = np.random.default_rng(100 + seed)
    nq, nk, d = 5, 11, 4
    q, k, v = _rand(rng, nq, d), _rand(rng, nk, d), 3 * _rand(rng, nk, d)
    scale = 1.3
    causal = bool(seed % 2)
    vis = ora.visible_mask(np.arange(nq), nq, nk, nk, causal)
    o_ref, l_ref = oracle.attn_fwd(q[None, None], k[None, None], v[None, None], scale, causal)
    for edges in (_edges(rng, nk), list(range(nk + 1)), [0, nk]):
        o, l = ora.online_softmax_attention(q, k, v, scale, edges, vis)
        np.testing.assert_allclose(o, o_ref[0, 0], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(l, l_ref[0, 0], rtol=1e-13, atol=1e-13)


def test_online_recurrence_with_fully_masked_leading_block():
    rng = np.random.default_rng(13)
    nq, nk, d = 3, 8, 2
    q, k, v = _rand(rng, nq, d), _rand(rng, nk, d), _rand(rng, nk, d)
    vis = np.ones((nq, nk), dtype=bool)
    vis[:, :4] = False
    o, l = ora.online_softmax_attention(q, k, v, 1.0, [0, 4, 8], vis)
    o_ref, l_ref = oracle.attn_fwd(q[None, None], k[None, None, 4:], v[None, None, 4:], 1.0, False)
    np.testing.assert_allclose(o, o_ref[0, 0], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(l, l_ref[0, 0], rtol=1e-14, atol=1e-14)


def test_online_recurrence_demo_shape():
    # The article's demo self-check: B2 H4 N256 d32, blocks of 64, seed 0.
    rng = np.random.default_rng(0)
    q, k, v = (_rand(rng, 2, 4, 256, 32) for _ in range(3))
    o_ref, l_ref = oracle.attn_fwd(q, k, v)
    worst = 0.0
    for b in range(2):
        for h in range(4):
            o, _ = ora.online_softmax_attention(q[b, h], k[b, h], v[b, h], 32 ** -0.5,
                                                list(range(0, 257, 64)))
            worst = max(worst, float(np.abs(o - o_ref[b, h]).max()))
    assert worst < 1e-12


# --------------------------------------------------------------------------
# backward: finite differences and identities
# --------------------------------------------------------------------------

BWD_CASES = [
    (1, 2, 1, 6, 6, 4, False, None),
    (1, 2, 1, 6, 6, 4, True, None),
    (1, 2, 2, 5, 8, 4, True, None),
    (2, 2, 1, 5, 7, 3, False, [7, 4]),
    (1, 2, 1, 7, 5, 3, True, None),     # Nq > Nk: leading rows fully masked
]


@pytest.mark.parametrize("case", BWD_CASES)
def test_backward_matches_central_finite_differences(case):
    B, Hq, Hkv, Nq, Nk, D, causal, kv_lens = case
    rng = np.random.default_rng(21)
    q, k, v = _rand(rng, B, Hq, Nq, D), _rand(rng, B, Hkv, Nk, D), _rand(rng, B, Hkv, Nk, D)
    do = _rand(rng, B, Hq, Nq, D)
    scale = 0.9
    dq, dk, dv, *_ = oracle.attn_bwd(q, k, v, do, scale, causal, kv_lens)

    def loss(q_, k_, v_):
        o, _ = oracle.attn_fwd(q_, k_, v_, scale, causal, kv_lens)
        return float(np.sum(do * o))

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (loss(**{a + "_": b for a, b in args_p.items()})
                        - loss(**{a + "_": b for a, b in args_m.items()})) / (2 * h)
        err = np.abs(num - g).max() / max(np.abs(g).max(), 1e-30)
        assert err < 1e-6, (name, err)


def test_backward_identities():
    rng = np.random.default_rng(22)
    B, Hq, Hkv, N, D = 2, 4, 2, 9, 5
    q, k, v, do = (_rand(rng, B, H, N, D) for H in (Hq, Hkv, Hkv, Hq))
    G = Hq // Hkv
    for causal in (False, True):
        dq, dk, dv, o, lse, delta = oracle.attn_bwd(q, k, v, do, 0.7, causal)
        # Di = rowsum(dO * O)
        np.testing.assert_allclose(delta, np.sum(do * o, axis=-1), rtol=1e-14, atol=1e-14)
        # sum_j dK_j = 0 (shift invariance of softmax in K)
        np.testing.assert_allclose(dk.sum(axis=2), 0, atol=1e-12)
        # sum_j dV_j = sum over the group's query heads of sum_i dO_i
        grp = do.reshape(B, Hkv, G, N, D).sum(axis=(2, 3))
        np.testing.assert_allclose(dv.sum(axis=2), grp, rtol=1e-12, atol=1e-12)
        # forward part equals the forward oracle
        o2, l2 = oracle.attn_fwd(q, k, v, 0.7, causal)
        np.testing.assert_allclose(o, o2, rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(lse, l2, rtol=1e-14, atol=1e-14)


def test_backward_gqa_equals_mha_summed_over_group():
    rng = np.random.default_rng(23)
    B, Hq, Hkv, N, D = 1, 4, 2, 6, 3
    q, k, v, do = (_rand(rng, B, H, N, D) for H in (Hq, Hkv, Hkv, Hq))
    G = Hq // Hkv
    dq, dk, dv, *_ = oracle.attn_bwd(q, k, v, do, 0.5, True)
    dq2, dk2, dv2, *_ = oracle.attn_bwd(q, np.repeat(k, G, 1), np.repeat(v, G, 1), do, 0.5, True)
    np.testing.assert_allclose(dq, dq2, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(dk, dk2.reshape(B, Hkv, G, N, D).sum(2), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dv, dv2.reshape(B, Hkv, G, N, D).sum(2), rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------
# decode: split + merge == one shot; decode == forward with Nq = 1
# --------------------------------------------------------------------------

def test_decode_equals_forward_with_one_query():
    rng = np.random.default_rng(31)
    Bs, Hq, Hkv, Lmax, D = 3, 4, 2, 13, 4
    q = _rand(rng, Bs, Hq, D)
    kc, vc = _rand(rng, Bs, Hkv, Lmax, D), _rand(rng, Bs, Hkv, Lmax, D)
    lens = [13, 5, 1]
    o, lse = oracle.attn_decode(q, kc, vc, lens, 0.6)
    for causal in (False, True):
        of, lf = oracle.attn_fwd(q[:, :, None], kc, vc, 0.6, causal, kv_lens=lens)
        np.testing.assert_allclose(o, of[:, :, 0], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(lse, lf[:, :, 0], rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("L,split", [(1, 4), (7, 4), (8, 4), (23, 5), (2048, 2048), (3000, 2048)])
def test_split_merge_equals_one_shot(L, split):
    rng = np.random.default_rng(32 + L)
    D = 6
    q, k, v = _rand(rng, D), _rand(rng, L, D), _rand(rng, L, D)
    o_p, l_p = ora.decode_split_partials(q, k, v, 0.4, split)
    assert len(l_p) == -(-L // split)
    o, lse = ora.merge_partials(o_p, l_p)
    o_ref, l_ref = oracle.attn_decode(q[None, None], k[None, None], v[None, None], [L], 0.4)
    np.testing.assert_allclose(o, o_ref[0, 0], rtol=1e-13, atol=1e-14)
    assert abs(lse - l_ref[0, 0]) < 1e-12


def test_merge_of_nothing_is_zero_and_neg_inf():
    o, lse = ora.merge_partials(np.zeros((0, 3)), np.zeros(0))
    assert np.all(o == 0) and lse == -math.inf
    o, lse = oracle.attn_decode(np.ones((1, 1, 3)), np.ones((1, 1, 4, 3)), np.ones((1, 1, 4, 3)), [0])
    assert np.all(o == 0) and np.isneginf(lse).all()


# --------------------------------------------------------------------------
# planted mistakes: each corrupted copy of the oracle fails a pin above
# --------------------------------------------------------------------------

def _mut_fwd_drop_scale(q, k, v, scale, causal, kv_lens=None):
    return oracle.attn_fwd(q, k, v, 1.0, causal, kv_lens)


def _mut_fwd_top_left_causal(q, k, v, scale, causal, kv_lens=None):
    # aligns the causal diagonal to the top-left instead of the bottom-right
    B, Hq, Nq, D = q.shape
    Nk = k.shape[2]
    if not causal or Nq == Nk:
        return oracle.attn_fwd(q, k, v, scale, causal, kv_lens)
    o = np.zeros(q.shape)
    lse = np.full(q.shape[:3], -np.inf)
    for i in range(Nq):
        oo, ll = oracle.attn_fwd(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1], scale, False)
        o[:, :, i], lse[:, :, i] = oo[:, :, 0], ll[:, :, 0]
    return o, lse


def _mut_fwd_interleaved_gqa(q, k, v, scale, causal, kv_lens=None):
    Hq, Hkv = q.shape[1], k.shape[1]
    idx = [h % Hkv for h in range(Hq)]
    return oracle.attn_fwd(q, k[:, idx], v[:, idx], scale, causal, kv_lens)


@pytest.mark.parametrize("mutant", [_mut_fwd_drop_scale, _mut_fwd_top_left_causal,
                                    _mut_fwd_interleaved_gqa])
def test_planted_forward_mistakes_are_caught_by_brute_force(mutant):
    caught = False
    for case in TINY_CASES:
        B, Hq, Hkv, Nq, Nk, D, causal, kv_lens = case
        rng = np.random.default_rng(1234)
        q, k, v = _rand(rng, B, Hq, Nq, D), _rand(rng, B, Hkv, Nk, D), _rand(rng, B, Hkv, Nk, D)
        o, _ = mutant(q, k, v, 0.7, causal, kv_lens)
        ob, _ = brute_fwd(q, k, v, 0.7, causal, kv_lens)
        if not np.allclose(o, ob, rtol=1e-10, atol=1e-12):
            caught = True
            break
    assert caught


def test_planted_backward_sign_mistake_is_caught_by_finite_differences():
    rng = np.random.default_rng(24)
    q, k, v, do = (_rand(rng, 1, 1, 4, 3) for _ in range(4))
    dq, dk, dv, o, lse, delta = oracle.attn_bwd(q, k, v, do, 1.0, False)
    # corrupted dQ: dS = P * (dP + D) instead of P * (dP - D)
    s = q[0, 0] @ k[0, 0].T
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    dp = do[0, 0] @ v[0, 0].T
    dq_bad = (p * (dp + delta[0, 0][:, None])) @ k[0, 0]
    h = 1e-6
    num = np.zeros((4, 3))
    for i in range(4):
        for t in range(3):
            qp, qm = q.copy(), q.copy()
            qp[0, 0, i, t] += h
            qm[0, 0, i, t] -= h
            num[i, t] = (np.sum(do * oracle.attn_fwd(qp, k, v, 1.0)[0])
                         - np.sum(do * oracle.attn_fwd(qm, k, v, 1.0)[0])) / (2 * h)
    assert np.abs(num - dq[0, 0]).max() < 1e-7
    assert np.abs(num - dq_bad).max() > 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_dq_rows_equal_the_full_backward(causal):
    # attn_bwd is pinned by central finite differences; the sampled-row form must agree
    rng = np.random.default_rng(31)
    q, k, v, do = (rng.standard_normal(s) for s in ((2, 4, 37, 16), (2, 2, 45, 16), (2, 2, 45, 16), (2, 4, 37, 16)))
    full = ora.attn_bwd(q, k, v, do, None, causal, [45, 20])[0]
    rows = [0, 5, 36, 17]
    part = ora.attn_bwd_dq_rows(q, k, v, do, rows, None, causal, [45, 20])
    np.testing.assert_allclose(part, full[:, :, rows], rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(37, 45), (45, 37), (40, 40)], ids=["nq<nk", "nq>nk", "square"])
def test_sampled_dkdv_rows_equal_the_full_backward(causal, shape, monkeypatch):
    # attn_bwd is pinned by central finite differences; the sampled-key form must agree
    # for GQA (sums over the group), kv_len (keys past it have zero gradients) and both
    # causal alignments; a small chunk size also exercises the skipped row chunks
    nq, nk = shape
    rng = np.random.default_rng(32)
    q, do = rng.standard_normal((2, 4, nq, 16)), rng.standard_normal((2, 4, nq, 16))
    k, v = rng.standard_normal((2, 2, nk, 16)), rng.standard_normal((2, 2, nk, 16))
    kv_lens = [nk, 20]
    _, dk, dv = ora.attn_bwd(q, k, v, do, None, causal, kv_lens)[:3]
    keys = [0, 1, 19, 20, nk - 1, 7, 7]
    for chunk in (1 << 25, 64):
        monkeypatch.setattr(ora, "_CHUNK_ELEMS", chunk)
        pk, pv = ora.attn_bwd_dkdv_rows(q, k, v, do, keys, None, causal, kv_lens)
        np.testing.assert_allclose(pk, dk[:, :, keys], rtol=0, atol=1e-12)
        np.testing.assert_allclose(pv, dv[:, :, keys], rtol=0, atol=1e-12)
    assert np.all(pk[1, :, 3:5] == 0) and np.all(pv[1, :, 3:5] == 0)  # keys 20, nk-1 >= kv_len 20


def test_sampled_dkdv_rows_catch_a_row_sum_over_sampled_keys_only():
    # a plausible slip: D_i (or P) formed from the sampled key columns alone; the pin
    # above would catch it, and so does this direct comparison with the full backward
    rng = np.random.default_rng(33)
    q, k, v, do = (rng.standard_normal((1, 1, 30, 8)) for _ in range(4))
    dk = ora.attn_bwd(q, k, v, do, None, True)[1]
    keys = [0, 3, 29]
    s = (q[0, 0] @ k[0, 0].T) / np.sqrt(8)
    vis = ora.visible_mask(np.arange(30), 30, 30, 30, True)
    p, _ = ora._softmax_rows(s, vis)
    pj = p[:, keys]
    di_bad = np.sum(do[0, 0] * (pj @ v[0, 0, keys]), axis=-1)      # O from sampled keys only
    dk_bad = ((pj * (do[0, 0] @ v[0, 0, keys].T - di_bad[:, None])).T @ q[0, 0]) / np.sqrt(8)
    good = ora.attn_bwd_dkdv_rows(q, k, v, do, keys, None, True)[0][0, 0]
    np.testing.assert_allclose(good, dk[0, 0, keys], rtol=0, atol=1e-12)
    assert np.abs(dk_bad - dk[0, 0, keys]).max() > 1e-3


def test_nan_inputs_reach_exactly_the_rows_that_see_them():
    # IEEE arithmetic on the plain definition: a NaN in query row i makes row i's O and
    # LSE NaN; a NaN in key row j makes O and LSE NaN for the rows that see j (causal:
    # i >= j); every other row equals the result without the NaN (masked pairs and
    # missing keys never enter a row's softmax).  A row with no visible key keeps
    # O = 0, LSE = -inf.
    rng = np.random.default_rng(40)
    q, k, v = (rng.standard_normal((1, 2, 12, 8)) for _ in range(3))
    o0, l0 = oracle.attn_fwd(q, k, v, None, True)
    qn = q.copy()
    qn[0, 1, 5, 3] = np.nan
    o, l = oracle.attn_fwd(qn, k, v, None, True)
    bad = np.zeros((2, 12), bool)
    bad[1, 5] = True
    assert np.all(np.isnan(o[0][bad])) and np.all(np.isnan(l[0][bad]))
    np.testing.assert_array_equal(o[0][~bad], o0[0][~bad])
    np.testing.assert_array_equal(l[0][~bad], l0[0][~bad])
    kn = k.copy()
    kn[0, 0, 7, 2] = np.nan
    o, l = oracle.attn_fwd(q, kn, v, None, True)
    bad = np.zeros((2, 12), bool)
    bad[0, 7:] = True
    assert np.all(np.isnan(o[0][bad])) and np.all(np.isnan(l[0][bad]))
    np.testing.assert_array_equal(o[0][~bad], o0[0][~bad])
    # a NaN key past kv_len does not exist
    o, l = oracle.attn_fwd(q, kn, v, None, True, kv_lens=[7])
    assert np.all(np.isfinite(o[0, :, :])) and not np.any(np.isnan(l))
    # decode: a NaN key poisons every query head of its KV head
    qd = rng.standard_normal((1, 4, 8))
    kc, vc = rng.standard_normal((1, 2, 20, 8)), rng.standard_normal((1, 2, 20, 8))
    kc[0, 1, 3, 0] = np.nan
    od, ld = oracle.attn_decode(qd, kc, vc, [20])
    assert np.all(np.isnan(od[0, 2:])) and np.all(np.isnan(ld[0, 2:]))
    assert np.all(np.isfinite(od[0, :2])) and np.all(np.isfinite(ld[0, :2]))
