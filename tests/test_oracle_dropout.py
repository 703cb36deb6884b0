"""Pins of the oracle's dropout: the Philox4x32-10 generator against its published
known-answer vectors, the element-to-byte mapping against scalar brute force, the
dropout forward against the plain forward (p = 0) and against scalar loops, the
keep rate, the dropout backward against central finite differences, and checked
slices (absolute batch / head offsets) against the whole computation.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import dropout as dr

GOLD = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")


def test_philox_known_answer_vectors():
    for vec in json.load(open(GOLD))["vectors"]:
        ctr = np.array([int(x, 16) for x in vec["ctr"]], dtype=np.uint64)
        key = np.array([int(x, 16) for x in vec["key"]], dtype=np.uint64)
        out = dr.philox4x32_10(ctr, key)
        assert [int(x) for x in out] == [int(x, 16) for x in vec["out"]]


def test_mask_bytes_match_scalar_mapping():
    # the mapping written out for one element at a time, with Python integers
    b, h, seed = 1, 3, 0x1234_5678_9ABC
    rows, nk = [0, 5, 77], 70
    got = dr.mask_bytes(b, h, rows, nk, seed)
    for r, i in enumerate(rows):
        for j in range(nk):
            ctr = np.array([2 * (j // 32) + (j // 4) % 2, i, h, b], dtype=np.uint64)
            key = np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint64)
            words = [int(x) for x in dr.philox4x32_10(ctr, key)]
            n = 4 * ((j // 8) % 4) + j % 4
            assert got[r, j] == (words[n // 4] >> (8 * (n % 4))) & 0xFF


def test_keep_rate_and_scale():
    for p in (0.1, 0.25, 0.5):
        t = dr.threshold(p)
        z = dr.keep_mask(0, 0, range(256), 512, 7, p)
        keep = (256 - t) / 256
        n = z.size
        assert abs(z.mean() - keep) < 5 * math.sqrt(keep * (1 - keep) / n)
        assert dr.keep_scale(p) * keep == 1.0
    assert dr.threshold(0.0) == 0 and dr.keep_scale(0.0) == 1.0


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_dropout_is_the_plain_forward(causal):
    rng = np.random.default_rng(1)
    q, k, v = _rand(rng, 1, 4, 40, 8), _rand(rng, 1, 2, 50, 8), _rand(rng, 1, 2, 50, 8)
    o, lse = dr.attn_fwd_dropout(q, k, v, 0.0, 5, None, causal)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, None, causal)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(lse, lse_ref)


def test_dropout_forward_matches_scalar_loops():
    rng = np.random.default_rng(2)
    q, k, v = _rand(rng, 1, 2, 6, 4), _rand(rng, 1, 1, 9, 4), _rand(rng, 1, 1, 9, 4)
    p, seed, scale = 0.3, 99, 0.5
    o, _ = dr.attn_fwd_dropout(q, k, v, p, seed, scale, True)
    ks = dr.keep_scale(p)
    for h in range(2):
        z = dr.keep_mask(0, h, range(6), 9, seed, p)
        for i in range(6):
            keys = [j for j in range(9) if j <= i + 3]
            s = [scale * sum(q[0, h, i, t] * k[0, 0, j, t] for t in range(4)) for j in keys]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            l = sum(e)
            for t in range(4):
                ref = sum(e[n] / l * (ks if z[i, j] else 0.0) * v[0, 0, j, t] for n, j in enumerate(keys))
                assert abs(o[0, h, i, t] - ref) < 1e-12


def test_dropout_backward_matches_finite_differences():
    rng = np.random.default_rng(3)
    q, k, v, do = _rand(rng, 1, 2, 7, 4), _rand(rng, 1, 1, 9, 4), _rand(rng, 1, 1, 9, 4), _rand(rng, 1, 2, 7, 4)
    p, seed = 0.25, 11
    dq, dk, dv, _, _ = dr.attn_bwd_dropout(q, k, v, do, p, seed, None, True)

    def loss(q_, k_, v_):
        return float(np.sum(dr.attn_fwd_dropout(q_, k_, v_, p, seed, None, True)[0] * do))

    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - g[idx]) < 1e-6, (name, idx, fd, g[idx])


def test_dropout_is_unbiased_over_seeds():
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng, 1, 1, 4, 8), _rand(rng, 1, 1, 64, 8), _rand(rng, 1, 1, 64, 8)
    o_ref, _ = oracle.attn_fwd(q, k, v)
    acc = np.zeros_like(o_ref)
    n = 400
    for seed in range(n):
        acc += dr.attn_fwd_dropout(q, k, v, 0.5, seed)[0]
    assert np.abs(acc / n - o_ref).max() < 0.1


def test_a_slice_with_its_offsets_is_the_slice_of_the_whole():
    # bh0 lets sampled (batch, head) slices of a large workload be checked on their own:
    # each slice with its offsets must equal the same slice of the whole computation,
    # and without the offsets it must not (the mask depends on the absolute indices)
    rng = np.random.default_rng(5)
    q, k, v, do = (rng.standard_normal((2, 3, 40, 8)) for _ in range(4))
    seed, p = 0x1234_5678_9ABC, 0.3
    o, lse = dr.attn_fwd_dropout(q, k, v, p, seed, None, True)
    g = dr.attn_bwd_dropout(q, k, v, do, p, seed, None, True)
    for b, h in ((1, 2), (0, 1)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        os_, ls = dr.attn_fwd_dropout(q[sl], k[sl], v[sl], p, seed, None, True, bh0=(b, h))
        np.testing.assert_array_equal(os_[0, 0], o[b, h])
        np.testing.assert_array_equal(ls[0, 0], lse[b, h])
        gs = dr.attn_bwd_dropout(q[sl], k[sl], v[sl], do[sl], p, seed, None, True, bh0=(b, h))
        for full, part in zip(g[:3], gs[:3]):
            np.testing.assert_allclose(part[0, 0], full[b, h], rtol=0, atol=1e-12)
        assert np.abs(dr.attn_fwd_dropout(q[sl], k[sl], v[sl], p, seed, None, True)[0][0, 0] - o[b, h]).max() > 1e-3
