"""GPU parity of fa_fwd against the fp64 oracle (element by element).

Tolerances: O max-abs <= 1e-2 (plus half a bf16 ulp of the reference when O is
written in bf16) and LSE max-abs <= 1e-3, both for bf16 inputs; the same for the
fp32 path.  Inputs are the seeded draws of io_aware_tiled_10_amd.inputs, given to
both sides bit for bit.
"""

import numpy as np
import pytest
import torch

import io_aware_tiled_10_amd as fa
import oracle
from io_aware_tiled_10_amd import inputs
from tests.helpers import DEV, assert_fwd_close, say, to_dev, to_host

pytestmark = pytest.mark.gpu

SMALL = [
    # name, B, Hq, Hkv, Nq, Nk, D, causal, kv_lens
    ("mha_ragged_noncausal_d128", 2, 2, 2, 300, 300, 128, False, None),
    ("mha_ragged_causal_d128", 2, 2, 2, 300, 300, 128, True, None),
    ("gqa_causal_d128", 1, 8, 2, 257, 257, 128, True, None),
    ("mqa_noncausal_d64", 1, 4, 1, 200, 333, 64, False, None),
    ("causal_nq_lt_nk", 1, 2, 1, 100, 333, 128, True, None),
    ("causal_nq_gt_nk_masked_rows", 1, 2, 2, 200, 70, 128, True, None),
    ("kvlens_noncausal", 3, 2, 1, 130, 300, 128, False, [300, 1, 0]),
    ("kvlens_causal_d64", 2, 4, 2, 150, 260, 64, True, [17, 259]),
    ("single_row_single_key", 1, 1, 1, 1, 1, 128, False, None),
    ("single_row_causal", 1, 2, 1, 1, 129, 128, True, None),
    ("exact_tiles", 1, 2, 2, 256, 256, 128, True, None),
    # several 256-row causal tiles, whose last steps skip blocks per wave, with the
    # diagonal offset by Nk - Nq (blocks not aligned to the tile)
    ("mha_causal_tiles_nq_lt_nk", 1, 2, 2, 1000, 1300, 128, True, None),
    ("mha_causal_tiles_nq_gt_nk", 1, 2, 2, 1100, 700, 64, True, None),
    # causal GQA tiles of 128 rows x 2 heads and of 64 rows x 4 heads
    ("gqa2_causal_tiles", 1, 4, 2, 700, 700, 128, True, None),
    ("gqa4_causal_tiles_kvlens", 2, 8, 2, 600, 650, 128, True, [650, 333]),
]


def run_case(B, Hq, Hkv, Nq, Nk, D, causal, kv_lens, out_dtype, seed=0, poison=False):
    x = inputs.attention_inputs(B, Hq, Hkv, Nq, Nk, D, "bf16", seed=seed)
    q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    kl = None
    if kv_lens is not None:
        kl = torch.tensor(kv_lens, dtype=torch.int32, device=DEV)
        if poison:
            for b, L in enumerate(kv_lens):
                k[b, :, L:] = float("nan")
                v[b, :, L:] = float("nan")
    o, lse = fa.fwd(q, k, v, causal=causal, kv_lens=kl, out_dtype=out_dtype)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(x.q, x.k, x.v, None, causal, kv_lens)
    return to_host(o), to_host(lse), o_ref, lse_ref


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["oF32", "oBF16"])
def test_fwd_bf16_matches_oracle(case, out_dtype):
    name, B, Hq, Hkv, Nq, Nk, D, causal, kv_lens = case
    say(f"fwd case {name} out={out_dtype}")
    o, lse, o_ref, lse_ref = run_case(B, Hq, Hkv, Nq, Nk, D, causal, kv_lens, out_dtype)
    err = assert_fwd_close(o, lse, o_ref, lse_ref, out_dtype == torch.bfloat16)
    say(f"  max|dO| = {err:.3e}")
    if out_dtype == torch.float32:
        # fp32 output: only bf16 rounding of P separates the kernel from exact
        assert err < 4e-3


def test_fwd_nan_poisoned_padding_is_never_read():
    say("fwd poisoned padding")
    o, lse, o_ref, lse_ref = run_case(2, 4, 2, 96, 300, 128, True, [77, 300], torch.float32, poison=True)
    assert_fwd_close(o, lse, o_ref, lse_ref, False)


def test_fwd_fp32_config_c1():
    # fp32 B1 H2 N256 D64 non-causal, full oracle comparison
    say("fwd fp32 c1")
    x = inputs.attention_inputs(1, 2, 2, 256, 256, 64, "fp32", seed=0)
    q, k, v = (to_dev(a, torch.float32) for a in (x.q, x.k, x.v))
    o, lse = fa.fwd(q, k, v, causal=False)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(x.q, x.k, x.v)
    err = assert_fwd_close(to_host(o), to_host(lse), o_ref, lse_ref, False)
    assert err < 1e-5, err


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp32_ragged(causal):
    x = inputs.attention_inputs(2, 2, 1, 100, 150, 64, "fp32", seed=3)
    q, k, v = (to_dev(a, torch.float32) for a in (x.q, x.k, x.v))
    o, lse = fa.fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(x.q, x.k, x.v, None, causal)
    assert assert_fwd_close(to_host(o), to_host(lse), o_ref, lse_ref, False) < 1e-5


# The fp32 forward takes 16-row tiles (each row over 16 threads) when 64-row tiles would
# give fewer than two per compute unit, else 64-row tiles of eight waves: these shapes
# (B1 H64 GQA 8:1, 512 and 520 rows, 5 and 9 row tiles of 64 past 512 in all) take the
# second path, with a ragged tail and Nq != Nk.
FP32_WIDE = [
    ("h64_n512", 64, 8, 512, 512, False),
    ("h64_n520_causal", 64, 8, 520, 520, True),
    ("h64_nq520_nk700_causal", 64, 8, 520, 700, True),
]


@pytest.mark.parametrize("case", FP32_WIDE, ids=[c[0] for c in FP32_WIDE])
def test_fwd_fp32_many_tiles(case):
    name, Hq, Hkv, Nq, Nk, causal = case
    say(f"fwd fp32 {name}")
    x = inputs.attention_inputs(1, Hq, Hkv, Nq, Nk, 64, "fp32", seed=11)
    q, k, v = (to_dev(a, torch.float32) for a in (x.q, x.k, x.v))
    o, lse = fa.fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(x.q, x.k, x.v, None, causal)
    assert assert_fwd_close(to_host(o), to_host(lse), o_ref, lse_ref, False) < 1e-5


def test_fwd_gqa_equals_mha_with_repeated_kv():
    x = inputs.attention_inputs(1, 8, 2, 200, 200, 128, "bf16", seed=5)
    q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    o1, l1 = fa.fwd(q, k, v, causal=True, out_dtype=torch.float32)
    kr, vr = k.repeat_interleave(4, dim=1), v.repeat_interleave(4, dim=1)
    o2, l2 = fa.fwd(q, kr, vr, causal=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fwd_strided_layout_bnhd():
    # [B, N, H, D] memory (the flash-attn layout) passed through strides
    x = inputs.attention_inputs(2, 4, 2, 130, 130, 128, "bf16", seed=6)
    qn = to_dev(x.q).transpose(1, 2).contiguous().transpose(1, 2)
    kn = to_dev(x.k).transpose(1, 2).contiguous().transpose(1, 2)
    vn = to_dev(x.v).transpose(1, 2).contiguous().transpose(1, 2)
    o, lse = fa.fwd(qn, kn, vn, causal=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(x.q, x.k, x.v, None, True)
    assert_fwd_close(to_host(o), to_host(lse), o_ref, lse_ref, False)


def test_fwd_is_deterministic():
    x = inputs.attention_inputs(1, 4, 1, 513, 513, 128, "bf16", seed=7)
    q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    a = fa.fwd(q, k, v, causal=True)
    b = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def _score_pattern(x, pattern):
    """Reshape the score landscape (values stay bf16-exact, both sides get them)."""
    q, k = x.q.copy(), x.k.copy()
    Nk = k.shape[2]
    if pattern == "rising":      # later key blocks outscore earlier ones by > 2^8
        k = k * (1.0 + 5.0 * np.arange(Nk, dtype=np.float32) / Nk)[None, None, :, None]
    elif pattern == "peaky":     # score spread of ~8 natural units per sigma
        q = q * 8.0
    elif pattern == "negative":  # every score of a row shifted far below zero
        k[..., 0] = 240.0
        q[..., 0] = -np.abs(q[..., 0]) - 4.0
    return inputs.bf16_round(q), inputs.bf16_round(k)


@pytest.mark.parametrize("pattern", ["rising", "peaky", "negative"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("D", [128, 64])
def test_fwd_exponent_reference_moves(pattern, causal, D):
    # The exponent reference is moved only when a block's probability sum outgrows
    # its bound; these score landscapes force such moves in the middle of rows, and
    # rows whose every score is far below zero.
    say(f"fwd reference move {pattern} causal={causal} D={D}")
    x = inputs.attention_inputs(1, 4, 2, 300, 700, D, "bf16", seed=12)
    qn, kn = _score_pattern(x, pattern)
    o, lse = fa.fwd(to_dev(qn), to_dev(kn), to_dev(x.v), causal=causal, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(qn, kn, x.v, None, causal)
    # P is rounded to bf16 (relative error <= 2^-8) before the second product while the
    # row sum keeps fp32, so |O - O_ref| <= 2^-8 max|v|; a row dominated by a few keys
    # (the peaky landscape) gets near that, past the 1e-2 of the N(0,1) workloads.
    tol_o = 2.0 ** -8 * float(np.abs(x.v).max()) + 1e-3
    assert_fwd_close(to_host(o), to_host(lse), o_ref, lse_ref, False, tol_o=tol_o)


def test_fwd_empty_key_set_gives_zero_and_neg_inf():
    x = inputs.attention_inputs(1, 2, 2, 40, 0, 128, "bf16", seed=8)
    q = to_dev(x.q)
    k = torch.zeros((1, 2, 0, 128), dtype=torch.bfloat16, device=DEV)  # may carry a NULL pointer
    o, lse = fa.fwd(q, k, k, causal=False, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


# --------------------------------------------------------------------------------------
# full-size workloads, launched as the benchmark launches them; sampled rows vs oracle
# --------------------------------------------------------------------------------------

FULL = [
    ("c3_gqa_causal_16k", 1, 32, 8, 16384, 128, True),
]
WHOLE = [
    ("c2_noncausal", 4, 16, 16, 2048, 128, False),
    ("c2_causal", 4, 16, 16, 2048, 128, True),
]


@pytest.mark.parametrize("case", WHOLE, ids=[c[0] for c in WHOLE])
def test_fwd_full_size_every_row(case):
    # B4 H16 N2048 D128: the oracle covers every output element in a few seconds
    name, B, Hq, Hkv, N, D, causal = case
    say(f"fwd whole {name}")
    x = inputs.attention_inputs(B, Hq, Hkv, N, N, D, "bf16", seed=0)
    q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    o, lse = fa.fwd(q, k, v, causal=causal)              # bf16 O, as timed
    o32, lse32 = fa.fwd(q, k, v, causal=causal, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(x.q, x.k, x.v, None, causal)
    e32 = assert_fwd_close(to_host(o32), to_host(lse32), o_ref, lse_ref, False)
    e16 = assert_fwd_close(to_host(o), to_host(lse), o_ref, lse_ref, True)
    say(f"  max|dO| fp32 out {e32:.3e}, bf16 out {e16:.3e}")
    assert torch.equal(lse, lse32)


@pytest.mark.parametrize("case", FULL, ids=[c[0] for c in FULL])
def test_fwd_full_size_sampled_rows(case):
    name, B, Hq, Hkv, N, D, causal = case
    say(f"fwd full {name}")
    x = inputs.attention_inputs(B, Hq, Hkv, N, N, D, "bf16", seed=0)
    q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    o, lse = fa.fwd(q, k, v, causal=causal)              # bf16 O, as timed
    o32, lse32 = fa.fwd(q, k, v, causal=causal, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, N - 1], rng.integers(0, N, 27)]))
    rt = torch.from_numpy(rows).to(DEV)
    heads = sorted(set([0, Hq - 1] + list(rng.integers(0, Hq, 3))))
    bs = sorted(set([0, B - 1]))
    for b in bs:
        for h in heads:
            o_ref, lse_ref = oracle.attn_fwd(x.q[b:b + 1, h:h + 1], x.k[b:b + 1, h // (Hq // Hkv):h // (Hq // Hkv) + 1],
                                             x.v[b:b + 1, h // (Hq // Hkv):h // (Hq // Hkv) + 1], None, causal,
                                             rows=rows)
            assert_fwd_close(to_host(o32[b, h, rt])[None, None], to_host(lse32[b, h, rt])[None, None],
                             o_ref, lse_ref, False)
            assert_fwd_close(to_host(o[b, h, rt])[None, None], to_host(lse[b, h, rt])[None, None],
                             o_ref, lse_ref, True)
    # properties that hold at any size: finite outputs, LSE agreement of both dtypes
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    assert torch.equal(lse, lse32)
