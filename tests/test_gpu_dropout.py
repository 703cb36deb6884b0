"""GPU parity of dropout on P (fa_fwd_dropout / fa_bwd_dropout) against the fp64
oracle, which draws the same Philox4x32-10 mask from its own implementation.

The mask itself is compared bit for bit: with V the identity (D >= Nk), O[i, j] is
P_ij * Z_ij / keep, so the kernel's kept set is exactly the non-zero entries of O.
"""

import numpy as np
import pytest
import torch

import io_aware_tiled_10_amd as fa
from io_aware_tiled_10_amd import inputs
from oracle import dropout as odr
from tests.helpers import DEV, assert_fwd_close, rel_l2, say, to_dev, to_host

pytestmark = pytest.mark.gpu

SEED = 0x5EED_0123_4567


def test_dropout_mask_is_the_generators_bit_for_bit():
    say("dropout mask")
    B, H, Nq, Nk, D = 2, 3, 300, 128, 128
    x = inputs.attention_inputs(B, H, H, Nq, Nk, D, "bf16", seed=31)
    v = np.zeros((B, H, Nk, D), np.float32)
    v[:, :, np.arange(Nk), np.arange(Nk)] = 1.0
    for p in (0.1, 0.5, 0.95):
        for causal in (False, True):
            o, _ = fa.fwd_dropout(to_dev(x.q), to_dev(x.k), to_dev(v), p, SEED, causal=causal,
                                  out_dtype=torch.float32)
            torch.cuda.synchronize()
            kept = to_host(o) != 0
            for b in range(B):
                for h in range(H):
                    z = odr.keep_mask(b, h, range(Nq), Nk, SEED, p)
                    if causal:  # only the visible pairs carry a probability
                        z &= np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + (Nk - Nq)
                    assert np.array_equal(kept[b, h], z), (p, causal, b, h)


CASES = [
    # name, B, Hq, Hkv, Nq, Nk, D, causal, kv_lens
    ("mha_ragged_causal", 1, 2, 2, 300, 300, 128, True, None),
    ("gqa_noncausal", 2, 4, 2, 200, 257, 128, False, None),
    ("kvlens_d64", 2, 2, 1, 150, 260, 64, True, [17, 259]),
    # mid sizes: the kernels' block loops run for many trips
    ("gqa4_n1100_causal", 1, 8, 2, 1100, 1100, 128, True, None),
    ("mha_d64_nq900_nk1300_kvlens", 2, 2, 2, 900, 1300, 64, True, [1300, 611]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("p_drop", [0.1, 0.5, 0.95])
def test_dropout_forward_and_backward_match_oracle(case, p_drop):
    name, B, Hq, Hkv, Nq, Nk, D, causal, kv_lens = case
    say(f"dropout {name} p={p_drop}")
    x = inputs.attention_inputs(B, Hq, Hkv, Nq, Nk, D, "bf16", seed=7, with_grad=True)
    q, k, v, do = to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.do)
    kl = torch.tensor(kv_lens, dtype=torch.int32, device=DEV) if kv_lens is not None else None
    o32, lse32 = fa.fwd_dropout(q, k, v, p_drop, SEED, causal=causal, kv_lens=kl, out_dtype=torch.float32)
    o, lse = fa.fwd_dropout(q, k, v, p_drop, SEED, causal=causal, kv_lens=kl)
    dq, dk, dv = fa.bwd_dropout(q, k, v, o, do, lse, p_drop, SEED, causal=causal, kv_lens=kl)
    torch.cuda.synchronize()
    o_ref, lse_ref = odr.attn_fwd_dropout(x.q, x.k, x.v, p_drop, SEED, None, causal, kv_lens)
    assert_fwd_close(to_host(o32), to_host(lse32), o_ref, lse_ref, False,
                     tol_o=2.0 ** -8 * odr.keep_scale(p_drop) * float(np.abs(x.v).max()) + 1e-3)
    ref = odr.attn_bwd_dropout(x.q, x.k, x.v, x.do, p_drop, SEED, None, causal, kv_lens)
    for nm, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref[:3]):
        e = rel_l2(to_host(g), r)
        say(f"  {nm} rel-L2 {e:.3e}")
        assert e <= 2e-2, (nm, e)


def test_zero_dropout_is_the_plain_forward_and_seeds_matter():
    x = inputs.attention_inputs(1, 2, 2, 200, 200, 128, "bf16", seed=8)
    q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    a = fa.fwd_dropout(q, k, v, 0.0, SEED, causal=True)
    b = fa.fwd(q, k, v, causal=True)
    c1 = fa.fwd_dropout(q, k, v, 0.2, 1, causal=True)
    c2 = fa.fwd_dropout(q, k, v, 0.2, 1, causal=True)
    c3 = fa.fwd_dropout(q, k, v, 0.2, 2, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(c1[0], c2[0]) and not torch.equal(c1[0], c3[0])
    assert torch.equal(c1[1], b[1])  # the log-sum-exp is that of the undropped scores


def test_dropout_full_size_c4_sampled_heads():
    # the timed dropout workload: B2 H16 N4096 D128 causal, p = 0.1, launched as the
    # benchmark launches it; two whole (batch, head) slices against the oracle, which
    # draws each slice's mask at its absolute (batch, head) index
    say("dropout full c4")
    B, H, N, D, p = 2, 16, 4096, 128, 0.1
    seed = 0x5EED
    x = inputs.attention_inputs(B, H, H, N, N, D, "bf16", seed=0, with_grad=True)
    q, k, v, do = to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.do)
    o32, lse32 = fa.fwd_dropout(q, k, v, p, seed, causal=True, out_dtype=torch.float32)
    o, lse = fa.fwd_dropout(q, k, v, p, seed, causal=True)
    dq, dk, dv = fa.bwd_dropout(q, k, v, o, do, lse, p, seed, causal=True)
    torch.cuda.synchronize()
    for t in (o, dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    for b, h in ((0, 0), (1, 11)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = odr.attn_bwd_dropout(x.q[sl], x.k[sl], x.v[sl], x.do[sl], p, seed, None, True, bh0=(b, h))
        assert_fwd_close(to_host(o32[sl]), to_host(lse32[sl]), ref[3], ref[4], False,
                         tol_o=2.0 ** -8 * odr.keep_scale(p) * float(np.abs(x.v[sl]).max()) + 1e-3)
        for nm, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref[:3]):
            e = rel_l2(to_host(g[sl]), r)
            say(f"  b{b} h{h} {nm} rel-L2 {e:.3e}")
            assert e <= 2e-2, (b, h, nm, e)
