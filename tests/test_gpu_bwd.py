"""GPU parity of fa_bwd against the fp64 oracle.

Pass: relative L2 error <= 2e-2 for each of dQ, dK, dV (whole tensor, fp64).  The
backward is fed O and LSE from fa_fwd on the same inputs, as a training step
would; the oracle runs its own fp64 forward.
"""

import numpy as np
import pytest
import torch

import io_aware_tiled_10_amd as fa
import oracle
from io_aware_tiled_10_amd import inputs
from tests.helpers import DEV, rel_l2, say, to_dev, to_host

pytestmark = pytest.mark.gpu

SMALL = [
    # name, B, Hq, Hkv, Nq, Nk, D, causal, kv_lens
    ("mha_causal_ragged", 1, 2, 2, 300, 300, 128, True, None),
    ("mha_noncausal_ragged", 2, 2, 2, 200, 200, 128, False, None),
    ("gqa_causal", 1, 4, 2, 257, 257, 128, True, None),
    ("d64_causal", 1, 2, 1, 190, 190, 64, True, None),
    ("nq_lt_nk_causal", 1, 2, 2, 70, 300, 128, True, None),
    ("nq_gt_nk_causal", 1, 2, 2, 260, 100, 128, True, None),
    ("kvlens", 2, 2, 1, 150, 300, 128, False, [300, 45]),
    ("tiny", 1, 1, 1, 3, 5, 128, False, None),
]


def run(B, Hq, Hkv, Nq, Nk, D, causal, kv_lens, seed=0):
    x = inputs.attention_inputs(B, Hq, Hkv, Nq, Nk, D, "bf16", seed=seed, with_grad=True)
    q, k, v, do = to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.do)
    kl = torch.tensor(kv_lens, dtype=torch.int32, device=DEV) if kv_lens is not None else None
    o, lse = fa.fwd(q, k, v, causal=causal, kv_lens=kl)
    dq, dk, dv = fa.bwd(q, k, v, o, do, lse, causal=causal, kv_lens=kl)
    torch.cuda.synchronize()
    return x, (to_host(dq), to_host(dk), to_host(dv))


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_bwd_matches_oracle(case):
    name, B, Hq, Hkv, Nq, Nk, D, causal, kv_lens = case
    say(f"bwd case {name}")
    x, got = run(B, Hq, Hkv, Nq, Nk, D, causal, kv_lens)
    ref = oracle.attn_bwd(x.q, x.k, x.v, x.do, None, causal, kv_lens)[:3]
    for nm, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert np.all(np.isfinite(g)), nm
        e = rel_l2(g, r)
        say(f"  {nm} rel-L2 {e:.3e}")
        assert e <= 2e-2, (nm, e)
    if kv_lens is not None:
        for b, L in enumerate(kv_lens):
            assert np.all(got[1][b, :, L:] == 0) and np.all(got[2][b, :, L:] == 0)


def test_bwd_full_size_c4_all_heads():
    # B2 H16 N4096 D128 causal; heads are independent (MHA), so every (batch, head)
    # slice is checked whole, against the oracle's backward of that slice
    say("bwd full c4")
    B, H, N, D = 2, 16, 4096, 128
    x = inputs.attention_inputs(B, H, H, N, N, D, "bf16", seed=0, with_grad=True)
    q, k, v, do = to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.do)
    o, lse = fa.fwd(q, k, v, causal=True)
    dq, dk, dv = fa.bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    worst = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for b, h in ((b, h) for b in range(B) for h in range(H)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oracle.attn_bwd(x.q[sl], x.k[sl], x.v[sl], x.do[sl], None, True)[:3]
        for nm, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            e = rel_l2(to_host(g[b:b + 1, h:h + 1]), r)
            worst[nm] = max(worst[nm], e)
            assert e <= 2e-2, (b, h, nm, e)
    say("  worst rel-L2 over the 32 slices: " + ", ".join(f"{k} {v:.3e}" for k, v in worst.items()))


def test_bwd_is_deterministic():
    # no atomics anywhere in the backward: two calls give identical bits
    say("bwd determinism")
    x = inputs.attention_inputs(1, 8, 2, 300, 300, 128, "bf16", seed=4, with_grad=True)
    q, k, v, do = to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.do)
    o, lse = fa.fwd(q, k, v, causal=True)
    a = fa.bwd(q, k, v, o, do, lse, causal=True)
    b = fa.bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    for x1, x2 in zip(a, b):
        assert torch.equal(x1, x2)


def test_bwd_strided_layout_bnhd_gives_the_same_bits():
    # [B, N, H, D] memory (the flash-attn layout) for every input and gradient, passed
    # through strides: the kernels do the same arithmetic, so the results are identical
    say("bwd strided layout")
    x = inputs.attention_inputs(2, 4, 2, 200, 200, 128, "bf16", seed=9, with_grad=True)
    q, k, v, do = to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.do)
    o, lse = fa.fwd(q, k, v, causal=True)
    ref = fa.bwd(q, k, v, o, do, lse, causal=True)

    def bnhd(t):
        return t.transpose(1, 2).contiguous().transpose(1, 2)

    qn, kn, vn, on, don = (bnhd(t) for t in (q, k, v, o, do))
    grads = (bnhd(torch.empty_like(q)), bnhd(torch.empty_like(k)), bnhd(torch.empty_like(v)))
    got = fa.bwd(qn, kn, vn, on, don, lse, causal=True, grads=grads)
    torch.cuda.synchronize()
    assert not grads[0].is_contiguous()
    for g, r in zip(got, ref):
        assert torch.equal(g, r)


def test_bwd_gqa_full_size_c3_shape():
    # B1 Hq32 Hkv8 N16384 D128 causal, launched as the benchmark launches it.  Against
    # the oracle: sampled dQ rows of three query heads, and sampled dK / dV key rows of
    # two KV heads (each summed over its 4 query heads).  Key 0 is seen by every query
    # row, so the first group's oracle forms all 4 x 16384 rows; the last group's keys
    # lie in the final 256 rows.  A property that holds at any size, over all keys:
    # dK / dV equal the MHA backward on K / V repeated for each query head, summed
    # over the group.
    say("bwd GQA full c3 shape")
    B, Hq, Hkv, N, D = 1, 32, 8, 16384, 128
    x = inputs.attention_inputs(B, Hq, Hkv, N, N, D, "bf16", seed=0, with_grad=True)
    q, k, v, do = to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.do)
    o, lse = fa.fwd(q, k, v, causal=True)
    dq, dk, dv = fa.bwd(q, k, v, o, do, lse, causal=True)
    kr = k.repeat_interleave(Hq // Hkv, dim=1).contiguous()
    vr = v.repeat_interleave(Hq // Hkv, dim=1).contiguous()
    o2, lse2 = fa.fwd(q, kr, vr, causal=True)
    _, dk2, dv2 = fa.bwd(q, kr, vr, o2, do, lse2, causal=True)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    dk_sum = dk2.float().view(B, Hkv, Hq // Hkv, N, D).sum(2)
    dv_sum = dv2.float().view(B, Hkv, Hq // Hkv, N, D).sum(2)
    for nm, g, r in (("dk", dk, dk_sum), ("dv", dv, dv_sum)):
        e = rel_l2(to_host(g), to_host(r))
        say(f"  {nm} vs summed MHA rel-L2 {e:.3e}")
        assert e <= 1e-2, (nm, e)
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, N - 1], rng.integers(0, N, 11)]))
    for h in (0, 13, 31):
        g = h // (Hq // Hkv)
        ref = oracle.attn_bwd_dq_rows(x.q[:, h:h + 1], x.k[:, g:g + 1], x.v[:, g:g + 1], x.do[:, h:h + 1],
                                      rows, None, True)
        e = rel_l2(to_host(dq[:, h:h + 1, rows]), ref)
        say(f"  h{h} sampled dq rel-L2 {e:.3e}")
        assert e <= 2e-2, (h, e)
    G = Hq // Hkv
    key_sets = {0: np.unique(np.concatenate([[0, 1, 127, 128, 8191, 8192, N - 2, N - 1],
                                               rng.integers(0, N, 8)])),
                Hkv - 1: np.unique(np.concatenate([[N - 256, N - 129, N - 128, N - 1],
                                                     rng.integers(N - 256, N, 8)]))}
    for g, keys in key_sets.items():
        hs = slice(g * G, (g + 1) * G)
        dk_ref, dv_ref = oracle.attn_bwd_dkdv_rows(x.q[:, hs], x.k[:, g:g + 1], x.v[:, g:g + 1], x.do[:, hs],
                                                   keys, None, True)
        for nm, t, r in (("dk", dk, dk_ref), ("dv", dv, dv_ref)):
            e = rel_l2(to_host(t[:, g:g + 1, keys]), r)
            say(f"  kv head {g}: {len(keys)} sampled {nm} rows rel-L2 {e:.3e}")
            assert e <= 2e-2, (g, nm, e)
