"""GPU parity on seeded random shapes.  Forward and backward: batch, head counts and
grouping, query and key lengths (including Nq != Nk, so causal rows with no visible key
occur), head dimension, causal flag and per-batch key lengths.  Decode: batch, grouping,
cache lengths (zero included) and chunk length.  Each case is drawn from a fixed seed and
every output is compared with the fp64 oracle.
"""

import numpy as np
import pytest
import torch

import io_aware_tiled_10_amd as fa
import oracle
from io_aware_tiled_10_amd import inputs
from tests.helpers import DEV, assert_fwd_close, rel_l2, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def draw_case(seed: int):
    rng = np.random.default_rng([seed, 31])
    B = int(rng.integers(1, 3))
    Hkv = int(rng.integers(1, 3))
    G = int(rng.choice([1, 2, 4]))
    Nq = int(rng.integers(1, 301))
    Nk = int(rng.integers(1, 301))
    D = int(rng.choice([64, 128]))
    causal = bool(rng.integers(0, 2))
    kv_lens = [int(x) for x in rng.integers(0, Nk + 1, size=B)] if rng.integers(0, 2) else None
    return B, Hkv * G, Hkv, Nq, Nk, D, causal, kv_lens


CASES = list(range(24))


@pytest.mark.parametrize("seed", CASES)
def test_random_shape_fwd_bwd_match_oracle(seed):
    B, Hq, Hkv, Nq, Nk, D, causal, kv_lens = draw_case(seed)
    say(f"random shape {seed}: B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Nk{Nk} D{D} causal={causal} kv_lens={kv_lens}")
    x = inputs.attention_inputs(B, Hq, Hkv, Nq, Nk, D, "bf16", seed=100 + seed, with_grad=True)
    q, k, v, do = to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.do)
    kl = torch.tensor(kv_lens, dtype=torch.int32, device=DEV) if kv_lens is not None else None
    o32, lse32 = fa.fwd(q, k, v, causal=causal, kv_lens=kl, out_dtype=torch.float32)
    o, lse = fa.fwd(q, k, v, causal=causal, kv_lens=kl)
    dq, dk, dv = fa.bwd(q, k, v, o, do, lse, causal=causal, kv_lens=kl)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(x.q, x.k, x.v, None, causal, kv_lens)
    assert_fwd_close(to_host(o32), to_host(lse32), o_ref, lse_ref, False)
    assert_fwd_close(to_host(o), to_host(lse), o_ref, lse_ref, True)
    ref = oracle.attn_bwd(x.q, x.k, x.v, x.do, None, causal, kv_lens)
    for nm, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref[:3]):
        gh = to_host(g)
        assert np.all(np.isfinite(gh)), nm
        e = rel_l2(gh, r)
        say(f"  {nm} rel-L2 {e:.3e}")
        assert e <= 2e-2, (nm, e)


def draw_decode_case(seed: int):
    rng = np.random.default_rng([seed, 37])
    Bs = int(rng.integers(1, 6))
    Hkv = int(rng.integers(1, 3))
    G = int(rng.choice([1, 2, 4, 8]))
    lens = [int(x) for x in rng.integers(0, 5000, size=Bs)]
    if seed % 3 == 0:
        lens[0] = 0  # a sequence with an empty cache: O = 0, LSE = -inf
    split = int(rng.choice([128, 256, 1024, 2048, 4096]))
    return Bs, Hkv * G, Hkv, lens, split


@pytest.mark.parametrize("seed", list(range(8)))
def test_random_shape_decode_matches_oracle(seed):
    Bs, Hq, Hkv, lens, split = draw_decode_case(seed)
    say(f"random decode {seed}: Bs{Bs} Hq{Hq} Hkv{Hkv} lens={lens} split={split}")
    rng = np.random.default_rng([seed, 41])
    d = inputs.DecodeInputs(np.array(lens), inputs.bf16_round(rng.standard_normal((Bs, Hq, 128), dtype=np.float32)),
                            Hkv, 128, seed=200 + seed)
    lmax = max(max(lens), 1)
    kc, vc = d.dense_cache(lmax)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o, lse = fa.decode(to_dev(d.q), to_dev(kc), to_dev(vc), sl, max_len=lmax, split_len=split,
                       out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_decode(d.q, kc, vc, lens)
    assert_fwd_close(to_host(o), to_host(lse), o_ref, lse_ref, False)
