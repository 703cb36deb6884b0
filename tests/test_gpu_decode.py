"""GPU parity of fa_decode (split-KV + merge) against the fp64 oracle.

The cache beyond each sequence's length is filled with NaN: any read of it into a
result would show up as a non-finite output.
"""

import numpy as np
import pytest
import torch

import io_aware_tiled_10_amd as fa
import oracle
from io_aware_tiled_10_amd import inputs
from tests.helpers import DEV, assert_fwd_close, dense_cache_on_device, say, to_host

pytestmark = pytest.mark.gpu


build_cache = dense_cache_on_device


def oracle_decode(d: inputs.DecodeInputs, seqs):
    o = np.zeros((len(seqs), d.q.shape[1], d.D))
    lse = np.zeros((len(seqs), d.q.shape[1]))
    for n, s in enumerate(seqs):
        k, v = d.kv(s)
        oo, ll = oracle.attn_decode(d.q[s:s + 1], k[None], v[None], [int(d.seq_lens[s])])
        o[n], lse[n] = oo[0], ll[0]
    return o, lse


SMALL = [
    # name, Hq, Hkv, D, lens, split, out dtype
    ("gqa4_d128_mixed", 8, 2, 128, [1, 31, 100, 2048, 2049, 5000], 2048, torch.bfloat16),
    ("gqa4_d128_small_split", 8, 2, 128, [1, 33, 129, 700, 1000], 128, torch.float32),
    ("mha_d64", 4, 4, 64, [5, 64, 300, 3000], 256, torch.float32),
    ("mqa_40_heads_two_head_blocks", 40, 1, 128, [1, 77, 2500], 512, torch.float32),
    ("zero_length_sequence", 8, 2, 128, [0, 50, 0], 128, torch.float32),
    # long chunks: each of a workgroup's two waves walks up to 64 (split 4096) or 128
    # (split 8192) 32-key blocks; and a chunk length that is not a power of two
    ("gqa4_d128_split4096", 8, 2, 128, [1, 4095, 4096, 4097, 9000], 4096, torch.bfloat16),
    ("gqa8_d64_split8192", 16, 2, 64, [383, 8191, 8192, 8193, 20000], 8192, torch.float32),
    ("gqa4_d128_split384", 8, 2, 128, [383, 384, 385, 1000, 3000], 384, torch.float32),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_decode_matches_oracle(case):
    name, Hq, Hkv, D, lens, split, odt = case
    say(f"decode case {name}")
    rng = np.random.default_rng(5)
    d = inputs.DecodeInputs(np.array(lens, dtype=np.int64),
                            inputs.bf16_round(rng.standard_normal((len(lens), Hq, D), dtype=np.float32)),
                            Hkv, D, seed=9)
    lmax = max(max(lens), 1) + 37
    kc, vc = build_cache(d, lmax)
    q = torch.from_numpy(d.q).to(DEV).to(torch.bfloat16)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o, lse = fa.decode(q, kc, vc, sl, max_len=max(lens), split_len=split, out_dtype=odt)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_decode(d, range(len(lens)))
    err = assert_fwd_close(to_host(o), to_host(lse), o_ref, lse_ref, odt == torch.bfloat16)
    say(f"  max|dO| = {err:.3e}")
    if odt == torch.float32:
        assert err < 4e-3


def test_decode_is_deterministic():
    rng = np.random.default_rng(6)
    lens = [3000, 4097, 1]
    d = inputs.DecodeInputs(np.array(lens), inputs.bf16_round(rng.standard_normal((3, 8, 128), dtype=np.float32)),
                            2, 128, seed=2)
    kc, vc = build_cache(d, 4200)
    q = torch.from_numpy(d.q).to(DEV).to(torch.bfloat16)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    a = fa.decode(q, kc, vc, sl, max_len=4200, split_len=1024)
    b = fa.decode(q, kc, vc, sl, max_len=4200, split_len=1024)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_full_size_c5_every_sequence():
    # 64 sequences, Hq 32, Hkv 8, D 128, lengths U[1024, 32768], chunks of 2048
    say("decode full c5")
    d = inputs.decode_inputs(64, 32, 8, 128, 1024, 32768, seed=0)
    lmax = 32768
    kc, vc = build_cache(d, lmax)
    q = torch.from_numpy(d.q).to(DEV).to(torch.bfloat16)
    sl = torch.tensor(d.seq_lens, dtype=torch.int32, device=DEV)
    o, lse = fa.decode(q, kc, vc, sl, max_len=lmax, split_len=2048)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    seqs = list(range(64))
    o_ref, lse_ref = oracle_decode(d, seqs)
    assert_fwd_close(to_host(o[seqs]), to_host(lse[seqs]), o_ref, lse_ref, True)


def test_decode_strided_cache_layout_gives_the_same_bits():
    # a [Bs, Lmax, Hkv, D] cache (heads interleaved per position) passed through strides
    rng = np.random.default_rng(7)
    lens = [2500, 700, 4100]
    d = inputs.DecodeInputs(np.array(lens), inputs.bf16_round(rng.standard_normal((3, 8, 128), dtype=np.float32)),
                            2, 128, seed=3)
    kc, vc = build_cache(d, 4200)
    q = torch.from_numpy(d.q).to(DEV).to(torch.bfloat16)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    a = fa.decode(q, kc, vc, sl, max_len=4200, split_len=1024)
    kn = kc.transpose(1, 2).contiguous().transpose(1, 2)
    vn = vc.transpose(1, 2).contiguous().transpose(1, 2)
    b = fa.decode(q, kn, vn, sl, max_len=4200, split_len=1024)
    torch.cuda.synchronize()
    assert kn.stride(2) == 2 * 128 and torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])

