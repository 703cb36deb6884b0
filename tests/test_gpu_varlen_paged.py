"""GPU parity of the packed variable-length forward (fa_fwd_varlen) and of the
paged-cache decode (fa_decode_paged) against the fp64 oracle.

Both variants only change how rows are addressed, so besides the oracle they are
checked bitwise against the dense forward / contiguous decode on the same data.
Packed rows past the last offset, page rows past a sequence and spare pages hold
NaN: any read of them into a result would show as a non-finite output.
"""

import numpy as np
import pytest
import torch

import io_aware_tiled_10_amd as fa
import oracle
from io_aware_tiled_10_amd import inputs
from tests.helpers import (DEV, assert_fwd_close, dense_cache_on_device, paged_pools, say, to_dev,
                           to_host)

pytestmark = pytest.mark.gpu

# ------------------------------------------------------------------------------------
# packed variable-length forward
# ------------------------------------------------------------------------------------

VARLEN = [
    # name, lens_q, lens_k, Hq, Hkv, D, causal
    ("ragged_causal_d128", [300, 513, 77, 1], [300, 513, 77, 1], 4, 2, 128, True),
    ("ragged_noncausal_d128", [300, 64, 257], [450, 700, 33], 4, 1, 128, False),
    ("empty_q_and_k_seqs", [40, 0, 260, 30], [0, 50, 260, 90], 2, 2, 128, True),
    ("nq_gt_nk_masked_rows_d64", [200, 129], [70, 300], 4, 2, 64, True),
    # groups of 4 query heads per KV head, causal: tiles of 64 rows x 4 heads
    ("gqa4_causal_ragged", [700, 65, 300], [700, 65, 300], 8, 2, 128, True),
    ("gqa4_causal_nq_ne_nk_d64", [150, 400], [300, 390], 8, 2, 64, True),
    # mid sizes: long block loops beside short sequences in one packed batch
    ("gqa4_causal_mid_sizes", [1500, 2049, 33, 900], [1500, 2049, 33, 900], 8, 2, 128, True),
]


def run_varlen(lq, lk, Hq, Hkv, D, causal, out_dtype, pad_rows=5):
    x = inputs.varlen_inputs(lq, lk, Hq, Hkv, D, "bf16", seed=21)
    nanrows = lambda a: np.concatenate([a, np.full((pad_rows,) + a.shape[1:], np.nan, np.float32)])
    q, k, v = to_dev(nanrows(x.q)), to_dev(nanrows(x.k)), to_dev(nanrows(x.v))
    cu_q = torch.from_numpy(x.cu_q).to(DEV)
    cu_k = torch.from_numpy(x.cu_k).to(DEV)
    o, lse = fa.fwd_varlen(q, k, v, cu_q, cu_k, max(lq), causal=causal, out_dtype=out_dtype)
    torch.cuda.synchronize()
    tq = int(x.cu_q[-1])
    o_ref, lse_ref = oracle.attn_fwd_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, None, causal)
    return x, (q, k, v, cu_q, cu_k), to_host(o[:tq]), to_host(lse[:, :tq]), o_ref, lse_ref


@pytest.mark.parametrize("case", VARLEN, ids=[c[0] for c in VARLEN])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["oF32", "oBF16"])
def test_fwd_varlen_matches_oracle(case, out_dtype):
    name, lq, lk, Hq, Hkv, D, causal = case
    say(f"fwd_varlen {name} out={out_dtype}")
    _, _, o, lse, o_ref, lse_ref = run_varlen(lq, lk, Hq, Hkv, D, causal, out_dtype)
    err = assert_fwd_close(o, lse, o_ref, lse_ref, out_dtype == torch.bfloat16)
    if out_dtype == torch.float32:
        assert err < 4e-3


@pytest.mark.parametrize("case", VARLEN[:2], ids=[c[0] for c in VARLEN[:2]])
def test_fwd_varlen_equals_dense_forward_per_sequence(case):
    # the same tiles, relative to each sequence's first row: bit for bit the dense call
    name, lq, lk, Hq, Hkv, D, causal = case
    say(f"fwd_varlen vs dense {name}")
    x, (q, k, v, cu_q, cu_k), *_ = run_varlen(lq, lk, Hq, Hkv, D, causal, torch.float32)
    o, lse = fa.fwd_varlen(q, k, v, cu_q, cu_k, max(lq), causal=causal, out_dtype=torch.float32)
    for b in range(len(lq)):
        q0, q1, k0, k1 = (int(t) for t in (x.cu_q[b], x.cu_q[b + 1], x.cu_k[b], x.cu_k[b + 1]))
        od, ld = fa.fwd(q[q0:q1].transpose(0, 1)[None], k[k0:k1].transpose(0, 1)[None],
                        v[k0:k1].transpose(0, 1)[None], causal=causal, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(o[q0:q1], od[0].transpose(0, 1)) and torch.equal(lse[:, q0:q1], ld[0])


def test_fwd_varlen_many_sequences_full_tiles():
    # 24 sequences of U[1, 1200] rows, GQA 4:1, causal: several tiles per sequence
    lens = [int(x) for x in inputs.ragged_lengths(24, 1, 1200, seed=3)]
    say(f"fwd_varlen 24 seqs, total {sum(lens)}")
    _, _, o, lse, o_ref, lse_ref = run_varlen(lens, lens, 8, 2, 128, True, torch.bfloat16)
    assert_fwd_close(o, lse, o_ref, lse_ref, True)


# ------------------------------------------------------------------------------------
# paged-cache decode
# ------------------------------------------------------------------------------------

PAGED = [
    # name, Hq, Hkv, D, lens, page, split, row-major heads, out dtype
    ("p16_d128", 8, 2, 128, [1, 15, 16, 17, 100, 2049, 3000], 16, 2048, False, torch.float32),
    ("p32_d128_split128", 8, 2, 128, [1, 31, 33, 129, 700], 32, 128, False, torch.float32),
    ("p64_rowmajor", 8, 2, 128, [64, 65, 1000, 4097], 64, 1024, True, torch.bfloat16),
    ("p256_d64_mha", 4, 4, 64, [5, 255, 256, 257, 3000], 256, 256, False, torch.float32),
    ("p16_d64_rowmajor_zero_len", 8, 1, 64, [0, 50, 0, 17], 16, 128, True, torch.float32),
    # 4096-key chunks: a wave's blocks 32-63 take their pages from the second page-id register
    ("p16_d128_split4096", 8, 2, 128, [1, 2049, 4095, 4096, 4097, 9000], 16, 4096, False, torch.float32),
    ("p128_d64_split4096", 8, 2, 64, [2100, 4096, 8191], 128, 4096, True, torch.bfloat16),
]


def paged_inputs(Hq, Hkv, D, lens, page, rowmajor, seed=9):
    rng = np.random.default_rng(seed)
    d = inputs.DecodeInputs(np.array(lens, dtype=np.int64),
                            inputs.bf16_round(rng.standard_normal((len(lens), Hq, D), dtype=np.float32)),
                            Hkv, D, seed=seed)
    lmax = max(max(lens), 1)
    kc, vc = dense_cache_on_device(d, lmax)
    kp, vp, table = paged_pools(kc, vc, lens, page, seed=seed, spare=3, row_major_heads=rowmajor)
    q = torch.from_numpy(d.q).to(DEV).to(torch.bfloat16)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    return d, q, sl, kc, vc, kp, vp, table


def oracle_decode(d, seqs):
    o = np.zeros((len(seqs), d.q.shape[1], d.D))
    lse = np.zeros((len(seqs), d.q.shape[1]))
    for n, s in enumerate(seqs):
        k, v = d.kv(s)
        oo, ll = oracle.attn_decode(d.q[s:s + 1], k[None], v[None], [int(d.seq_lens[s])])
        o[n], lse[n] = oo[0], ll[0]
    return o, lse


@pytest.mark.parametrize("case", PAGED, ids=[c[0] for c in PAGED])
def test_decode_paged_matches_oracle_and_contiguous(case):
    name, Hq, Hkv, D, lens, page, split, rowmajor, odt = case
    say(f"decode_paged {name}")
    d, q, sl, kc, vc, kp, vp, table = paged_inputs(Hq, Hkv, D, lens, page, rowmajor)
    o, lse = fa.decode_paged(q, kp, vp, table, sl, max_len=max(lens), split_len=split, out_dtype=odt)
    oc, lc = fa.decode(q, kc, vc, sl, max_len=max(lens), split_len=split, out_dtype=odt)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_decode(d, range(len(lens)))
    err = assert_fwd_close(to_host(o), to_host(lse), o_ref, lse_ref, odt == torch.bfloat16)
    if odt == torch.float32:
        assert err < 4e-3
    # the same blocks and chunks as the contiguous decode: bit for bit its result
    assert torch.equal(o, oc) and torch.equal(lse, lc)


def test_decode_paged_page_id_outside_pool_reads_zeros():
    lens = [100, 70]
    d, q, sl, kc, vc, kp, vp, table = paged_inputs(8, 2, 128, lens, 16, False, seed=4)
    table[0, 2] = kp.shape[0] + 5    # positions 32..47 of sequence 0
    table[1, 0] = -7                 # positions 0..15 of sequence 1
    o, lse = fa.decode_paged(q, kp, vp, table, sl, max_len=100, split_len=128, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref = np.zeros((2, 8, 128))
    lse_ref = np.zeros((2, 8))
    for s, (lo, hi) in enumerate([(32, 48), (0, 16)]):
        k, v = d.kv(s)
        k, v = k.copy(), v.copy()
        k[:, lo:hi] = 0.0
        v[:, lo:hi] = 0.0
        oo, ll = oracle.attn_decode(d.q[s:s + 1], k[None], v[None], [lens[s]])
        o_ref[s], lse_ref[s] = oo[0], ll[0]
    assert_fwd_close(to_host(o), to_host(lse), o_ref, lse_ref, False)


@pytest.mark.parametrize("page", [16, 256])
def test_decode_paged_full_size_c5(page):
    # 64 sequences, Hq 32, Hkv 8, D 128, lengths U[1024, 32768], chunks of 2048
    say(f"decode_paged full c5 page {page}")
    d = inputs.decode_inputs(64, 32, 8, 128, 1024, 32768, seed=0)
    kc, vc = dense_cache_on_device(d, 32768)
    kp, vp, table = paged_pools(kc, vc, d.seq_lens, page, seed=1)
    q = torch.from_numpy(d.q).to(DEV).to(torch.bfloat16)
    sl = torch.tensor(d.seq_lens, dtype=torch.int32, device=DEV)
    lmax = int(d.seq_lens.max())  # the table covers the longest sequence
    o, lse = fa.decode_paged(q, kp, vp, table, sl, max_len=lmax, split_len=2048)
    oc, lc = fa.decode(q, kc, vc, sl, max_len=lmax, split_len=2048)
    torch.cuda.synchronize()
    assert torch.equal(o, oc) and torch.equal(lse, lc)
    seqs = [int(np.argmin(d.seq_lens)), int(np.argmax(d.seq_lens)), 5]
    o_ref, lse_ref = oracle_decode(d, seqs)
    assert_fwd_close(to_host(o[seqs]), to_host(lse[seqs]), o_ref, lse_ref, True)
