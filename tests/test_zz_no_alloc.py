"""fa_decode_noalloc (the decode whose partials live in the library's static per-device
array) against fa_decode (caller-supplied workspace) through the C ABI: the same
kernels on the same inputs, so the outputs must be bit-identical.  Two calls in a row,
the second smaller than the first, so the second reuses an array holding the first
call's partials; the second is also checked against the oracle.
"""

import numpy as np
import pytest
import torch

import io_aware_tiled_10_amd as fa
import oracle
from io_aware_tiled_10_amd import inputs
from tests.helpers import DEV, assert_fwd_close, dense_cache_on_device, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def case(lens, Hq, Hkv, seed):
    rng = np.random.default_rng(seed)
    lens = np.array(lens)
    d = inputs.DecodeInputs(lens, inputs.bf16_round(rng.standard_normal((len(lens), Hq, 128), dtype=np.float32)),
                            Hkv, 128, seed=seed)
    lmax = int(lens.max())
    kc, vc = dense_cache_on_device(d, lmax)
    return d, to_dev(d.q), kc, vc, torch.tensor(lens, dtype=torch.int32, device=DEV), lmax


def both(q, kc, vc, sl, lmax, split, out_dtype):
    ref_o, ref_l = fa.decode(q, kc, vc, sl, max_len=lmax, split_len=split, out_dtype=out_dtype)
    o = torch.empty_like(ref_o)
    lse = torch.empty_like(ref_l)
    fa.decode_noalloc(q, kc, vc, sl, out=o, lse_out=lse, max_len=lmax, split_len=split)
    torch.cuda.synchronize()
    return o, lse, ref_o, ref_l


def test_noalloc_decode_equals_the_workspace_decode_on_two_calls_in_a_row():
    say("noalloc decode: call 1 (16 sequences up to 32768 keys, 16 chunks)")
    lens1 = np.random.default_rng(70).integers(1024, 32768, size=16, endpoint=True)
    lens1[0] = 32768
    _, q, kc, vc, sl, lmax = case(lens1, 32, 8, 70)
    o, lse, ro, rl = both(q, kc, vc, sl, lmax, 2048, torch.bfloat16)
    assert torch.equal(o, ro) and torch.equal(lse, rl)
    assert torch.isfinite(o.float()).all()
    del q, kc, vc
    say("noalloc decode: call 2 (5 sequences up to 5000 keys, fp32 out)")
    d, q, kc, vc, sl, lmax = case([1, 5000, 2048, 0, 777], 8, 2, 71)
    o, lse, ro, rl = both(q, kc, vc, sl, lmax, 1024, torch.float32)
    assert torch.equal(o, ro) and torch.equal(lse, rl)
    o_ref = np.zeros((5, 8, 128))
    l_ref = np.full((5, 8), -np.inf)
    for s in range(5):
        if d.seq_lens[s]:
            k, v = d.kv(s)
            oo, ll = oracle.attn_decode(d.q[s:s + 1], k[None], v[None], [int(d.seq_lens[s])])
            o_ref[s], l_ref[s] = oo[0], ll[0]
    assert_fwd_close(to_host(o), to_host(lse), o_ref, l_ref, False)


def test_noalloc_decode_refuses_work_beyond_its_array():
    # 64 sequences x 32 heads x 33 chunks of partials exceed 32 MiB: refused on the host
    q = torch.zeros((64, 32, 128), dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros((64, 8, 1, 128), dtype=torch.bfloat16, device=DEV).expand(64, 8, 33 * 1024, 128)
    sl = torch.full((64,), 33 * 1024, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    with pytest.raises(fa.FaError, match="WORKSPACE"):
        fa.decode_noalloc(q, kc, kc, sl, out=out, split_len=1024)
