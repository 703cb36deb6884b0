"""The Python binding's argument checks, on the CPU.

The C ABI takes raw pointers: it trusts element types, the contiguity of LSE and of the
length / offset arrays, and the sizes of caller-supplied outputs.  The binding checks
them and raises ValueError before any library call.  Host tensors reach every check
except the last one (a GPU device is required), so each case here changes one property
of an otherwise valid host argument set and expects its specific message.
"""

import pytest
import torch

from io_aware_tiled_10_amd import binding as fb

bf = torch.bfloat16


def fwd_set(B=2, Hq=4, Hkv=2, N=16, D=64):
    q = torch.zeros(B, Hq, N, D, dtype=bf)
    k = torch.zeros(B, Hkv, N, D, dtype=bf)
    return q, k, k.clone()


def test_valid_host_arguments_stop_at_the_device_check():
    q, k, v = fwd_set()
    with pytest.raises(ValueError, match="GPU device"):
        fb.fwd(q, k, v)
    with pytest.raises(ValueError, match="GPU device"):
        fb.fwd(q, k, v, kv_lens=torch.tensor([16, 3], dtype=torch.int32))


@pytest.mark.parametrize("bad,match", [
    (dict(kv_lens=torch.tensor([16, 3])), "kv_lens has dtype torch.int64"),       # int64 default
    (dict(kv_lens=torch.tensor([16], dtype=torch.int32)), "kv_lens must be a 1-D tensor of 2"),
    (dict(kv_lens=torch.tensor([[16, 3]], dtype=torch.int32)), "kv_lens must be a 1-D"),
    (dict(kv_lens=torch.tensor([16, 0, 3, 0], dtype=torch.int32)[::2]), "kv_lens must be contiguous"),
    (dict(lse_out=torch.zeros(2, 4, 16, dtype=bf)), "lse_out has dtype"),
    (dict(lse_out=torch.zeros(2, 4, 15)), "lse_out has shape"),
    (dict(lse_out=torch.zeros(2, 16, 4).transpose(1, 2)), "lse_out must be contiguous"),
    (dict(out=torch.zeros(2, 4, 16, 32, dtype=bf)), "out has shape"),
    (dict(out=torch.zeros(2, 4, 16, 64, dtype=torch.float16)), "out has dtype"),
])
def test_forward_rejections(bad, match):
    q, k, v = fwd_set()
    with pytest.raises(ValueError, match=match):
        fb.fwd(q, k, v, **bad)
    with pytest.raises(ValueError, match=match):
        fb.fwd_dropout(q, k, v, 0.1, 1, **bad)


def test_forward_input_rejections():
    q, k, v = fwd_set()
    with pytest.raises(ValueError, match="v has dtype"):
        fb.fwd(q, k, v.float())
    with pytest.raises(ValueError, match="differ in shape"):
        fb.fwd(q, k, v[:, :, :8])
    with pytest.raises(ValueError, match="batch or head dim"):
        fb.fwd(q, k[:1], v[:1])
    with pytest.raises(ValueError, match="4 dimensions"):
        fb.fwd(q[0], k, v)
    with pytest.raises(ValueError, match="q has dtype"):
        fb.fwd(q.half(), k.half(), v.half())


def bwd_set():
    q, k, v = fwd_set()
    return q, k, v, q.clone(), q.clone(), torch.zeros(2, 4, 16)


@pytest.mark.parametrize("which,bad,match", [
    ("lse", torch.zeros(2, 4, 16, dtype=bf), "lse has dtype"),
    ("lse", torch.zeros(2, 4, 17), "lse has shape"),
    ("lse", torch.zeros(2, 16, 4).transpose(1, 2), "lse must be contiguous"),
    ("lse", None, "lse .* is required"),
    ("o", torch.zeros(2, 4, 16, 64), "o has dtype"),
    ("do", torch.zeros(2, 4, 8, 64, dtype=bf), "do has shape"),
])
def test_backward_input_rejections(which, bad, match):
    q, k, v, o, do, lse = bwd_set()
    args = dict(q=q, k=k, v=v, o=o, do=do, lse=lse)
    args[which] = bad
    with pytest.raises(ValueError, match=match):
        fb.bwd(**args)
    with pytest.raises(ValueError, match=match):
        fb.bwd_dropout(p_drop=0.1, seed=1, **args)


def test_backward_gradient_and_workspace_rejections():
    q, k, v, o, do, lse = bwd_set()
    with pytest.raises(ValueError, match="dk has shape"):
        fb.bwd(q, k, v, o, do, lse, grads=(torch.empty_like(q), torch.empty_like(q), torch.empty_like(v)))
    with pytest.raises(ValueError, match="dv has dtype"):
        fb.bwd(q, k, v, o, do, lse, grads=(torch.empty_like(q), torch.empty_like(k), torch.empty_like(v).float()))
    with pytest.raises(ValueError, match="kv_lens has dtype"):
        fb.bwd(q, k, v, o, do, lse, kv_lens=torch.tensor([3, 4]))
    with pytest.raises(ValueError, match="GPU device"):
        fb.bwd(q, k, v, o, do, lse)
    with pytest.raises(ValueError, match="q has dtype"):
        fb.bwd(q.float(), k.float(), v.float(), o.float(), do.float(), lse)


def dec_set(Bs=3, Hq=8, Hkv=2, L=64, D=128):
    q = torch.zeros(Bs, Hq, D, dtype=bf)
    kc = torch.zeros(Bs, Hkv, L, D, dtype=bf)
    return q, kc, kc.clone(), torch.tensor([5, 64, 1], dtype=torch.int32)


@pytest.mark.parametrize("bad,match", [
    (dict(seq_lens=torch.tensor([5, 64, 1])), "seq_lens has dtype"),
    (dict(seq_lens=torch.tensor([5, 64], dtype=torch.int32)), "seq_lens must be a 1-D tensor of 3"),
    (dict(seq_lens=None), "seq_lens is required"),
    (dict(lse_out=torch.zeros(3, 8, dtype=bf)), "lse_out has dtype"),
    (dict(lse_out=torch.zeros(8, 3).t()), "lse_out must be contiguous"),
    (dict(out=torch.zeros(3, 8, 64, dtype=bf)), "out has shape"),
    (dict(workspace=torch.zeros(64, dtype=torch.uint8)[::2]), "workspace must be contiguous"),
])
def test_decode_rejections(bad, match):
    q, kc, vc, sl = dec_set()
    args = dict(seq_lens=sl)
    args.update(bad)
    with pytest.raises(ValueError, match=match):
        fb.decode(q, kc, vc, **args)


def test_decode_input_rejections():
    q, kc, vc, sl = dec_set()
    with pytest.raises(ValueError, match="k_cache has dtype"):
        fb.decode(q, kc.float(), vc.float(), sl)
    with pytest.raises(ValueError, match="differ in shape"):
        fb.decode(q, kc, vc[:, :, :32], sl)
    with pytest.raises(ValueError, match="sequences or head dim"):
        fb.decode(q[:2], kc, vc, sl[:2])
    with pytest.raises(ValueError, match="GPU device"):
        fb.decode(q, kc, vc, sl)


def test_paged_decode_rejections():
    q = torch.zeros(2, 8, 128, dtype=bf)
    pool = torch.zeros(10, 2, 16, 128, dtype=bf)
    table = torch.zeros(2, 4, dtype=torch.int32)
    sl = torch.tensor([30, 64], dtype=torch.int32)
    with pytest.raises(ValueError, match="block_table has dtype"):
        fb.decode_paged(q, pool, pool, table.long(), sl, max_len=64)
    with pytest.raises(ValueError, match="block_table must be"):
        fb.decode_paged(q, pool, pool, table[:1], sl, max_len=64)
    with pytest.raises(ValueError, match="seq_lens has dtype"):
        fb.decode_paged(q, pool, pool, table, sl.long(), max_len=64)
    with pytest.raises(ValueError, match="GPU device"):
        fb.decode_paged(q, pool, pool, table, sl, max_len=64)


def test_varlen_rejections():
    q = torch.zeros(40, 4, 64, dtype=bf)
    k = torch.zeros(40, 2, 64, dtype=bf)
    cu = torch.tensor([0, 10, 40], dtype=torch.int32)
    with pytest.raises(ValueError, match="cu_seqlens_q has dtype"):
        fb.fwd_varlen(q, k, k, cu.long(), cu, 30)
    with pytest.raises(ValueError, match="cu_seqlens_k must be a 1-D tensor of 3"):
        fb.fwd_varlen(q, k, k, cu, cu[:2], 30)
    with pytest.raises(ValueError, match="lse_out has shape"):
        fb.fwd_varlen(q, k, k, cu, cu, 30, lse_out=torch.zeros(40, 4))
    with pytest.raises(ValueError, match="GPU device"):
        fb.fwd_varlen(q, k, k, cu, cu, 30)


def test_fp8_rejections():
    x = torch.zeros(1, 2, 100, 128, dtype=bf)
    with pytest.raises(ValueError, match="x has dtype"):
        fb.quantize_fp8(x.float())
    with pytest.raises(ValueError, match="scales_out has shape"):
        fb.quantize_fp8(x, scales_out=torch.zeros(1, 2, 1))
    with pytest.raises(ValueError, match="GPU device"):
        fb.quantize_fp8(x)
    q8 = torch.zeros(1, 2, 100, 128, dtype=torch.uint8)
    k8 = torch.zeros(1, 1, 100, 128, dtype=torch.uint8)
    v = torch.zeros(1, 1, 100, 128, dtype=bf)
    qs, ks = torch.ones(1, 2, 2), torch.ones(1, 1, 2)
    with pytest.raises(ValueError, match="q_scales has shape"):
        fb.fwd_fp8(q8, qs[:, :, :1], k8, ks, v)
    with pytest.raises(ValueError, match="k8 has dtype"):
        fb.fwd_fp8(q8, qs, k8.to(bf), ks, v)
    with pytest.raises(ValueError, match="GPU device"):
        fb.fwd_fp8(q8, qs, k8, ks, v)
