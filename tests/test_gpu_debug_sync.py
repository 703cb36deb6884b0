"""Race canary: the FA_DEBUG_SYNC build of the library (every counted s_waitcnt a full
wait, every fence-free barrier preceded by a full drain of the wave's loads and LDS
reads) must give bit-identical outputs to the normal build on every entry point.  The
kernels' arithmetic does not depend on timing, so a difference would mean that some
counted wait lets a wave read LDS or registers before the data it needs has landed.
"""

import ctypes
import os

import numpy as np
import pytest
import torch

import io_aware_tiled_10_amd as fa
from io_aware_tiled_10_amd import binding, inputs
from tests.helpers import DEV, dense_cache_on_device, paged_pools, say, to_dev

pytestmark = pytest.mark.gpu

DEBUG_LIB = os.path.join(os.path.dirname(binding._LIB_PATH), "libfa_debugsync.so")


def both_builds(fn):
    """fn() under the normal build, then under the debug-sync build (cloned outputs)."""
    a = [t.clone() for t in fn()]
    torch.cuda.synchronize()
    prev = binding.use_library(DEBUG_LIB)
    try:
        b = [t.clone() for t in fn()]
        torch.cuda.synchronize()
    finally:
        binding.restore_library(prev)
    return a, b


def same_bits(a, b):
    return all(torch.equal(x.view(torch.uint8) if x.dtype != torch.uint8 else x,
                           y.view(torch.uint8) if y.dtype != torch.uint8 else y)
               for x, y in zip(a, b))


def test_debug_sync_build_exists_and_differs():
    assert os.path.exists(DEBUG_LIB), "build the library (python -m io_aware_tiled_10_amd.build)"
    assert open(DEBUG_LIB, "rb").read() != open(binding._LIB_PATH, "rb").read()


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
def test_forward_paths_give_the_same_bits(causal):
    say(f"debug-sync fwd causal={causal}")
    x = inputs.attention_inputs(2, 8, 2, 1100, 1100, 128, "bf16", seed=51)
    q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    kl = torch.tensor([1100, 613], dtype=torch.int32, device=DEV)
    x64 = inputs.attention_inputs(1, 4, 2, 700, 700, 64, "bf16", seed=52)
    q64, k64, v64 = to_dev(x64.q), to_dev(x64.k), to_dev(x64.v)
    xf = inputs.attention_inputs(1, 2, 2, 256, 256, 64, "fp32", seed=53)
    qf, kf, vf = (to_dev(t, torch.float32) for t in (xf.q, xf.k, xf.v))

    def run():
        o1, l1 = fa.fwd(q, k, v, causal=causal, kv_lens=kl)
        o2, l2 = fa.fwd(q64, k64, v64, causal=causal, out_dtype=torch.float32)
        o3, l3 = fa.fwd_dropout(q, k, v, 0.1, 99, causal=causal)
        o4, l4 = fa.fwd(qf, kf, vf, causal=causal)
        q8, qs = fa.quantize_fp8(q)
        k8, ks = fa.quantize_fp8(k)
        o5, l5 = fa.fwd_fp8(q8, qs, k8, ks, v, causal=causal)
        return o1, l1, o2, l2, o3, l3, o4, l4, q8, qs, o5, l5

    a, b = both_builds(run)
    assert same_bits(a, b)


def test_varlen_forward_gives_the_same_bits():
    say("debug-sync varlen")
    lens = [700, 1, 0, 1300, 257]
    x = inputs.varlen_inputs(lens, lens, 8, 2, 128, "bf16", seed=54)
    q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    cu = torch.from_numpy(x.cu_q).to(DEV)
    a, b = both_builds(lambda: fa.fwd_varlen(q, k, v, cu, cu, max(lens), causal=True))
    assert same_bits(a, b)


@pytest.mark.parametrize("drop", [0.0, 0.1], ids=["plain", "dropout"])
def test_backward_gives_the_same_bits(drop):
    say(f"debug-sync bwd p={drop}")
    x = inputs.attention_inputs(2, 8, 2, 900, 900, 128, "bf16", seed=55, with_grad=True)
    q, k, v, do = to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.do)
    x64 = inputs.attention_inputs(1, 2, 1, 500, 500, 64, "bf16", seed=56, with_grad=True)
    q6, k6, v6, do6 = to_dev(x64.q), to_dev(x64.k), to_dev(x64.v), to_dev(x64.do)
    if drop == 0:
        o, lse = fa.fwd(q, k, v, causal=True)
        o6, lse6 = fa.fwd(q6, k6, v6, causal=False)
        run = lambda: (*fa.bwd(q, k, v, o, do, lse, causal=True),
                       *fa.bwd(q6, k6, v6, o6, do6, lse6, causal=False))
    else:
        o, lse = fa.fwd_dropout(q, k, v, drop, 5, causal=True)
        o6, lse6 = fa.fwd_dropout(q6, k6, v6, drop, 5, causal=False)
        run = lambda: (*fa.bwd_dropout(q, k, v, o, do, lse, drop, 5, causal=True),
                       *fa.bwd_dropout(q6, k6, v6, o6, do6, lse6, drop, 5, causal=False))
    a, b = both_builds(run)
    assert same_bits(a, b)


def test_decode_contiguous_and_paged_give_the_same_bits():
    say("debug-sync decode")
    rng = np.random.default_rng(57)
    lens = np.array([1, 2048, 2049, 9000, 5000, 31])
    d = inputs.DecodeInputs(lens, inputs.bf16_round(rng.standard_normal((6, 8, 128), dtype=np.float32)), 2, 128,
                            seed=8)
    kc, vc = dense_cache_on_device(d, 9000)
    q = to_dev(d.q)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    kp, vp, table = paged_pools(kc, vc, lens, 16, seed=3)

    def run():
        o1, l1 = fa.decode(q, kc, vc, sl, max_len=9000, split_len=2048)
        o2, l2 = fa.decode_paged(q, kp, vp, table, sl, max_len=9000, split_len=1024)
        return o1, l1, o2, l2

    a, b = both_builds(run)
    assert same_bits(a, b)
