"""GPU parity of the E4M3 path: fa_quantize_fp8 bit for bit against the oracle's
two-pass quantiser, and fa_fwd_fp8 against the oracle's FP8 forward (which quantises
the same bf16 inputs itself and attends with the dequantised Q and K in fp64).

Given the quantised values, the kernel's remaining arithmetic is that of the bf16
forward (exact E4M3 products, fp32 sums, bf16 P), so the forward tolerances apply.
"""

import numpy as np
import pytest
import torch

import io_aware_tiled_10_amd as fa
from io_aware_tiled_10_amd import inputs
from oracle import fp8 as ofp8
from tests.helpers import DEV, assert_fwd_close, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def test_quantize_matches_oracle_bit_for_bit():
    say("quantize fp8")
    x = inputs.attention_inputs(2, 3, 3, 150, 150, 128, "bf16", seed=13).q
    x[1, 2, 64:128] = 0.0           # an all-zero block
    x[0, 1, 5, 7] = -0.0
    x[0, 0, 3] *= 40.0              # a block with a wide range (subnormal codes appear)
    x = inputs.bf16_round(x)
    codes, sc = fa.quantize_fp8(to_dev(x))
    torch.cuda.synchronize()
    ref_codes, ref_sc = ofp8.quantize_blocks(x, 64)
    np.testing.assert_array_equal(sc.cpu().numpy(), ref_sc)
    np.testing.assert_array_equal(codes.cpu().numpy(), ref_codes)


CASES = [
    # name, B, Hq, Hkv, Nq, Nk, causal, kv_lens
    ("mha_ragged_noncausal", 2, 2, 2, 300, 300, False, None),
    ("gqa_ragged_causal", 1, 8, 2, 257, 257, True, None),
    ("causal_nq_lt_nk", 1, 2, 1, 100, 333, True, None),
    ("kvlens", 2, 2, 1, 130, 300, False, [300, 61]),
    # mid sizes: the block loop runs for many trips, across many 64-row scale blocks
    ("gqa4_n1100_causal", 1, 8, 2, 1100, 1100, True, None),
    ("mha_nq700_nk1500_kvlens_causal", 2, 2, 2, 700, 1500, True, [1500, 333]),
]


def run_fp8(B, Hq, Hkv, Nq, Nk, causal, kv_lens, out_dtype, seed=0):
    x = inputs.attention_inputs(B, Hq, Hkv, Nq, Nk, 128, "bf16", seed=seed)
    q8, qs = fa.quantize_fp8(to_dev(x.q))
    k8, ks = fa.quantize_fp8(to_dev(x.k))
    kl = torch.tensor(kv_lens, dtype=torch.int32, device=DEV) if kv_lens is not None else None
    o, lse = fa.fwd_fp8(q8, qs, k8, ks, to_dev(x.v), causal=causal, kv_lens=kl, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return x, to_host(o), to_host(lse)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["oF32", "oBF16"])
def test_fwd_fp8_matches_oracle(case, out_dtype):
    name, B, Hq, Hkv, Nq, Nk, causal, kv_lens = case
    say(f"fwd_fp8 {name} out={out_dtype}")
    x, o, lse = run_fp8(B, Hq, Hkv, Nq, Nk, causal, kv_lens, out_dtype)
    qc, qd = ofp8.quantize_blocks(x.q, 64)
    kc, kd = ofp8.quantize_blocks(x.k, 64)
    qf = ofp8.dequantize_blocks(qc, qd, 64)
    kf = ofp8.dequantize_blocks(kc, kd, 64)
    import oracle
    o_ref, lse_ref = oracle.attn_fwd(qf, kf, x.v, None, causal, kv_lens)
    err = assert_fwd_close(o, lse, o_ref, lse_ref, out_dtype == torch.bfloat16)
    say(f"  max|dO| = {err:.3e}")


def test_fwd_fp8_close_to_the_bf16_forward():
    # the quantisation error itself: E4M3 keeps 3 mantissa bits, so the FP8 result is
    # near, not equal to, the bf16 forward
    x, o, lse = run_fp8(1, 4, 2, 300, 300, True, None, torch.float32, seed=3)
    import oracle
    o_ref, lse_ref = oracle.attn_fwd(x.q, x.k, x.v, None, True)
    assert np.abs(o - o_ref).max() < 0.2 and np.abs(lse - lse_ref).max() < 0.1


def test_fwd_fp8_full_size_c3_sampled_rows():
    # B1 Hq32 Hkv8 N16384 D128 causal, quantised on the GPU; sampled rows of three heads
    say("fwd_fp8 full c3")
    B, Hq, Hkv, N = 1, 32, 8, 16384
    x = inputs.attention_inputs(B, Hq, Hkv, N, N, 128, "bf16", seed=0)
    q8, qs = fa.quantize_fp8(to_dev(x.q))
    k8, ks = fa.quantize_fp8(to_dev(x.k))
    o, lse = fa.fwd_fp8(q8, qs, k8, ks, to_dev(x.v), causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 63, 64, 255, 256, N - 1], rng.integers(0, N, 10)]))
    import oracle
    for h in (0, 17, 31):
        g = h // (Hq // Hkv)
        qc, qd = ofp8.quantize_blocks(x.q[:, h:h + 1], 64)
        kc, kd = ofp8.quantize_blocks(x.k[:, g:g + 1], 64)
        o_ref, lse_ref = oracle.attn_fwd(ofp8.dequantize_blocks(qc, qd, 64), ofp8.dequantize_blocks(kc, kd, 64),
                                         x.v[:, g:g + 1], None, True, None, rows)
        assert_fwd_close(to_host(o[:, h:h + 1, rows]), to_host(lse[:, h:h + 1, rows]), o_ref, lse_ref, True)
