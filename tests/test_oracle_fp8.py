"""Pins of the oracle's E4M3 block quantisation and FP8 forward (no GPU).

The encoder is pinned to torch's float8_e4m3fn conversion (an independent library
routine) on random values, on every exact tie and on every code; the two-pass
quantiser to the properties the article's formula fixes (the block maximum lands on
448, the step is max|x| / 448, the rounding error is at most half an E4M3 step); the
FP8 forward to the plain forward on inputs that quantise without loss.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8
from io_aware_tiled_10_amd import inputs


def torch_codes(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encoder_matches_torch_on_random_values():
    rng = np.random.default_rng(0)
    parts = [rng.uniform(-448, 448, 100000), rng.standard_normal(100000) * 3,
             rng.uniform(-2 ** -6, 2 ** -6, 50000), rng.uniform(-1, 1, 50000) * 2.0 ** rng.integers(-12, 8, 50000)]
    x = np.concatenate(parts).astype(np.float32)
    np.testing.assert_array_equal(fp8.e4m3_encode(x), torch_codes(x))


def test_encoder_ties_go_to_the_even_code():
    v = fp8.e4m3_values()
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)   # exact in fp32
    for s in (1.0, -1.0):
        np.testing.assert_array_equal(fp8.e4m3_encode(s * mids), torch_codes(s * mids))
    codes = fp8.e4m3_encode(mids)
    assert np.all(codes % 2 == 0)


def test_decode_is_exact_for_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    np.testing.assert_array_equal(fp8.e4m3_decode(codes), ref.astype(np.float64))
    assert fp8.e4m3_decode(np.uint8(0x7E)) == 448.0
    assert fp8.e4m3_decode(np.uint8(0x01)) == 2.0 ** -9
    np.testing.assert_array_equal(fp8.e4m3_encode(fp8.e4m3_values()), np.arange(0x7F, dtype=np.uint8))


def test_block_quantiser_properties():
    rng = np.random.default_rng(1)
    x = inputs.bf16_round(rng.standard_normal((2, 3, 150, 64)).astype(np.float32))
    x[1, 2, 64:128] = 0.0                                       # an all-zero block
    codes, delta = fp8.quantize_blocks(x, 64)
    assert delta.shape == (2, 3, 3) and delta.dtype == np.float32
    assert delta[1, 2, 1] == 1.0 and np.all(codes[1, 2, 64:128] == 0)
    for b in range(2):
        for h in range(3):
            for j in range(3):
                xs = x[b, h, 64 * j:64 * (j + 1)]
                if not np.any(xs):
                    continue
                assert delta[b, h, j] == np.float32(np.abs(xs).max()) / np.float32(448.0)
                # the element of largest magnitude lands on +-448
                cs = codes[b, h, 64 * j:64 * (j + 1)]
                assert np.max(np.abs(fp8.e4m3_decode(cs))) == 448.0
    xd = fp8.dequantize_blocks(codes, delta, 64)
    # half an E4M3 step: relative 2^-4 for normal values, absolute 2^-10 * Delta below
    rep = np.repeat(delta.astype(np.float64), 64, axis=2)[:, :, :150, None]
    err = np.abs(xd - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * rep) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_planted_fnuz_range_is_caught():
    # a quantiser using 240 (the E4M3 "fnuz" maximum) instead of 448 breaks the pin above
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1, 1, 64, 16)).astype(np.float32)
    d_bad = np.float32(np.abs(x).max()) / np.float32(240.0)
    codes_bad = fp8.e4m3_encode(x / d_bad)
    assert np.max(np.abs(fp8.e4m3_decode(codes_bad))) != 448.0


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_forward_equals_plain_forward_on_exact_inputs(causal):
    # Q and K built as Delta * (E4M3 values) with max code 448 per block quantise with
    # no loss, so the FP8 forward must equal the plain forward on them
    rng = np.random.default_rng(3)
    vals = fp8.e4m3_values()
    def exact(shape, block):
        c = rng.integers(0, 0x7F, size=shape)
        c[:, :, ::block, 0] = 0x7E                                # each block holds 448
        sgn = np.where(rng.random(shape) < 0.5, -1.0, 1.0)
        d = 2.0 ** rng.integers(-8, -5, size=(shape[0], shape[1], (shape[2] + block - 1) // block))
        return (sgn * vals[c] * np.repeat(d, block, axis=2)[:, :, :shape[2], None]).astype(np.float32)
    q, k = exact((1, 2, 100, 32), 64), exact((1, 1, 130, 32), 64)
    v = rng.standard_normal((1, 1, 130, 32))
    qc, qd = fp8.quantize_blocks(q, 64)
    kc, kd = fp8.quantize_blocks(k, 64)
    np.testing.assert_array_equal(fp8.dequantize_blocks(qc, qd, 64), q)
    o8, l8 = fp8.attn_fwd_fp8(qc, qd, kc, kd, v, 64, None, causal)
    o, l = oracle.attn_fwd(q, k, v, None, causal)
    np.testing.assert_array_equal(o8, o)
    np.testing.assert_array_equal(l8, l)
