"""Host-side checks of the seeded input generators (no attention arithmetic)."""

import numpy as np
import torch

from io_aware_tiled_10_amd import inputs


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000, dtype=np.float32) * 10
    # exact ties: values halfway between two bf16 numbers
    ties = ((np.arange(1, 2000, dtype=np.uint32) << 16) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = inputs.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(inputs.bf16_round(x), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_attention_inputs_are_seeded_and_bf16_valued():
    a = inputs.attention_inputs(1, 2, 1, 8, 8, 4, "bf16", seed=3, with_grad=True)
    b = inputs.attention_inputs(1, 2, 1, 8, 8, 4, "bf16", seed=3, with_grad=True)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v), (a.do, b.do)):
        np.testing.assert_array_equal(x, y)
        np.testing.assert_array_equal(inputs.bf16_round(x), x)
    c = inputs.attention_inputs(1, 2, 1, 8, 8, 4, "fp32", seed=3)
    assert not np.array_equal(inputs.bf16_round(c.q), c.q)


def test_decode_inputs_lengths_and_per_sequence_regeneration():
    d = inputs.decode_inputs(64, 32, 8, 128, 1024, 32768, seed=0)
    assert d.seq_lens.min() >= 1024 and d.seq_lens.max() <= 32768
    assert int(d.seq_lens.sum()) == 1101299
    assert int(np.sum(-(-d.seq_lens // 2048))) == 567
    small = inputs.decode_inputs(3, 4, 2, 8, 5, 9, seed=1)
    k1, v1 = small.kv(1)
    k2, v2 = small.kv(1)
    np.testing.assert_array_equal(k1, k2)
    kb, vb = small.kv_bits(1)
    np.testing.assert_array_equal((kb.astype(np.uint32) << 16).view(np.float32), k1)
    kc, vc = small.dense_cache(lmax=10)
    assert np.isnan(kc[1, :, int(small.seq_lens[1]):]).all()
    np.testing.assert_array_equal(kc[1, :, :int(small.seq_lens[1])], k1)


def test_varlen_offsets_and_shapes():
    x = inputs.varlen_inputs([3, 0, 5], [4, 2, 5], 4, 2, 8, "bf16", seed=1)
    np.testing.assert_array_equal(x.cu_q, [0, 3, 3, 8])
    np.testing.assert_array_equal(x.cu_k, [0, 4, 6, 11])
    assert x.q.shape == (8, 4, 8) and x.k.shape == (11, 2, 8) and x.v.shape == (11, 2, 8)
    np.testing.assert_array_equal(inputs.bf16_round(x.q), x.q)


def test_paged_cache_places_every_position_once():
    dec = inputs.decode_inputs(4, 4, 2, 8, 1, 50, seed=2)
    pc = inputs.paged_cache(dec, 16, seed=3, spare_pages=5)
    used = []
    for s, L in enumerate(dec.seq_lens):
        k, v = dec.kv(s)
        n = (int(L) + 15) // 16
        assert np.all(pc.block_table[s, n:] == -1)
        for t in range(int(L)):
            page = pc.block_table[s, t // 16]
            np.testing.assert_array_equal(pc.k_pages[page, :, t % 16], k[:, t])
            np.testing.assert_array_equal(pc.v_pages[page, :, t % 16], v[:, t])
        used += list(pc.block_table[s, :n])
    assert len(set(used)) == len(used)
    assert pc.k_pages.shape[0] == len(used) + 5
