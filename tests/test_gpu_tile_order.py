"""Tile order with many (batch entry, KV head) groups per XCD.

When one XCD holds more groups than its L2 can serve at once, the kernels take its groups
a few at a time: one at a time without the causal mask (every tile does the same work),
and with it enough groups for a few tiles per compute unit, longest first inside each
batch of groups.  These shapes make every XCD take its groups in several batches, so a
tile that the order skipped or ran twice would leave rows unwritten or wrong.  Outputs are
pre-filled with NaN; every row must come out finite, the forward must match the oracle on
every (batch entry, head) slice and the backward on slices spread over the batch.
"""

import numpy as np
import pytest
import torch

import io_aware_tiled_10_amd as fa
import oracle
from io_aware_tiled_10_amd import inputs
from tests.helpers import DEV, assert_fwd_close, rel_l2, say, to_dev, to_host

pytestmark = pytest.mark.gpu

# name, B, H, N, D, causal: 16 x 16 groups = 32 per XCD; with 4 tiles of 256 rows per group
# the causal forward takes them 16 at a time and the causal dK/dV kernel (8 key tiles per
# group) 16 at a time; 8 x 16 groups without the mask are taken one at a time
CASES = [
    ("b16h16n1024_causal", 16, 16, 1024, 64, True),
    ("b8h16n512_noncausal", 8, 16, 512, 64, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_grouped_tile_order_covers_every_tile(case):
    name, B, H, N, D, causal = case
    say(f"tile order {name}")
    x = inputs.attention_inputs(B, H, H, N, N, D, "bf16", seed=31, with_grad=True)
    q, k, v, do = to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.do)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=DEV)
    fa.fwd(q, k, v, causal=causal, out=o, lse_out=lse)
    grads = tuple(torch.full_like(t, float("nan")) for t in (q, k, v))
    fa.bwd(q, k, v, o, do, lse, causal=causal, grads=grads)
    torch.cuda.synchronize()
    oh, lh = to_host(o), to_host(lse)
    gh = [to_host(g) for g in grads]
    assert np.all(np.isfinite(oh)) and np.all(np.isfinite(lh))
    for nm, g in zip(("dq", "dk", "dv"), gh):
        assert np.all(np.isfinite(g)), nm

    for b in range(B):  # the forward of every slice, one batch entry at a time
        o_ref, l_ref = oracle.attn_fwd(x.q[b:b + 1], x.k[b:b + 1], x.v[b:b + 1], None, causal)
        assert_fwd_close(oh[b:b + 1], lh[b:b + 1], o_ref, l_ref, True)
    say(f"  forward: all {B * H} slices match the oracle")

    for b, h in [(0, 0), (0, H - 1), (B // 2, 3), (B // 2 + 1, H // 2), (B - 1, 7), (B - 1, H - 1)]:
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oracle.attn_bwd(x.q[sl], x.k[sl], x.v[sl], x.do[sl], None, causal)[:3]
        for nm, g, r in zip(("dq", "dk", "dv"), gh, ref):
            e = rel_l2(g[sl], r)
            assert e <= 2e-2, (b, h, nm, e)
    say("  backward: sampled slices match the oracle")
