"""The entry points under HIP graph capture.

A forward, the backward that consumes its O and LSE, and the allocation-free decode are
captured once into one graph, with every buffer allocated before the capture.  The graph
is replayed several times with eager work (the outputs overwritten) and synchronisations
between the replays.  Every replay must give the bits of the same calls made eagerly:
all three paths are deterministic, and none of them records a memset.  The eager
results are also checked against the oracle, so the replays are too.
"""

import numpy as np
import pytest
import torch

import io_aware_tiled_10_amd as fa
import oracle
from io_aware_tiled_10_amd import inputs
from tests.helpers import DEV, assert_fwd_close, dense_cache_on_device, rel_l2, say, to_dev, to_host

pytestmark = pytest.mark.gpu


class Buffers:
    """Outputs of one forward + backward + decode pass."""

    def __init__(self, q, k, dq_lens):
        self.o = torch.empty_like(q)
        self.lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
        self.grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(k))
        self.od = torch.empty(dq_lens, dtype=torch.bfloat16, device=DEV)
        self.ld = torch.empty(dq_lens[:2], dtype=torch.float32, device=DEV)

    def tensors(self):
        return [self.o, self.lse, *self.grads, self.od, self.ld]


def test_fwd_bwd_decode_graph_replays_match_eager():
    say("graph: fwd + bwd (B1 Hq8 Hkv2 N1000 D128 causal) + noalloc decode (3 sequences)")
    B, Hq, Hkv, N, D = 1, 8, 2, 1000, 128
    x = inputs.attention_inputs(B, Hq, Hkv, N, N, D, "bf16", seed=90, with_grad=True)
    q, k, v, do = to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.do)
    ws = torch.empty(fa.binding.bwd_workspace_bytes(q, k, v), dtype=torch.uint8, device=DEV)

    lens = np.array([900, 3000, 17])
    rng = np.random.default_rng(91)
    dd = inputs.DecodeInputs(lens, inputs.bf16_round(rng.standard_normal((3, 8, D), dtype=np.float32)),
                             2, D, seed=91)
    lmax = int(lens.max())
    kc, vc = dense_cache_on_device(dd, lmax)
    qd = to_dev(dd.q)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)

    def body(bf):
        fa.fwd(q, k, v, causal=True, out=bf.o, lse_out=bf.lse)
        fa.bwd(q, k, v, bf.o, do, bf.lse, causal=True, workspace=ws, grads=bf.grads)
        fa.decode_noalloc(qd, kc, vc, sl, out=bf.od, lse_out=bf.ld, max_len=lmax, split_len=1024)

    eager = Buffers(q, k, tuple(qd.shape))
    body(eager)
    torch.cuda.synchronize()

    # the eager pass against the oracle
    o_ref, l_ref = oracle.attn_fwd(x.q, x.k, x.v, None, True)
    assert_fwd_close(to_host(eager.o), to_host(eager.lse), o_ref, l_ref, True)
    dq_r, dk_r, dv_r = oracle.attn_bwd(x.q, x.k, x.v, x.do, None, True)[:3]
    for nm, g, r in zip(("dq", "dk", "dv"), eager.grads, (dq_r, dk_r, dv_r)):
        e = rel_l2(to_host(g), r)
        say(f"  eager {nm} rel-L2 {e:.3e}")
        assert e <= 2e-2, (nm, e)
    od_ref = np.zeros((3, 8, D))
    ld_ref = np.full((3, 8), -np.inf)
    for s in range(3):
        kk, vv = dd.kv(s)
        oo, ll = oracle.attn_decode(dd.q[s:s + 1], kk[None], vv[None], [int(lens[s])])
        od_ref[s], ld_ref[s] = oo[0], ll[0]
    assert_fwd_close(to_host(eager.od), to_host(eager.ld), od_ref, ld_ref, True)

    graphed = Buffers(q, k, tuple(qd.shape))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one pass on a side stream before capture
        body(graphed)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body(graphed)
    torch.cuda.synchronize()

    for rep in range(3):
        for t in graphed.tensors():  # eager work between replays: overwrite every output
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv", "decode o", "decode lse"),
                              graphed.tensors(), eager.tensors()):
            assert torch.equal(a, b), (rep, name)
        say(f"  replay {rep}: bit-identical to the eager pass")
    del g
