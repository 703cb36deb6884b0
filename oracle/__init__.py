"""fp64 CPU oracle for exact attention -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg import this package.  It shares no code with the HIP library.
"""

from .attention import (  # noqa: F401
    attn_bwd,
    attn_bwd_dkdv_rows,
    attn_bwd_dq_rows,
    attn_decode,
    attn_decode_paged,
    attn_fwd,
    attn_fwd_varlen,
    decode_split_partials,
    materialised_score_bytes,
    merge_partials,
    online_softmax_attention,
    visible_mask,
)
