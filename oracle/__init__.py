"""fp64 CPU oracle of the Slow-Fast Inference decode-attention path (``sfi_oracle``).

Test infrastructure only: ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it; it never imports the product package and the product never
imports it.  Every function is pinned by closed forms, library routines, brute force and
invariants in ``tests/test_oracle.py`` (the pages print no worked example).
"""
from .sfi_oracle import (  # noqa: F401
    candidate_range,
    recent_range,
    paged_rows,
    softmax_attention,
    dense_attention,
    group_scores,
    select_topk,
    pack_compact,
    sparse_decode,
    mixed,
    refresh_loop,
    append_token,
    indexed_decode,
    head_scores,
    indexed_decode_heads,
    draft_refresh_loop,
)
