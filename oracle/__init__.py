"""Plain, slow, fp64 CPU oracle for the Slow-Fast Inference decode-attention path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package imports, calls or
links anything here; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path: it never imports the product package and the product never imports it.

What it computes, with the passages it follows (SFI page =
thelatestinai.com/papers/2603.12038, "Slow-Fast Inference: Training-Free
Inference Acceleration via Within-Sentence Support Stability"):

* ``dense_attention``  - the slow step attends densely over the whole context (SFI page,
  Fig. 2 caption), plain softmax attention over every visible key; with
  ``t_q > 1`` it is the full-context causal verification of draft tokens
  (SparseSpec-L abstract, page 1 and page 3).
* ``group_scores``     - the masked attention logits the slow step collects over
  the allowed candidate set (SFI page, Fig. 2 caption), one row per KV head,
  summed over the query heads (and query tokens) that share that KV head
  (the per-head attention statistics of the SparseSpec-L abstract).
* ``select_topk``      - the Selector that refreshes the selected memory from
  those logits (SFI page, Abstract and Fig. 2): exact top-k, lowest index wins
  ties, output in ascending position order.
* ``pack_compact``     - sink and selected tokens packed into a contiguous
  compact buffer (SFI page, Fig. 3B).
* ``sparse_decode``    - the fast step: attention over the managed sparse state
  sink + selected + recent (Fig. 2), with sink and selected read from the
  compact buffer and recent read in place from paged KV (Fig. 3B).
* ``indexed_decode``   - the fast step with sink, selected and recent rows all read
  in place from paged KV through the block table (attention restricted to an index
  set).
* ``head_scores`` / ``indexed_decode_heads`` - per-query-head selection: the
  slow step's logits kept per query head, and the fast step with one set per query
  head (the per-head statistics of the SparseSpec-L abstract, not summed).
* ``draft_refresh_loop`` - draft steps of a layer stack whose designated layer
  attends densely and refreshes the selected set every step (ASPIRE abstract,
  page 1: intra-draft refresh layer).
* ``mixed``            - drafting and verifying requests in one batched call
  (ASPIRE abstract, page 1: one mixed forward pass for both kinds).

The pages print no worked example, so no value here is pinned to a number on
the pages; every function is pinned instead by closed forms, library routines,
brute force and invariants in ``tests/test_oracle.py``.
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
