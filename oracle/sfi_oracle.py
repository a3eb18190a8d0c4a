"""fp64 reference definitions of the SFI decode-attention path (test infrastructure only).

Citations name the page and the part of it that states the operation:
  SFI page     = "Slow-Fast Inference: Training-Free Inference Acceleration via
                  Within-Sentence Support Stability" (thelatestinai.com/papers/2603.12038)
  SparseSpec-L = "A Sparse Glimpse of the Whole: Train-Free Self-Speculative Decoding"
                  abstract (pages 1 and 3)
  ASPIRE       = ASPIRE abstract (page 1)

Conventions shared by every function (the pages fix none of them; each is one
of the readings listed in the design notes):
  * a paged pool has shape [num_pages, Hkv, page_size, d]; token j of a request
    sits at [block_table_row[j // page_size], g, j % page_size];
  * L counts every token of the request including its t_q query tokens; query
    token t sits at position L - t_q + t and sees keys [0, L - t_q + t];
  * query head h reads KV head h // G with G = Hq / Hkv;
  * logits are scale * q . k (scale is normally 1/sqrt(d)).

All arithmetic is float64.  Pools may be given as float arrays or, with
``kv_dtype="bf16"``, as raw uint16 bfloat16 bits, which are widened exactly.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np


# --------------------------------------------------------------------------- helpers

def _widen(rows: np.ndarray, kv_dtype: str) -> np.ndarray:
    """Exact float64 values of stored rows (bf16 bits are the top half of an fp32)."""
    if kv_dtype == "bf16":
        rows = (np.asarray(rows, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    return np.asarray(rows, dtype=np.float64)


def candidate_range(L: int, t_q: int, n_sink: int, n_recent: int) -> Tuple[int, int]:
    """The allowed candidate set of a slow step as a position range [lo, hi).

    SFI page, Fig. 2 caption: the slow step collects masked logits "over the
    allowed candidate set"; the fast state is sink + selected + recent, so sink
    and recent tokens are kept anyway and are not candidates.  The recent
    window is taken at the first query token (position L - t_q), so every
    candidate is visible to every query token of the call.
    """
    lo = n_sink
    hi = max(lo, L - t_q + 1 - n_recent)
    return lo, hi


def recent_range(L: int, n_sink: int, n_recent: int) -> Tuple[int, int]:
    """Recent tokens of a fast step, read in place from paged KV (SFI page, Fig. 3B):
    the last n_recent positions, never reaching into the sink."""
    start = min(max(n_sink, L - n_recent), L)
    return start, L


def paged_rows(pool: np.ndarray, block_table_row: np.ndarray, g: int,
               positions: Sequence[int], page_size: int = 16) -> np.ndarray:
    """Rows of KV head g at the given logical positions, located through the block table
    (paged KV, SFI page Fig. 3B).  Returns the stored values unchanged."""
    positions = np.asarray(positions, dtype=np.int64)
    pages = np.asarray(block_table_row, dtype=np.int64)[positions // page_size]
    return pool[pages, g, positions % page_size, :]


# --------------------------------------------------------------------------- attention

def softmax_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                      visible: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """out[r] = sum_j softmax_j(scale * q[r] . K[j]) V[j];  lse[r] = log sum_j exp(scale * q[r] . K[j]).

    q: [R, d], K and V: [N, d], visible: optional [R, N] booleans (False = key not seen).
    The maximum is subtracted before exponentiating, which leaves the result unchanged.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    s = scale * (q @ K.T)
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    l = w.sum(axis=1, keepdims=True)
    out = (w @ V) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


def dense_attention(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                    block_table_row: np.ndarray, L: int, scale: float, Hkv: int,
                    kv_dtype: str = "f32", groups: Optional[Sequence[int]] = None,
                    page_size: int = 16) -> Tuple[np.ndarray, np.ndarray]:
    """Dense attention of one request over its whole paged KV [0, L).

    SFI page, Fig. 2 caption: a slow step performs dense attention.  With
    t_q > 1 rows this is full-context verification of t_q draft tokens
    (SparseSpec-L abstract), causal: query token t sees keys [0, L - t_q + t].

    q: [t_q, Hq, d] values.  Returns out [t_q, Hq, d] and lse [t_q, Hq] (rows of
    KV heads not in ``groups`` are left as NaN).
    """
    q = np.asarray(q, dtype=np.float64)
    t_q, Hq, d = q.shape
    G = Hq // Hkv
    out = np.full((t_q, Hq, d), np.nan)
    lse = np.full((t_q, Hq), np.nan)
    pos = np.arange(L)
    for g in (range(Hkv) if groups is None else groups):
        K = _widen(paged_rows(k_pool, block_table_row, g, pos, page_size), kv_dtype)
        V = _widen(paged_rows(v_pool, block_table_row, g, pos, page_size), kv_dtype)
        for t in range(t_q):
            last = L - t_q + t
            rows = q[t, g * G:(g + 1) * G, :]
            o, l = softmax_attention(rows, K[:last + 1], V[:last + 1], scale)
            out[t, g * G:(g + 1) * G, :] = o
            lse[t, g * G:(g + 1) * G] = l
    return out, lse


def group_scores(q: np.ndarray, k_pool: np.ndarray, block_table_row: np.ndarray, L: int,
                 scale: float, Hkv: int, n_sink: int, n_recent: int, stride: int,
                 kv_dtype: str = "f32", groups: Optional[Sequence[int]] = None,
                 page_size: int = 16) -> np.ndarray:
    """Masked logits handed to the Selector, one row per KV head.

    SFI page, Fig. 2 caption: the slow step gathers the attention logits of the
    candidate set, masked elsewhere.  Row g holds, for each candidate position
    j, the logits scale * q . k_j summed over every query head of group g and
    every query token of the call (per-head statistics of verification,
    SparseSpec-L abstract); positions outside the candidate set hold -inf.

    q: [t_q, Hq, d] values.  Returns [Hkv, stride] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    t_q, Hq, d = q.shape
    G = Hq // Hkv
    lo, hi = candidate_range(L, t_q, n_sink, n_recent)
    S = np.full((Hkv, stride), -np.inf)
    if hi <= lo:
        return S
    pos = np.arange(lo, hi)
    for g in (range(Hkv) if groups is None else groups):
        K = _widen(paged_rows(k_pool, block_table_row, g, pos, page_size), kv_dtype)
        acc = np.zeros(hi - lo)
        for t in range(t_q):
            for h in range(g * G, (g + 1) * G):
                acc += scale * (K @ q[t, h])
        S[g, lo:hi] = acc
    return S


# --------------------------------------------------------------------------- Selector

def select_topk(scores_row: np.ndarray, lo: int, hi: int, k: int) -> np.ndarray:
    """The Selector on one KV head's logits (SFI page, Abstract and Fig. 2: the slow
    step refreshes the selected memory from the masked logits).

    Among candidate positions [lo, hi) take the k_eff = min(k, hi - lo) that come
    first when ordered by score descending and, for equal scores, by position
    ascending (-0.0 equals +0.0; -inf is the lowest score).  Returns int32 [k]:
    the chosen positions in ascending order, then -1 padding.
    """
    n = max(0, hi - lo)
    k_eff = min(k, n)
    out = np.full(k, -1, dtype=np.int32)
    if k_eff == 0:
        return out
    j = np.arange(lo, hi, dtype=np.int64)
    s = np.asarray(scores_row[lo:hi], dtype=np.float64)
    order = np.lexsort((j, -s))          # primary key -s, secondary key j
    out[:k_eff] = np.sort(j[order[:k_eff]])
    return out


# --------------------------------------------------------------------------- pack

def pack_compact(k_pool: np.ndarray, v_pool: np.ndarray, block_table_row: np.ndarray, L: int,
                 n_sink: int, sel: np.ndarray, cap: int,
                 page_size: int = 16) -> Tuple[np.ndarray, np.ndarray, int]:
    """Compact buffer of one request (SFI page, Fig. 3B: sink and selected tokens packed
    into a contiguous buffer).

    With ns = min(n_sink, L) and k_eff = the number of entries of sel[0] before its first
    negative one, row i < ns + k_eff of KV head g is the stored row at position i
    (i < ns) or sel[g][i - ns]; the copy is bitwise.  A position outside [0, L) or behind
    an invalid block-table entry gives a zero row (reading: the pages pack only selected
    positions, which lie in [0, L) on valid pages; anything else packs as zeros).
    sel: [Hkv, k].  Returns ck, cv of shape [Hkv, cap, d] (rows past n_compact are zero)
    and n_compact.
    """
    Hkv = k_pool.shape[1]
    d = k_pool.shape[3]
    num_pages = k_pool.shape[0]
    sel = np.asarray(sel)
    ns_eff = min(n_sink, L)
    neg = np.flatnonzero(sel[0] < 0) if Hkv > 0 else np.zeros(0, int)
    k_eff = int(neg[0]) if len(neg) else sel.shape[1]
    n_c = ns_eff + k_eff
    ck = np.zeros((Hkv, cap, d), dtype=k_pool.dtype)
    cv = np.zeros((Hkv, cap, d), dtype=v_pool.dtype)
    bt = np.asarray(block_table_row, dtype=np.int64)
    for g in range(Hkv):
        pos = np.concatenate([np.arange(ns_eff), np.asarray(sel[g][:k_eff], dtype=np.int64)])
        inside = (pos >= 0) & (pos < L)
        page = np.full(len(pos), -1, dtype=np.int64)
        page[inside] = bt[pos[inside] // page_size]
        ok = inside & (page >= 0) & (page < num_pages)
        rows = np.flatnonzero(ok)
        ck[g, rows] = paged_rows(k_pool, bt, g, pos[ok], page_size)
        cv[g, rows] = paged_rows(v_pool, bt, g, pos[ok], page_size)
    return ck, cv, n_c


# --------------------------------------------------------------------------- fast step

def sparse_decode(q: np.ndarray, ck: np.ndarray, cv: np.ndarray, n_compact: int,
                  k_pool: np.ndarray, v_pool: np.ndarray, block_table_row: np.ndarray, L: int,
                  n_sink: int, n_recent: int, scale: float, kv_dtype: str = "f32",
                  groups: Optional[Sequence[int]] = None,
                  page_size: int = 16) -> Tuple[np.ndarray, np.ndarray]:
    """Fast step of one request (SFI page, Fig. 2: attention over the managed sparse
    state sink + selected + recent; Fig. 3B: sink and selected come from the compact
    buffer, recent is read in place from paged KV).

    q: [Hq, d] values; ck, cv: [Hkv, cap, d] stored rows, of which [0, n_compact) are
    used.  Returns out [Hq, d] and lse [Hq].
    """
    q = np.asarray(q, dtype=np.float64)
    Hq, d = q.shape
    Hkv = ck.shape[0]
    G = Hq // Hkv
    rs, re = recent_range(L, n_sink, n_recent)
    out = np.full((Hq, d), np.nan)
    lse = np.full(Hq, np.nan)
    for g in (range(Hkv) if groups is None else groups):
        K = np.concatenate([_widen(ck[g, :n_compact], kv_dtype),
                            _widen(paged_rows(k_pool, block_table_row, g, np.arange(rs, re), page_size), kv_dtype)])
        V = np.concatenate([_widen(cv[g, :n_compact], kv_dtype),
                            _widen(paged_rows(v_pool, block_table_row, g, np.arange(rs, re), page_size), kv_dtype)])
        o, l = softmax_attention(q[g * G:(g + 1) * G], K, V, scale)
        out[g * G:(g + 1) * G] = o
        lse[g * G:(g + 1) * G] = l
    return out, lse


def _valid_page(block_table_row: np.ndarray, pos: int, num_pages: int, page_size: int) -> bool:
    e = int(block_table_row[pos // page_size])
    return 0 <= e < num_pages


def indexed_decode(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, block_table_row: np.ndarray, L: int,
                   n_sink: int, n_recent: int, sel: np.ndarray, scale: float, kv_dtype: str = "f32",
                   page_size: int = 16) -> Tuple[np.ndarray, np.ndarray]:
    """Fast step over sink + selected + recent with every row read in place from paged KV
    (attention restricted to an index set; SFI page, Fig. 2 for the three parts).  For KV
    head g the attended positions are, in this order: [0, min(n_sink, L)), the entries of
    sel[g] that lie in [0, L) (negative entries are padding), then the recent range.  A
    position behind an invalid block-table entry is skipped.  q: [Hq, d] values;
    sel: [Hkv, k].  Returns out [Hq, d] and lse [Hq]."""
    q = np.asarray(q, dtype=np.float64)
    Hq, d = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    num_pages = k_pool.shape[0]
    rs, re = recent_range(L, n_sink, n_recent)
    out = np.empty((Hq, d))
    lse = np.empty(Hq)
    for g in range(Hkv):
        chosen = [int(s) for s in np.asarray(sel[g]) if 0 <= int(s) < L]
        pos = list(range(min(n_sink, L))) + chosen + list(range(rs, re))
        pos = np.asarray([p for p in pos if _valid_page(block_table_row, p, num_pages, page_size)], dtype=np.int64)
        K = _widen(paged_rows(k_pool, block_table_row, g, pos, page_size), kv_dtype)
        V = _widen(paged_rows(v_pool, block_table_row, g, pos, page_size), kv_dtype)
        o, l = softmax_attention(q[g * G:(g + 1) * G], K, V, scale)
        out[g * G:(g + 1) * G] = o
        lse[g * G:(g + 1) * G] = l
    return out, lse


def head_scores(q: np.ndarray, k_pool: np.ndarray, block_table_row: np.ndarray, L: int, scale: float, Hkv: int,
                n_sink: int, n_recent: int, stride: int, kv_dtype: str = "f32", page_size: int = 16) -> np.ndarray:
    """Masked logits kept per query head (the per-head statistics of the SparseSpec-L
    abstract, not summed over the group): row h holds scale * q_h . k_j for each candidate
    position j of the slow step (SFI page, Fig. 2) and -inf elsewhere; query head h reads
    KV head h // G.  q: [Hq, d] values (one query token).  Returns [Hq, stride] float64."""
    q = np.asarray(q, dtype=np.float64)
    Hq = q.shape[0]
    G = Hq // Hkv
    lo, hi = candidate_range(L, 1, n_sink, n_recent)
    S = np.full((Hq, stride), -np.inf)
    if hi <= lo:
        return S
    pos = np.arange(lo, hi)
    for h in range(Hq):
        K = _widen(paged_rows(k_pool, block_table_row, h // G, pos, page_size), kv_dtype)
        S[h, lo:hi] = scale * (K @ q[h])
    return S


def indexed_decode_heads(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, block_table_row: np.ndarray,
                         L: int, n_sink: int, n_recent: int, sel: np.ndarray, scale: float, kv_dtype: str = "f32",
                         page_size: int = 16) -> Tuple[np.ndarray, np.ndarray]:
    """Fast step with one selected set per query head: query head h attends over sink +
    the valid entries of sel[h] + recent of KV head h // G, every row read in place (as
    indexed_decode, with the set chosen per head).  q: [Hq, d] values; sel: [Hq, k].
    Returns out [Hq, d] and lse [Hq]."""
    q = np.asarray(q, dtype=np.float64)
    Hq, d = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    num_pages = k_pool.shape[0]
    rs, re = recent_range(L, n_sink, n_recent)
    out = np.empty((Hq, d))
    lse = np.empty(Hq)
    for h in range(Hq):
        chosen = [int(s) for s in np.asarray(sel[h]) if 0 <= int(s) < L]
        pos = list(range(min(n_sink, L))) + chosen + list(range(rs, re))
        pos = np.asarray([p for p in pos if _valid_page(block_table_row, p, num_pages, page_size)], dtype=np.int64)
        K = _widen(paged_rows(k_pool, block_table_row, h // G, pos, page_size), kv_dtype)
        V = _widen(paged_rows(v_pool, block_table_row, h // G, pos, page_size), kv_dtype)
        o, l = softmax_attention(q[h:h + 1], K, V, scale)
        out[h] = o[0]
        lse[h] = l[0]
    return out, lse


def draft_refresh_loop(q_steps: np.ndarray, pools: Sequence[Tuple[np.ndarray, np.ndarray]],
                       block_table_row: np.ndarray, L0: int, n_sink: int, n_recent: int, k: int, refresh_layer: int,
                       sel0: np.ndarray, scale: float, kv_dtype: str = "f32", scores_at=None):
    """Draft steps of a stack of layers with an intra-draft refresh layer (ASPIRE
    abstract, page 1: full attention at one designated layer during drafting refreshes
    the sparse context at every draft step).  Reading: the designated layer attends
    densely and its masked group logits give, through the Selector, the selected set
    that every other layer attends over (sink + selected + recent, read in place);
    layers before the designated one use the previous step's set, layers after it the
    new one.  Step t decodes position L0 + t (length L0 + t + 1), whose K/V is in the pools.

    q_steps: [T, n_layers, Hq, d] values; pools[l] = (k_pool, v_pool); sel0: [Hkv, k],
    the set before the first step.  scores_at(t), when given, supplies step t's logits
    [Hkv, n] (the device's own, so selections can be compared bit for bit).
    Returns per step a list over layers of (out [Hq, d], lse [Hq]) and the selection
    [Hkv, k] made at that step."""
    sel = np.array(sel0, dtype=np.int64, copy=True)
    Hkv = pools[0][0].shape[1]
    res = []
    for t in range(q_steps.shape[0]):
        L = L0 + t + 1
        outs = []
        for layer, (kp, vp) in enumerate(pools):
            q = q_steps[t, layer]
            if layer == refresh_layer:
                o, l = dense_attention(q[None], kp, vp, block_table_row, L, scale, Hkv, kv_dtype=kv_dtype)
                outs.append((o[0], l[0]))
                S = scores_at(t) if scores_at is not None else \
                    group_scores(q[None], kp, block_table_row, L, scale, Hkv, n_sink, n_recent, L, kv_dtype=kv_dtype)
                lo, hi = candidate_range(L, 1, n_sink, n_recent)
                sel = np.stack([select_topk(S[g], lo, hi, k) for g in range(Hkv)])
            else:
                outs.append(indexed_decode(q, kp, vp, block_table_row, L, n_sink, n_recent, sel, scale, kv_dtype))
        res.append((outs, sel.copy()))
    return res


# --------------------------------------------------------------------------- mixed draft / verify

def mixed(modes: Sequence[int], t_q: Sequence[int], q_rows: Sequence[np.ndarray], ck: np.ndarray,
          cv: np.ndarray, n_compact: Sequence[int], k_pool: np.ndarray, v_pool: np.ndarray,
          block_table: np.ndarray, seq_lens: Sequence[int], n_sink: int, n_recent: int,
          scale: float, Hkv: int, stride: int, kv_dtype: str = "f32",
          groups: Optional[Sequence[int]] = None):
    """Drafting and verifying requests served by one call (ASPIRE abstract: a unified
    mixed forward).  Request b with mode 0 drafts: one query token, fast step over its
    compact buffer plus recent tokens.  Mode 1 verifies t_q[b] draft tokens densely and
    also yields its masked logits.  q_rows[b]: [t_q[b], Hq, d].

    Returns per request a tuple (out, lse, scores-or-None).
    """
    res = []
    for b, mode in enumerate(modes):
        if mode == 0:
            o, l = sparse_decode(q_rows[b][0], ck[b], cv[b], int(n_compact[b]), k_pool, v_pool,
                                 block_table[b], int(seq_lens[b]), n_sink, n_recent, scale,
                                 kv_dtype, groups)
            res.append((o[None], l[None], None))
        else:
            o, l = dense_attention(q_rows[b], k_pool, v_pool, block_table[b], int(seq_lens[b]),
                                   scale, Hkv, kv_dtype, groups)
            S = group_scores(q_rows[b], k_pool, block_table[b], int(seq_lens[b]), scale, Hkv,
                             n_sink, n_recent, stride, kv_dtype, groups)
            res.append((o, l, S))
    return res


# --------------------------------------------------------------------------- KV append

def append_token(k_pool: np.ndarray, v_pool: np.ndarray, block_table_row: np.ndarray, L: int,
                 k_new: np.ndarray, v_new: np.ndarray, page_size: int = 16):
    """Pools after storing the decoded token's K/V (k_new, v_new: [Hkv, d] stored rows) at
    position L - 1 of one request, the slot a fast step then reads in place as its newest
    recent token (SFI page, Fig. 3B).  A position behind an invalid block-table entry is
    not stored.  Returns copies of the two pools."""
    k2, v2 = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    if L < 1:
        return k2, v2
    page = int(block_table_row[(L - 1) // page_size])
    if 0 <= page < k_pool.shape[0]:
        k2[page, :, (L - 1) % page_size, :] = k_new
        v2[page, :, (L - 1) % page_size, :] = v_new
    return k2, v2


# --------------------------------------------------------------------------- refresh schedule

def refresh_loop(q_steps: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, block_table_row: np.ndarray,
                 L0: int, Hkv: int, n_sink: int, n_recent: int, k: int, interval: int, scale: float,
                 cap: int, kv_dtype: str = "f32", scores_at=None):
    """One request's decode steps with a slow step every ``interval`` steps and fast steps
    between (SFI page, Fig. 2 and its caption: slow steps perform dense attention and refresh
    the selected memory from the masked logits; fast steps attend over sink + selected +
    recent; the pages' own trigger is a sentence boundary, here a fixed interval).

    Step t decodes the token at position L0 + t, so its length is L = L0 + t + 1; its queries
    are q_steps[t] [Hq, d].  A slow step (t % interval == 0) outputs dense attention over
    [0, L), forms the candidate logits, selects per KV head and packs the compact buffer.  A
    fast step attends over that compact buffer and the recent window at its own L.
    ``scores_at(t)`` may return the [Hkv, >= L] logits to select from (the fp32 values a
    device produced); by default the function's own logits are used.

    Returns per step (out [Hq, d], lse [Hq], sel [Hkv, k] or None, logits or None).
    """
    res = []
    ck = cv = None
    n_c = 0
    for t in range(len(q_steps)):
        q = np.asarray(q_steps[t], dtype=np.float64)
        L = L0 + t + 1
        if t % interval == 0:
            out, lse = dense_attention(q[None], k_pool, v_pool, block_table_row, L, scale, Hkv, kv_dtype)
            S = group_scores(q[None], k_pool, block_table_row, L, scale, Hkv, n_sink, n_recent, L, kv_dtype)
            S_sel = S if scores_at is None else scores_at(t)
            lo, hi = candidate_range(L, 1, n_sink, n_recent)
            sel = np.stack([select_topk(S_sel[g], lo, hi, k) for g in range(Hkv)])
            ck, cv, n_c = pack_compact(k_pool, v_pool, block_table_row, L, n_sink, sel, cap)
            res.append((out[0], lse[0], sel, S))
        else:
            out, lse = sparse_decode(q, ck, cv, n_c, k_pool, v_pool, block_table_row, L, n_sink, n_recent,
                                     scale, kv_dtype)
            res.append((out, lse, None, None))
    return res
