"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test checks one oracle function against a closed form, a hand-derived
fixture under tests/golden/, a library routine that computes the same
quantity by another route (torch SDPA, scipy softmax / logsumexp, einsum on a
scatter-built logical KV), brute force over tiny inputs, or an invariant of
the definition.  The pages print no worked example, so no value is pinned to
a number printed on the pages.
"""
import itertools
import json
import math
import os
import re

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O
from sfi_synth import PAGE_SIZE, bf16_values, make_case, qwen06b_decode_case, tiny_case

GOLD = os.path.join(os.path.dirname(__file__), "golden")
_SPECIAL = {"ln2": math.log(2.0), "ln3": math.log(3.0), "ln4": math.log(4.0),
            "-inf": -math.inf, "-0.0": -0.0}


def _num(x):
    if isinstance(x, list):
        return [_num(v) for v in x]
    return _SPECIAL[x] if isinstance(x, str) else float(x)


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _logical(pool, bt_row, L, g):
    """Logical rows [0, L) of KV head g, built by scattering every physical page
    to where the block table says it belongs (the inverse of the oracle's gather)."""
    d = pool.shape[-1]
    out = np.zeros((L, d), dtype=pool.dtype)
    for lp, phys in enumerate(bt_row):
        if phys < 0:
            continue
        for s in range(PAGE_SIZE):
            j = lp * PAGE_SIZE + s
            if j < L:
                out[j] = pool[phys, g, s]
    return out


def _sdpa(q, K, V, scale, mask=None, causal=False):
    """torch's scaled_dot_product_attention in float64 on the CPU, one head."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, None]
    kt = torch.from_numpy(np.asarray(K, np.float64))[None, None]
    vt = torch.from_numpy(np.asarray(V, np.float64))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=m, is_causal=causal, scale=scale)[0, 0].numpy()


# --------------------------------------------------------------------------- softmax attention

def test_single_key_returns_its_value_exactly():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((5, 64))
    K = rng.standard_normal((1, 64))
    V = rng.standard_normal((1, 64))
    out, lse = O.softmax_attention(q, K, V, 0.125)
    assert np.array_equal(out, np.repeat(V, 5, axis=0))
    np.testing.assert_allclose(lse, 0.125 * (q @ K[0]), rtol=0, atol=1e-12)


def test_zero_query_gives_mean_value():
    rng = np.random.default_rng(1)
    K = rng.standard_normal((37, 16))
    V = rng.standard_normal((37, 16))
    out, lse = O.softmax_attention(np.zeros((2, 16)), K, V, 0.25)
    np.testing.assert_allclose(out, np.repeat(V.mean(axis=0, keepdims=True), 2, 0), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, np.log(37.0), rtol=0, atol=1e-13)


def test_constant_values_pass_through():
    rng = np.random.default_rng(2)
    K = rng.standard_normal((50, 8)) * 3
    out, _ = O.softmax_attention(rng.standard_normal((3, 8)), K, np.full((50, 8), 1.75), 0.5)
    np.testing.assert_allclose(out, 1.75, rtol=0, atol=1e-13)


def test_weights_sum_to_one_and_match_scipy_softmax():
    rng = np.random.default_rng(3)
    n = 24
    q = rng.standard_normal((4, n))
    K = rng.standard_normal((n, n)) * 2
    w, lse = O.softmax_attention(q, K, np.eye(n), 0.3)   # identity values expose the weights
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(w, scipy.special.softmax(0.3 * q @ K.T, axis=1), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(0.3 * q @ K.T, axis=1), rtol=0, atol=1e-12)


def test_matches_torch_sdpa_with_mask():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((6, 32))
    K = rng.standard_normal((40, 32))
    V = rng.standard_normal((40, 32))
    vis = rng.random((6, 40)) < 0.6
    vis[:, 0] = True
    out, _ = O.softmax_attention(q, K, V, 0.17, visible=vis)
    np.testing.assert_allclose(out, _sdpa(q, K, V, 0.17, mask=vis), rtol=0, atol=1e-12)


def test_golden_two_keys():
    g = _gold("attention_two_keys.json")
    out, lse = O.softmax_attention(np.array([_num(g["q"])]), np.array(_num(g["k"])),
                                   np.array(_num(g["v"])), g["scale"])
    np.testing.assert_allclose(out[0], _num(g["out"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0], _num(g["lse"]), rtol=0, atol=1e-14)


# --------------------------------------------------------------------------- paged dense / verify

@pytest.mark.parametrize("G", [1, 2, 4])
def test_dense_matches_sdpa_on_scatter_built_kv(G):
    Hkv = 2
    c = make_case(11 + G, name="t", B=2, Hq=G * Hkv, Hkv=Hkv, d=64, dtype="bf16",
                  seq_lens=[77, 130], n_sink=4, n_recent=8, k_sel=8, spare_pages=3)
    K, V, Q = c.kv.k_values(), c.kv.v_values(), c.q_values()
    for b in range(c.B):
        L = int(c.seq_lens[b])
        out, lse = O.dense_attention(Q[b], c.kv.k, c.kv.v, c.kv.block_table[b], L, c.scale,
                                     c.Hkv, kv_dtype="bf16")
        for h in range(c.Hq):
            g = h // G
            Kl, Vl = _logical(K, c.kv.block_table[b], L, g), _logical(V, c.kv.block_table[b], L, g)
            ref = _sdpa(Q[b, :, h], Kl, Vl, c.scale)
            np.testing.assert_allclose(out[:, h], ref, rtol=0, atol=1e-12)
            ref_lse = scipy.special.logsumexp(c.scale * Q[b, 0, h].astype(np.float64) @ Kl.T.astype(np.float64))
            np.testing.assert_allclose(lse[0, h], ref_lse, rtol=0, atol=1e-12)


def test_verify_all_positions_are_queries_matches_sdpa_causal():
    rng = np.random.default_rng(5)
    L, d = 23, 16
    pool_k = rng.standard_normal((2, 1, PAGE_SIZE, d)).astype(np.float32)
    pool_v = rng.standard_normal((2, 1, PAGE_SIZE, d)).astype(np.float32)
    bt = np.array([1, 0], dtype=np.int32)
    q = rng.standard_normal((L, 1, d))
    out, _ = O.dense_attention(q, pool_k, pool_v, bt, L, 0.3, 1)
    Kl, Vl = _logical(pool_k, bt, L, 0), _logical(pool_v, bt, L, 0)
    np.testing.assert_allclose(out[:, 0], _sdpa(q[:, 0], Kl, Vl, 0.3, causal=True), rtol=0, atol=1e-12)


@pytest.mark.parametrize("t_q", [2, 8, 16])
def test_verify_causal_offset_matches_masked_sdpa(t_q):
    c = make_case(21 + t_q, name="t", B=1, Hq=8, Hkv=2, d=32, dtype="bf16", seq_lens=[100],
                  n_sink=4, n_recent=16, k_sel=8, t_q=t_q)
    Q, K, V = c.q_values(), c.kv.k_values(), c.kv.v_values()
    L = 100
    out, _ = O.dense_attention(Q[0], c.kv.k, c.kv.v, c.kv.block_table[0], L, c.scale, 2, kv_dtype="bf16")
    rows = np.arange(t_q)[:, None] + (L - t_q)      # position of each draft token
    mask = np.arange(L)[None, :] <= rows
    for h in range(8):
        Kl, Vl = _logical(K, c.kv.block_table[0], L, h // 4), _logical(V, c.kv.block_table[0], L, h // 4)
        np.testing.assert_allclose(out[:, h], _sdpa(Q[0, :, h], Kl, Vl, c.scale, mask=mask),
                                   rtol=0, atol=1e-12)


def test_golden_causal_verify():
    g = _gold("causal_verify_tiny.json")
    k = np.zeros((1, 1, PAGE_SIZE, 1))
    v = np.zeros((1, 1, PAGE_SIZE, 1))
    k[0, 0, :3, 0] = np.array(_num(g["k"]))[:, 0]
    v[0, 0, :3, 0] = np.array(_num(g["v"]))[:, 0]
    q = np.array(_num(g["q"]))[:, None, :]
    bt = np.array([0], dtype=np.int32)
    out, lse = O.dense_attention(q, k, v, bt, g["L"], g["scale"], 1)
    np.testing.assert_allclose(out[:, 0, :], _num(g["out"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[:, 0], _num(g["lse"]), rtol=0, atol=1e-14)
    S = O.group_scores(q, k, bt, g["L"], g["scale"], 1, 0, 0, 3)
    assert S[0].tolist() == _num(g["scores"])


# --------------------------------------------------------------------------- candidate set and logits

def test_candidate_counts_of_the_workloads():
    assert O.candidate_range(1024, 1, 4, 32) == (4, 992)          # tiny fp32 case: 988 candidates
    assert O.candidate_range(16384, 1, 4, 64) == (4, 16320)       # 16K decode layer: 16316
    assert O.candidate_range(65536, 1, 4, 256) == (4, 65280)      # 64K refresh: 65276
    assert O.candidate_range(131072, 8, 4, 256) == (4, 130809)    # verify of 8 drafts at 128K
    assert O.candidate_range(10, 1, 4, 32) == (4, 4)              # short request: none
    assert O.recent_range(1032, 4, 32) == (1000, 1032)
    assert O.recent_range(20, 4, 32) == (4, 20)
    assert O.recent_range(2, 4, 32) == (2, 2)


@pytest.mark.parametrize("t_q", [1, 3])
def test_group_scores_match_einsum_on_logical_kv(t_q):
    c = make_case(31, name="t", B=1, Hq=8, Hkv=2, d=64, dtype="bf16", seq_lens=[300],
                  n_sink=4, n_recent=20, k_sel=8, t_q=t_q)
    L = 300
    S = O.group_scores(c.q_values()[0], c.kv.k, c.kv.block_table[0], L, c.scale, 2, 4, 20, 320,
                       kv_dtype="bf16")
    lo, hi = 4, L - t_q + 1 - 20
    Q = torch.from_numpy(c.q_values()[0].astype(np.float64)).view(t_q, 2, 4, 64)
    for g in range(2):
        Kl = torch.from_numpy(_logical(c.kv.k_values(), c.kv.block_table[0], L, g).astype(np.float64))
        ref = c.scale * torch.einsum("thd,jd->j", Q[:, g], Kl).numpy()
        np.testing.assert_allclose(S[g, lo:hi], ref[lo:hi], rtol=1e-13, atol=1e-12)
        assert np.all(np.isneginf(S[g, :lo])) and np.all(np.isneginf(S[g, hi:]))


def test_planted_keys_have_closed_form_scores():
    # float32 inputs: a planted key is exactly fp32(4 * mean of the group's queries)
    c = make_case(41, name="t", B=1, Hq=4, Hkv=1, d=64, dtype="f32", seq_lens=[512],
                  n_sink=4, n_recent=32, k_sel=16, hh_per_head=6)
    S = O.group_scores(c.q_values()[0], c.kv.k, c.kv.block_table[0], 512, c.scale, 1, 4, 32, 512)
    qbar = c.q_values()[0, 0].astype(np.float64).mean(axis=0)
    closed = 4.0 * c.scale * 4 * float(qbar @ qbar)          # sum over G = 4 heads of scale*q_h.(4 qbar)
    np.testing.assert_allclose(S[0, c.planted[(0, 0)]], closed, rtol=1e-6)


# --------------------------------------------------------------------------- Selector

def _brute_topk(s, lo, k):
    """The unique subset whose every member beats every non-member under (score desc, index asc)."""
    n = len(s)
    k_eff = min(k, n)
    beats = lambda a, b: (s[a] > s[b]) or (s[a] == s[b] and a < b)
    hits = [sub for sub in itertools.combinations(range(n), k_eff)
            if all(beats(a, b) for a in sub for b in range(n) if b not in sub)]
    assert len(hits) == 1
    return [lo + i for i in hits[0]] + [-1] * (k - k_eff)


def test_selector_brute_force_tiny():
    rng = np.random.default_rng(6)
    vals = np.array([-np.inf, -1.0, -0.0, 0.0, 0.5, 2.0], dtype=np.float32)
    for trial in range(150):
        n = int(rng.integers(1, 11))
        lo = int(rng.integers(0, 4))
        row = np.full(lo + n + 2, np.nan, dtype=np.float32)
        row[lo:lo + n] = rng.choice(vals, size=n)
        for k in range(1, n + 3):
            got = O.select_topk(row, lo, lo + n, k).tolist()
            assert got == _brute_topk([float(x) for x in row[lo:lo + n]], lo, k), (trial, k)


def test_selector_golden():
    g = _gold("selector_ties.json")
    row = np.array(_num(g["scores"]), dtype=np.float32)
    for k, want in g["expected"].items():
        assert O.select_topk(row, g["lo"], g["hi"], int(k)).tolist() == want


def test_selector_all_equal_and_oversized_k():
    row = np.full(40, 1.5, dtype=np.float32)
    assert O.select_topk(row, 4, 30, 7).tolist() == list(range(4, 11))
    assert O.select_topk(row, 4, 30, 30).tolist() == list(range(4, 30)) + [-1] * 4
    assert O.select_topk(row, 4, 4, 3).tolist() == [-1, -1, -1]


def test_planted_heavy_hitters_are_selected():
    c = tiny_case(1)
    L = int(c.seq_lens[0])
    S = O.group_scores(c.q_values()[0], c.kv.k, c.kv.block_table[0], L, c.scale, 1, c.n_sink,
                       c.n_recent, L)
    lo, hi = O.candidate_range(L, 1, c.n_sink, c.n_recent)
    sel = O.select_topk(S[0], lo, hi, c.k_sel)
    assert set(c.planted[(0, 0)].tolist()) <= set(sel.tolist())
    assert np.all(np.diff(sel) > 0) and sel.min() >= lo and sel.max() < hi


# --------------------------------------------------------------------------- pack and fast step

def test_pack_is_a_bitwise_gather_and_idempotent():
    c = qwen06b_decode_case(7, L=700, frac=(1, 4))
    L = 700
    rng = np.random.default_rng(8)
    lo, hi = O.candidate_range(L, 1, c.n_sink, c.n_recent)
    sel = np.stack([np.sort(rng.choice(np.arange(lo, hi), 50, replace=False)) for _ in range(c.Hkv)])
    sel = np.concatenate([sel, -np.ones((c.Hkv, 5), np.int64)], axis=1)
    ck, cv, n_c = O.pack_compact(c.kv.k, c.kv.v, c.kv.block_table[0], L, c.n_sink, sel, 64)
    assert n_c == 54 and ck.dtype == np.uint16
    for g in range(c.Hkv):
        Kl = _logical(c.kv.k, c.kv.block_table[0], L, g)
        Vl = _logical(c.kv.v, c.kv.block_table[0], L, g)
        pos = list(range(4)) + sel[g, :50].tolist()
        assert np.array_equal(ck[g, :n_c], Kl[pos]) and np.array_equal(cv[g, :n_c], Vl[pos])
    ck2, cv2, n_c2 = O.pack_compact(c.kv.k, c.kv.v, c.kv.block_table[0], L, c.n_sink, sel, 64)
    assert n_c2 == n_c and np.array_equal(ck, ck2) and np.array_equal(cv, cv2)


def _full_selection(L, c):
    lo, hi = O.candidate_range(L, 1, c.n_sink, c.n_recent)
    return np.tile(np.arange(lo, hi), (c.Hkv, 1))


def test_fast_step_at_full_retention_equals_dense():
    c = qwen06b_decode_case(9, L=900, frac=(1, 1))
    L = 900
    sel = _full_selection(L, c)
    ck, cv, n_c = O.pack_compact(c.kv.k, c.kv.v, c.kv.block_table[0], L, c.n_sink, sel, sel.shape[1] + 4)
    out_s, lse_s = O.sparse_decode(c.q_values()[0, 0], ck, cv, n_c, c.kv.k, c.kv.v, c.kv.block_table[0],
                                   L, c.n_sink, c.n_recent, c.scale, kv_dtype="bf16")
    out_d, lse_d = O.dense_attention(c.q_values()[0], c.kv.k, c.kv.v, c.kv.block_table[0], L, c.scale,
                                     c.Hkv, kv_dtype="bf16")
    np.testing.assert_allclose(out_s, out_d[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_s, lse_d[0], rtol=0, atol=1e-12)


def test_fast_step_equals_masked_dense_and_ignores_row_order():
    c = tiny_case(3)
    L = 1029                                        # five tokens appended after the slow step at 1024
    rng = np.random.default_rng(10)
    lo, hi = O.candidate_range(1024, 1, c.n_sink, c.n_recent)
    sel = np.sort(rng.choice(np.arange(lo, hi), c.k_sel, replace=False))[None]
    ck, cv, n_c = O.pack_compact(c.kv.k, c.kv.v, c.kv.block_table[0], 1024, c.n_sink, sel, 80)
    q = c.extra_q_values()[4, 0]
    out, _ = O.sparse_decode(q, ck, cv, n_c, c.kv.k, c.kv.v, c.kv.block_table[0], L, c.n_sink,
                             c.n_recent, c.scale)
    keep = np.zeros(L, bool)
    keep[:4] = True
    keep[sel[0]] = True
    keep[L - 32:] = True
    Kl = _logical(c.kv.k, c.kv.block_table[0], L, 0)
    Vl = _logical(c.kv.v, c.kv.block_table[0], L, 0)
    for h in range(4):
        ref = _sdpa(q[h:h + 1], Kl, Vl, c.scale, mask=keep[None, :])
        np.testing.assert_allclose(out[h:h + 1], ref, rtol=0, atol=1e-12)
    perm = rng.permutation(n_c)
    ck_p, cv_p = ck.copy(), cv.copy()
    ck_p[0, :n_c], cv_p[0, :n_c] = ck[0, perm], cv[0, perm]
    out_p, _ = O.sparse_decode(q, ck_p, cv_p, n_c, c.kv.k, c.kv.v, c.kv.block_table[0], L, c.n_sink,
                               c.n_recent, c.scale)
    np.testing.assert_allclose(out_p, out, rtol=0, atol=1e-13)


def test_mixed_dispatches_per_request():
    c = make_case(51, name="t", B=3, Hq=8, Hkv=2, d=32, dtype="bf16", seq_lens=[200, 180, 240],
                  n_sink=4, n_recent=16, k_sel=20, t_q=4)
    rng = np.random.default_rng(12)
    cap = 32
    cks, cvs, ncs = [], [], []
    for b in range(3):
        L = int(c.seq_lens[b])
        lo, hi = O.candidate_range(L, 1, 4, 16)
        sel = np.stack([np.sort(rng.choice(np.arange(lo, hi), 20, replace=False)) for _ in range(2)])
        ck, cv, n_c = O.pack_compact(c.kv.k, c.kv.v, c.kv.block_table[b], L, 4, sel, cap)
        cks.append(ck), cvs.append(cv), ncs.append(n_c)
    ck, cv = np.stack(cks), np.stack(cvs)
    Q = c.q_values()
    modes, tq = [0, 1, 0], [1, 4, 1]
    res = O.mixed(modes, tq, [Q[0, :1], Q[1], Q[2, :1]], ck, cv, ncs, c.kv.k, c.kv.v,
                  c.kv.block_table, c.seq_lens, 4, 16, c.scale, 2, 256, kv_dtype="bf16")
    o0, _ = O.sparse_decode(Q[0, 0], ck[0], cv[0], ncs[0], c.kv.k, c.kv.v, c.kv.block_table[0], 200,
                            4, 16, c.scale, kv_dtype="bf16")
    assert np.array_equal(res[0][0][0], o0) and res[0][2] is None
    o1, _ = O.dense_attention(Q[1], c.kv.k, c.kv.v, c.kv.block_table[1], 180, c.scale, 2, kv_dtype="bf16")
    assert np.array_equal(res[1][0], o1) and res[1][2].shape == (2, 256)


def test_pack_writes_zero_rows_past_the_end_and_behind_invalid_pages():
    c = make_case(43, name="pz", B=1, Hq=4, Hkv=2, d=32, dtype="f32", seq_lens=[200], capacity=[240], n_sink=4,
                  n_recent=16, k_sel=6)
    bt = c.kv.block_table[0].copy()
    bt[3] = -1                                     # positions 48..63
    sel = np.array([[10, 50, 205, 100, -1, 7], [11, 12, 13, 14, 15, 16]], np.int32)
    ck, cv, n_c = O.pack_compact(c.kv.k, c.kv.v, bt, 200, 4, sel, 12)
    assert n_c == 4 + 4                            # head 0's entries before its first negative one
    Kl, Vl = _logical(c.kv.k, bt, 240, 0), _logical(c.kv.v, bt, 240, 0)
    np.testing.assert_array_equal(ck[0, :5], Kl[[0, 1, 2, 3, 10]])
    np.testing.assert_array_equal(cv[0, :5], Vl[[0, 1, 2, 3, 10]])
    assert not ck[0, 5].any() and not cv[0, 5].any()      # 50: behind the invalid page
    assert not ck[0, 6].any() and not cv[0, 6].any()      # 205: past L = 200
    np.testing.assert_array_equal(ck[0, 7], Kl[100])
    assert not ck[:, 8:].any()                           # rows past n_compact stay zero
    np.testing.assert_array_equal(ck[1, 4:8], _logical(c.kv.k, bt, 240, 1)[[11, 12, 13, 14]])


# --------------------------------------------------------------------------- KV append

def test_append_token_stores_one_row_and_a_dominant_new_key_returns_its_value():
    c = make_case(41, name="ap", B=1, Hq=4, Hkv=2, d=64, dtype="f32", seq_lens=[300], capacity=[310], n_sink=4,
                  n_recent=16, k_sel=8)
    rng = np.random.default_rng(3)
    L = 305                                      # decoding position 304
    q = c.q_values()[0, 0]
    k_new = np.stack([40.0 * q[g * 2:(g + 1) * 2].mean(axis=0) for g in range(2)]).astype(np.float32)
    v_new = rng.standard_normal((2, 64)).astype(np.float32)
    k2, v2 = O.append_token(c.kv.k, c.kv.v, c.kv.block_table[0], L, k_new, v_new)
    for g in range(2):
        np.testing.assert_array_equal(O.paged_rows(k2, c.kv.block_table[0], g, [L - 1])[0], k_new[g])
        np.testing.assert_array_equal(O.paged_rows(v2, c.kv.block_table[0], g, [L - 1])[0], v_new[g])
    changed = np.argwhere(np.any(k2 != c.kv.k, axis=-1))
    assert len(changed) == 2 and np.all(changed[:, 2] == (L - 1) % PAGE_SIZE)
    # the new key dominates every query of its group: the fast step returns its value
    ck, cv, n_c = O.pack_compact(k2, v2, c.kv.block_table[0], L, 4, np.full((2, 8), -1, np.int32), 12)
    out, _ = O.sparse_decode(q, ck, cv, n_c, k2, v2, c.kv.block_table[0], L, 4, 16, c.scale)
    for h in range(4):
        np.testing.assert_allclose(out[h], v_new[h // 2], rtol=0, atol=1e-12)


def test_append_token_behind_an_invalid_page_or_at_length_zero_stores_nothing():
    c = make_case(42, name="ap", B=1, Hq=4, Hkv=2, d=64, dtype="f32", seq_lens=[100], capacity=[112], n_sink=4,
                  n_recent=16, k_sel=8)
    bt = c.kv.block_table[0].copy()
    bt[6] = -1                                   # the page of position 100
    kn = np.ones((2, 64), np.float32)
    for row, L in ((bt, 101), (c.kv.block_table[0], 0)):
        k2, v2 = O.append_token(c.kv.k, c.kv.v, row, L, kn, kn)
        np.testing.assert_array_equal(k2, c.kv.k)
        np.testing.assert_array_equal(v2, c.kv.v)


# --------------------------------------------------------------------------- refresh schedule

def _drift(seed=31, q_gain=1.0, hh=12):
    from sfi_synth import drifting_case
    dc = drifting_case(seed, B=1, Hq=4, Hkv=2, d=64, dtype="f32", L0=[700], steps=40, period=16, hh=hh,
                       n_sink=4, n_recent=32, k_sel=24, noise=0.0)
    c = dc.case
    q = dc.q_step_values()[:, 0] * q_gain          # [steps, Hq, d]
    return dc, c, q


def test_refresh_loop_every_step_is_dense_attention_on_scatter_built_kv():
    """interval = 1: every step is a slow step, i.e. dense attention over [0, L0 + t + 1)."""
    dc, c, q = _drift()
    res = O.refresh_loop(q[:6], c.kv.k, c.kv.v, c.kv.block_table[0], 700, c.Hkv, 4, 32, 24, 1, c.scale, 4 + 24)
    for t, (out, lse, sel, S) in enumerate(res):
        L = 700 + t + 1
        assert sel is not None and S is not None
        for h in range(c.Hq):
            Kl = _logical(c.kv.k, c.kv.block_table[0], L, h // 2)
            Vl = _logical(c.kv.v, c.kv.block_table[0], L, h // 2)
            np.testing.assert_allclose(out[h], _sdpa(q[t, h][None], Kl, Vl, c.scale)[0], rtol=0, atol=1e-12)


def test_refresh_loop_fast_steps_match_dense_while_the_support_holds_all_mass():
    """Queries 30x larger make every key outside the epoch's planted support weigh exactly
    zero in fp64 (logit gaps > 745).  A fast step after a refresh in the same epoch then
    equals dense attention; after an epoch shift without refresh it does not."""
    dc, c, q = _drift(q_gain=30.0)
    res = O.refresh_loop(q, c.kv.k, c.kv.v, c.kv.block_table[0], 700, c.Hkv, 4, 32, 24, 8, c.scale, 4 + 24)
    for t, (out, lse, sel, S) in enumerate(res):
        L = 700 + t + 1
        dense, dlse = O.dense_attention(q[t][None], c.kv.k, c.kv.v, c.kv.block_table[0], L, c.scale, c.Hkv)
        last_refresh = t - t % 8
        same_epoch = last_refresh // dc.period == t // dc.period
        if same_epoch:
            np.testing.assert_allclose(out, dense[0], rtol=0, atol=1e-10)
        else:
            assert np.abs(out - dense[0]).max() > 0.1, t


def test_refresh_loop_selects_the_current_support_after_a_refresh():
    dc, c, q = _drift()
    res = O.refresh_loop(q, c.kv.k, c.kv.v, c.kv.block_table[0], 700, c.Hkv, 4, 32, 24, 8, c.scale, 4 + 24)
    for t in range(0, 40, 8):
        sel = res[t][2]
        for g in range(c.Hkv):
            assert set(dc.support[t // dc.period, 0, g].tolist()) <= set(sel[g].tolist()), (t, g)


# --------------------------------------------------------------------------- indexed fast step, draft refresh

def _positions_sdpa(q_rows, pool_k, pool_v, bt_row, L, g, pos, scale):
    """SDPA over the scatter-built logical rows at an explicit position list."""
    Kl = _logical(pool_k, bt_row, L, g)[pos]
    Vl = _logical(pool_v, bt_row, L, g)[pos]
    return _sdpa(q_rows, Kl, Vl, scale)


def test_indexed_decode_over_every_candidate_is_dense_attention():
    c = make_case(51, name="ix", B=1, Hq=4, Hkv=2, d=64, dtype="f32", seq_lens=[333], n_sink=4, n_recent=16, k_sel=8)
    L, bt = 333, c.kv.block_table[0]
    lo, hi = O.candidate_range(L, 1, 4, 16)
    sel = np.stack([np.arange(lo, hi)] * 2).astype(np.int32)
    q = c.q_values()[0, 0]
    out, _ = O.indexed_decode(q, c.kv.k, c.kv.v, bt, L, 4, 16, sel, c.scale)
    for g in range(2):
        ref = _positions_sdpa(q[2 * g:2 * g + 2], c.kv.k, c.kv.v, bt, L, g, np.arange(L), c.scale)
        np.testing.assert_allclose(out[2 * g:2 * g + 2], ref, rtol=0, atol=1e-12)


def test_indexed_decode_skips_padding_out_of_range_entries_and_invalid_pages():
    c = make_case(52, name="ix", B=1, Hq=4, Hkv=2, d=64, dtype="f32", seq_lens=[400], capacity=[480], n_sink=4,
                  n_recent=16, k_sel=8)
    L = 400
    bt = c.kv.block_table[0].copy()
    bt[10] = -1                                    # positions 160..175 unusable
    sel = np.array([[7, 165, 200, 450, -1, -1], [12, 40, 399 + 30, 300, -1, 171]], np.int32)
    q = c.q_values()[0, 0]
    out, _ = O.indexed_decode(q, c.kv.k, c.kv.v, bt, L, 4, 16, sel, c.scale)
    kept = {0: [7, 200], 1: [12, 40, 300]}         # 165 / 171 sit on the dropped page, 450 / 429 are past L
    for g in range(2):
        pos = np.array([0, 1, 2, 3] + kept[g] + list(range(384, 400)))
        ref = _positions_sdpa(q[2 * g:2 * g + 2], c.kv.k, c.kv.v, bt, L, g, pos, c.scale)
        np.testing.assert_allclose(out[2 * g:2 * g + 2], ref, rtol=0, atol=1e-12)


def test_indexed_decode_equals_pack_then_compact_fast_step():
    c = make_case(53, name="ix", B=1, Hq=8, Hkv=2, d=64, dtype="bf16", seq_lens=[900], n_sink=4, n_recent=32,
                  k_sel=40)
    L, bt = 900, c.kv.block_table[0]
    rng = np.random.default_rng(5)
    sel = np.stack([np.sort(rng.choice(np.arange(4, 868), 40, replace=False)) for _ in range(2)]).astype(np.int32)
    q = c.q_values()[0, 0]
    a, la = O.indexed_decode(q, c.kv.k, c.kv.v, bt, L, 4, 32, sel, c.scale, kv_dtype="bf16")
    ck, cv, n_c = O.pack_compact(c.kv.k, c.kv.v, bt, L, 4, sel, 44)
    b, lb = O.sparse_decode(q, ck, cv, n_c, c.kv.k, c.kv.v, bt, L, 4, 32, c.scale, kv_dtype="bf16")
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)
    np.testing.assert_allclose(la, lb, rtol=0, atol=1e-13)


def _layers(c, n, seed):
    rng = np.random.default_rng(seed)
    pools = [(c.kv.k, c.kv.v)]
    for _ in range(n - 1):
        pools.append((rng.standard_normal(c.kv.k.shape).astype(np.float32),
                      rng.standard_normal(c.kv.v.shape).astype(np.float32)))
    return pools


def test_draft_refresh_layer_attends_densely_and_selects_its_top_k():
    c = make_case(54, name="dr", B=1, Hq=4, Hkv=2, d=32, dtype="f32", seq_lens=[300], capacity=[310], n_sink=4,
                  n_recent=16, k_sel=12)
    bt, L0, k = c.kv.block_table[0], 299, 12
    pools = _layers(c, 3, 1)
    q = np.random.default_rng(2).standard_normal((3, 3, 4, 32))
    sel0 = np.full((2, k), -1, np.int32)
    res = O.draft_refresh_loop(q, pools, bt, L0, 4, 16, k, 1, sel0, c.scale)
    for t, (outs, sel) in enumerate(res):
        L = L0 + t + 1
        kp, vp = pools[1]
        for g in range(2):
            Kl = _logical(kp, bt, L, g)
            ref = _sdpa(q[t, 1, 2 * g:2 * g + 2], Kl, _logical(vp, bt, L, g), c.scale)
            np.testing.assert_allclose(outs[1][0][2 * g:2 * g + 2], ref, rtol=0, atol=1e-12)
            # brute force: group-summed logits over the candidates, best k by (score desc, position asc)
            cand = range(4, L - 16)
            sc = {j: sum(float(q[t, 1, h] @ Kl[j]) for h in (2 * g, 2 * g + 1)) for j in cand}
            best = sorted(cand, key=lambda j: (-sc[j], j))[:k]
            assert sel[g].tolist() == sorted(best), (t, g)


def test_draft_refresh_layers_before_the_refresh_layer_use_the_previous_set():
    c = make_case(55, name="dr", B=1, Hq=4, Hkv=2, d=32, dtype="f32", seq_lens=[300], capacity=[310], n_sink=4,
                  n_recent=16, k_sel=10)
    bt, L0, k = c.kv.block_table[0], 299, 10
    pools = _layers(c, 3, 3)
    q = np.random.default_rng(4).standard_normal((4, 3, 4, 32))
    sel0 = np.stack([np.arange(4, 14), np.arange(20, 30)]).astype(np.int32)
    res = O.draft_refresh_loop(q, pools, bt, L0, 4, 16, k, 1, sel0, c.scale)
    prev = sel0
    for t, (outs, sel) in enumerate(res):
        L = L0 + t + 1
        assert not np.array_equal(prev, sel)       # the set moves, so the two layers see different sets
        for layer, use in ((0, prev), (2, sel)):
            kp, vp = pools[layer]
            for g in range(2):
                pos = np.array(list(range(4)) + use[g].tolist() + list(range(L - 16, L)))
                ref = _positions_sdpa(q[t, layer, 2 * g:2 * g + 2], kp, vp, bt, L, g, pos, c.scale)
                np.testing.assert_allclose(outs[layer][0][2 * g:2 * g + 2], ref, rtol=0, atol=1e-12)
        prev = sel


def test_draft_refresh_at_full_retention():
    """k covers every candidate: a layer after the refresh layer is dense attention; a layer
    before it misses exactly the position that left the recent window since the last refresh."""
    c = make_case(56, name="dr", B=1, Hq=4, Hkv=2, d=32, dtype="f32", seq_lens=[200], capacity=[210], n_sink=4,
                  n_recent=16, k_sel=8)
    bt, L0 = c.kv.block_table[0], 199
    pools = _layers(c, 3, 5)
    q = np.random.default_rng(6).standard_normal((3, 3, 4, 32))
    k = 200
    sel0 = np.stack([np.r_[np.arange(4, 183), -np.ones(21, int)]] * 2).astype(np.int32)   # the candidates at L = 199
    res = O.draft_refresh_loop(q, pools, bt, L0, 4, 16, k, 1, sel0, c.scale)
    for t, (outs, _) in enumerate(res):
        L = L0 + t + 1
        for layer, pos in ((2, np.arange(L)), (0, np.setdiff1d(np.arange(L), [L - 17]))):
            kp, vp = pools[layer]
            for g in range(2):
                ref = _positions_sdpa(q[t, layer, 2 * g:2 * g + 2], kp, vp, bt, L, g, pos, c.scale)
                np.testing.assert_allclose(outs[layer][0][2 * g:2 * g + 2], ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- per-query-head selection

def test_head_scores_are_per_head_dot_products_over_the_candidates():
    c = make_case(57, name="hs", B=1, Hq=8, Hkv=2, d=32, dtype="bf16", seq_lens=[260], n_sink=4, n_recent=16,
                  k_sel=8)
    L, bt = 260, c.kv.block_table[0]
    q = c.q_values()[0, 0]
    S = O.head_scores(q, c.kv.k, bt, L, c.scale, 2, 4, 16, 300, kv_dtype="bf16")
    assert np.all(np.isneginf(S[:, :4])) and np.all(np.isneginf(S[:, 244:]))
    for h in range(8):
        Kl = torch.from_numpy(bf16_values(_logical(c.kv.k, bt, L, h // 4)).astype(np.float64))
        ref = (Kl @ torch.from_numpy(q[h].astype(np.float64))).numpy() * c.scale
        np.testing.assert_allclose(S[h, 4:244], ref[4:244], rtol=0, atol=1e-12)
    # their sum over a group is the group's logit row
    Sg = O.group_scores(q[None], c.kv.k, bt, L, c.scale, 2, 4, 16, 300, kv_dtype="bf16")
    np.testing.assert_allclose(S.reshape(2, 4, 300).sum(axis=1)[:, 4:244], Sg[:, 4:244], rtol=0, atol=1e-11)


def test_per_head_sets_equal_to_the_group_set_give_the_group_fast_step():
    c = make_case(58, name="hs", B=1, Hq=8, Hkv=2, d=32, dtype="f32", seq_lens=[500], n_sink=4, n_recent=16,
                  k_sel=20)
    L, bt = 500, c.kv.block_table[0]
    rng = np.random.default_rng(9)
    sel = np.stack([np.sort(rng.choice(np.arange(4, 484), 20, replace=False)) for _ in range(2)]).astype(np.int32)
    q = c.q_values()[0, 0]
    a, la = O.indexed_decode_heads(q, c.kv.k, c.kv.v, bt, L, 4, 16, np.repeat(sel, 4, axis=0), c.scale)
    b, lb = O.indexed_decode(q, c.kv.k, c.kv.v, bt, L, 4, 16, sel, c.scale)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)
    np.testing.assert_allclose(la, lb, rtol=0, atol=1e-13)


def test_per_head_fast_step_attends_each_heads_own_positions():
    c = make_case(59, name="hs", B=1, Hq=4, Hkv=1, d=32, dtype="f32", seq_lens=[300], n_sink=4, n_recent=16,
                  k_sel=6)
    L, bt = 300, c.kv.block_table[0]
    rng = np.random.default_rng(10)
    sel = np.stack([np.r_[np.sort(rng.choice(np.arange(4, 284), 5, replace=False)), -1] for _ in range(4)])
    q = c.q_values()[0, 0]
    out, _ = O.indexed_decode_heads(q, c.kv.k, c.kv.v, bt, L, 4, 16, sel.astype(np.int32), c.scale)
    for h in range(4):
        pos = np.array([0, 1, 2, 3] + sel[h, :5].tolist() + list(range(284, 300)))
        ref = _positions_sdpa(q[h:h + 1], c.kv.k, c.kv.v, bt, L, 0, pos, c.scale)
        np.testing.assert_allclose(out[h:h + 1], ref, rtol=0, atol=1e-12)


def test_oracle_is_independent_of_the_product():
    here = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle")
    for fn in os.listdir(here):
        if fn.endswith(".py"):
            src = open(os.path.join(here, fn)).read()
            for mod in ("sparse_kv_cache_sfi_amd", "sfi_synth"):
                assert not re.search(r"^\s*(import|from)\s+" + mod, src, re.M), (fn, mod)
