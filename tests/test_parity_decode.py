"""GPU parity of the t_q = 1 attention paths against the fp64 oracle (through the C ABI).

Slow step (dense + masked logits) and fast step (compact + recent), at sizes the
oracle finishes in seconds that still span several splits, tiles and a ragged
tail, plus edge cases: one key, empty compact segment, requests shorter than the
sink, invalid block-table entries.  Tolerances: out 2e-3 max-abs, lse 1e-3,
logits within the forward error bound of fp32 summation (tests/_gpu.py).
"""
import zlib

import numpy as np
import pytest
import torch

import oracle as O
from sfi_synth import make_case, tiny_case, qwen06b_decode_case
from _gpu import DEV, LSE_TOL, OUT_TOL, DevCase, assert_close, dev_array, host_bits, score_bound

pytestmark = pytest.mark.gpu


def _dense_check(sfi, c, dc, with_scores=True, stride=None):
    out, lse, scores = sfi.dense_attn_with_stats(dc.q, dc.k, dc.v, dc.bt, dc.lens, max_seq_len=dc.max_seq_len,
                                                 n_sink=c.n_sink, n_recent=c.n_recent, scale=c.scale,
                                                 with_scores=with_scores, score_stride=stride)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    sc = scores.cpu().numpy() if scores is not None else None
    Q, K = c.q_values(), c.kv.k_values()
    G = c.G
    for b in range(c.B):
        L = int(c.seq_lens[b])
        ref_o, ref_l = O.dense_attention(c.q_values()[b], c.kv.k, c.kv.v, c.kv.block_table[b], L, c.scale, c.Hkv,
                                         kv_dtype=c.dtype)
        assert_close(out[b], ref_o, OUT_TOL, f"out b={b}")
        assert_close(lse[b], ref_l, LSE_TOL, f"lse b={b}")
        if sc is None:
            continue
        ref_s = O.group_scores(Q[b], c.kv.k, c.kv.block_table[b], L, c.scale, c.Hkv, c.n_sink, c.n_recent,
                               sc.shape[-1], kv_dtype=c.dtype)
        lo, hi = O.candidate_range(L, 1, c.n_sink, c.n_recent)
        for g in range(c.Hkv):
            assert np.all(np.isneginf(sc[b, g, :lo])) and np.all(np.isneginf(sc[b, g, hi:])), (b, g)
            if hi > lo:
                rows = O.paged_rows(K, c.kv.block_table[b], g, np.arange(lo, hi))
                bound = score_bound(Q[b, 0, g * G:(g + 1) * G], rows, c.scale)
                assert_close(sc[b, g, lo:hi], ref_s[g, lo:hi], bound, f"scores b={b} g={g}")
    return out, lse, sc


DENSE_CASES = [
    ("tiny_fp32", lambda: tiny_case(1)),
    ("bf16_g2_d128_L3000", lambda: make_case(101, name="a", B=1, Hq=16, Hkv=8, d=128, dtype="bf16",
                                              seq_lens=[3000], n_sink=4, n_recent=64, k_sel=100, hh_per_head=40)),
    ("bf16_g4_ragged", lambda: make_case(102, name="b", B=3, Hq=8, Hkv=2, d=128, dtype="bf16",
                                          seq_lens=[1, 77, 2900], n_sink=4, n_recent=32, k_sel=64,
                                          hh_per_head=10, spare_pages=5)),
    ("bf16_g1_d64", lambda: make_case(103, name="c", B=2, Hq=4, Hkv=4, d=64, dtype="bf16",
                                       seq_lens=[700, 1500], n_sink=4, n_recent=16, k_sel=32)),
    ("bf16_g8_d128", lambda: make_case(104, name="d", B=2, Hq=16, Hkv=2, d=128, dtype="bf16",
                                        seq_lens=[1030, 513], n_sink=2, n_recent=16, k_sel=32)),
    ("f32_g2_d128", lambda: make_case(105, name="e", B=1, Hq=4, Hkv=2, d=128, dtype="f32",
                                       seq_lens=[2100], n_sink=4, n_recent=64, k_sel=32)),
    ("f32_g8_d64", lambda: make_case(106, name="f", B=1, Hq=8, Hkv=1, d=64, dtype="f32",
                                      seq_lens=[333], n_sink=4, n_recent=8, k_sel=16)),
    ("short_below_sink", lambda: make_case(107, name="g", B=2, Hq=8, Hkv=4, d=128, dtype="bf16",
                                            seq_lens=[3, 20], n_sink=4, n_recent=16, k_sel=8)),
    # 16 requests x 8 KV heads, several splits each
    ("bf16_b16_large_grid", lambda: make_case(108, name="g16", B=16, Hq=16, Hkv=8, d=128, dtype="bf16",
                                               seq_lens=list(range(2100, 2660, 35)), n_sink=4, n_recent=64,
                                               k_sel=64)),
]


def _splits(sfi, op, c, dc, cap=0):
    st, ns = sfi.plan_splits(op, B=c.B, Hq=c.Hq, Hkv=c.Hkv, d=c.d, bf16=c.dtype == "bf16",
                             max_pages=c.kv.max_pages, num_pages=c.kv.num_pages, max_seq_len=dc.max_seq_len,
                             cap=cap, n_recent=c.n_recent)
    return ns


@pytest.mark.parametrize("name,mk", DENSE_CASES, ids=[n for n, _ in DENSE_CASES])
def test_dense_slow_step_matches_oracle(gpu_lib, name, mk):
    c = mk()
    dc = DevCase(c)
    if "large_grid" in name:   # many units, each merged from several splits
        assert _splits(gpu_lib, 0, c, dc) >= 2
    _dense_check(gpu_lib, c, dc, stride=dc.max_seq_len + 37)


# The split-K merge has two forms at d 128: one output group per thread with every split in one
# batch of loads (up to 2 x 16 splits at two rows per unit, 16 at four), and the LDS form for more
# splits.  Each case states the form its plan takes.
MERGE_CASES = [
    # two rows per unit, 20 splits: the one-batch form
    ("g2_20_splits", dict(B=1, Hq=4, Hkv=2, seq_lens=[9000]), lambda ns: 16 < ns <= 32),
    # two rows per unit, 40 splits: the LDS form
    ("g2_40_splits", dict(B=1, Hq=4, Hkv=2, seq_lens=[20000]), lambda ns: ns > 32),
    # four rows per unit, 24 splits: the LDS form (one lane per group takes at most 16)
    ("g4_24_splits", dict(B=1, Hq=8, Hkv=2, seq_lens=[6000]), lambda ns: 16 < ns <= 32),
]


@pytest.mark.parametrize("name,kw,form", MERGE_CASES, ids=[n for n, _, _ in MERGE_CASES])
def test_dense_slow_step_under_both_merge_forms(gpu_lib, name, kw, form):
    c = make_case(150 + len(name), name=name, d=128, dtype="bf16", n_sink=4, n_recent=64, k_sel=64,
                  hh_per_head=20, **kw)
    dc = DevCase(c)
    assert form(_splits(gpu_lib, 0, c, dc))
    _dense_check(gpu_lib, c, dc)


def test_dense_without_scores_and_determinism(gpu_lib):
    c = make_case(110, name="h", B=2, Hq=16, Hkv=8, d=128, dtype="bf16", seq_lens=[2500, 900], n_sink=4,
                  n_recent=64, k_sel=64)
    dc = DevCase(c)
    o1, l1, _ = _dense_check(gpu_lib, c, dc, with_scores=False)
    o2, l2, _ = _dense_check(gpu_lib, c, dc, with_scores=False)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_bound_calls_repeat_the_direct_calls(gpu_lib):
    """bind() marshals a call once; replaying it gives bit-identical results to the direct call."""
    c = make_case(112, name="bind", B=2, Hq=16, Hkv=8, d=128, dtype="bf16", seq_lens=[3000, 1200], n_sink=4,
                  n_recent=64, k_sel=200)
    dc = DevCase(c)
    o1, l1, s1 = gpu_lib.dense_attn_with_stats(dc.q[:, :1].contiguous(), dc.k, dc.v, dc.bt, dc.lens,
                                               max_seq_len=dc.max_seq_len, n_sink=4, n_recent=64)
    sel1 = gpu_lib.select_topk(s1, dc.lens, k=200, n_sink=4, n_recent=64)
    o2, l2, s2 = torch.empty_like(o1), torch.empty_like(l1), torch.empty_like(s1)
    sel2 = torch.empty_like(sel1)
    ws = torch.zeros(gpu_lib.workspace_size("dense", k_pool=dc.k, block_table=dc.bt, Hq=16, dtype=torch.bfloat16,
                                            max_seq_len=dc.max_seq_len), dtype=torch.uint8, device=DEV)
    dense = gpu_lib.bind(gpu_lib.dense_attn_with_stats, dc.q[:, :1].contiguous(), dc.k, dc.v, dc.bt, dc.lens,
                         max_seq_len=dc.max_seq_len, n_sink=4, n_recent=64, out=o2, lse=l2, scores=s2, workspace=ws)
    select = gpu_lib.bind(gpu_lib.select_topk, s2, dc.lens, k=200, n_sink=4, n_recent=64, sel_idx=sel2)
    for _ in range(2):
        dense()
        select()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(s1, s2) and torch.equal(sel1, sel2)
    # Buffers the entry point allocates itself (outputs, workspace) stay with the bound call.
    auto = gpu_lib.bind(gpu_lib.dense_attn_with_stats, dc.q[:, :1].contiguous(), dc.k, dc.v, dc.bt, dc.lens,
                        max_seq_len=dc.max_seq_len, n_sink=4, n_recent=64)
    auto()
    torch.cuda.synchronize()
    o3, l3, s3 = auto.outputs
    assert torch.equal(o1, o3) and torch.equal(l1, l3) and torch.equal(s1, s3)


def test_bound_calls_keep_the_tensors_they_were_given(gpu_lib):
    """A bound call holds its tensors: temporaries passed to bind() are not freed and reused."""
    c = make_case(113, name="keep", B=2, Hq=16, Hkv=8, d=128, dtype="bf16", seq_lens=[2500, 900], n_sink=4,
                  n_recent=64, k_sel=128)
    dc = DevCase(c)
    rng = np.random.default_rng(3)
    sel = dev_array(np.stack([_random_selection(rng, c, int(c.seq_lens[b]), 128) for b in range(2)]))
    ck, cv, nc = gpu_lib.pack_compact(dc.k, dc.v, dc.bt, dc.lens, sel, n_sink=4, cap=132, max_seq_len=dc.max_seq_len)
    kw = dict(n_sink=4, n_recent=64, max_seq_len=dc.max_seq_len)
    o1, l1 = gpu_lib.sparse_decode_attn(dc.q[:, 0].contiguous(), dc.k, dc.v, dc.bt, dc.lens, ck, cv, nc, **kw)
    call = gpu_lib.bind(gpu_lib.sparse_decode_attn, dc.q[:, 0].contiguous(), dc.k, dc.v, dc.bt, dc.lens, ck.clone(),
                        cv.clone(), nc.clone(), **kw)
    torch.cuda.synchronize()
    churn = [torch.full_like(ck, float("nan")) for _ in range(4)] + [torch.full_like(dc.q, float("nan"))]
    call()
    torch.cuda.synchronize()
    o2, l2 = call.outputs
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    del churn


def test_dense_is_invariant_to_physical_page_order(gpu_lib):
    c = make_case(111, name="i", B=1, Hq=8, Hkv=4, d=128, dtype="bf16", seq_lens=[1800], n_sink=4,
                  n_recent=32, k_sel=64, spare_pages=7)
    dc = DevCase(c)
    o1, l1, s1 = _dense_check(gpu_lib, c, dc)
    # Move every page to a new physical slot and rewrite the block table accordingly.
    rng = np.random.default_rng(5)
    perm = rng.permutation(c.kv.num_pages)
    k2, v2 = np.empty_like(c.kv.k), np.empty_like(c.kv.v)
    k2[perm], v2[perm] = c.kv.k, c.kv.v
    bt2 = np.where(c.kv.block_table >= 0, perm[np.maximum(c.kv.block_table, 0)], -1).astype(np.int32)
    out, lse, sc = gpu_lib.dense_attn_with_stats(dc.q, dev_array(k2), dev_array(v2), dev_array(bt2), dc.lens,
                                                 max_seq_len=dc.max_seq_len, n_sink=c.n_sink,
                                                 n_recent=c.n_recent)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), o1) and np.array_equal(lse.cpu().numpy(), l1)
    assert np.array_equal(sc.cpu().numpy(), s1)


def test_invalid_block_table_entries_are_skipped(gpu_lib):
    c = make_case(112, name="j", B=1, Hq=4, Hkv=2, d=128, dtype="bf16", seq_lens=[640], n_sink=4,
                  n_recent=32, k_sel=16)
    bt = c.kv.block_table.copy()
    bt[0, 7] = -5                       # page 7 (positions 112..127) unusable
    bt[0, 9] = c.kv.num_pages + 100     # page 9 (positions 144..159) out of the pool
    dc = DevCase(c)
    out, lse, sc = gpu_lib.dense_attn_with_stats(dc.q, dc.k, dc.v, dev_array(bt), dc.lens,
                                                 max_seq_len=dc.max_seq_len, n_sink=4, n_recent=32)
    torch.cuda.synchronize()
    keep = np.ones(640, bool)
    keep[112:128] = False
    keep[144:160] = False
    pos = np.arange(640)[keep]
    for g in range(2):
        K = O.paged_rows(c.kv.k_values(), c.kv.block_table[0], g, pos)
        V = O.paged_rows(c.kv.v_values(), c.kv.block_table[0], g, pos)
        ref, _ = O.softmax_attention(c.q_values()[0, 0, 2 * g:2 * g + 2], K, V, c.scale)
        assert_close(out.cpu().numpy()[0, 0, 2 * g:2 * g + 2], ref, OUT_TOL, f"g={g}")
    s = sc.cpu().numpy()
    assert np.all(np.isneginf(s[0, :, 112:128])) and np.all(np.isneginf(s[0, :, 144:160]))


# --------------------------------------------------------------------------- fast step

def _random_selection(rng, c, L, k):
    lo, hi = O.candidate_range(L, 1, c.n_sink, c.n_recent)
    k_eff = min(k, hi - lo)
    sel = np.full((c.Hkv, k), -1, np.int32)
    for g in range(c.Hkv):
        sel[g, :k_eff] = np.sort(rng.choice(np.arange(lo, hi), k_eff, replace=False))
    return sel


def _fast_step_check(sfi, c, dc, sels, cap, L_fast, q_fast_store, q_fast_vals):
    """Pack the given selections on the GPU, run the fast step at lengths L_fast, compare to the oracle."""
    sel_d = dev_array(np.stack(sels).astype(np.int32))
    ck, cv, nc = sfi.pack_compact(dc.k, dc.v, dc.bt, dc.lens, sel_d, n_sink=c.n_sink, cap=cap,
                                  max_seq_len=dc.max_seq_len)
    lens_f = dc.lens_tensor(L_fast)
    out, lse = sfi.sparse_decode_attn(dev_array(q_fast_store), dc.k, dc.v, dc.bt, lens_f, ck, cv, nc,
                                      n_sink=c.n_sink, n_recent=c.n_recent, max_seq_len=dc.max_seq_len,
                                      scale=c.scale)
    torch.cuda.synchronize()
    out, lse, ncn = out.cpu().numpy(), lse.cpu().numpy(), nc.cpu().numpy()
    for b in range(c.B):
        rck, rcv, rnc = O.pack_compact(c.kv.k, c.kv.v, c.kv.block_table[b], int(c.seq_lens[b]), c.n_sink,
                                       sels[b], cap)
        assert ncn[b] == rnc
        ref_o, ref_l = O.sparse_decode(q_fast_vals[b], rck, rcv, rnc, c.kv.k, c.kv.v, c.kv.block_table[b],
                                       int(L_fast[b]), c.n_sink, c.n_recent, c.scale, kv_dtype=c.dtype)
        assert_close(out[b], ref_o, OUT_TOL, f"fast out b={b}")
        assert_close(lse[b], ref_l, LSE_TOL, f"fast lse b={b}")
    return out, lse


FAST_CASES = [
    ("tiny_fp32", lambda: tiny_case(2), 64),
    ("bf16_g2_L4000_k600", lambda: make_case(121, name="a", B=1, Hq=16, Hkv=8, d=128, dtype="bf16",
                                              seq_lens=[4000], capacity=[4010], n_sink=4, n_recent=64,
                                              k_sel=600), 600),
    ("bf16_g4_ragged", lambda: make_case(122, name="b", B=3, Hq=8, Hkv=2, d=128, dtype="bf16",
                                          seq_lens=[300, 5000, 2047], capacity=[310, 5010, 2050], n_sink=4,
                                          n_recent=256, k_sel=1024), 1024),
    ("f32_g2_d128", lambda: make_case(123, name="c", B=2, Hq=4, Hkv=2, d=128, dtype="f32",
                                       seq_lens=[900, 1200], capacity=[905, 1205], n_sink=4, n_recent=32,
                                       k_sel=200), 200),
    ("bf16_g8_d64", lambda: make_case(124, name="d", B=1, Hq=8, Hkv=1, d=64, dtype="bf16",
                                       seq_lens=[2000], capacity=[2003], n_sink=4, n_recent=48, k_sel=333), 333),
    # 16 requests x 8 KV heads, several splits each
    ("bf16_b16_large_grid", lambda: make_case(125, name="e16", B=16, Hq=16, Hkv=8, d=128, dtype="bf16",
                                               seq_lens=list(range(1500, 3100, 100)),
                                               capacity=list(range(1504, 3104, 100)), n_sink=4, n_recent=64,
                                               k_sel=1024), 1024),
]


@pytest.mark.parametrize("name,mk,k", FAST_CASES, ids=[n for n, _, _ in FAST_CASES])
def test_fast_step_matches_oracle(gpu_lib, name, mk, k):
    c = mk()
    dc = DevCase(c)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    sels = [_random_selection(rng, c, int(c.seq_lens[b]), k) for b in range(c.B)]
    cap = c.n_sink + k + 3
    if "large_grid" in name:   # many units, each merged from several splits
        assert _splits(gpu_lib, 1, c, dc, cap=cap) >= 2
    # Fast step a few tokens after the slow step (appended tokens already sit in the pool).
    L_fast = np.minimum(c.seq_lens + 3, c.kv.max_pages * 16).astype(np.int32)
    qv = c.q_values()[:, 0]
    _fast_step_check(gpu_lib, c, dc, sels, cap, L_fast, c.q[:, 0], qv)


@pytest.mark.parametrize("recent_split", ["1", "0"])
def test_fast_step_under_both_split_plans(gpu_lib, recent_split, monkeypatch):
    # 1 request x 8 KV heads, 1984 compact slots + 64 recent tokens: by default 16 compact splits and the
    # recent window as a 17th split of its own; SFI_TUNE_RECENT_SPLIT=0 cuts the 2048 rows into 16 even
    # splits.  Both plans against the oracle.
    monkeypatch.setenv("SFI_TUNE_RECENT_SPLIT", recent_split)
    c = make_case(126, name="rs", B=1, Hq=16, Hkv=8, d=128, dtype="bf16", seq_lens=[4000], capacity=[4010],
                  n_sink=4, n_recent=64, k_sel=1980)
    dc = DevCase(c)
    k = 1980
    cap = c.n_sink + k
    assert _splits(gpu_lib, 1, c, dc, cap=cap) == (17 if recent_split == "1" else 16)
    rng = np.random.default_rng(126)
    sels = [_random_selection(rng, c, int(c.seq_lens[b]), k) for b in range(c.B)]
    L_fast = np.minimum(c.seq_lens + 3, c.kv.max_pages * 16).astype(np.int32)
    _fast_step_check(gpu_lib, c, dc, sels, cap, L_fast, c.q[:, 0], c.q_values()[:, 0])


def test_fast_step_at_full_retention_equals_dense(gpu_lib):
    c = qwen06b_decode_case(131, L=3072, frac=(1, 1))
    dc = DevCase(c)
    L = 3072
    lo, hi = O.candidate_range(L, 1, c.n_sink, c.n_recent)
    sel = [np.tile(np.arange(lo, hi, dtype=np.int32), (c.Hkv, 1))]
    out_s, lse_s = _fast_step_check(gpu_lib, c, dc, sel, hi, np.array([L], np.int32), c.q[:, 0],
                                    c.q_values()[:, 0])
    out_d, lse_d, _ = gpu_lib.dense_attn_with_stats(dc.q, dc.k, dc.v, dc.bt, dc.lens, max_seq_len=dc.max_seq_len,
                                                    with_scores=False)
    torch.cuda.synchronize()
    assert_close(out_s, out_d.cpu().numpy()[:, 0], OUT_TOL, "sparse@100% vs dense")


def test_fast_step_single_key_returns_its_value_exactly(gpu_lib):
    for dtype in ("f32", "bf16"):
        c = make_case(132, name="s", B=1, Hq=4, Hkv=2, d=128, dtype=dtype, seq_lens=[64], n_sink=1, n_recent=0,
                      k_sel=1)
        dc = DevCase(c)
        sel = np.full((1, 2, 1), -1, np.int32)   # no selected token: compact = the single sink row
        ck, cv, nc = gpu_lib.pack_compact(dc.k, dc.v, dc.bt, dc.lens, dev_array(sel), n_sink=1, cap=4,
                                          max_seq_len=dc.max_seq_len)
        out, lse = gpu_lib.sparse_decode_attn(dev_array(c.q[:, 0]), dc.k, dc.v, dc.bt, dc.lens, ck, cv, nc,
                                              n_sink=1, n_recent=0, max_seq_len=dc.max_seq_len)
        torch.cuda.synchronize()
        assert int(nc.cpu()[0]) == 1
        V0 = O.paged_rows(c.kv.v_values(), c.kv.block_table[0], 0, [0])[0]
        V1 = O.paged_rows(c.kv.v_values(), c.kv.block_table[0], 1, [0])[0]
        o = out.cpu().numpy()[0]
        assert np.array_equal(o[0], V0) and np.array_equal(o[1], V0)
        assert np.array_equal(o[2], V1) and np.array_equal(o[3], V1)


def test_fast_step_empty_compact_and_empty_state(gpu_lib):
    c = make_case(133, name="e", B=2, Hq=4, Hkv=2, d=128, dtype="bf16", seq_lens=[200, 200], n_sink=4,
                  n_recent=16, k_sel=8)
    dc = DevCase(c)
    ck = torch.zeros((2, 2, 16, 128), dtype=torch.bfloat16, device=DEV)
    cv = torch.zeros_like(ck)
    nc = torch.tensor([0, 0], dtype=torch.int32, device=DEV)
    lens = dc.lens_tensor([200, 3])          # request 1: shorter than the sink -> no recent tokens either
    out, lse = gpu_lib.sparse_decode_attn(dev_array(c.q[:, 0]), dc.k, dc.v, dc.bt, lens, ck, cv, nc, n_sink=4,
                                          n_recent=16, max_seq_len=dc.max_seq_len)
    torch.cuda.synchronize()
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    for g in range(2):
        K = O.paged_rows(c.kv.k_values(), c.kv.block_table[0], g, np.arange(184, 200))
        V = O.paged_rows(c.kv.v_values(), c.kv.block_table[0], g, np.arange(184, 200))
        ref, _ = O.softmax_attention(c.q_values()[0, 0, 2 * g:2 * g + 2], K, V, c.scale)
        assert_close(o[0, 2 * g:2 * g + 2], ref, OUT_TOL, "recent only")
    assert np.all(o[1] == 0) and np.all(np.isneginf(l[1]))


def test_tiny_sequence_one_slow_step_then_eight_fast_steps(gpu_lib):
    """The tiny fp32 workload: slow step at L=1024 (dense + logits + top-64 + pack), then eight fast steps
    at L = 1025..1032, each seeing one more appended token."""
    c = tiny_case(7)
    dc = DevCase(c)
    L = 1024
    out, lse, sc = _dense_check(gpu_lib, c, dc)
    lo, hi = O.candidate_range(L, 1, c.n_sink, c.n_recent)
    sel = gpu_lib.select_topk(torch.from_numpy(sc).to(DEV), dc.lens, k=c.k_sel, n_sink=c.n_sink,
                              n_recent=c.n_recent)
    ref_sel = O.select_topk(sc[0, 0], lo, hi, c.k_sel)
    assert np.array_equal(sel.cpu().numpy()[0, 0], ref_sel)
    assert set(c.planted[(0, 0)].tolist()) <= set(ref_sel.tolist())
    cap = c.n_sink + c.k_sel
    ck, cv, nc = gpu_lib.pack_compact(dc.k, dc.v, dc.bt, dc.lens, sel, n_sink=c.n_sink, cap=cap,
                                      max_seq_len=dc.max_seq_len)
    rck, rcv, rnc = O.pack_compact(c.kv.k, c.kv.v, c.kv.block_table[0], L, c.n_sink, ref_sel[None], cap)
    for step in range(8):
        Lf = L + 1 + step
        out, lse = gpu_lib.sparse_decode_attn(dev_array(c.extra_q[step]), dc.k, dc.v, dc.bt, dc.lens_tensor([Lf]),
                                              ck, cv, nc, n_sink=c.n_sink, n_recent=c.n_recent,
                                              max_seq_len=dc.max_seq_len)
        torch.cuda.synchronize()
        ref_o, ref_l = O.sparse_decode(c.extra_q_values()[step, 0], rck, rcv, rnc, c.kv.k, c.kv.v,
                                       c.kv.block_table[0], Lf, c.n_sink, c.n_recent, c.scale)
        assert_close(out.cpu().numpy()[0], ref_o, OUT_TOL, f"step {step}")
        assert_close(lse.cpu().numpy()[0], ref_l, LSE_TOL, f"step {step}")


@pytest.mark.parametrize("L", [64, 65, 128, 129, 255, 256, 257, 2048, 2049, 4096, 4097])
def test_slow_step_logits_at_tile_and_split_boundaries(gpu_lib, L):
    """Lengths on and one past the slow step's iteration (64 tokens), iteration-pair (128) and split
    boundaries; the plan gives these lengths 64 to 320 tokens per split, some not a whole number of
    pairs (192, 320).  Each split keeps its logits in LDS and writes them after its loop, so every
    boundary decides which positions a split writes.  The plain slow step is checked against the
    oracle; the variant that leaves its combine to a later launch must write the same logits, bit for
    bit."""
    c = make_case(1200 + L, name="tb", B=2, Hq=16, Hkv=8, d=128, dtype="bf16", seq_lens=[L, max(1, L - 1)],
                  n_sink=4, n_recent=64, k_sel=8, hh_per_head=2)
    dc = DevCase(c)
    stride = dc.max_seq_len + 5
    _, _, sc = _dense_check(gpu_lib, c, dc, stride=stride)
    _, _, sc_d, _ = gpu_lib.dense_attn_with_stats_deferred(dc.q, dc.k, dc.v, dc.bt, dc.lens,
                                                           max_seq_len=dc.max_seq_len, n_sink=c.n_sink,
                                                           n_recent=c.n_recent, scale=c.scale, score_stride=stride)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(sc_d).view(np.uint32), sc.view(np.uint32))
