"""GPU parity of the MFMA multi-query causal verification (t_q > 1) against the fp64 oracle.

Outputs within 2e-3 max-abs and lse within 1e-3; the verification statistics
(masked logits summed over every query token and head of the group) within the
fp32 forward error bound.  Cases span one and several splits, ragged request
lengths, d = 64 and 128, 2 to 32 query rows per KV head, and invalid pages.
"""
import numpy as np
import pytest
import torch

import oracle as O
from sfi_synth import make_case
from _gpu import LSE_TOL, OUT_TOL, DevCase, assert_close, dev_array, score_bound

pytestmark = pytest.mark.gpu


def _verify_check(sfi, c, dc, bt=None, with_scores=True, stride=None):
    bt_dev = dc.bt if bt is None else dev_array(bt)
    bt_np = c.kv.block_table if bt is None else bt
    out, lse, sc = sfi.dense_attn_with_stats(dc.q, dc.k, dc.v, bt_dev, dc.lens, max_seq_len=dc.max_seq_len,
                                             n_sink=c.n_sink, n_recent=c.n_recent, scale=c.scale,
                                             with_scores=with_scores, score_stride=stride)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    sc = sc.cpu().numpy() if sc is not None else None
    Q, K = c.q_values(), c.kv.k_values()
    G = c.G
    for b in range(c.B):
        L = int(c.seq_lens[b])
        ref_o, ref_l = O.dense_attention(Q[b], c.kv.k, c.kv.v, bt_np[b], L, c.scale, c.Hkv, kv_dtype=c.dtype)
        assert_close(out[b], ref_o, OUT_TOL, f"out b={b}")
        assert_close(lse[b], ref_l, LSE_TOL, f"lse b={b}")
        if sc is None:
            continue
        ref_s = O.group_scores(Q[b], c.kv.k, bt_np[b], L, c.scale, c.Hkv, c.n_sink, c.n_recent, sc.shape[-1],
                               kv_dtype=c.dtype)
        lo, hi = O.candidate_range(L, c.t_q, c.n_sink, c.n_recent)
        for g in range(c.Hkv):
            assert np.all(np.isneginf(sc[b, g, :lo])) and np.all(np.isneginf(sc[b, g, hi:])), (b, g)
            if hi > lo:
                rows = O.paged_rows(K, bt_np[b], g, np.arange(lo, hi))
                qg = Q[b][:, g * G:(g + 1) * G, :].reshape(-1, c.d)
                assert_close(sc[b, g, lo:hi], ref_s[g, lo:hi], score_bound(qg, rows, c.scale), f"scores b={b} g={g}")
    return out, lse, sc


CASES = [
    ("g4_tq8_d128_ragged", dict(B=2, Hq=8, Hkv=2, d=128, t_q=8, seq_lens=[300, 1000])),
    ("g4_tq8_d128_long", dict(B=1, Hq=8, Hkv=2, d=128, t_q=8, seq_lens=[9000])),
    ("g2_tq4_d64", dict(B=2, Hq=4, Hkv=2, d=64, t_q=4, seq_lens=[777, 64])),
    ("g1_tq2_d128", dict(B=1, Hq=2, Hkv=2, d=128, t_q=2, seq_lens=[1500])),
    ("g2_tq16_d128", dict(B=1, Hq=4, Hkv=2, d=128, t_q=16, seq_lens=[2100])),
    ("g8_tq4_d128", dict(B=1, Hq=16, Hkv=2, d=128, t_q=4, seq_lens=[1234])),
    ("g4_tq8_short", dict(B=2, Hq=8, Hkv=2, d=128, t_q=8, seq_lens=[8, 40])),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[n for n, _ in CASES])
def test_verify_matches_oracle(gpu_lib, name, kw):
    c = make_case(300 + len(name), name=name, dtype="bf16", n_sink=4, n_recent=32, k_sel=64, hh_per_head=12, **kw)
    dc = DevCase(c)
    _verify_check(gpu_lib, c, dc, stride=dc.max_seq_len + 5)


def test_verify_without_scores_is_deterministic(gpu_lib):
    c = make_case(311, name="v", B=1, Hq=8, Hkv=2, d=128, dtype="bf16", t_q=8, seq_lens=[5000], n_sink=4,
                  n_recent=32, k_sel=64)
    dc = DevCase(c)
    o1, l1, _ = _verify_check(gpu_lib, c, dc, with_scores=False)
    o2, l2, _ = _verify_check(gpu_lib, c, dc, with_scores=False)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_verify_skips_invalid_pages(gpu_lib):
    c = make_case(312, name="v", B=1, Hq=8, Hkv=2, d=128, dtype="bf16", t_q=8, seq_lens=[900], n_sink=4,
                  n_recent=32, k_sel=64)
    dc = DevCase(c)
    bt = c.kv.block_table.copy()
    bt[0, 3] = -1
    out, lse, sc = gpu_lib.dense_attn_with_stats(dc.q, dc.k, dc.v, dev_array(bt), dc.lens,
                                                 max_seq_len=dc.max_seq_len, n_sink=4, n_recent=32)
    torch.cuda.synchronize()
    keep = np.ones(900, bool)
    keep[48:64] = False
    Q = c.q_values()[0]
    for t in range(8):
        pos = np.arange(900 - 8 + t + 1)
        pos = pos[keep[:len(pos)]]
        for g in range(2):
            K = O.paged_rows(c.kv.k_values(), c.kv.block_table[0], g, pos)
            V = O.paged_rows(c.kv.v_values(), c.kv.block_table[0], g, pos)
            ref, _ = O.softmax_attention(Q[t, 4 * g:4 * g + 4], K, V, c.scale)
            assert_close(out.cpu().numpy()[0, t, 4 * g:4 * g + 4], ref, OUT_TOL, f"t={t} g={g}")
    assert np.all(np.isneginf(sc.cpu().numpy()[0, :, 48:64]))


def test_verify_at_one_query_equals_the_slow_step(gpu_lib):
    """t_q = 1 goes through the vector kernel; a one-token verification through the MFMA path must agree
    with it (both within tolerance of the oracle, here compared directly)."""
    c = make_case(313, name="v", B=1, Hq=8, Hkv=2, d=128, dtype="bf16", t_q=2, seq_lens=[3000], n_sink=4,
                  n_recent=32, k_sel=64)
    dc = DevCase(c)
    out2, _, sc2 = gpu_lib.dense_attn_with_stats(dc.q, dc.k, dc.v, dc.bt, dc.lens, max_seq_len=dc.max_seq_len,
                                                 n_sink=4, n_recent=32)
    q1 = dc.q[:, 1:2].contiguous()            # the last query token alone, at position L - 1
    out1, _, _ = gpu_lib.dense_attn_with_stats(q1, dc.k, dc.v, dc.bt, dc.lens, max_seq_len=dc.max_seq_len,
                                               n_sink=4, n_recent=32)
    torch.cuda.synchronize()
    assert_close(out2.cpu().numpy()[0, 1], out1.cpu().numpy()[0, 0], 2 * OUT_TOL, "mfma vs vector")
