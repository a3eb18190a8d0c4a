"""GPU parity of per-query-head selection: the slow step with one logit row per query
head (sfi_dense_attn_with_head_stats), the Selector over those rows, and the fast
step with one selected set per query head (sfi_sparse_decode_indexed_attn with
per_head = 1), against the oracle's head_scores / select_topk / indexed_decode_heads.
Logits within the fp32 forward-error bound, selections bit-exact given the GPU's
logits, outputs within 2e-3 and lse within 1e-3.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle as O
from sfi_synth import bf16_bits, make_case
from _gpu import DEV, LSE_TOL, OUT_TOL, DevCase, assert_close, dev_array, host_bits, score_bound

pytestmark = pytest.mark.gpu


HEAD_CASES = [
    ("bf16_g2_ragged", lambda: make_case(401, name="hd_a", B=3, Hq=16, Hkv=8, d=128, dtype="bf16",
                                          seq_lens=[700, 3000, 1500], n_sink=4, n_recent=64, k_sel=200), 200),
    ("bf16_g4_d128", lambda: make_case(402, name="hd_b", B=2, Hq=32, Hkv=8, d=128, dtype="bf16",
                                        seq_lens=[4000, 2222], n_sink=4, n_recent=64, k_sel=256, hh_per_head=16), 256),
    ("f32_g8_d64", lambda: make_case(403, name="hd_c", B=1, Hq=8, Hkv=1, d=64, dtype="f32", seq_lens=[1800],
                                      n_sink=4, n_recent=32, k_sel=100), 100),
]


@pytest.mark.parametrize("name,mk,k", HEAD_CASES, ids=[n for n, _, _ in HEAD_CASES])
def test_head_stats_select_and_per_head_fast_step(gpu_lib, name, mk, k):
    c = mk()
    dc = DevCase(c)
    q1 = dc.q[:, 0].contiguous()
    out, lse, S = gpu_lib.dense_attn_with_head_stats(q1, dc.k, dc.v, dc.bt, dc.lens, max_seq_len=dc.max_seq_len,
                                                     n_sink=c.n_sink, n_recent=c.n_recent, scale=c.scale)
    sel = torch.empty((c.B, c.Hq, k), dtype=torch.int32, device=DEV)
    gpu_lib.select_topk(S, dc.lens, k=k, n_sink=c.n_sink, n_recent=c.n_recent, sel_idx=sel)
    L_fast = np.minimum(c.seq_lens + 0, c.kv.max_pages * 16).astype(np.int32)
    fo, fl = gpu_lib.sparse_decode_indexed_attn(q1, dc.k, dc.v, dc.bt, dc.lens, sel, n_sink=c.n_sink,
                                                n_recent=c.n_recent, max_seq_len=dc.max_seq_len, scale=c.scale,
                                                per_head=True)
    torch.cuda.synchronize()
    out, lse, S, sel = out.cpu().numpy(), lse.cpu().numpy(), S.cpu().numpy(), sel.cpu().numpy()
    fo, fl = fo.cpu().numpy(), fl.cpu().numpy()
    qv = c.q_values()[:, 0]
    kv_vals = c.kv.k_values()
    for b in range(c.B):
        L = int(c.seq_lens[b])
        ro, rl = O.dense_attention(qv[b][None], c.kv.k, c.kv.v, c.kv.block_table[b], L, c.scale, c.Hkv,
                                   kv_dtype=c.dtype)
        assert_close(out[b], ro[0], OUT_TOL, f"dense out b={b}")
        assert_close(lse[b], rl[0], LSE_TOL, f"dense lse b={b}")
        RS = O.head_scores(qv[b], c.kv.k, c.kv.block_table[b], L, c.scale, c.Hkv, c.n_sink, c.n_recent,
                           dc.max_seq_len, kv_dtype=c.dtype)
        lo, hi = O.candidate_range(L, 1, c.n_sink, c.n_recent)
        assert np.all(np.isneginf(S[b][:, :lo])) and np.all(np.isneginf(S[b][:, hi:]))
        for h in range(c.Hq):
            rows = O.paged_rows(kv_vals, c.kv.block_table[b], h // c.G, np.arange(lo, hi))
            assert_close(S[b, h, lo:hi], RS[h, lo:hi], score_bound(qv[b, h][None], rows, c.scale), f"S b={b} h={h}")
            ref_sel = O.select_topk(S[b, h].astype(np.float64), lo, hi, k)
            assert np.array_equal(sel[b, h], ref_sel), (b, h)
        o2, l2 = O.indexed_decode_heads(qv[b], c.kv.k, c.kv.v, c.kv.block_table[b], int(L_fast[b]), c.n_sink,
                                        c.n_recent, sel[b], c.scale, kv_dtype=c.dtype)
        assert_close(fo[b], o2, OUT_TOL, f"fast out b={b}")
        assert_close(fl[b], l2, LSE_TOL, f"fast lse b={b}")


def test_per_head_sets_equal_across_the_group_match_the_group_fast_step(gpu_lib):
    c = make_case(404, name="hd_d", B=2, Hq=16, Hkv=4, d=128, dtype="bf16", seq_lens=[2500, 900], n_sink=4,
                  n_recent=64, k_sel=300)
    dc = DevCase(c)
    rng = np.random.default_rng(zlib.crc32(b"hd_d"))
    sel = np.full((2, 4, 300), -1, np.int32)
    for b in range(2):
        lo, hi = O.candidate_range(int(c.seq_lens[b]), 1, 4, 64)
        for g in range(4):
            n = min(300, hi - lo)
            sel[b, g, :n] = np.sort(rng.choice(np.arange(lo, hi), n, replace=False))
    q1 = dc.q[:, 0].contiguous()
    kw = dict(n_sink=4, n_recent=64, max_seq_len=dc.max_seq_len, scale=c.scale)
    go, gl = gpu_lib.sparse_decode_indexed_attn(q1, dc.k, dc.v, dc.bt, dc.lens, dev_array(sel), **kw)
    ho, hl = gpu_lib.sparse_decode_indexed_attn(q1, dc.k, dc.v, dc.bt, dc.lens, dev_array(np.repeat(sel, 4, axis=1)),
                                                per_head=True, **kw)
    torch.cuda.synchronize()
    assert_close(ho.cpu().numpy(), go.cpu().numpy().astype(np.float64), 1e-5, "out")
    assert_close(hl.cpu().numpy(), gl.cpu().numpy().astype(np.float64), 1e-5, "lse")


def test_per_head_fast_step_with_append_stores_each_kv_head_once(gpu_lib):
    c = make_case(405, name="hd_e", B=2, Hq=16, Hkv=4, d=128, dtype="bf16", seq_lens=[1200, 640],
                  capacity=[1210, 650], n_sink=4, n_recent=32, k_sel=64)
    dc = DevCase(c)
    rng = np.random.default_rng(11)
    sel = np.full((2, 16, 64), -1, np.int32)
    for b in range(2):
        lo, hi = O.candidate_range(int(c.seq_lens[b]), 1, 4, 32)
        for h in range(16):
            sel[b, h] = np.sort(rng.choice(np.arange(lo, hi), 64, replace=False))
    x = rng.standard_normal((2, 2, 4, 128)).astype(np.float32)
    kn, vn = bf16_bits(x[0]), bf16_bits(x[1])
    L = (c.seq_lens + 1).astype(np.int32)
    fo, fl = gpu_lib.sparse_decode_indexed_attn(dc.q[:, 0].contiguous(), dc.k, dc.v, dc.bt, dc.lens_tensor(L),
                                                dev_array(sel), n_sink=4, n_recent=32, max_seq_len=dc.max_seq_len,
                                                scale=c.scale, per_head=True, k_new=dev_array(kn), v_new=dev_array(vn))
    torch.cuda.synchronize()
    kp, vp = c.kv.k, c.kv.v
    for b in range(2):
        kp, vp = O.append_token(kp, vp, c.kv.block_table[b], int(L[b]), kn[b], vn[b])
    np.testing.assert_array_equal(host_bits(dc.k), kp)
    np.testing.assert_array_equal(host_bits(dc.v), vp)
    qv = c.q_values()[:, 0]
    fo, fl = fo.cpu().numpy(), fl.cpu().numpy()
    for b in range(2):
        ro, rl = O.indexed_decode_heads(qv[b], kp, vp, c.kv.block_table[b], int(L[b]), 4, 32, sel[b], c.scale,
                                        kv_dtype="bf16")
        assert_close(fo[b], ro, OUT_TOL, f"out b={b}")
        assert_close(fl[b], rl, LSE_TOL, f"lse b={b}")
