"""GPU parity at the library's size limits.

* The longest context a call accepts (max_seq_len = 256 splits x 4096 tokens =
  1,048,576): slow step with logits (256 splits per KV head), the Selector's
  streaming variant for rows beyond 65536 candidates, pack and fast step, against
  the oracle on every KV head (2 KV heads keep the pools at 1 GiB).
* The largest mixed launch (64 requests, alternating draft / verify), every request
  checked.
"""
import numpy as np
import pytest
import torch

import oracle as O
from sfi_synth import make_case
from _gpu import DEV, LSE_TOL, OUT_TOL, DevCase, assert_close, dev_array, host_bits, score_bound

pytestmark = pytest.mark.gpu

MAX_TOKENS = 256 * 4096


def test_longest_context_slow_step_selector_pack_and_fast_step(gpu_lib):
    L = MAX_TOKENS
    c = make_case(501, name="max", B=1, Hq=8, Hkv=2, d=128, dtype="bf16", seq_lens=[L], n_sink=4, n_recent=256,
                  k_sel=4096, hh_per_head=64)
    dc = DevCase(c)
    assert dc.max_seq_len == L
    st, ns = gpu_lib.plan_splits(0, B=1, Hq=8, Hkv=2, d=128, bf16=True, max_pages=c.kv.max_pages,
                                 num_pages=c.kv.num_pages, max_seq_len=L)
    assert ns == 256 and st == 4096
    k, cap = c.k_sel, c.n_sink + c.k_sel
    out, lse, sc = gpu_lib.dense_attn_with_stats(dc.q, dc.k, dc.v, dc.bt, dc.lens, max_seq_len=L, n_sink=4,
                                                 n_recent=256)
    sel = gpu_lib.select_topk(sc, dc.lens, k=k, n_sink=4, n_recent=256)
    ck, cv, nc = gpu_lib.pack_compact(dc.k, dc.v, dc.bt, dc.lens, sel, n_sink=4, cap=cap, max_seq_len=L)
    fo, fl = gpu_lib.sparse_decode_attn(dc.q[:, 0].contiguous(), dc.k, dc.v, dc.bt, dc.lens, ck, cv, nc, n_sink=4,
                                        n_recent=256, max_seq_len=L)
    torch.cuda.synchronize()
    qv = c.q_values()[0, 0]
    bt = c.kv.block_table[0]
    ro, rl = O.dense_attention(qv[None], c.kv.k, c.kv.v, bt, L, c.scale, 2, kv_dtype="bf16")
    assert_close(out.cpu().numpy()[0, 0], ro[0], OUT_TOL, "dense out")
    assert_close(lse.cpu().numpy()[0, 0], rl[0], LSE_TOL, "dense lse")
    S = sc.cpu().numpy()[0]
    lo, hi = O.candidate_range(L, 1, 4, 256)
    kvals = c.kv.k_values()
    rng = np.random.default_rng(5)
    for g in range(2):
        # logits: sampled positions plus the planted ones, within the fp32 bound
        pos = np.unique(np.r_[rng.integers(lo, hi, 4096), c.planted[(0, g)], lo, hi - 1])
        ref = O.group_scores(qv[None], c.kv.k, bt, L, c.scale, 2, 4, 256, L, kv_dtype="bf16", groups=[g])[g, pos]
        rows = O.paged_rows(kvals, bt, g, pos)
        assert_close(S[g, pos], ref, score_bound(qv[4 * g:4 * g + 4], rows, c.scale), f"logits g={g}")
        assert np.all(np.isneginf(S[g, :lo])) and np.all(np.isneginf(S[g, hi:]))
    got_sel = sel.cpu().numpy()[0]
    ref_sel = np.stack([O.select_topk(S[g].astype(np.float64), lo, hi, k) for g in range(2)])
    assert np.array_equal(got_sel, ref_sel)
    for g in range(2):
        assert set(c.planted[(0, g)].tolist()) <= set(got_sel[g].tolist())
    rck, rcv, rnc = O.pack_compact(c.kv.k, c.kv.v, bt, L, 4, ref_sel, cap)
    assert int(nc.cpu()[0]) == rnc
    assert np.array_equal(host_bits(ck)[0], rck) and np.array_equal(host_bits(cv)[0], rcv)
    so, sl = O.sparse_decode(qv, rck, rcv, rnc, c.kv.k, c.kv.v, bt, L, 4, 256, c.scale, kv_dtype="bf16")
    assert_close(fo.cpu().numpy()[0], so, OUT_TOL, "fast out")
    assert_close(fl.cpu().numpy()[0], sl, LSE_TOL, "fast lse")


def test_mixed_launch_at_its_largest_batch(gpu_lib):
    B = 64
    rng = np.random.default_rng(6)
    lens = rng.integers(200, 1400, size=B).tolist()
    c = make_case(502, name="mix64", B=B, Hq=8, Hkv=2, d=128, dtype="bf16", t_q=4, seq_lens=lens, n_sink=4,
                  n_recent=32, k_sel=48)
    dc = DevCase(c)
    modes = [b % 2 for b in range(B)]
    sel = np.full((B, 2, 48), -1, np.int32)
    for b in range(B):
        lo, hi = O.candidate_range(lens[b], 1, 4, 32)
        for g in range(2):
            sel[b, g] = np.sort(rng.choice(np.arange(lo, hi), 48, replace=False))
    cap = 52
    ck, cv, nc = gpu_lib.pack_compact(dc.k, dc.v, dc.bt, dc.lens, dev_array(sel), n_sink=4, cap=cap,
                                      max_seq_len=dc.max_seq_len)
    t_q = [1 if m == 0 else 4 for m in modes]
    q_packed = np.concatenate([c.q[b, -1:] if modes[b] == 0 else c.q[b] for b in range(B)], axis=0)
    out, lse, sc = gpu_lib.mixed_attn(dev_array(q_packed), dc.k, dc.v, dc.bt, dc.lens, modes, t_q, ck, cv, nc,
                                      n_sink=4, n_recent=32, max_seq_len=dc.max_seq_len, scale=c.scale)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    row0 = np.concatenate([[0], np.cumsum(t_q)])
    for b in range(B):
        Qv = c.q_values()[b]
        L = lens[b]
        r = int(row0[b])
        if modes[b] == 0:
            rck, rcv, rnc = O.pack_compact(c.kv.k, c.kv.v, c.kv.block_table[b], L, 4, sel[b], cap)
            ro, rl = O.sparse_decode(Qv[-1], rck, rcv, rnc, c.kv.k, c.kv.v, c.kv.block_table[b], L, 4, 32, c.scale,
                                     kv_dtype="bf16")
            assert_close(out[r], ro, OUT_TOL, f"draft out b={b}")
            assert_close(lse[r], rl, LSE_TOL, f"draft lse b={b}")
        else:
            ro, rl = O.dense_attention(Qv, c.kv.k, c.kv.v, c.kv.block_table[b], L, c.scale, 2, kv_dtype="bf16")
            assert_close(out[r:r + 4], ro, OUT_TOL, f"verify out b={b}")
            assert_close(lse[r:r + 4], rl, LSE_TOL, f"verify lse b={b}")
