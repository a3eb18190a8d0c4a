"""GPU parity of the slow step whose split-K combine runs in a later launch.

sfi_dense_attn_with_stats_deferred leaves the slow step's split partials in the
workspace; after the Selector, sfi_sparse_decode_indexed_attn_merge (the fast step
over the selection, read in place) packs the compact buffer and merges the partials
into out and lse in the same launch.  The three calls must give out, lse, scores,
sel_idx and the compact buffer bit-identical to sfi_dense_attn_with_stats,
sfi_select_topk and sfi_pack_compact (which the other parity files check against
the oracle); the 16K layer is also checked against the fp64 oracle directly.  Cases
cover one and many splits, query groups of 1, 2, 4 and 8, fp32 and bf16, d 64 and
128, requests with fewer candidates than k, long rows, and both forms of the
launch's pack (blocks of their own, rows written by the attention).
"""
import numpy as np
import pytest
import torch

import oracle as O
from sfi_synth import make_case, qwen06b_decode_case, tiny_case
from _gpu import DEV, LSE_TOL, OUT_TOL, DevCase, assert_close, dev_array

pytestmark = pytest.mark.gpu

NAMES = ("out", "lse", "scores", "sel_idx", "compact_k", "compact_v", "n_compact")


def _bits(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    a = t.numpy()
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _zero_compact(dc, cap):
    """Compact buffers zeroed first: rows past n_compact are never written, so the two runs compare whole."""
    B, Hkv, d = int(dc.bt.shape[0]), int(dc.k.shape[1]), int(dc.k.shape[3])
    return (torch.zeros((B, Hkv, cap, d), dtype=dc.k.dtype, device=DEV),
            torch.zeros((B, Hkv, cap, d), dtype=dc.k.dtype, device=DEV))


def _pair(sfi, dc, n_sink, n_recent, k, workspace=None):
    """Deferred slow step, Selector, then the launch that packs and finishes the slow step."""
    out, lse, sc, ws = sfi.dense_attn_with_stats_deferred(dc.q, dc.k, dc.v, dc.bt, dc.lens,
                                                          max_seq_len=dc.max_seq_len, n_sink=n_sink,
                                                          n_recent=n_recent, workspace=workspace)
    sel = sfi.select_topk(sc, dc.lens, k=k, n_sink=n_sink, n_recent=n_recent)
    ck, cv = _zero_compact(dc, n_sink + k)
    nc = torch.empty((dc.q.shape[0],), dtype=torch.int32, device=DEV)
    sfi.sparse_decode_indexed_attn_merge(dc.q[:, -1].contiguous(), dc.k, dc.v, dc.bt, dc.lens, sel, n_sink=n_sink,
                                         n_recent=n_recent, max_seq_len=dc.max_seq_len, slow_out=out,
                                         slow_lse=lse, slow_workspace=ws, compact_k=ck, compact_v=cv,
                                         n_compact=nc)
    return out, lse, sc, sel, ck, cv, nc


def _separate(sfi, dc, n_sink, n_recent, k):
    out, lse, sc = sfi.dense_attn_with_stats(dc.q, dc.k, dc.v, dc.bt, dc.lens, max_seq_len=dc.max_seq_len,
                                             n_sink=n_sink, n_recent=n_recent)
    sel = sfi.select_topk(sc, dc.lens, k=k, n_sink=n_sink, n_recent=n_recent)
    ck, cv = _zero_compact(dc, n_sink + k)
    ck, cv, nc = sfi.pack_compact(dc.k, dc.v, dc.bt, dc.lens, sel, n_sink=n_sink, cap=n_sink + k,
                                  max_seq_len=dc.max_seq_len, compact_k=ck, compact_v=cv)
    return out, lse, sc, sel, ck, cv, nc


def _check_identical(sfi, c, k, n_splits_min=1):
    dc = DevCase(c)
    d = c.q.shape[-1]
    _, ns = sfi.plan_splits(0, B=c.B, Hq=c.Hq, Hkv=c.Hkv, d=d, bf16=(c.dtype == "bf16"),
                            max_pages=int(dc.bt.shape[1]), num_pages=int(dc.k.shape[0]), max_seq_len=dc.max_seq_len)
    assert ns >= n_splits_min, ns
    ref = _separate(sfi, dc, c.n_sink, c.n_recent, k)
    got = _pair(sfi, dc, c.n_sink, c.n_recent, k)
    torch.cuda.synchronize()
    for name, x, y in zip(NAMES, got, ref):
        assert np.array_equal(_bits(x), _bits(y)), f"{c.name}: {name} differs from the separate calls (splits {ns})"
    return dc, got


@pytest.mark.parametrize("name,mk,k,min_splits", [
    ("tiny_fp32_d64_g4", lambda: tiny_case(3), 64, 2),
    ("ragged_bf16_g4", lambda: make_case(611, name="ragged", B=3, Hq=16, Hkv=4, d=128, dtype="bf16",
                                         seq_lens=[5000, 333, 9000], n_sink=4, n_recent=64, k_sel=300,
                                         hh_per_head=10), 300, 2),
    ("g1_d64_bf16", lambda: make_case(612, name="g1", B=2, Hq=4, Hkv=4, d=64, dtype="bf16", seq_lens=[3000, 100],
                                      n_sink=4, n_recent=64, k_sel=200), 200, 2),
    ("g8_bf16", lambda: make_case(613, name="g8", B=2, Hq=64, Hkv=8, d=128, dtype="bf16", seq_lens=[6000, 2500],
                                  n_sink=4, n_recent=64, k_sel=512, hh_per_head=20), 512, 2),
    ("one_split_fp32", lambda: make_case(614, name="one_split", B=32, Hq=16, Hkv=8, d=64, dtype="f32",
                                         seq_lens=[300 + 7 * i for i in range(32)], n_sink=4, n_recent=32,
                                         k_sel=100), 100, 1),
])
def test_deferred_pair_equals_separate_calls(gpu_lib, name, mk, k, min_splits):
    _check_identical(gpu_lib, mk(), k, min_splits)


def test_deferred_pair_rows_beyond_the_register_selector(gpu_lib):
    """Rows of more than 65536 candidates (the streaming Selector variant) with the merge."""
    c = make_case(615, name="long", B=1, Hq=8, Hkv=2, d=128, dtype="bf16", seq_lens=[70000], n_sink=4,
                  n_recent=64, k_sel=2048)
    _check_identical(gpu_lib, c, 2048, 2)


def test_deferred_pair_16k_layer_matches_oracle(gpu_lib):
    c = qwen06b_decode_case(1000, L=16384, B=1, frac=(1, 8))
    dc, (out, lse, sc, sel, _, _, _) = _check_identical(gpu_lib, c, c.k_sel, 2)
    L = int(c.seq_lens[0])
    ref_o, ref_l = O.dense_attention(c.q_values()[0], c.kv.k, c.kv.v, c.kv.block_table[0], L, c.scale, c.Hkv,
                                     kv_dtype=c.dtype)
    assert_close(out.cpu().numpy()[0], ref_o, OUT_TOL, "16K out")
    assert_close(lse.cpu().numpy()[0], ref_l, LSE_TOL, "16K lse")
    lo, hi = O.candidate_range(L, 1, c.n_sink, c.n_recent)
    scn, seln = sc.cpu().numpy(), sel.cpu().numpy()
    for g in (0, 5):
        assert np.array_equal(seln[0, g], O.select_topk(scn[0, g], lo, hi, c.k_sel)), f"selection g={g}"


def test_deferred_pair_after_other_calls_on_one_workspace(gpu_lib):
    """A ticket-merged slow step on the same workspace before the deferred calls changes nothing."""
    sfi = gpu_lib
    c = make_case(616, name="shared", B=2, Hq=16, Hkv=8, d=128, dtype="bf16", seq_lens=[4096, 3001], n_sink=4,
                  n_recent=64, k_sel=256)
    dc = DevCase(c)
    ref = _separate(sfi, dc, 4, 64, 256)
    ws = torch.zeros(sfi.workspace_size("dense", k_pool=dc.k, block_table=dc.bt, Hq=16, dtype=torch.bfloat16,
                                        max_seq_len=dc.max_seq_len), dtype=torch.uint8, device=DEV)
    for _ in range(2):
        sfi.dense_attn_with_stats(dc.q, dc.k, dc.v, dc.bt, dc.lens, max_seq_len=dc.max_seq_len, n_sink=4,
                                  n_recent=64, workspace=ws)
        got = _pair(sfi, dc, 4, 64, 256, workspace=ws)
        torch.cuda.synchronize()
        for name, x, y in zip(NAMES, got, ref):
            assert np.array_equal(_bits(x), _bits(y)), name


def _three_launch(sfi, dc, q1, n_sink, n_recent, k):
    """Deferred slow step, Selector, then one launch with the fast step over the index set, the pack and
    the slow step's combine."""
    out, lse, sc, ws = sfi.dense_attn_with_stats_deferred(dc.q, dc.k, dc.v, dc.bt, dc.lens,
                                                          max_seq_len=dc.max_seq_len, n_sink=n_sink,
                                                          n_recent=n_recent)
    sel = sfi.select_topk(sc, dc.lens, k=k, n_sink=n_sink, n_recent=n_recent)
    ck, cv = _zero_compact(dc, n_sink + k)
    nc = torch.empty((dc.q.shape[0],), dtype=torch.int32, device=DEV)
    fo, fl = sfi.sparse_decode_indexed_attn_merge(q1, dc.k, dc.v, dc.bt, dc.lens, sel, n_sink=n_sink,
                                                  n_recent=n_recent, max_seq_len=dc.max_seq_len, slow_out=out,
                                                  slow_lse=lse, slow_workspace=ws, compact_k=ck, compact_v=cv,
                                                  n_compact=nc)
    return out, lse, sc, sel, ck, cv, nc, fo, fl


@pytest.mark.parametrize("name,mk,k", [
    ("tiny_fp32_d64_g4", lambda: tiny_case(3), 64),
    ("ragged_bf16_g4", lambda: make_case(621, name="ragged", B=3, Hq=16, Hkv=4, d=128, dtype="bf16",
                                         seq_lens=[5000, 333, 9000], n_sink=4, n_recent=64, k_sel=300,
                                         hh_per_head=10), 300),
    ("g8_bf16", lambda: make_case(623, name="g8", B=2, Hq=64, Hkv=8, d=128, dtype="bf16", seq_lens=[6000, 2500],
                                  n_sink=4, n_recent=64, k_sel=512, hh_per_head=20), 512),
    ("one_split_fp32", lambda: make_case(624, name="one_split", B=32, Hq=16, Hkv=8, d=64, dtype="f32",
                                         seq_lens=[300 + 7 * i for i in range(32)], n_sink=4, n_recent=32,
                                         k_sel=100), 100),
    ("no_sink_g1", lambda: make_case(625, name="no_sink", B=2, Hq=4, Hkv=4, d=64, dtype="bf16",
                                     seq_lens=[3000, 90], n_sink=0, n_recent=64, k_sel=200), 200),
    ("layer_16k", lambda: qwen06b_decode_case(1000, L=16384, B=1, frac=(1, 8)), None),
    ("batch16_g4", lambda: make_case(627, name="b16", B=16, Hq=32, Hkv=8, d=128, dtype="bf16",
                                     seq_lens=[2000 + 131 * i for i in range(16)], n_sink=4, n_recent=256,
                                     k_sel=384, hh_per_head=16), None),
])
def test_three_launch_step_equals_separate_calls(gpu_lib, name, mk, k):
    """Slow step + Selector + one launch (index-set fast step, pack, combine) against the plain slow step,
    Selector, pack and fast step over the compact buffer: all nine outputs bit for bit."""
    sfi = gpu_lib
    c = mk()
    k = c.k_sel if k is None else k
    dc = DevCase(c)
    q1 = dev_array(np.ascontiguousarray(c.q[:, -1]))
    ref = list(_separate(sfi, dc, c.n_sink, c.n_recent, k))
    ref += list(sfi.sparse_decode_attn(q1, dc.k, dc.v, dc.bt, dc.lens, ref[4], ref[5], ref[6], n_sink=c.n_sink,
                                       n_recent=c.n_recent, max_seq_len=dc.max_seq_len))
    got = _three_launch(sfi, dc, q1, c.n_sink, c.n_recent, k)
    torch.cuda.synchronize()
    for nm, x, y in zip(NAMES, got, ref):
        assert np.array_equal(_bits(x), _bits(y)), f"{name}: {nm} differs from the separate calls"
    # The fast step over the index set walks all k entries of a selection row (padding as masked rows),
    # the one over the compact buffer only the filled ones: with padding their split boundaries fall on
    # other tokens, so the sums round in another order.  Bit for bit when every row is full.
    full = bool((ref[3].cpu().numpy() >= 0).all())
    for nm, x, y in zip(("fast_out", "fast_lse"), got[7:], ref[7:]):
        if full:
            assert np.array_equal(_bits(x), _bits(y)), f"{name}: {nm} differs from the separate calls"
        else:
            assert_close(x.cpu().numpy(), y.cpu().numpy(), 1e-5, f"{name}: {nm}")


def test_three_launch_step_rejects_shared_workspaces(gpu_lib):
    sfi = gpu_lib
    c = make_case(626, name="ws", B=1, Hq=16, Hkv=8, d=128, dtype="bf16", seq_lens=[4096], n_sink=4, n_recent=64,
                  k_sel=256)
    dc = DevCase(c)
    out, lse, sc, ws = sfi.dense_attn_with_stats_deferred(dc.q, dc.k, dc.v, dc.bt, dc.lens,
                                                          max_seq_len=dc.max_seq_len, n_sink=4, n_recent=64)
    sel = sfi.select_topk(sc, dc.lens, k=256, n_sink=4, n_recent=64)
    ck, cv = _zero_compact(dc, 260)
    nc = torch.empty((1,), dtype=torch.int32, device=DEV)
    with pytest.raises(sfi.SfiError, match="overlap"):
        sfi.sparse_decode_indexed_attn_merge(dev_array(np.ascontiguousarray(c.q[:, -1])), dc.k, dc.v, dc.bt, dc.lens,
                                             sel, n_sink=4, n_recent=64, max_seq_len=dc.max_seq_len, slow_out=out,
                                             slow_lse=lse, slow_workspace=ws, compact_k=ck, compact_v=cv,
                                             n_compact=nc, workspace=ws)


def test_pack_in_blocks_or_in_attention_work_groups_agree(gpu_lib, monkeypatch):
    """The fused launch packs in work-groups of its own (few packed rows) or in the attention's work-groups
    (many); both forms give all outputs bit for bit, with and without the deferred combine.
    SFI_TUNE_PACK_IN_ATTN_BYTES forces each form."""
    sfi = gpu_lib
    c = make_case(628, name="modes", B=4, Hq=16, Hkv=8, d=128, dtype="bf16", seq_lens=[3000, 5000, 700, 4100],
                  n_sink=4, n_recent=64, k_sel=256, hh_per_head=12)
    dc = DevCase(c)
    q1 = dev_array(np.ascontiguousarray(c.q[:, -1]))
    got = {}
    for thr in ("1", str(1 << 60)):
        monkeypatch.setenv("SFI_TUNE_PACK_IN_ATTN_BYTES", thr)
        three = _three_launch(sfi, dc, q1, c.n_sink, c.n_recent, 256)
        sel = three[3]
        ck, cv = _zero_compact(dc, c.n_sink + 256)
        nc = torch.empty((c.B,), dtype=torch.int32, device=DEV)
        fo, fl = sfi.sparse_decode_indexed_attn(q1, dc.k, dc.v, dc.bt, dc.lens, sel, n_sink=c.n_sink,
                                                n_recent=c.n_recent, max_seq_len=dc.max_seq_len, compact_k=ck,
                                                compact_v=cv, n_compact=nc)
        torch.cuda.synchronize()
        got[thr] = list(three) + [ck, cv, nc, fo, fl]
    names = list(NAMES) + ["fast_out", "fast_lse", "ck2", "cv2", "nc2", "fo2", "fl2"]
    for nm, x, y in zip(names, got["1"], got[str(1 << 60)]):
        assert np.array_equal(_bits(x), _bits(y)), f"{nm} differs between the two pack forms"
