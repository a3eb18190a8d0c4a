"""GPU parity of the fast step over an index set read in place
(sfi_sparse_decode_indexed_attn) and of the draft-step driver with an intra-draft
refresh layer (sparse_kv_cache_sfi_amd.schedule.DraftRefresh).

The indexed fast step is checked against the oracle's indexed_decode (out 2e-3,
lse 1e-3) on ragged batches with padded selections, entries past the request's end,
invalid pages, an empty selection and an appended token, and bit for bit against
sfi_pack_compact + sfi_sparse_decode_attn when every entry is valid.  The driver is
checked step by step against the oracle's draft_refresh_loop, selecting from the
logits the GPU produced (themselves within the fp32 bound of the oracle's), so every
selection must match exactly.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle as O
from sfi_synth import bf16_bits, bf16_values, drifting_case, make_case
from _gpu import DEV, LSE_TOL, OUT_TOL, DevCase, assert_close, dev_array, host_bits, score_bound

pytestmark = pytest.mark.gpu


def _selection(rng, c, L, k, pad=0):
    """k_eff = min(k - pad, candidates) sorted candidates per KV head, then -1 padding."""
    lo, hi = O.candidate_range(L, 1, c.n_sink, c.n_recent)
    k_eff = max(0, min(k - pad, hi - lo))
    sel = np.full((c.Hkv, k), -1, np.int32)
    for g in range(c.Hkv):
        if k_eff:
            sel[g, :k_eff] = np.sort(rng.choice(np.arange(lo, hi), k_eff, replace=False))
    return sel


def _indexed(sfi, c, dc, sels, L, bt_d=None, **kw):
    out, lse = sfi.sparse_decode_indexed_attn(dc.q[:, 0].contiguous(), dc.k, dc.v, dc.bt if bt_d is None else bt_d,
                                              dc.lens_tensor(L), dev_array(np.stack(sels).astype(np.int32)),
                                              n_sink=c.n_sink, n_recent=c.n_recent, max_seq_len=dc.max_seq_len,
                                              scale=c.scale, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _check_vs_oracle(c, out, lse, sels, L, bt=None, pools=None):
    bt = c.kv.block_table if bt is None else bt
    kp, vp = (c.kv.k, c.kv.v) if pools is None else pools
    qv = c.q_values()[:, 0]
    for b in range(c.B):
        if L[b] == 0:
            assert np.all(out[b] == 0) and np.all(np.isneginf(lse[b])), b
            continue
        ro, rl = O.indexed_decode(qv[b], kp, vp, bt[b], int(L[b]), c.n_sink, c.n_recent, sels[b], c.scale,
                                  kv_dtype=c.dtype)
        assert_close(out[b], ro, OUT_TOL, f"out b={b}")
        assert_close(lse[b], rl, LSE_TOL, f"lse b={b}")


CASES = [
    ("bf16_g2_ragged_padded", lambda: make_case(301, name="ix_a", B=3, Hq=16, Hkv=8, d=128, dtype="bf16",
                                                 seq_lens=[300, 5000, 2047], n_sink=4, n_recent=64, k_sel=600),
     600, 37),
    ("f32_g2_d128", lambda: make_case(302, name="ix_b", B=2, Hq=4, Hkv=2, d=128, dtype="f32", seq_lens=[900, 1200],
                                       n_sink=4, n_recent=32, k_sel=200), 200, 0),
    ("bf16_g8_d64", lambda: make_case(303, name="ix_c", B=1, Hq=8, Hkv=1, d=64, dtype="bf16", seq_lens=[2000],
                                       n_sink=4, n_recent=48, k_sel=333), 333, 5),
    ("bf16_g4_16k_2pct", lambda: make_case(304, name="ix_d", B=2, Hq=32, Hkv=8, d=128, dtype="bf16",
                                            seq_lens=[16384, 9000], n_sink=4, n_recent=64, k_sel=256), 256, 0),
    ("bf16_b16_large_grid", lambda: make_case(305, name="ix_e", B=16, Hq=16, Hkv=8, d=128, dtype="bf16",
                                               seq_lens=list(range(1500, 3100, 100)), n_sink=4, n_recent=64,
                                               k_sel=700), 700, 0),
    # compact splits of 576 rows: the compact fast step starts them at rotated iterations, so the two
    # variants are compared with the oracle only
    ("bf16_b16_long_splits", lambda: make_case(307, name="ix_g", B=16, Hq=16, Hkv=8, d=128, dtype="bf16",
                                                seq_lens=list(range(1500, 3100, 100)), n_sink=4, n_recent=64,
                                                k_sel=1024), 1024, 0),
]


@pytest.mark.parametrize("name,mk,k,pad", CASES, ids=[n[0] for n in CASES])
def test_indexed_fast_step_matches_oracle(gpu_lib, name, mk, k, pad):
    c = mk()
    dc = DevCase(c)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    L = c.seq_lens.astype(np.int32)
    sels = [_selection(rng, c, int(L[b]), k, pad) for b in range(c.B)]
    out, lse = _indexed(gpu_lib, c, dc, sels, L)
    _check_vs_oracle(c, out, lse, sels, L)
    st, ns = gpu_lib.plan_splits(1, B=c.B, Hq=c.Hq, Hkv=c.Hkv, d=c.d, bf16=c.dtype == "bf16",
                                 max_pages=c.kv.max_pages, num_pages=c.kv.num_pages, max_seq_len=dc.max_seq_len,
                                 cap=c.n_sink + k, n_recent=c.n_recent)
    if pad == 0 and all(int(L[b]) - c.n_sink - c.n_recent >= k for b in range(c.B)) and st < 8 * 64:
        # every entry valid and no compact split long enough for a rotated start (8 iterations of 64
        # rows): bit-identical to packing the same rows and the compact fast step
        sel_d = dev_array(np.stack(sels).astype(np.int32))
        ck, cv, nc = gpu_lib.pack_compact(dc.k, dc.v, dc.bt, dc.lens, sel_d, n_sink=c.n_sink, cap=c.n_sink + k,
                                          max_seq_len=dc.max_seq_len)
        o2, l2 = gpu_lib.sparse_decode_attn(dc.q[:, 0].contiguous(), dc.k, dc.v, dc.bt, dc.lens, ck, cv, nc,
                                            n_sink=c.n_sink, n_recent=c.n_recent, max_seq_len=dc.max_seq_len,
                                            scale=c.scale)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(o2.cpu().numpy(), out)
        np.testing.assert_array_equal(l2.cpu().numpy(), lse)


def test_indexed_entries_past_the_end_invalid_pages_and_empty_selection(gpu_lib):
    c = make_case(306, name="ix_f", B=3, Hq=8, Hkv=2, d=128, dtype="bf16", seq_lens=[700, 1300, 3],
                  capacity=[800, 1300, 16], n_sink=4, n_recent=32, k_sel=64)
    dc = DevCase(c)
    bt = c.kv.block_table.copy()
    bt[0, 20] = -1                                  # positions 320..335 of request 0
    bt[1, 5] = c.kv.num_pages + 9                   # positions 80..95 of request 1
    rng = np.random.default_rng(7)
    sels = [_selection(rng, c, int(c.seq_lens[b]), 64) for b in range(3)]
    sels[0][0, 3] = 750                             # past L (700)
    sels[0][1, 10] = -1                             # padding in the middle
    sels[0][1, 11] = 325                            # on the invalid page
    sels[1][0, :] = -1                              # empty selection: sink + recent only
    L = c.seq_lens.astype(np.int32)
    out, lse = _indexed(gpu_lib, c, dc, sels, L, bt_d=dev_array(bt))
    _check_vs_oracle(c, out, lse, sels, L, bt=bt)


def test_indexed_with_zero_k_is_sink_plus_recent(gpu_lib):
    c = make_case(307, name="ix_g", B=2, Hq=8, Hkv=2, d=128, dtype="bf16", seq_lens=[900, 40], n_sink=4,
                  n_recent=32, k_sel=8)
    dc = DevCase(c)
    sels = [np.zeros((2, 0), np.int32)] * 2
    L = c.seq_lens.astype(np.int32)
    out, lse = _indexed(gpu_lib, c, dc, sels, L)
    _check_vs_oracle(c, out, lse, sels, L)


def test_indexed_recent_window_alone(gpu_lib):
    # no sink and no selection (cap 0): the fast step attends the recent window only
    c = make_case(308, name="ix_h", B=2, Hq=8, Hkv=2, d=128, dtype="bf16", seq_lens=[900, 20], n_sink=0,
                  n_recent=32, k_sel=8)
    dc = DevCase(c)
    sels = [np.zeros((2, 0), np.int32)] * 2
    L = c.seq_lens.astype(np.int32)
    out, lse = _indexed(gpu_lib, c, dc, sels, L)
    _check_vs_oracle(c, out, lse, sels, L)


def test_indexed_with_append_stores_and_attends_the_new_token(gpu_lib):
    c = make_case(308, name="ix_h", B=2, Hq=16, Hkv=8, d=128, dtype="bf16", seq_lens=[1000, 2500],
                  capacity=[1010, 2510], n_sink=4, n_recent=64, k_sel=128)
    dc = DevCase(c)
    rng = np.random.default_rng(8)
    sels = [_selection(rng, c, int(c.seq_lens[b]), 128) for b in range(2)]
    x = rng.standard_normal((2, 2, 8, 128)).astype(np.float32)
    kn, vn = bf16_bits(x[0]), bf16_bits(x[1])
    L = (c.seq_lens + 1).astype(np.int32)
    out, lse = _indexed(gpu_lib, c, dc, sels, L, k_new=dev_array(kn), v_new=dev_array(vn))
    kp, vp = c.kv.k, c.kv.v
    for b in range(2):
        kp, vp = O.append_token(kp, vp, c.kv.block_table[b], int(L[b]), kn[b], vn[b])
    np.testing.assert_array_equal(host_bits(dc.k), kp)
    np.testing.assert_array_equal(host_bits(dc.v), vp)
    _check_vs_oracle(c, out, lse, sels, L, pools=(kp, vp))


# --------------------------------------------------------------------------- draft steps with a refresh layer

@pytest.mark.parametrize("refresh_layer", [0, 2])
def test_draft_refresh_driver_matches_the_oracle_loop(gpu_lib, refresh_layer):
    from sparse_kv_cache_sfi_amd.schedule import DraftRefresh
    steps, k, n_layers = 12, 48, 4
    dc0 = drifting_case(71, B=2, Hq=8, Hkv=2, d=128, dtype="bf16", L0=[1500, 2600], steps=steps, period=4, hh=16,
                        n_sink=4, n_recent=32, k_sel=k)
    c = dc0.case
    rng = np.random.default_rng(72)
    # every layer shares the block table; layer 0 is the drifting case's own pool
    pools_h = [(c.kv.k, c.kv.v)] + [(bf16_bits(rng.standard_normal(c.kv.k.shape).astype(np.float32)),
                                     bf16_bits(rng.standard_normal(c.kv.v.shape).astype(np.float32)))
                                    for _ in range(n_layers - 1)]
    pools = [(dev_array(kp), dev_array(vp)) for kp, vp in pools_h]
    bt = dev_array(c.kv.block_table)
    max_len = c.kv.max_pages * 16
    qs = dc0.q_step_values()                                   # [steps, B, Hq, d], the refresh layer's queries
    other = rng.standard_normal((steps, n_layers, c.B, c.Hq, c.d)).astype(np.float32)
    q_bits = bf16_bits(other)
    q_bits[:, refresh_layer] = dc0.q_steps                     # stored bits of the drifting queries
    q_vals = bf16_values(q_bits)                               # [steps, n_layers, B, Hq, d]
    q = torch.empty((n_layers, c.B, c.Hq, c.d), dtype=torch.bfloat16, device=DEV)
    lens = torch.empty((c.B,), dtype=torch.int32, device=DEV)
    L0 = c.seq_lens.astype(np.int64)
    sel0 = np.stack([_selection(np.random.default_rng(b), c, int(L0[b]), k) for b in range(c.B)])
    drv = DraftRefresh(pools, bt, q, lens, max_seq_len=max_len, n_sink=4, n_recent=32, k=k,
                       refresh_layer=refresh_layer, sel0=dev_array(sel0))
    outs, lses, sels, scores = [], [], [], []
    for t in range(steps):
        q.copy_(dev_array(q_bits[t]))
        lens.copy_(torch.from_numpy((L0 + t + 1).astype(np.int32)))
        drv.step()
        torch.cuda.synchronize()
        outs.append(drv.out.cpu().numpy().copy())
        lses.append(drv.lse.cpu().numpy().copy())
        sels.append(drv.sel.cpu().numpy().copy())
        scores.append(drv.scores.cpu().numpy().copy())
    assert np.array_equal(q_vals[:, refresh_layer], qs)
    for b in range(c.B):
        res = O.draft_refresh_loop(q_vals[:, :, b], pools_h, c.kv.block_table[b], int(L0[b]), 4, 32, k,
                                   refresh_layer, sel0[b], c.scale, kv_dtype="bf16",
                                   scores_at=lambda t: scores[t][b].astype(np.float64))
        for t, (layer_res, sel) in enumerate(res):
            assert np.array_equal(sels[t][b], sel), (t, b)
            L = int(L0[b]) + t + 1
            lo, hi = O.candidate_range(L, 1, 4, 32)
            kp, _ = pools_h[refresh_layer]
            for g in range(c.Hkv):
                rows = O.paged_rows(bf16_values(kp), c.kv.block_table[b], g, np.arange(lo, hi))
                bound = score_bound(q_vals[t, refresh_layer, b, g * c.G:(g + 1) * c.G], rows, c.scale)
                assert_close(scores[t][b, g, lo:hi], O.group_scores(q_vals[t, refresh_layer, b][None], kp,
                                                                    c.kv.block_table[b], L, c.scale, c.Hkv, 4, 32,
                                                                    L, kv_dtype="bf16", groups=[g])[g, lo:hi],
                             bound, f"scores t={t} b={b} g={g}")
            for layer, (ro, rl) in enumerate(layer_res):
                assert_close(outs[t][layer, b], ro, OUT_TOL, f"out t={t} layer={layer} b={b}")
                assert_close(lses[t][layer, b], rl, LSE_TOL, f"lse t={t} layer={layer} b={b}")


# --------------------------------------------------------------------------- packing while attending

def _sentinel_like(shape, dtype):
    t = torch.empty(shape, dtype=dtype, device=DEV)
    t.view(torch.int16 if dtype == torch.bfloat16 else torch.int32).fill_(0x3f3f)
    return t


PACK_CASES = [
    ("bf16_g2_ragged_padded", lambda: make_case(311, name="pk_a", B=3, Hq=16, Hkv=8, d=128, dtype="bf16",
                                                 seq_lens=[300, 5000, 2047], n_sink=4, n_recent=64, k_sel=600),
     600, 37, False),
    ("f32_g2", lambda: make_case(312, name="pk_b", B=2, Hq=4, Hkv=2, d=128, dtype="f32", seq_lens=[900, 1200],
                                  n_sink=4, n_recent=32, k_sel=200), 200, 0, False),
    ("bf16_g4_per_head", lambda: make_case(313, name="pk_c", B=2, Hq=16, Hkv=4, d=128, dtype="bf16",
                                            seq_lens=[2500, 900], n_sink=4, n_recent=64, k_sel=128), 128, 0, True),
]


@pytest.mark.parametrize("name,mk,k,pad,per_head", PACK_CASES, ids=[n[0] for n in PACK_CASES])
def test_indexed_fast_step_packs_exactly_like_pack_compact(gpu_lib, name, mk, k, pad, per_head):
    c = mk()
    dc = DevCase(c)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    units = c.Hq if per_head else c.Hkv
    L = c.seq_lens.astype(np.int32)
    sels = []
    for b in range(c.B):
        s_ = np.concatenate([_selection(rng, c, int(L[b]), k, pad) for _ in range(units // c.Hkv)])
        sels.append(s_)
    sel = np.stack(sels).astype(np.int32)
    if not per_head:
        sel[0, 0, 5] = int(L[0]) + 3            # past the end: a zero row
        sel[min(1, c.B - 1), 1, 7] = -1         # padding in the middle: no row
    sel_d = dev_array(sel)
    cap = c.n_sink + k + 2
    kdt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
    kw = dict(n_sink=c.n_sink, n_recent=c.n_recent, max_seq_len=dc.max_seq_len, scale=c.scale, per_head=per_head)
    q1 = dc.q[:, 0].contiguous()
    ck1, cv1 = _sentinel_like((c.B, units, cap, c.d), kdt), _sentinel_like((c.B, units, cap, c.d), kdt)
    nc1 = torch.full((c.B,), -5, dtype=torch.int32, device=DEV)
    o1, l1 = gpu_lib.sparse_decode_indexed_attn(q1, dc.k, dc.v, dc.bt, dc.lens, sel_d, compact_k=ck1,
                                                compact_v=cv1, n_compact=nc1, **kw)
    o0, l0 = gpu_lib.sparse_decode_indexed_attn(q1, dc.k, dc.v, dc.bt, dc.lens, sel_d, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o0) and torch.equal(l1, l0)
    ibits = torch.int16 if kdt == torch.bfloat16 else torch.int32
    if per_head:
        # the gather-pack has no per-query-head form: the reference packs each query head's set from its
        # KV head's rows on the host (pools with every KV head repeated for its G query heads)
        kr, vr = np.repeat(c.kv.k, c.G, axis=1), np.repeat(c.kv.v, c.G, axis=1)
        got_k, got_v, got_n = host_bits(ck1), host_bits(cv1), nc1.cpu().numpy()
        for b in range(c.B):
            rck, rcv, rnc = O.pack_compact(kr, vr, c.kv.block_table[b], int(L[b]), c.n_sink, sel[b], cap)
            assert got_n[b] == rnc, b
            assert np.array_equal(got_k[b, :, :rnc], rck[:, :rnc]) and np.array_equal(got_v[b, :, :rnc], rcv[:, :rnc])
        return
    ck2, cv2 = _sentinel_like((c.B, units, cap, c.d), kdt), _sentinel_like((c.B, units, cap, c.d), kdt)
    nc2 = torch.full((c.B,), -5, dtype=torch.int32, device=DEV)
    gpu_lib.pack_compact(dc.k, dc.v, dc.bt, dc.lens, sel_d, n_sink=c.n_sink, cap=cap, max_seq_len=dc.max_seq_len,
                         compact_k=ck2, compact_v=cv2, n_compact=nc2)
    torch.cuda.synchronize()
    assert torch.equal(nc1, nc2)
    assert torch.equal(ck1.view(ibits), ck2.view(ibits))
    assert torch.equal(cv1.view(ibits), cv2.view(ibits))
    # and the packed buffer serves the compact fast step like any other
    if pad == 0:
        o2, l2 = gpu_lib.sparse_decode_attn(q1, dc.k, dc.v, dc.bt, dc.lens, ck1, cv1, nc1, n_sink=c.n_sink,
                                            n_recent=c.n_recent, max_seq_len=dc.max_seq_len, scale=c.scale)
        torch.cuda.synchronize()
        qv = c.q_values()[:, 0]
        for b in range(c.B):
            rck, rcv, rnc = O.pack_compact(c.kv.k, c.kv.v, c.kv.block_table[b], int(L[b]), c.n_sink, sel[b], cap)
            ro, rl = O.sparse_decode(qv[b], rck, rcv, rnc, c.kv.k, c.kv.v, c.kv.block_table[b], int(L[b]),
                                     c.n_sink, c.n_recent, c.scale, kv_dtype=c.dtype)
            assert_close(o2.cpu().numpy()[b], ro, OUT_TOL, f"compact after fused pack b={b}")


def test_indexed_pack_with_invalid_pages_and_append(gpu_lib):
    c = make_case(314, name="pk_d", B=2, Hq=8, Hkv=2, d=128, dtype="bf16", seq_lens=[700, 1300],
                  capacity=[710, 1310], n_sink=4, n_recent=32, k_sel=64)
    dc = DevCase(c)
    bt = c.kv.block_table.copy()
    bt[0, 20] = -1
    bt[1, 5] = c.kv.num_pages + 9
    bt_d = dev_array(bt)
    rng = np.random.default_rng(15)
    sel = np.stack([_selection(rng, c, int(c.seq_lens[b]), 64) for b in range(2)]).astype(np.int32)
    sel[0, 1, 3] = 325                              # on the invalid page: a zero row
    sel_d = dev_array(sel)
    L = (c.seq_lens + 1).astype(np.int32)
    lens = dc.lens_tensor(L)
    x = rng.standard_normal((2, 2, 2, 128)).astype(np.float32)
    kn, vn = dev_array(bf16_bits(x[0])), dev_array(bf16_bits(x[1]))
    ck1, cv1 = _sentinel_like((2, 2, 68, 128), torch.bfloat16), _sentinel_like((2, 2, 68, 128), torch.bfloat16)
    nc1 = torch.zeros((2,), dtype=torch.int32, device=DEV)
    kw = dict(n_sink=4, n_recent=32, max_seq_len=dc.max_seq_len, scale=c.scale)
    o1, l1 = gpu_lib.sparse_decode_indexed_attn(dc.q[:, 0].contiguous(), dc.k, dc.v, bt_d, lens, sel_d, k_new=kn,
                                                v_new=vn, compact_k=ck1, compact_v=cv1, n_compact=nc1, **kw)
    ck2, cv2 = _sentinel_like((2, 2, 68, 128), torch.bfloat16), _sentinel_like((2, 2, 68, 128), torch.bfloat16)
    nc2 = torch.zeros((2,), dtype=torch.int32, device=DEV)
    gpu_lib.pack_compact(dc.k, dc.v, bt_d, lens, sel_d, n_sink=4, cap=68, max_seq_len=dc.max_seq_len,
                         compact_k=ck2, compact_v=cv2, n_compact=nc2)
    torch.cuda.synchronize()
    assert torch.equal(nc1, nc2)
    assert torch.equal(ck1.view(torch.int16), ck2.view(torch.int16))
    assert torch.equal(cv1.view(torch.int16), cv2.view(torch.int16))


def test_binding_rejects_selections_and_buffers_that_disagree_with_the_pools(gpu_lib):
    """Sizes the library takes from its descriptors must agree with the pools; the binding refuses a
    mismatch before anything is launched (a per-query-head selection is not a gather-pack input)."""
    c = make_case(315, name="pk_e", B=2, Hq=16, Hkv=4, d=128, dtype="bf16", seq_lens=[600, 900], n_sink=4,
                  n_recent=32, k_sel=16)
    dc = DevCase(c)
    per_head_sel = torch.zeros((2, 16, 16), dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="KV heads"):
        gpu_lib.pack_compact(dc.k, dc.v, dc.bt, dc.lens, per_head_sel, n_sink=4, cap=20, max_seq_len=dc.max_seq_len)
    wrong = torch.zeros((2, 16, 20, 128), dtype=torch.bfloat16, device=DEV)
    nc = torch.zeros((2,), dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="KV heads"):
        gpu_lib.sparse_decode_attn(dc.q[:, 0].contiguous(), dc.k, dc.v, dc.bt, dc.lens, wrong, wrong, nc, n_sink=4,
                                   n_recent=32, max_seq_len=dc.max_seq_len)
    with pytest.raises(ValueError, match="block_table"):
        gpu_lib.dense_attn_with_stats(dc.q[:1], dc.k, dc.v, dc.bt, dc.lens[:1], max_seq_len=dc.max_seq_len)
