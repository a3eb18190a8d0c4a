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
    if pad == 0 and all(int(L[b]) - c.n_sink - c.n_recent >= k for b in range(c.B)):
        # every entry valid: bit-identical to packing the same rows and the compact fast step
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
