"""GPU parity of the fast step with KV append (sfi_sparse_decode_append_attn).

The launch stores the decoded token's K/V at position seq_lens[b] - 1 of each
request's pages and attends over sink + selected + recent with that row read from
the arguments.  Checked against the oracle's append_token followed by its fast step:
outputs within tolerance, the pools bit-exact after the launch (one row per (b, g)
written, nothing else touched), and outputs bit-identical to a store followed by the
plain fast step.  Edge cases: an empty recent window (stored, not attended), an
invalid page at the new position (neither), an empty request, a new token opening a
page.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle as O
from sfi_synth import bf16_bits, bf16_values, make_case
from _gpu import DEV, LSE_TOL, OUT_TOL, DevCase, assert_close, dev_array, host_bits

pytestmark = pytest.mark.gpu


def _new_kv(seed, c):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((2, c.B, c.Hkv, c.d)).astype(np.float32)
    if c.dtype == "bf16":
        st = bf16_bits(x)
        return st[0], st[1], bf16_values(st[0]), bf16_values(st[1])
    return x[0], x[1], x[0].astype(np.float64), x[1].astype(np.float64)


def _selection(rng, c, L, k):
    lo, hi = O.candidate_range(L, 1, c.n_sink, c.n_recent)
    k_eff = max(0, min(k, hi - lo))
    sel = np.full((c.Hkv, k), -1, np.int32)
    for g in range(c.Hkv):
        if k_eff:
            sel[g, :k_eff] = np.sort(rng.choice(np.arange(lo, hi), k_eff, replace=False))
    return sel


def _run(sfi, c, k, L_new, bt=None, n_recent=None, seed=0):
    """Pack at the case's lengths, then one fused append + fast step at lengths L_new.
    Returns (device outputs, pools after, oracle pools after, oracle outputs)."""
    n_recent = c.n_recent if n_recent is None else n_recent
    bt = c.kv.block_table if bt is None else bt     # oracle outputs only for the case's own table
    dc = DevCase(c)
    bt_d = dev_array(bt.astype(np.int32))
    rng = np.random.default_rng(zlib.crc32(f"{c.name}/{seed}".encode()))
    sels = np.stack([_selection(rng, c, int(c.seq_lens[b]), k) for b in range(c.B)]).astype(np.int32)
    cap = c.n_sink + k
    ck, cv, nc = sfi.pack_compact(dc.k, dc.v, bt_d, dc.lens, dev_array(sels), n_sink=c.n_sink, cap=cap,
                                  max_seq_len=dc.max_seq_len)
    kn, vn, kn_val, vn_val = _new_kv(seed + 7, c)
    lens = dc.lens_tensor(L_new)
    out, lse = sfi.sparse_decode_attn(dc.q[:, 0].contiguous(), dc.k, dc.v, bt_d, lens, ck, cv, nc, n_sink=c.n_sink,
                                      n_recent=n_recent, max_seq_len=dc.max_seq_len, scale=c.scale,
                                      k_new=dev_array(kn), v_new=dev_array(vn))
    torch.cuda.synchronize()
    got = (out.cpu().numpy(), lse.cpu().numpy(), host_bits(dc.k), host_bits(dc.v))
    ref_k, ref_v = c.kv.k, c.kv.v
    refs = []
    qv = c.q_values()[:, 0]
    for b in range(c.B):
        ref_k, ref_v = O.append_token(ref_k, ref_v, bt[b], int(L_new[b]), kn[b], vn[b])
    for b in range(c.B if bt is c.kv.block_table else 0):
        if L_new[b] == 0:              # empty state: zero output, lse = -inf
            refs.append(None)
            continue
        rck, rcv, rnc = O.pack_compact(c.kv.k, c.kv.v, bt[b], int(c.seq_lens[b]), c.n_sink, sels[b], cap)
        refs.append(O.sparse_decode(qv[b], rck, rcv, rnc, ref_k, ref_v, bt[b], int(L_new[b]), c.n_sink, n_recent,
                                    c.scale, kv_dtype=c.dtype))
    # the same fast step after a separate store: bit-identical outputs
    out2, lse2 = sfi.sparse_decode_attn(dc.q[:, 0].contiguous(), dc.k, dc.v, bt_d, lens, ck, cv, nc,
                                        n_sink=c.n_sink, n_recent=n_recent, max_seq_len=dc.max_seq_len,
                                        scale=c.scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out2.cpu().numpy(), got[0])
    np.testing.assert_array_equal(lse2.cpu().numpy(), got[1])
    return got, (ref_k, ref_v), refs, (kn_val, vn_val)


def _check(got, ref_pools, refs):
    out, lse, k_after, v_after = got
    np.testing.assert_array_equal(k_after, ref_pools[0])
    np.testing.assert_array_equal(v_after, ref_pools[1])
    for b, ref in enumerate(refs):
        if ref is None:
            assert np.all(out[b] == 0) and np.all(np.isneginf(lse[b])), b
            continue
        ro, rl = ref
        assert_close(out[b], ro, OUT_TOL, f"out b={b}")
        assert_close(lse[b], rl, LSE_TOL, f"lse b={b}")


CASES = [
    ("bf16_g2_ragged", lambda: make_case(201, name="ap_a", B=3, Hq=16, Hkv=8, d=128, dtype="bf16",
                                          seq_lens=[300, 4000, 2047], capacity=[310, 4010, 2060], n_sink=4,
                                          n_recent=64, k_sel=512), 512),
    ("f32_g2_d128", lambda: make_case(202, name="ap_b", B=2, Hq=4, Hkv=2, d=128, dtype="f32",
                                       seq_lens=[900, 1200], capacity=[905, 1205], n_sink=4, n_recent=32,
                                       k_sel=200), 200),
    ("bf16_g8_d64", lambda: make_case(203, name="ap_c", B=1, Hq=8, Hkv=1, d=64, dtype="bf16",
                                       seq_lens=[2000], capacity=[2003], n_sink=4, n_recent=48, k_sel=333), 333),
    ("bf16_b16_large_grid", lambda: make_case(204, name="ap_d", B=16, Hq=16, Hkv=8, d=128, dtype="bf16",
                                               seq_lens=list(range(1500, 3100, 100)),
                                               capacity=list(range(1504, 3104, 100)), n_sink=4, n_recent=64,
                                               k_sel=1024), 1024),
]


@pytest.mark.parametrize("name,mk,k", CASES, ids=[n for n, _, _ in CASES])
def test_fused_append_matches_store_then_fast_step(gpu_lib, name, mk, k):
    c = mk()
    L_new = (c.seq_lens + 1).astype(np.int32)
    got, ref_pools, refs, _ = _run(gpu_lib, c, k, L_new)
    _check(got, ref_pools, refs)


def test_append_opening_a_page_and_an_empty_request(gpu_lib):
    # request 0: new token at position 320 (first row of page 20); request 1: empty
    c = make_case(205, name="ap_e", B=2, Hq=8, Hkv=2, d=128, dtype="bf16", seq_lens=[320, 0],
                  capacity=[336, 16], n_sink=4, n_recent=16, k_sel=32)
    L_new = np.array([321, 0], np.int32)
    got, ref_pools, refs, _ = _run(gpu_lib, c, 32, L_new)
    _check(got, ref_pools, refs)


def test_append_with_empty_recent_window_stores_without_attending(gpu_lib):
    c = make_case(206, name="ap_f", B=2, Hq=8, Hkv=2, d=128, dtype="bf16", seq_lens=[700, 1100],
                  capacity=[710, 1110], n_sink=4, n_recent=0, k_sel=64)
    L_new = (c.seq_lens + 1).astype(np.int32)
    got, ref_pools, refs, _ = _run(gpu_lib, c, 64, L_new, n_recent=0)
    _check(got, ref_pools, refs)
    assert not np.array_equal(got[2], c.kv.k)      # the row was stored


def test_append_behind_an_invalid_page_is_neither_stored_nor_attended(gpu_lib):
    c = make_case(207, name="ap_g", B=1, Hq=8, Hkv=2, d=128, dtype="bf16", seq_lens=[999], capacity=[1010],
                  n_sink=4, n_recent=32, k_sel=64)
    bt = c.kv.block_table.copy()
    bt[0, 999 // 16] = -1                          # the page of positions 992..1007
    got, ref_pools, _, _ = _run(gpu_lib, c, 64, np.array([1000], np.int32), bt=bt, seed=3)
    out, lse, k_after, v_after = got
    np.testing.assert_array_equal(k_after, c.kv.k)
    np.testing.assert_array_equal(v_after, c.kv.v)
    # reference: the compact rows, then the recent positions 968..991 (992..999 sit on the dropped page)
    rng = np.random.default_rng(zlib.crc32(f"{c.name}/3".encode()))
    sel = _selection(rng, c, 999, 64)
    ck, cv, n_c = O.pack_compact(c.kv.k, c.kv.v, bt[0], 999, 4, sel, 68)
    pos = np.arange(968, 992)
    qv = c.q_values()[0, 0]
    for g in range(2):
        K = np.concatenate([bf16_values(ck[g, :n_c]), O.paged_rows(c.kv.k_values(), bt[0], g, pos)])
        V = np.concatenate([bf16_values(cv[g, :n_c]), O.paged_rows(c.kv.v_values(), bt[0], g, pos)])
        ro, rl = O.softmax_attention(qv[4 * g:4 * g + 4], K, V, c.scale)
        assert_close(out[0, 4 * g:4 * g + 4], ro, OUT_TOL, f"out g={g}")
        assert_close(lse[0, 4 * g:4 * g + 4], rl, LSE_TOL, f"lse g={g}")


def test_dominant_appended_key_returns_its_value(gpu_lib):
    c = make_case(208, name="ap_h", B=1, Hq=4, Hkv=2, d=64, dtype="f32", seq_lens=[600], capacity=[610],
                  n_sink=4, n_recent=16, k_sel=16)
    dc = DevCase(c)
    q = c.q_values()[0, 0]
    kn = np.stack([40.0 * q[2 * g:2 * g + 2].mean(axis=0) for g in range(2)]).astype(np.float32)[None]
    vn = np.random.default_rng(9).standard_normal((1, 2, 64)).astype(np.float32)
    ck = torch.zeros((1, 2, 20, 64), dtype=torch.float32, device=DEV)
    nc = torch.zeros((1,), dtype=torch.int32, device=DEV)
    out, _ = gpu_lib.sparse_decode_attn(dc.q[:, 0].contiguous(), dc.k, dc.v, dc.bt, dc.lens_tensor([601]), ck,
                                        ck.clone(), nc, n_sink=4, n_recent=16, max_seq_len=dc.max_seq_len,
                                        scale=c.scale, k_new=dev_array(kn), v_new=dev_array(vn))
    torch.cuda.synchronize()
    o = out.cpu().numpy()[0]
    for h in range(4):
        assert_close(o[h], vn[0, h // 2].astype(np.float64), 1e-5, f"h={h}")
