"""GPU parity of the mixed draft / verify launch against the fp64 oracle.

Drafting requests (one query token, fast step over compact + recent) and
verifying requests (t_q draft tokens, dense causal attention with the summed
logits) share one launch.  Small cases are checked on every output; the 128K
speculative mix (4 drafting + 4 verifying requests, 32 query heads on 8 KV
heads) is checked at full size on sampled (request, KV head) units.
"""
import numpy as np
import pytest
import torch

import oracle as O
from sfi_synth import make_case, specmix128k_case
from _gpu import DEV, LSE_TOL, OUT_TOL, DevCase, assert_close, dev_array, score_bound

pytestmark = pytest.mark.gpu


def _selection(rng, c, k):
    sel = np.full((c.B, c.Hkv, k), -1, np.int32)
    for b in range(c.B):
        lo, hi = O.candidate_range(int(c.seq_lens[b]), 1, c.n_sink, c.n_recent)
        k_eff = min(k, hi - lo)
        for g in range(c.Hkv):
            sel[b, g, :k_eff] = np.sort(rng.choice(np.arange(lo, hi), k_eff, replace=False))
    return sel


def _run_mixed(sfi, c, dc, modes, k, seed, with_scores=True):
    """Pack a random selection for every request, build the packed query rows, launch."""
    rng = np.random.default_rng(seed)
    sel = _selection(rng, c, k)
    cap = c.n_sink + k
    ck, cv, nc = sfi.pack_compact(dc.k, dc.v, dc.bt, dc.lens, dev_array(sel), n_sink=c.n_sink, cap=cap,
                                  max_seq_len=dc.max_seq_len)
    t_q = [1 if m == 0 else c.t_q for m in modes]
    # drafting requests use their last query token (position L - 1), verifying ones all t_q tokens
    rows = [c.q[b, -1:] if modes[b] == 0 else c.q[b] for b in range(c.B)]
    q_packed = np.concatenate(rows, axis=0)
    out, lse, sc = sfi.mixed_attn(dev_array(q_packed), dc.k, dc.v, dc.bt, dc.lens, modes, t_q, ck, cv, nc,
                                  n_sink=c.n_sink, n_recent=c.n_recent, max_seq_len=dc.max_seq_len, scale=c.scale,
                                  with_scores=with_scores)
    torch.cuda.synchronize()
    return sel, cap, t_q, out.cpu().numpy(), lse.cpu().numpy(), (sc.cpu().numpy() if sc is not None else None)


def _check_request(c, b, mode, sel, cap, row0, t_q, out, lse, sc, groups=None):
    Qv = c.q_values()[b]
    L = int(c.seq_lens[b])
    gs = range(c.Hkv) if groups is None else groups
    G = c.G
    if mode == 0:
        ck, cv, n_c = O.pack_compact(c.kv.k, c.kv.v, c.kv.block_table[b], L, c.n_sink, sel[b], cap)
        ref_o, ref_l = O.sparse_decode(Qv[-1], ck, cv, n_c, c.kv.k, c.kv.v, c.kv.block_table[b], L, c.n_sink,
                                       c.n_recent, c.scale, kv_dtype=c.dtype, groups=groups)
        for g in gs:
            hs = slice(g * G, (g + 1) * G)
            assert_close(out[row0, hs], ref_o[hs], OUT_TOL, f"draft out b={b} g={g}")
            assert_close(lse[row0, hs], ref_l[hs], LSE_TOL, f"draft lse b={b} g={g}")
    else:
        ref_o, ref_l = O.dense_attention(Qv, c.kv.k, c.kv.v, c.kv.block_table[b], L, c.scale, c.Hkv,
                                         kv_dtype=c.dtype, groups=groups)
        for g in gs:
            hs = slice(g * G, (g + 1) * G)
            assert_close(out[row0:row0 + t_q, hs], ref_o[:, hs], OUT_TOL, f"verify out b={b} g={g}")
            assert_close(lse[row0:row0 + t_q, hs], ref_l[:, hs], LSE_TOL, f"verify lse b={b} g={g}")
        if sc is not None:
            ref_s = O.group_scores(Qv, c.kv.k, c.kv.block_table[b], L, c.scale, c.Hkv, c.n_sink, c.n_recent,
                                   sc.shape[-1], kv_dtype=c.dtype, groups=list(gs))
            lo, hi = O.candidate_range(L, t_q, c.n_sink, c.n_recent)
            for g in gs:
                assert np.all(np.isneginf(sc[b, g, :lo])) and np.all(np.isneginf(sc[b, g, hi:]))
                rows = O.paged_rows(c.kv.k_values(), c.kv.block_table[b], g, np.arange(lo, hi))
                bound = score_bound(Qv[:, g * G:(g + 1) * G].reshape(-1, c.d), rows, c.scale)
                assert_close(sc[b, g, lo:hi], ref_s[g, lo:hi], bound, f"verify scores b={b} g={g}")


@pytest.mark.parametrize("modes", [[0, 1, 0, 1], [1, 1, 1], [0, 0], [1, 0, 0, 0, 1]],
                         ids=["alternating", "all_verify", "all_draft", "ends_verify"])
def test_mixed_matches_oracle(gpu_lib, modes):
    B = len(modes)
    lens = [700, 2500, 1300, 4100, 333][:B]
    c = make_case(400 + B, name="mix", B=B, Hq=8, Hkv=2, d=128, dtype="bf16", t_q=8, seq_lens=lens, n_sink=4,
                  n_recent=64, k_sel=96, hh_per_head=20)
    dc = DevCase(c)
    sel, cap, t_q, out, lse, sc = _run_mixed(gpu_lib, c, dc, modes, 96, 7)
    row0 = np.concatenate([[0], np.cumsum(t_q)])
    for b in range(B):
        _check_request(c, b, modes[b], sel, cap, int(row0[b]), t_q[b], out, lse, sc)


def test_mixed_equals_separate_calls(gpu_lib):
    """One mixed launch gives the same numbers as the separate fast-step and verification calls."""
    modes = [0, 1, 1, 0]
    c = make_case(410, name="mix", B=4, Hq=16, Hkv=4, d=128, dtype="bf16", t_q=4, seq_lens=[3000, 2000, 5000, 900],
                  n_sink=4, n_recent=32, k_sel=128)
    dc = DevCase(c)
    sel, cap, t_q, out, lse, sc = _run_mixed(gpu_lib, c, dc, modes, 128, 3)
    o_v, l_v, s_v = gpu_lib.dense_attn_with_stats(dc.q, dc.k, dc.v, dc.bt, dc.lens, max_seq_len=dc.max_seq_len,
                                                  n_sink=4, n_recent=32)
    ck, cv, nc = gpu_lib.pack_compact(dc.k, dc.v, dc.bt, dc.lens, dev_array(sel), n_sink=4, cap=cap,
                                      max_seq_len=dc.max_seq_len)
    o_d, l_d = gpu_lib.sparse_decode_attn(dev_array(np.ascontiguousarray(c.q[:, -1])), dc.k, dc.v, dc.bt, dc.lens,
                                          ck, cv, nc, n_sink=4, n_recent=32, max_seq_len=dc.max_seq_len)
    torch.cuda.synchronize()
    o_v, s_v, o_d = o_v.cpu().numpy(), s_v.cpu().numpy(), o_d.cpu().numpy()
    row0 = np.concatenate([[0], np.cumsum(t_q)])
    for b in range(4):
        if modes[b] == 0:
            assert_close(out[row0[b]], o_d[b], 1e-5, f"draft b={b}")
        else:
            assert_close(out[row0[b]:row0[b] + 4], o_v[b], 1e-5, f"verify b={b}")
            assert_close(sc[b], s_v[b], 1e-4, f"scores b={b}")


def test_speculative_mix_128k_sampled(gpu_lib):
    """4 drafting requests (one token, 5 % retention: sink 4 + selected + recent 256) and 4 verifying requests
    (8 draft tokens, dense causal) at KV length 131072, 32 query heads / 8 KV heads, in one launch."""
    c = specmix128k_case(5)
    dc = DevCase(c)
    modes = c.modes.tolist()
    sel, cap, t_q, out, lse, sc = _run_mixed(gpu_lib, c, dc, modes, c.k_sel, 11)
    row0 = np.concatenate([[0], np.cumsum(t_q)])
    for b, g in [(0, 0), (3, 7), (4, 0), (6, 3), (7, 6)]:
        _check_request(c, b, modes[b], sel, cap, int(row0[b]), t_q[b], out, lse, sc, groups=[g])
    assert np.all(np.isfinite(out))
