"""GPU parity of the slow step that carries the previous layer's maintenance.

sfi_dense_attn_with_refresh runs layer i+1's slow step and, in the same launch,
layer i's Selector and pack (SFI page, Fig. 3A: maintenance of layer i overlaps
layer i+1's attention).  Every output must be bit-identical to the three separate
calls made in order; the Selector result is also checked against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle as O
from sfi_synth import make_case
from _gpu import DEV, DevCase, dev_array

pytestmark = pytest.mark.gpu


def _layers(seed, lens, Hq=16, Hkv=8, d=128, n_sink=4, n_recent=64, k=300, dtype="bf16"):
    li = make_case(seed, name="li", B=len(lens), Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, seq_lens=lens, n_sink=n_sink,
                   n_recent=n_recent, k_sel=k, hh_per_head=8)
    lj = make_case(seed + 1, name="lj", B=len(lens), Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, seq_lens=lens,
                   n_sink=n_sink, n_recent=n_recent, k_sel=k)
    return li, DevCase(li), lj, DevCase(lj)


def _check(sfi, li, di, lj, dj, k, r_scores=None, r_n_sink=None, r_n_recent=None, pack=True):
    r_n_sink = li.n_sink if r_n_sink is None else r_n_sink
    r_n_recent = li.n_recent if r_n_recent is None else r_n_recent
    cap = r_n_sink + k + 5
    if r_scores is None:
        _, _, r_scores = sfi.dense_attn_with_stats(di.q, di.k, di.v, di.bt, di.lens, max_seq_len=di.max_seq_len,
                                                   n_sink=r_n_sink, n_recent=r_n_recent)
    # separate calls, in order
    o1, l1, s1 = sfi.dense_attn_with_stats(dj.q, dj.k, dj.v, dj.bt, dj.lens, max_seq_len=dj.max_seq_len,
                                           n_sink=lj.n_sink, n_recent=lj.n_recent)
    sel1 = sfi.select_topk(r_scores, di.lens, k=k, n_sink=r_n_sink, n_recent=r_n_recent)
    ck1 = torch.full((li.B, li.Hkv, cap, li.d), 7, dtype=di.k.dtype, device=DEV)
    cv1 = torch.full_like(ck1, 7)
    nc1 = torch.full((li.B,), -9, dtype=torch.int32, device=DEV)
    sfi.pack_compact(di.k, di.v, di.bt, di.lens, sel1, n_sink=r_n_sink, cap=cap, max_seq_len=di.max_seq_len,
                     compact_k=ck1, compact_v=cv1, n_compact=nc1)
    # one launch
    ck2, cv2 = torch.full_like(ck1, 7), torch.full_like(cv1, 7)
    nc2 = torch.full_like(nc1, -9)
    o2, l2, s2, sel2, _, _, _ = sfi.dense_attn_with_refresh(
        dj.q, dj.k, dj.v, dj.bt, dj.lens, max_seq_len=dj.max_seq_len, n_sink=lj.n_sink, n_recent=lj.n_recent,
        r_k_pool=di.k, r_v_pool=di.v, r_block_table=di.bt, r_max_seq_len=di.max_seq_len, r_scores=r_scores,
        r_n_sink=r_n_sink, r_n_recent=r_n_recent, k=k, cap=cap, compact_k=ck2, compact_v=cv2, n_compact=nc2,
        pack=pack)
    if not pack:   # selection only rode along: the compact buffers are untouched until packed
        torch.cuda.synchronize()
        assert bool((ck2 == 7).all()) and bool((nc2 == -9).all())
        sfi.pack_compact(di.k, di.v, di.bt, di.lens, sel2, n_sink=r_n_sink, cap=cap, max_seq_len=di.max_seq_len,
                         compact_k=ck2, compact_v=cv2, n_compact=nc2)
    torch.cuda.synchronize()
    for name, x, y in (("out", o1, o2), ("lse", l1, l2), ("scores", s1, s2), ("sel", sel1, sel2),
                       ("compact_k", ck1, ck2), ("compact_v", cv1, cv2), ("n_compact", nc1, nc2)):
        assert torch.equal(x, y), name
    sc = r_scores.cpu().numpy()
    got = sel2.cpu().numpy()
    for b in range(li.B):
        lo, hi = O.candidate_range(int(li.seq_lens[b]), 1, r_n_sink, r_n_recent)
        for g in range(li.Hkv):
            assert np.array_equal(got[b, g], O.select_topk(sc[b, g], lo, hi, k)), (b, g)


@pytest.mark.parametrize("lens,k", [([5000, 1300, 3], 300), ([20000], 2048), ([700, 9000], 5000)],
                         ids=["ragged_short", "long_row", "k_above_candidates"])
def test_refresh_launch_equals_separate_calls(gpu_lib, lens, k):
    li, di, lj, dj = _layers(500 + len(lens), lens, k=k)
    _check(gpu_lib, li, di, lj, dj, k)


def test_refresh_launch_with_ties_and_unaligned_rows(gpu_lib):
    """Quantised logits (many exact ties, signed zeros, -inf) in rows whose stride is not a
    multiple of four, with a sink that leaves the candidates unaligned: the riders' scalar path."""
    lens = [3000, 2500]
    li, di, lj, dj = _layers(520, lens, k=400)
    rng = np.random.default_rng(9)
    stride = di.max_seq_len + 3
    sc = (np.round(rng.standard_normal((2, li.Hkv, stride)) * 4) / 4).astype(np.float32)
    sc[0, 1, ::7] = -0.0
    sc[1, 2, ::5] = -np.inf
    _check(gpu_lib, li, di, lj, dj, 400, r_scores=torch.from_numpy(sc).to(DEV), r_n_sink=3, r_n_recent=17)


@pytest.mark.parametrize("lens,k", [([6000, 2100], 700), ([16384], 1980), ([30000], 2048)],
                         ids=["register_rows", "row_16k", "row_30k"])
def test_selection_only_rides(gpu_lib, lens, k):
    li, di, lj, dj = _layers(540 + lens[0] % 7, lens, k=k)
    _check(gpu_lib, li, di, lj, dj, k, pack=False)


def test_refresh_launch_d64_fp32(gpu_lib):
    li, di, lj, dj = _layers(530, [1800, 2600], Hq=8, Hkv=2, d=64, k=256, dtype="f32")
    _check(gpu_lib, li, di, lj, dj, 256)
