"""GPU parity of the Selector and the gather-pack: bit-exact against the oracle.

The oracle Selector is fed the very fp32 scores the GPU consumed, so both sides
take every comparison on the same values (an integer result decided by floating
point is compared at the kernel's precision).  Pack is a bitwise gather.
"""
import numpy as np
import pytest
import torch

import oracle as O
from sfi_synth import make_case, refresh64k_case
from _gpu import DEV, DevCase, dev_array, host_bits

pytestmark = pytest.mark.gpu


def _select_both(sfi, scores_np, lens, k, n_sink, n_recent, t_q=1):
    sc = torch.from_numpy(np.ascontiguousarray(scores_np, dtype=np.float32)).to(DEV)
    sel = sfi.select_topk(sc, torch.tensor(lens, dtype=torch.int32, device=DEV), k=k, n_sink=n_sink,
                          n_recent=n_recent, t_q=t_q)
    torch.cuda.synchronize()
    got = sel.cpu().numpy()
    B, H, _ = scores_np.shape
    for b in range(B):
        lo, hi = O.candidate_range(int(lens[b]), t_q, n_sink, n_recent)
        hi = min(hi, scores_np.shape[-1])
        lo = min(lo, hi)
        for g in range(H):
            ref = O.select_topk(scores_np[b, g], lo, hi, k)
            assert np.array_equal(got[b, g], ref), (b, g, k)
    return got


@pytest.mark.parametrize("n_sink", [3, 4], ids=["unaligned_rows", "aligned_rows"])
@pytest.mark.parametrize("k", [1, 2, 7, 64, 500, 999, 1000, 1001, 5000])
def test_selector_crafted_ties(gpu_lib, k, n_sink):
    rng = np.random.default_rng(k)
    B, H, stride = 3, 4, 1100
    vals = np.array([-np.inf, -3.0, -1.5, -0.0, 0.0, 0.25, 1.0, 2.0, 1e30, np.inf], dtype=np.float32)
    sc = rng.choice(vals, size=(B, H, stride)).astype(np.float32)
    sc[1, 2, :] = 1.5                       # one row entirely tied
    sc[2, 0, :] = -0.0                      # signed zeros only
    sc[2, 1, 500:] = 0.0
    lens = [1100, 900, 37]
    _select_both(gpu_lib, sc, lens, k, n_sink=n_sink, n_recent=5)


@pytest.fixture(params=["segments", "one_work_group"])
def select_path(request, monkeypatch):
    """Rows of >= 32768 candidates with a small k run over segments; the other value keeps every
    row on one work-group (tuning override), so both paths see the same rows."""
    if request.param == "one_work_group":
        monkeypatch.setenv("SFI_TUNE_SELECT_SEGMENTS", "0")
    return request.param


@pytest.mark.parametrize("k", [1, 33, 2048, 20000])
def test_selector_large_rows_quantised_scores(gpu_lib, k, select_path):
    rng = np.random.default_rng(100 + k)
    B, H, stride = 2, 3, 65536
    sc = (np.round(rng.standard_normal((B, H, stride)) * 8) / 8).astype(np.float32)   # many exact ties
    lens = [65536, 40000]
    _select_both(gpu_lib, sc, lens, k, n_sink=4, n_recent=256)


def test_selector_on_gpu_slow_step_scores_keeps_planted_keys(gpu_lib):
    c = make_case(201, name="p", B=2, Hq=16, Hkv=8, d=128, dtype="bf16", seq_lens=[6000, 4100], n_sink=4,
                  n_recent=64, k_sel=512, hh_per_head=100)
    dc = DevCase(c)
    _, _, scores = gpu_lib.dense_attn_with_stats(dc.q, dc.k, dc.v, dc.bt, dc.lens, max_seq_len=dc.max_seq_len,
                                                 n_sink=c.n_sink, n_recent=c.n_recent)
    torch.cuda.synchronize()
    sc = scores.cpu().numpy()
    got = _select_both(gpu_lib, sc, c.seq_lens.tolist(), c.k_sel, c.n_sink, c.n_recent)
    for (b, g), pos in c.planted.items():
        assert set(pos.tolist()) <= set(got[b, g].tolist())


def test_selector_is_deterministic(gpu_lib):
    rng = np.random.default_rng(3)
    sc = (np.round(rng.standard_normal((4, 8, 20000)) * 4) / 4).astype(np.float32)
    a = _select_both(gpu_lib, sc, [20000] * 4, 777, 4, 64)
    b = _select_both(gpu_lib, sc, [20000] * 4, 777, 4, 64)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_pack_bit_exact_and_idempotent(gpu_lib, dtype, d):
    c = make_case(210 + d, name="k", B=3, Hq=4, Hkv=2, d=d, dtype=dtype, seq_lens=[500, 130, 3], n_sink=4,
                  n_recent=16, k_sel=100)
    dc = DevCase(c)
    rng = np.random.default_rng(d)
    k, cap = 100, 110
    sel = np.full((3, 2, k), -1, np.int32)
    for b in range(3):
        lo, hi = O.candidate_range(int(c.seq_lens[b]), 1, 4, 16)
        k_eff = max(0, min(k, hi - lo))
        for g in range(2):
            if k_eff:
                sel[b, g, :k_eff] = np.sort(rng.choice(np.arange(lo, hi), k_eff, replace=False))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    ck = torch.full((3, 2, cap, d), 7.0, dtype=tdt, device=DEV)       # sentinel rows must survive past n_compact
    cv = torch.full((3, 2, cap, d), 7.0, dtype=tdt, device=DEV)
    nc = torch.full((3,), -9, dtype=torch.int32, device=DEV)
    for rep in range(2):
        gpu_lib.pack_compact(dc.k, dc.v, dc.bt, dc.lens, dev_array(sel), n_sink=4, cap=cap,
                             max_seq_len=dc.max_seq_len, compact_k=ck, compact_v=cv, n_compact=nc)
        torch.cuda.synchronize()
        gk, gv, gn = host_bits(ck), host_bits(cv), nc.cpu().numpy()
        for b in range(3):
            rk, rv, rn = O.pack_compact(c.kv.k, c.kv.v, c.kv.block_table[b], int(c.seq_lens[b]), 4, sel[b], cap)
            assert gn[b] == rn
            assert np.array_equal(gk[b, :, :rn], rk[:, :rn]) and np.array_equal(gv[b, :, :rn], rv[:, :rn])
            sentinel = host_bits(torch.full((1,), 7.0, dtype=tdt))[0]
            assert np.all(gk[b, :, rn:] == sentinel) and np.all(gv[b, :, rn:] == sentinel)


def test_refresh_64k_select_and_pack_match_oracle_on_sampled_rows(gpu_lib):
    """The 64K refresh workload at full size: 4 requests x 8 KV heads, top-2048 of 65276 candidates."""
    c = refresh64k_case(4)
    dc = DevCase(c)
    _, _, scores = gpu_lib.dense_attn_with_stats(dc.q, dc.k, dc.v, dc.bt, dc.lens, max_seq_len=dc.max_seq_len,
                                                 n_sink=c.n_sink, n_recent=c.n_recent, with_scores=True)
    sel = gpu_lib.select_topk(scores, dc.lens, k=c.k_sel, n_sink=c.n_sink, n_recent=c.n_recent)
    cap = c.n_sink + c.k_sel
    ck, cv, nc = gpu_lib.pack_compact(dc.k, dc.v, dc.bt, dc.lens, sel, n_sink=c.n_sink, cap=cap,
                                      max_seq_len=dc.max_seq_len)
    torch.cuda.synchronize()
    sc, gs, gk = scores.cpu().numpy(), sel.cpu().numpy(), host_bits(ck)
    assert np.all(nc.cpu().numpy() == cap)
    lo, hi = O.candidate_range(65536, 1, c.n_sink, c.n_recent)
    for b, g in [(0, 0), (1, 3), (2, 5), (3, 7)]:
        ref = O.select_topk(sc[b, g], lo, hi, c.k_sel)
        assert np.array_equal(gs[b, g], ref), (b, g)
        assert set(c.planted[(b, g)].tolist()) <= set(ref.tolist())
        rk, _, _ = O.pack_compact(c.kv.k, c.kv.v, c.kv.block_table[b], 65536, c.n_sink,
                                  np.repeat(ref[None], c.Hkv, 0), cap)
        assert np.array_equal(gk[b, g], rk[g])


@pytest.mark.parametrize("k", [7, 5000])
def test_selector_rows_beyond_the_register_variant(gpu_lib, k, select_path):
    """Rows longer than 65536 candidates (the verification statistics at 128K) take the streaming kernel."""
    rng = np.random.default_rng(200 + k)
    B, H, stride = 1, 2, 131072
    sc = (np.round(rng.standard_normal((B, H, stride)) * 16) / 16).astype(np.float32)
    _select_both(gpu_lib, sc, [131072], k, n_sink=4, n_recent=256, t_q=8)


def _key_to_float(keys):
    """Inverse of the Selector's order-preserving key map (positive floats have the top key bit set)."""
    keys = np.asarray(keys, dtype=np.uint64)
    bits = np.where(keys & 0x80000000, keys & 0x7FFFFFFF, (~keys) & 0xFFFFFFFF).astype(np.uint32)
    return bits.view(np.float32)


@pytest.mark.parametrize("stride,digits", [(4096, [(20, 12), (8, 12)]),
                                           (131072, [(24, 8), (16, 8), (8, 8)])],
                         ids=["register_rows", "streaming_rows"])
def test_selector_bin_that_holds_exactly_the_wanted_keys(gpu_lib, stride, digits, select_path):
    """A radix pass whose chosen bin holds exactly the keys still wanted settles the selection.

    Row h plants, at random positions, a keys in a higher bin of digit level h, m keys in the bin
    (two of them equal to the bin's lowest key, the rest above it), and keys just below the bin that
    share its higher digits, so no earlier level settles it; k = a + m.  The last row has no planted
    structure (continuous scores).  Selections must equal the oracle's top-k.
    """
    rng = np.random.default_rng(stride)
    H = len(digits) + 1
    n_sink, n_recent = 4, 16
    lo, hi = O.candidate_range(stride, 1, n_sink, n_recent)
    a, m = 5, 6
    sc = np.empty((1, H, stride), np.float32)
    for h, (shift, _) in enumerate(digits):
        bw = 1 << shift
        P = (0xC0000000 & ~((bw << 4) - 1)) | (5 << shift)   # digit 5 at this level, lower digits zero
        keys = rng.integers(0x10000000, 0x70000000, size=stride, dtype=np.uint64)   # negative floats
        planted = [P + 2 * bw + j for j in range(a)]
        planted += [P, P] + [P + int(x) for x in rng.choice(np.arange(1, min(bw, 1 << 16)), m - 2, replace=False)]
        planted += [P - 1 - j for j in range(3)]
        pos = rng.choice(np.arange(lo, hi), len(planted), replace=False)
        keys[pos] = planted
        sc[0, h] = _key_to_float(keys)
    sc[0, H - 1] = rng.standard_normal(stride).astype(np.float32)
    _select_both(gpu_lib, sc, [stride], a + m, n_sink=n_sink, n_recent=n_recent)
    for k in (1, 17, 300):
        _select_both(gpu_lib, sc, [stride], k, n_sink=n_sink, n_recent=n_recent)


@pytest.mark.parametrize("seg", [16384, 8192])
@pytest.mark.parametrize("k", [1, 100, 1024, 4095])
def test_selector_segments_with_ties_across_segment_boundaries(gpu_lib, k, seg, monkeypatch):
    """Long rows cut into segments: equal scores straddling segment boundaries, whole rows of one
    value, signed zeros and -inf, and ragged lengths that leave trailing segments short or empty.
    The lowest positions must win every tie, exactly as the one-work-group Selector and the oracle.
    98300 candidates make 6 segments of 16384 positions (the default size) or 12 of 8192."""
    if seg != 16384:
        monkeypatch.setenv("SFI_TUNE_SELECT_SEG", str(seg))
    rng = np.random.default_rng(300 + k)
    B, H, stride = 3, 4, 98304
    vals = np.array([-np.inf, -2.0, -0.0, 0.0, 0.5, 3.0, 3.0, 7.25], dtype=np.float32)
    sc = rng.choice(vals, size=(B, H, stride)).astype(np.float32)
    sc[0, 1, :] = 3.0                            # one value everywhere
    sc[1, 2, :] = -0.0
    sc[1, 2, ::3] = 0.0                          # signed zeros only
    for j in range(1, (stride - 4) // seg + 1):  # a band of the top value across every boundary
        sc[2, 3, 4 + j * seg - 40: 4 + j * seg + 40] = 9.5
    lens = [98304, 70001, 33000]
    _select_both(gpu_lib, sc, lens, k, n_sink=4, n_recent=64)
