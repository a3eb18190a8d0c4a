"""The fast step that allocates nothing (sfi_sparse_decode_attn_static) against the
workspace fast step (sfi_sparse_decode_attn) through the C ABI: the same kernels and
plan, so every output must match bit for bit, on two calls in a row (the second with a
smaller input, so the static scratch is reused with another layout) and after them a
call of the first shape again."""
import numpy as np
import pytest
import torch

from sfi_synth import make_case, qwen06b_decode_case
from _gpu import DEV, DevCase, dev_array

pytestmark = pytest.mark.gpu


def _packed(sfi, c, dc, k, seed):
    rng = np.random.default_rng(seed)
    L = c.seq_lens.astype(np.int64)
    sel = np.full((c.B, c.Hkv, k), -1, np.int32)
    for b in range(c.B):
        lo, hi = c.n_sink, max(c.n_sink, int(L[b]) - c.n_recent)
        n = min(k, hi - lo)
        for g in range(c.Hkv):
            if n > 0:
                sel[b, g, :n] = np.sort(rng.choice(np.arange(lo, hi), n, replace=False))
    cap = c.n_sink + k
    return sfi.pack_compact(dc.k, dc.v, dc.bt, dc.lens, dev_array(sel), n_sink=c.n_sink, cap=cap,
                            max_seq_len=dc.max_seq_len)


def _both(sfi, c, dc, ck, cv, nc):
    q1 = dc.q[:, 0].contiguous()
    kw = dict(n_sink=c.n_sink, n_recent=c.n_recent, max_seq_len=dc.max_seq_len, scale=c.scale)
    o1, l1 = sfi.sparse_decode_attn(q1, dc.k, dc.v, dc.bt, dc.lens, ck, cv, nc, **kw)
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    sfi.sparse_decode_attn_static(q1, dc.k, dc.v, dc.bt, dc.lens, ck, cv, nc, out=o2, lse=l2, **kw)
    torch.cuda.synchronize()
    return (o1, l1), (o2, l2)


def test_static_scratch_fast_step_equals_the_workspace_call_twice_then_smaller(gpu_lib):
    assert gpu_lib.load().sfi_static_scratch_bytes() == 8 << 20
    big = qwen06b_decode_case(41, L=16384, B=1, frac=(1, 8))      # 16K layer, 12.5 %: 16 splits per KV head
    small = make_case(42, name="na_s", B=3, Hq=8, Hkv=2, d=128, dtype="bf16", seq_lens=[700, 2100, 35],
                      n_sink=4, n_recent=32, k_sel=300)           # 3 requests, other split count
    runs = []
    for c, k, seed in ((big, big.k_sel, 1), (small, 300, 2), (big, big.k_sel, 3)):
        dc = DevCase(c)
        ck, cv, nc = _packed(gpu_lib, c, dc, k, seed)
        (o1, l1), (o2, l2) = _both(gpu_lib, c, dc, ck, cv, nc)
        assert torch.equal(o1, o2), "out differs from the workspace call"
        assert torch.equal(l1, l2), "lse differs from the workspace call"
        assert bool(torch.isfinite(o2).all())
        runs.append(o2.cpu())
    assert not torch.equal(runs[0], runs[2])   # different selections: a stale result would show


def test_static_scratch_fast_step_on_a_side_stream(gpu_lib):
    c = make_case(43, name="na_t", B=2, Hq=16, Hkv=8, d=128, dtype="bf16", seq_lens=[4000, 3000], n_sink=4,
                  n_recent=64, k_sel=512)
    dc = DevCase(c)
    ck, cv, nc = _packed(gpu_lib, c, dc, 512, 4)
    q1 = dc.q[:, 0].contiguous()
    kw = dict(n_sink=c.n_sink, n_recent=c.n_recent, max_seq_len=dc.max_seq_len, scale=c.scale)
    o1, l1 = gpu_lib.sparse_decode_attn(q1, dc.k, dc.v, dc.bt, dc.lens, ck, cv, nc, **kw)
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(s):
        o2 = torch.empty_like(o1)
        l2 = torch.empty_like(l1)
    gpu_lib.sparse_decode_attn_static(q1, dc.k, dc.v, dc.bt, dc.lens, ck, cv, nc, out=o2, lse=l2, stream=s, **kw)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
