"""The C-ABI library on the CPU: it loads, exports every symbol include/sfi.h declares,
rejects bad arguments with the documented status before launching anything, and
plans splits / workspaces consistently.  No compute call is made here (no GPU)."""
import ctypes
import os
import re

import pytest

import sparse_kv_cache_sfi_amd as sfi
from sparse_kv_cache_sfi_amd import SfiPagedKV, SfiShape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sfi.h")

FAKE = 0x10000            # a 16-byte aligned address; never dereferenced by a rejected call
MISALIGNED = 0x10004


@pytest.fixture(scope="module")
def lib():
    return sfi.load()


def declared_symbols():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^SFI_API\s+[\w\s\*]+?\b(sfi_\w+)\s*\(", src, re.M)))


def test_header_declares_the_entry_points():
    names = declared_symbols()
    for n in ("sfi_dense_attn_with_stats", "sfi_select_topk", "sfi_pack_compact", "sfi_sparse_decode_attn",
              "sfi_mixed_attn", "sfi_sparse_decode_append_attn",
              "sfi_sparse_decode_indexed_attn", "sfi_dense_attn_with_head_stats"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_symbols():
        assert hasattr(lib, n), n


def test_removed_entry_points_are_gone(lib):
    # the slow step that carried the previous layer's Selector and pack as extra
    # work-groups measured slower than running them serially; the pack that merged a
    # deferred slow step is superseded by the fused fast step + pack launch
    assert not hasattr(lib, "sfi_dense_attn_with_refresh")
    assert not hasattr(lib, "sfi_pack_compact_merge")


def test_version_and_status_strings(lib):
    assert lib.sfi_version() == 10000
    assert lib.sfi_status_string(0) == b"SFI_OK"
    assert lib.sfi_status_string(3) == b"SFI_ERR_WORKSPACE"
    assert lib.sfi_status_string(99) == b"SFI_ERR_UNKNOWN"


def _shape(B=1, Hq=16, Hkv=8, d=128, dtype=1, scale=0.088):
    return SfiShape(B, Hq, Hkv, d, dtype, scale)


def _kv(k=FAKE, v=FAKE, bt=FAKE, max_pages=1024, page=16, num_pages=1024, max_len=16384):
    return SfiPagedKV(k, v, bt, max_pages, page, num_pages, max_len)


def _dense(lib, shape, kv, q=FAKE, t_q=1, lens=FAKE, n_sink=4, n_recent=64, out=FAKE, lse=FAKE, scores=FAKE,
           stride=16384, ws=FAKE, ws_bytes=1 << 40):
    return lib.sfi_dense_attn_with_stats(ctypes.byref(shape) if shape is not None else None,
                                         ctypes.byref(kv) if kv is not None else None, q, t_q, lens, n_sink,
                                         n_recent, out, lse, scores, stride, ws, ws_bytes, None)


@pytest.mark.parametrize("mutate,status,msg", [
    (lambda a: a.update(shape=None), 1, "shape is NULL"),
    (lambda a: a.update(kv=None), 1, "kv descriptor"),
    (lambda a: a.update(shape=_shape(Hq=24)), 2, "1, 2, 4 or 8"),
    (lambda a: a.update(shape=_shape(Hq=15)), 1, "multiple"),
    (lambda a: a.update(shape=_shape(d=96)), 2, "head_dim"),
    (lambda a: a.update(shape=_shape(dtype=7)), 1, "dtype"),
    (lambda a: a.update(shape=_shape(scale=-1.0)), 1, "scale"),
    (lambda a: a.update(shape=_shape(B=0)), 1, "batch"),
    (lambda a: a.update(kv=_kv(page=32)), 2, "page_size"),
    (lambda a: a.update(kv=_kv(max_len=20000)), 1, "max_seq_len"),
    (lambda a: a.update(kv=_kv(max_pages=70000, max_len=(1 << 20) + 16)), 2, "exceeds"),
    (lambda a: a.update(kv=_kv(k=MISALIGNED)), 1, "aligned"),
    (lambda a: a.update(kv=_kv(bt=0)), 1, "non-NULL"),
    (lambda a: a.update(q=0), 1, "q is NULL"),
    (lambda a: a.update(q=MISALIGNED), 1, "q must be 16-byte aligned"),
    (lambda a: a.update(out=0), 1, "out is NULL"),
    (lambda a: a.update(lens=0), 1, "seq_lens"),
    (lambda a: a.update(t_q=0), 1, "t_q"),
    (lambda a: a.update(t_q=17), 1, "t_q"),
    (lambda a: a.update(n_sink=-1), 1, "n_sink"),
    (lambda a: a.update(stride=100), 1, "score_stride"),
    (lambda a: a.update(ws_bytes=10), 3, "workspace"),
    (lambda a: a.update(ws=0), 1, "workspace is NULL"),
    (lambda a: a.update(shape=_shape(dtype=0), t_q=4), 2, "bf16"),
    (lambda a: a.update(shape=_shape(Hq=64, Hkv=8), t_q=16), 2, "<= 32"),
    (lambda a: a.update(shape=_shape(Hq=32, Hkv=8), t_q=9), 2, "<= 32"),
])
def test_dense_rejects_bad_arguments(lib, mutate, status, msg):
    args = dict(shape=_shape(), kv=_kv())
    mutate(args)
    st = _dense(lib, **args)
    assert st == status, (st, lib.sfi_last_error())
    assert msg in lib.sfi_last_error().decode()


def test_select_rejects_bad_arguments(lib):
    ok = dict(scores=FAKE, B=1, H=8, stride=16384, lens=FAKE, t_q=1, ns=4, nr=64, k=100, sel=FAKE)

    def call(**kw):
        a = {**ok, **kw}
        return lib.sfi_select_topk(a["scores"], a["B"], a["H"], a["stride"], a["lens"], a["t_q"], a["ns"], a["nr"],
                                   a["k"], a["sel"], None, 0, None)
    assert call(scores=0) == 1
    assert call(sel=0) == 1
    assert call(k=0) == 1 and "k must be" in lib.sfi_last_error().decode()
    assert call(B=0) == 1
    assert call(stride=0) == 1
    assert call(t_q=0) == 1
    assert call(nr=-3) == 1
    # long rows need the candidate workspace: 65536 positions, top-2048 -> 8 segments
    assert call(stride=65536, k=2048) == 3 and "workspace" in lib.sfi_last_error().decode()


def test_select_workspace_size_covers_the_segment_candidates(lib):
    def size(B, H, stride, ns, k):
        out = ctypes.c_size_t(0)
        assert lib.sfi_select_topk_workspace_size(B, H, stride, ns, k, ctypes.byref(out)) == 0
        return out.value
    # 16K rows run on one work-group each: no workspace
    assert size(1, 8, 16384, 4, 1980) == 0
    # the 64K refresh: 4 requests x 8 KV heads, 65532 possible candidates -> 4 segments of 16383
    # positions, each keeping its top-2048 candidates, 8 bytes each (key, position)
    assert size(4, 8, 65536, 4, 2048) == 32 * 4 * 2048 * 8        # keys + positions
    # k too large for the segments to cut the row at least in half: one work-group per row
    assert size(4, 8, 65536, 4, 8192) == 0
    # 1,048,576 positions: 16 segments
    assert size(1, 1, 1 << 20, 4, 1024) == 16 * 1024 * 8
    # the candidate rows are padded to a multiple of four: 4 segments x top-2047 = 8188 -> 8188
    assert size(1, 1, 65536, 4, 2047) == ((4 * 2047 + 3) // 4 * 4) * 8
    # a k whose padding shows: 4 x 2045 = 8180 -> 8180; 3 segments (49148 positions) x 2045 = 6135 -> 6136
    assert size(1, 1, 49152, 4, 2045) == 6136 * 8


def test_pack_rejects_bad_arguments(lib):
    shape, kv = _shape(), _kv()

    def call(ck=FAKE, cv=FAKE, cap=200, k=100, n_sink=4, nc=FAKE, sel=FAKE):
        return lib.sfi_pack_compact(ctypes.byref(shape), ctypes.byref(kv), FAKE, n_sink, sel, k, ck, cv, cap, nc,
                                    None)
    assert call(cap=103) == 1 and "cap" in lib.sfi_last_error().decode()
    assert call(ck=MISALIGNED) == 1
    assert call(nc=0) == 1
    assert call(sel=0) == 1
    assert call(k=0) == 1
    assert call(n_sink=-1) == 1


def test_sparse_rejects_bad_arguments(lib):
    shape, kv = _shape(), _kv()

    def call(q=FAKE, ck=FAKE, cap=2048, nc=FAKE, ws=FAKE, ws_bytes=1 << 40, n_recent=64, out=FAKE):
        return lib.sfi_sparse_decode_attn(ctypes.byref(shape), ctypes.byref(kv), q, FAKE, 4, n_recent, ck, FAKE, cap,
                                          nc, out, FAKE, ws, ws_bytes, None)
    assert call(q=MISALIGNED) == 1
    assert call(ck=0) == 1
    assert call(nc=0) == 1
    assert call(cap=0) == 1
    assert call(n_recent=-1) == 1
    assert call(out=0) == 1
    assert call(ws_bytes=1) == 3


def test_sparse_append_rejects_bad_arguments(lib):
    shape, kv = _shape(), _kv()

    def call(kn=FAKE, vn=FAKE, q=FAKE, ws_bytes=1 << 40):
        return lib.sfi_sparse_decode_append_attn(ctypes.byref(shape), ctypes.byref(kv), q, kn, vn, FAKE, 4, 64, FAKE,
                                                 FAKE, 2048, FAKE, FAKE, FAKE, FAKE, ws_bytes, None)
    assert call(kn=0) == 1 and "k_new is NULL" in lib.sfi_last_error().decode()
    assert call(vn=0) == 1 and "v_new is NULL" in lib.sfi_last_error().decode()
    assert call(kn=MISALIGNED) == 1 and "aligned" in lib.sfi_last_error().decode()
    assert call(q=MISALIGNED) == 1
    assert call(ws_bytes=1) == 3


def test_sparse_indexed_rejects_bad_arguments(lib):
    shape = _shape()

    def call(sel=FAKE, k=64, kn=None, vn=None, q=FAKE, ws_bytes=1 << 40, kv=None, out=FAKE, per_head=0, ck=None,
             cap=0, nc=None):
        kv = kv or _kv()
        return lib.sfi_sparse_decode_indexed_attn(ctypes.byref(shape), ctypes.byref(kv), q, kn, vn, FAKE, 4, 64, sel,
                                                  k, per_head, ck, FAKE if ck else None, cap, nc, out, FAKE, FAKE,
                                                  ws_bytes, None)
    assert call(sel=0) == 1 and "sel_idx is NULL" in lib.sfi_last_error().decode()
    assert call(k=-1) == 1 and "k must be" in lib.sfi_last_error().decode()
    assert call(kn=FAKE) == 1 and "both" in lib.sfi_last_error().decode()
    assert call(kn=MISALIGNED, vn=FAKE) == 1 and "aligned" in lib.sfi_last_error().decode()
    assert call(q=MISALIGNED) == 1
    assert call(out=0) == 1
    assert call(k=20000, ws_bytes=1) == 3          # several splits: partials needed
    assert call(kv=_kv(num_pages=1 << 27)) == 2 and "slots" in lib.sfi_last_error().decode()
    assert call(per_head=2) == 1 and "per_head" in lib.sfi_last_error().decode()
    assert call(per_head=1, k=20000, ws_bytes=1) == 3
    assert call(ck=FAKE, cap=68) == 1 and "go together" in lib.sfi_last_error().decode()
    assert call(ck=FAKE, cap=67, nc=FAKE) == 1 and "cap" in lib.sfi_last_error().decode()
    assert call(ck=MISALIGNED, cap=68, nc=FAKE) == 1 and "aligned" in lib.sfi_last_error().decode()
    assert call(ck=FAKE, cap=20004, nc=FAKE, k=20000, ws_bytes=1) == 3


def test_dense_head_stats_rejects_bad_arguments(lib):
    shape, kv = _shape(), _kv()

    def call(scores=FAKE, stride=16384, q=FAKE, ws_bytes=1 << 40):
        return lib.sfi_dense_attn_with_head_stats(ctypes.byref(shape), ctypes.byref(kv), q, FAKE, 4, 64, FAKE, FAKE,
                                                  scores, stride, FAKE, ws_bytes, None)
    assert call(scores=0) == 1 and "scores is NULL" in lib.sfi_last_error().decode()
    assert call(stride=100) == 1 and "score_stride" in lib.sfi_last_error().decode()
    assert call(q=MISALIGNED) == 1
    assert call(ws_bytes=1) == 3


def test_workspace_queries_match_the_plan(lib):
    shape, kv = _shape(), _kv()
    st, ns = ctypes.c_int32(), ctypes.c_int32()
    assert lib.sfi_plan_splits(0, ctypes.byref(shape), ctypes.byref(kv), 1, 0, 0, ctypes.byref(st),
                               ctypes.byref(ns)) == 0
    size = ctypes.c_size_t()
    assert lib.sfi_dense_attn_workspace_size(ctypes.byref(shape), ctypes.byref(kv), 1, ctypes.byref(size)) == 0
    if ns.value > 1:
        assert size.value >= 16 * ns.value * (128 + 2) * 4
    else:
        assert size.value == 0


@pytest.mark.parametrize("B,Hkv,n_tok", [(1, 8, 16384), (1, 8, 256), (16, 8, 32768), (4, 8, 65536),
                                         (8, 8, 131072), (1, 1, 1), (3, 2, 3000), (64, 8, 100),
                                         (1, 1, 1 << 20), (1, 1, 300000)])
def test_split_plan_covers_every_token(B, Hkv, n_tok):
    st, ns = sfi.plan_splits(0, B=B, Hq=4 * Hkv, Hkv=Hkv, d=128, bf16=True, max_pages=(n_tok + 15) // 16,
                             num_pages=1, max_seq_len=n_tok)
    assert st % 64 == 0 and 64 <= st <= 4096
    assert ns * st >= n_tok and (ns - 1) * st < n_tok
    assert 1 <= ns <= 256
    assert ns == 1 or st >= 256 or B * Hkv * ns >= 2048


def test_split_plan_of_the_16k_decode_layer():
    # 1 request x 8 KV heads x 16384 tokens: 32 splits of 512 tokens -> 256 work-groups.
    assert sfi.plan_splits(0, B=1, Hq=16, Hkv=8, d=128, bf16=True, max_pages=1024, num_pages=1024,
                           max_seq_len=16384) == (512, 32)
    # fast step, 1.6 % retention: 192 compact slots + 64 recent -> one split (no split-K tail)
    assert sfi.plan_splits(1, B=1, Hq=16, Hkv=8, d=128, bf16=True, max_pages=1024, num_pages=1024,
                           max_seq_len=16384, cap=192, n_recent=64) == (256, 1)
    # 12.5 %: 1984 compact slots in 16 splits of 128 tokens, and the 64 recent tokens as a split of
    # their own (it waits for the block table): 136 work-groups
    assert sfi.plan_splits(1, B=1, Hq=16, Hkv=8, d=128, bf16=True, max_pages=1024, num_pages=1024,
                           max_seq_len=16384, cap=1984, n_recent=64) == (128, 17)
    # 25 %: one more work-group per unit would pass one per CU: 32 even splits of 128
    assert sfi.plan_splits(1, B=1, Hq=16, Hkv=8, d=128, bf16=True, max_pages=1024, num_pages=1024,
                           max_seq_len=16384, cap=4032, n_recent=64) == (128, 32)
    # batch 16: 128 units of two splits fill the 256 CUs
    assert sfi.plan_splits(1, B=16, Hq=16, Hkv=8, d=128, bf16=True, max_pages=1024, num_pages=1024,
                           max_seq_len=16384, cap=1984, n_recent=64) == (1024, 2)
    # batch 16 at 75 %: 12288 rows; cut at the cap (3 x 4096, 384 work-groups) half the CUs would
    # stream two long splits; four even splits of 3072 give every CU two
    assert sfi.plan_splits(1, B=16, Hq=16, Hkv=8, d=128, bf16=True, max_pages=1024, num_pages=1024,
                           max_seq_len=16384, cap=12224, n_recent=64) == (3072, 4)
    # 12305 rows: not 3 x 4096 + 17 but four even splits of 3136
    assert sfi.plan_splits(1, B=16, Hq=16, Hkv=8, d=128, bf16=True, max_pages=1024, num_pages=1024,
                           max_seq_len=16384, cap=12241, n_recent=64) == (3136, 4)
    # dense at batch 12 x 16K: five splits of 3328 (480 work-groups) instead of four of 4096 (384)
    assert sfi.plan_splits(0, B=12, Hq=16, Hkv=8, d=128, bf16=True, max_pages=1024, num_pages=1024,
                           max_seq_len=16384) == (3328, 5)
    # where the capped cut already fills whole waves it stays: batch 16 x 16K dense, 4 x 4096
    assert sfi.plan_splits(0, B=16, Hq=16, Hkv=8, d=128, bf16=True, max_pages=1024, num_pages=1024,
                           max_seq_len=16384) == (4096, 4)


def test_verification_splits_take_up_to_8192_tokens():
    # 4 verifying requests x 8 KV heads x 128K, 8 draft tokens: 16 splits of 8192 -> 512 work-groups, one wave
    assert sfi.plan_splits(0, B=4, Hq=32, Hkv=8, d=128, bf16=True, max_pages=8192, num_pages=32768,
                           max_seq_len=131072, t_q=8) == (8192, 16)
    # the decode kernels keep 4096: one request x 8 KV heads x 256K at t_q = 1 -> 64 splits of 4096
    assert sfi.plan_splits(0, B=1, Hq=16, Hkv=8, d=128, bf16=True, max_pages=16384, num_pages=16384,
                           max_seq_len=262144) == (4096, 64)


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        sfi.select_topk(torch.zeros((1, 1, 8)), torch.zeros(1, dtype=torch.int32), k=2, n_sink=0, n_recent=0)


def test_deferred_slow_step_rejects_bad_arguments(lib):
    shape, kv = _shape(), _kv()

    def dense(scores=FAKE, q=FAKE, ws_bytes=1 << 40):
        return lib.sfi_dense_attn_with_stats_deferred(ctypes.byref(shape), ctypes.byref(kv), q, FAKE, 4, 64, FAKE,
                                                      FAKE, scores, 16384, FAKE, ws_bytes, None)

    assert dense(scores=0) == 1 and "scores is NULL" in lib.sfi_last_error().decode()
    assert dense(q=MISALIGNED) == 1
    assert dense(ws_bytes=10) == 3



def test_indexed_fast_step_with_pack_and_combine_rejects_bad_arguments(lib):
    shape, kv = _shape(), _kv()
    WS = 0x100000

    def call(sel=FAKE, k=100, ck=FAKE, cap=200, nc=FAKE, slow_out=FAKE, ws=FAKE, ws_bytes=1 << 20, slow_ws=WS,
             slow_bytes=1 << 40, shape_=shape):
        return lib.sfi_sparse_decode_indexed_attn_merge(ctypes.byref(shape_), ctypes.byref(kv), FAKE, FAKE, 4, 64,
                                                        sel, k, ck, FAKE, cap, nc, FAKE, FAKE, ws, ws_bytes, slow_out,
                                                        FAKE, slow_ws, slow_bytes, None)

    assert call(ck=0) == 1
    assert call(ck=MISALIGNED) == 1
    assert call(nc=0) == 1 and "n_compact" in lib.sfi_last_error().decode()
    assert call(slow_out=0) == 1
    assert call(sel=0) == 1 and "sel_idx" in lib.sfi_last_error().decode()
    assert call(k=-1) == 1
    assert call(cap=50) == 1 and "cap" in lib.sfi_last_error().decode()
    assert call(slow_bytes=10) == 3
    assert call(ws=WS + 64) == 1 and "overlap" in lib.sfi_last_error().decode()
    assert call(shape_=_shape(d=96)) == 2


def test_static_scratch_fast_step_rejects_calls_beyond_its_scratch(lib, monkeypatch):
    # Many splits (tuning override of the work-group target) need more split-K scratch
    # than the static array holds: rejected on the host, before any device call.
    monkeypatch.setenv("SFI_TUNE_TARGET_WGS", "1000000")
    shape = sfi.SfiShape(8, 64, 8, 128, sfi.SFI_BF16, 0.088)
    kv = _kv()
    st = lib.sfi_sparse_decode_attn_static(ctypes.byref(shape), ctypes.byref(kv), FAKE, FAKE, 4, 64, FAKE, FAKE,
                                           16380, FAKE, FAKE, FAKE, None)
    assert st == sfi.SFI_ERR_WORKSPACE and "static scratch" in lib.sfi_last_error().decode()
    assert lib.sfi_static_scratch_bytes() == 8 << 20
