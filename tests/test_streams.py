"""Stream ordering of the slow-step maintenance (SFI page, Fig. 3A).

The Selector and pack of layer i run on an auxiliary stream after an event from the
main stream, while the main stream moves on to other work; the fast step that follows
waits on the auxiliary stream's event.  Its output, the compact buffer and n_compact
must be bit-identical to the fully serialised order on one stream.
"""
import numpy as np
import pytest
import torch

from sfi_synth import qwen06b_decode_case
from _gpu import DEV, DevCase, dev_array

pytestmark = pytest.mark.gpu


def _buffers(c, cap):
    B, Hq, Hkv, d = c.B, c.Hq, c.Hkv, c.d
    return dict(sc=torch.empty((B, Hkv, c.kv.max_pages * 16), dtype=torch.float32, device=DEV),
                sel=torch.empty((B, Hkv, c.k_sel), dtype=torch.int32, device=DEV),
                ck=torch.empty((B, Hkv, cap, d), dtype=torch.bfloat16, device=DEV),
                cv=torch.empty((B, Hkv, cap, d), dtype=torch.bfloat16, device=DEV),
                nc=torch.empty((B,), dtype=torch.int32, device=DEV),
                fo=torch.empty((B, Hq, d), dtype=torch.float32, device=DEV),
                fl=torch.empty((B, Hq), dtype=torch.float32, device=DEV))


def _slow_and_fast(sfi, c, dc, buf, main, aux, partner=None):
    cap = c.n_sink + c.k_sel
    sfi.dense_attn_with_stats(dc.q, dc.k, dc.v, dc.bt, dc.lens, max_seq_len=dc.max_seq_len, n_sink=c.n_sink,
                              n_recent=c.n_recent, scores=buf["sc"], stream=main)
    if aux is not main:
        e1 = torch.cuda.Event()
        e1.record(main)
        aux.wait_event(e1)
    sfi.select_topk(buf["sc"], dc.lens, k=c.k_sel, n_sink=c.n_sink, n_recent=c.n_recent, sel_idx=buf["sel"],
                    stream=aux)
    sfi.pack_compact(dc.k, dc.v, dc.bt, dc.lens, buf["sel"], n_sink=c.n_sink, cap=cap,
                     max_seq_len=dc.max_seq_len, compact_k=buf["ck"], compact_v=buf["cv"], n_compact=buf["nc"],
                     stream=aux)
    if partner is not None:
        partner(main)            # the main stream moves on while the auxiliary stream works
    if aux is not main:
        e2 = torch.cuda.Event()
        e2.record(aux)
        main.wait_event(e2)
    sfi.sparse_decode_attn(dev_array(np.ascontiguousarray(c.q[:, 0])), dc.k, dc.v, dc.bt, dc.lens, buf["ck"],
                           buf["cv"], buf["nc"], n_sink=c.n_sink, n_recent=c.n_recent, max_seq_len=dc.max_seq_len,
                           out=buf["fo"], lse=buf["fl"], stream=main)


def test_aux_stream_maintenance_matches_serial_order(gpu_lib):
    c = qwen06b_decode_case(301, L=6000, B=2, frac=(1, 8))
    dc = DevCase(c)
    other = qwen06b_decode_case(302, L=8000, B=2, frac=(1, 8))
    do = DevCase(other)
    main = torch.cuda.current_stream(DEV)
    aux = torch.cuda.Stream(device=DEV)

    def partner(stream):          # the next layer's slow step on other data
        gpu_lib.dense_attn_with_stats(do.q, do.k, do.v, do.bt, do.lens, max_seq_len=do.max_seq_len,
                                      n_sink=other.n_sink, n_recent=other.n_recent, stream=stream)

    cap = c.n_sink + c.k_sel
    serial, overlapped = _buffers(c, cap), _buffers(c, cap)
    _slow_and_fast(gpu_lib, c, dc, serial, main, main)
    for _ in range(3):
        _slow_and_fast(gpu_lib, c, dc, overlapped, main, aux, partner)
        torch.cuda.synchronize()
        for key in ("sel", "ck", "cv", "nc", "fo", "fl"):
            assert torch.equal(serial[key], overlapped[key]), key
