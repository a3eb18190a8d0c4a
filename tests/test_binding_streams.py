"""Host-side rule of the binding (CPU): a workspace the binding allocates for a call is
filled on the stream that call is launched on and recorded as used by that stream, so
neither its zero-fill nor a reuse of its memory can overtake the launch."""
import contextlib

import torch

import sparse_kv_cache_sfi_amd as sfi


class _FakeTensor:
    def __init__(self, n):
        self.n = n
        self.recorded = []

    def record_stream(self, s):
        self.recorded.append(s)


def test_allocated_workspace_is_filled_and_recorded_on_the_call_stream(monkeypatch):
    events = []
    current = object()
    call_stream = object()

    @contextlib.contextmanager
    def fake_stream(s):
        events.append(("enter", s))
        yield
        events.append(("exit", s))

    def fake_zeros(n, **kw):
        events.append(("zeros", n))
        return _FakeTensor(n)

    monkeypatch.setattr(torch.cuda, "stream", fake_stream)
    monkeypatch.setattr(torch.cuda, "current_stream", lambda device=None: current)
    monkeypatch.setattr(torch, "zeros", fake_zeros)

    ws = sfi._workspace(1024, None, "cuda:0", call_stream)
    assert events == [("enter", call_stream), ("zeros", 1024), ("exit", call_stream)]
    assert ws.recorded == [call_stream]

    events.clear()
    ws = sfi._workspace(64, None, "cuda:0", None)      # no stream given: the current one
    assert events == [("enter", current), ("zeros", 64), ("exit", current)]
    assert ws.recorded == [current]


def test_caller_workspace_and_empty_size_allocate_nothing(monkeypatch):
    monkeypatch.setattr(torch, "zeros", lambda *a, **k: (_ for _ in ()).throw(AssertionError("allocated")))
    assert sfi._workspace(0, None, "cuda:0", None) is None
