"""CPU checks of the Python binding's stream handling (no GPU: torch's stream
context, its allocator entry point and the library are replaced by recorders).

A workspace the binding allocates for a call must belong to the stream the
call's kernels are queued on.  Allocated under another stream, the caching
allocator could hand the block to new work on that stream as soon as the
tensor is dropped, while the kernels still use it.
"""
import types

import pytest
import torch

import store_kvi8r_quantize_amd as h3a


class _Recorder:
    def __init__(self):
        self.events = []
        self.current = "default"

    def stream(self, s):
        rec = self

        class Ctx:
            def __enter__(self):
                rec.events.append(("enter", s))
                rec._prev, rec.current = rec.current, s

            def __exit__(self, *a):
                rec.current = rec._prev
                rec.events.append(("exit", s))

        return Ctx()

    def empty(self, n, dtype=None, device=None):
        self.events.append(("alloc", n, self.current))
        return torch.zeros(n, dtype=dtype)


class _Fake:
    def __init__(self, shape, ptr):
        self.shape, self._ptr = tuple(shape), ptr
        self.device = "cuda:0"

    def is_contiguous(self):
        return True

    def dim(self):
        return len(self.shape)

    def data_ptr(self):
        return self._ptr


class _Lib:
    def __init__(self, need):
        self.need, self.calls = need, []

    def h3a_attention_workspace_bytes(self, *a):
        return self.need

    def _record(self, name):
        def f(*a):
            self.calls.append((name, a))
            return 0
        return f

    def __getattr__(self, name):
        return self._record(name)


@pytest.fixture
def rig(monkeypatch):
    rec = _Recorder()
    lib = _Lib(need=4096)
    side = types.SimpleNamespace(cuda_stream=0xABC, name="side")
    monkeypatch.setattr(torch.cuda, "stream", rec.stream)
    monkeypatch.setattr(torch, "empty", rec.empty)
    monkeypatch.setattr(h3a, "_load", lambda: lib)
    monkeypatch.setattr(h3a, "_lib", lib)
    monkeypatch.setattr(h3a, "_need", lambda *a: None)
    monkeypatch.setattr(h3a, "_out_flag", lambda out, mode: 0)
    monkeypatch.setattr(h3a, "_stream_obj", lambda t, s: side)
    return rec, lib, side


def test_workspace_allocated_under_the_given_stream(rig):
    rec, _, side = rig
    h3a._workspace(1000, "cuda:0", side)
    assert rec.events == [("enter", side), ("alloc", 1000, side), ("exit", side)]


@pytest.mark.parametrize("entry", ["attention", "routed", "host_kv"])
def test_entry_points_allocate_on_the_stream_they_launch_on(rig, monkeypatch, entry):
    rec, lib, side = rig
    q = _Fake((256, 2, 128), 0x1000)
    out = _Fake((256, 2, 128), 0x2000)
    if entry == "attention":
        kc, vc, sc = _Fake((2, 512, 128), 0x3000), _Fake((2, 512, 128), 0x4000), _Fake((2, 2, 512), 0x5000)
        h3a.h3a_attention(q, kc, vc, sc, out, q_chunk=128, mode="kvi8r")
    elif entry == "routed":
        kb, vb = _Fake((512, 2, 128), 0x3000), _Fake((512, 2, 128), 0x4000)
        store = (_Fake((2, 512, 128), 0x5000), _Fake((2, 512, 128), 0x6000), _Fake((2, 2, 512), 0x7000))
        h3a.h3a_attention_routed(q, kb, vb, store, out, exact_spans=[(0, 64)], q_chunk=128)
    else:
        monkeypatch.setattr(lib, "h3a_attention_host_kv_workspace_bytes", lambda *a: 8192, raising=False)
        host = [types.SimpleNamespace(device=types.SimpleNamespace(type="cpu"), dtype=torch.int8, shape=(2, 512, 128),
                                      is_contiguous=lambda: True, is_pinned=lambda: True, numel=lambda: 1,
                                      data_ptr=lambda: 0x9000) for _ in range(3)]
        h3a.h3a_attention_host_kv(q, *host, out, q_chunk=128, mode="kvi8r")
    allocs = [e for e in rec.events if e[0] == "alloc"]
    assert len(allocs) == 1 and allocs[0][2] is side
    name, args = [c for c in lib.calls if not c[0].endswith("_bytes")][-1]
    assert args[-1] == side.cuda_stream  # the kernels go to the stream the workspace belongs to
