"""HostBuffer.free() returns pinned memory only once no numpy array views it
(a traceback that keeps a view of a freed buffer would otherwise read freed
memory while a failure is reported).  CPU only: the allocation is replaced by
a ctypes buffer and the release is recorded."""
from __future__ import annotations

import ctypes

import numpy as np

from device_buffer_reuse_amd import avsg


def _fake(nbytes=64):
    hb = avsg.HostBuffer.__new__(avsg.HostBuffer)
    hb._raw = (ctypes.c_char * nbytes)()
    hb.ptr = ctypes.addressof(hb._raw)
    hb.shape, hb.dtype, hb.nbytes = (4, nbytes // 8), np.dtype(np.uint16), nbytes
    hb.array = np.frombuffer(hb._raw, dtype=np.uint16).reshape(hb.shape)
    return hb


def test_free_waits_for_views(monkeypatch):
    freed = []
    monkeypatch.setattr(avsg, "avsg_host_free", lambda p: freed.append(p) or 0)
    monkeypatch.setattr(avsg, "_pending_host_frees", [])
    a, b = _fake(), _fake()
    view = a.array[1][2:]          # a view of a view
    copy = b.array.copy()          # owns its memory
    pa, pb = a.ptr, b.ptr
    a.free()
    b.free()
    assert freed == [pb] and a.ptr is None and a.array is None
    assert view.sum() == 0         # still readable: not yet released
    del view
    a.free()                       # a later call retries the release
    assert sorted(freed) == sorted([pa, pb])
    assert avsg._pending_host_frees == []
    assert copy.shape == (4, 8)
