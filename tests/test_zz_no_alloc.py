"""avsg_step_static (no context, no caller workspace: the library's own
device array) against avsg_step through the C ABI, on the same seeded inputs:
slot state, buffer bytes, hit statistics and attention outputs must be
bit-identical, over consecutive calls whose sizes change (each later call
smaller than the one before, so stale contents of the shared array would
show).  Also: a configuration whose scratch exceeds the array is refused
before anything runs, and a missing per-unit status array is an argument
error."""
from __future__ import annotations

import numpy as np
import pytest

import tracegen as tg
from gpu_harness import ensure_lib, say

pytestmark = pytest.mark.gpu

# largest scratch first, each later one smaller (0.5 MB .. 4 KB)
SEQUENCE = [
    ("latent", tg.WORKLOADS[5].replace(batch=2, n_entries=3001, k=90, n_slots=300), 3),
    ("token", tg.WORKLOADS[2].replace(batch=3, n_kv_heads=2, n_q_heads=8, n_entries=5003, k=300,
                                      n_slots=1000), 4),
    ("mtp", tg.WORKLOADS[3].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=5003, k=200,
                                    n_slots=700), 3),
    ("lru_pages", tg.WORKLOADS[4].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=1001,
                                          k=37, n_slots=100), 4),
    ("token_small", tg.WORKLOADS[2].replace(batch=1, n_kv_heads=1, n_q_heads=4, n_entries=600,
                                            k=40, n_slots=64), 3),
]


def _state(avsg, cfg, lru):
    st = avsg.State(cfg)
    if lru:
        st.lifetimes.fill_(-1)   # an empty LRU buffer: stamps -1
    return st


def _same(a, b, what):
    assert a.shape == b.shape and bool((a == b).all()), what


def test_static_step_equals_context_step():
    import torch
    avsg = ensure_lib()
    sizes = [avsg.avsg_workspace_bytes(avsg.config_from_workload(w)) for _, w, _ in SEQUENCE]
    assert all(x > y for x, y in zip(sizes, sizes[1:])), sizes
    stream = torch.cuda.current_stream().cuda_stream
    for name, w, steps in SEQUENCE:
        say("[no-alloc] %s units=%d k=%d S=%d steps=%d" % (name, w.units, w.k, w.n_slots, steps))
        cfg = avsg.config_from_workload(w)
        assert avsg.avsg_workspace_bytes(cfg) <= avsg.STATIC_SCRATCH_BYTES
        host = avsg.HostBuffer((w.units, w.n_entries, w.row_elems))
        tg.fill_kv(w, out=host.array)
        sel = tg.selections(w, steps=steps)
        ctx = avsg.Context(cfg)
        a = _state(avsg, cfg, w.policy == "lru")
        b = _state(avsg, cfg, w.policy == "lru")
        ctx.reset(a.slot_table, a.lifetimes)
        try:
            for t in range(steps):
                s_dev = torch.from_numpy(sel[t]).cuda()
                q_dev = torch.from_numpy(tg.queries(w, t).view(np.int16)).cuda()
                ctx.step(s_dev, q_dev, host, a.buf_kv, a.slot_table, a.lifetimes, a.out, a.stats)
                st = avsg.avsg_step_static(cfg, t, stream, s_dev.data_ptr(), q_dev.data_ptr(),
                                           host.ptr, b.buf_kv.data_ptr(), b.slot_table.data_ptr(),
                                           b.lifetimes.data_ptr(), b.out.data_ptr(),
                                           b.stats.struct())
                assert st == avsg.OK, avsg.status_string(st)
                torch.cuda.synchronize()
                what = "%s t=%d" % (name, t)
                _same(a.slot_table, b.slot_table, what + " slot_table")
                _same(a.lifetimes, b.lifetimes, what + " lifetimes")
                _same(a.buf_kv, b.buf_kv, what + " buf_kv")
                _same(a.out, b.out, what + " out")
                for f in ("hit_flag", "sel_slot", "n_hit", "n_miss", "n_evict", "unit_status"):
                    _same(getattr(a.stats, f), getattr(b.stats, f), what + " " + f)
                assert int(b.stats.unit_status.abs().sum()) == 0
                assert t == 0 or int(b.stats.n_hit.sum()) > 0
            assert ctx.last_error() == avsg.OK
        finally:
            ctx.close()
            host.free()


def test_static_step_refuses_what_does_not_fit():
    avsg = ensure_lib()
    import torch
    # twice the latent workload's requests: its split partials alone exceed the array
    w = tg.WORKLOADS[5].replace(batch=128)
    cfg = avsg.config_from_workload(w)
    assert avsg.avsg_workspace_bytes(cfg) > avsg.STATIC_SCRATCH_BYTES
    hs = avsg.avsg_hit_stats(1, 1, 1, 1, 1, 1)   # never dereferenced: refused before any use
    st = avsg.avsg_step_static(cfg, 0, 0, 1, 1, 1, 1, 1, 1, 1, hs)
    assert st == avsg.ERR_UNSUPPORTED
    # no per-unit status array: nowhere to report data errors
    w = SEQUENCE[-1][1]
    cfg = avsg.config_from_workload(w)
    hs = avsg.avsg_hit_stats(1, 1, 1, 1, 1, None)
    assert avsg.avsg_step_static(cfg, 0, 0, 1, 1, 1, 1, 1, 1, 1, hs) == avsg.ERR_INVALID_ARG
    # a negative step counter
    hs = avsg.avsg_hit_stats(1, 1, 1, 1, 1, 1)
    assert avsg.avsg_step_static(cfg, -1, 0, 1, 1, 1, 1, 1, 1, 1, hs) == avsg.ERR_INVALID_ARG
    torch.cuda.synchronize()
