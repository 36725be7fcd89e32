"""Error handling, exactness without reuse, determinism and checkpoint/resume
of the HIP path, through the C ABI."""
from __future__ import annotations

import numpy as np
import pytest

import tracegen as tg
import oracle
from gpu_harness import Runner, say, ensure_lib

pytestmark = pytest.mark.gpu

W = tg.WORKLOADS[2].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=4000, k=200,
                            n_slots=600, steps=8)


def _run(w, sel, reset_each=False, host=None, stop=None):
    import torch
    run = Runner(w, host=host, track_buf=False)
    outs, stats = [], []
    for t in range(stop or w.steps):
        if reset_each:
            run.ctx.reset(run.st.slot_table, run.st.lifetimes)
            run.ctx.t = t
        run.gpu_step(sel[t], tg.queries(w, t))
        outs.append(run.st.out.cpu().numpy().copy())
        stats.append(run.st.stats.n_hit.cpu().numpy().copy())
    torch.cuda.synchronize()
    return run, outs, stats


def test_exact_without_reuse():
    """Emptying the buffer before every step (no reuse at all) changes which
    slots rows land in, but not the attention result: bit-identical output,
    since the kernels accumulate in selection order, not slot order."""
    say("[behaviour] exact without reuse")
    sel = tg.selections(W)
    a, oa, ha = _run(W, sel)
    b, ob_, hb = _run(W, sel, reset_each=True, host=a.host)
    for t in range(W.steps):
        assert np.array_equal(oa[t], ob_[t]), t
        assert (hb[t] == 0).all()
    assert sum(h.sum() for h in ha[1:]) > 0
    a.close(); b.close()


def test_deterministic_repeat():
    say("[behaviour] determinism")
    sel = tg.selections(W)
    a, oa, _ = _run(W, sel)
    b, ob_, _ = _run(W, sel, host=a.host)
    for t in range(W.steps):
        assert np.array_equal(oa[t], ob_[t])
    assert np.array_equal(a.st.slot_table.cpu().numpy(), b.st.slot_table.cpu().numpy())
    assert np.array_equal(a.st.buf_kv.cpu().numpy(), b.st.buf_kv.cpu().numpy())
    a.close(); b.close()


def test_checkpoint_resume():
    """State is slot_table, lifetimes, buffer and the step counter: restoring
    them reproduces the later steps bit for bit."""
    import torch
    say("[behaviour] checkpoint/resume")
    w = W.replace(policy="lru", n_buckets=4, steps=10)
    sel = tg.selections(w)
    run = Runner(w, track_buf=False)
    for t in range(5):
        run.gpu_step(sel[t], tg.queries(w, t))
    snap = (run.st.slot_table.clone(), run.st.lifetimes.clone(), run.st.buf_kv.clone(), run.ctx.t)
    outs = []
    for t in range(5, 10):
        run.gpu_step(sel[t], tg.queries(w, t))
        outs.append((run.st.out.clone(), run.st.slot_table.clone()))
    run.st.slot_table.copy_(snap[0]); run.st.lifetimes.copy_(snap[1]); run.st.buf_kv.copy_(snap[2])
    run.ctx.t = snap[3]
    for i, t in enumerate(range(5, 10)):
        run.gpu_step(sel[t], tg.queries(w, t))
        assert torch.equal(run.st.out, outs[i][0]) and torch.equal(run.st.slot_table, outs[i][1])
    # into a fresh context with its own workspace: no state lives in the
    # library between steps, so the restored arrays and counter suffice
    fresh = Runner(w, host=run.host, track_buf=False)
    fresh.st.slot_table.copy_(snap[0]); fresh.st.lifetimes.copy_(snap[1])
    fresh.st.buf_kv.copy_(snap[2])
    from device_buffer_reuse_amd import avsg
    assert fresh.ctx.rebuild_index(fresh.st.slot_table) == avsg.OK
    fresh.ctx.t = snap[3]
    for i, t in enumerate(range(5, 10)):
        fresh.gpu_step(sel[t], tg.queries(w, t))
        assert torch.equal(fresh.st.out, outs[i][0]) and torch.equal(fresh.st.slot_table, outs[i][1])
    fresh.close()
    run.close()


@pytest.mark.parametrize("kind", ["unsorted", "duplicate", "range", "capacity", "state_dup",
                                  "state_range", "state_life"])
def test_data_errors(kind):
    """A bad unit reports its error, keeps its state and outputs zeros; the
    other units proceed exactly as the oracle says."""
    import torch
    avsg = ensure_lib()
    say("[behaviour] data error %s" % kind)
    w = W.replace(n_q_tokens=2 if kind == "capacity" else 1, overlap_shared=0.0, n_slots=300,
                  steps=3)
    sel = tg.selections(w)
    run = Runner(w)
    for t in range(2):
        run.step_and_compare(t, sel[t], tg.queries(w, t))
    bad = 1
    s2 = sel[2].copy()
    if kind == "unsorted":
        s2[bad, 0, 5], s2[bad, 0, 6] = s2[bad, 0, 6], s2[bad, 0, 5]
    elif kind == "duplicate":
        s2[bad, 0, 6] = s2[bad, 0, 5]
    elif kind == "range":
        s2[bad, 0, -1] = w.n_entries
    elif kind == "capacity":
        pass  # two disjoint-ish lists of 200 over 300 slots
    elif kind.startswith("state"):
        st = run.st.slot_table[bad].cpu().numpy()
        occ = np.nonzero(st >= 0)[0]
        if kind == "state_dup":
            # give a second slot the id of a slot whose entry is selected again
            x = int(np.intersect1d(st[occ], s2[bad, 0])[0])
            other = int(occ[st[occ] != x][0])
            run.st.slot_table[bad, other] = x
            run.ob.slot_tok[bad, other] = x
        elif kind == "state_range":
            run.st.slot_table[bad, int(occ[0])] = w.n_entries + 3
            run.ob.slot_tok[bad, int(occ[0])] = w.n_entries + 3
        else:
            run.st.lifetimes[bad, int(occ[0])] = w.lifetime_L + 1
            run.ob.life[bad, int(occ[0])] = w.lifetime_L + 1
    before = run.st.slot_table.cpu().numpy().copy()
    r, _ = run.step_and_compare(2, s2, tg.queries(w, 2))
    want = {"unsorted": avsg.ERR_UNSORTED, "duplicate": avsg.ERR_UNSORTED, "range": avsg.ERR_RANGE,
            "capacity": avsg.ERR_CAPACITY}.get(kind, avsg.ERR_STATE)
    if kind == "capacity":
        assert (r["status"] == want).all()
    else:
        assert r["status"][bad] == want and (np.delete(r["status"], bad) == 0).all()
    assert np.array_equal(run.st.slot_table[bad].cpu().numpy(), before[bad])
    assert run.ctx.last_error() == want
    assert run.ctx.last_error() == avsg.OK   # cleared
    run.close()


def test_validate_state():
    import torch
    avsg = ensure_lib()
    say("[behaviour] validate_state")
    sel = tg.selections(W)
    run = Runner(W, track_buf=False)
    for t in range(3):
        run.gpu_step(sel[t], tg.queries(W, t))
    assert run.ctx.validate_state(run.st.slot_table, run.st.lifetimes) == avsg.OK
    assert run.ctx.rebuild_index(run.st.slot_table) == avsg.OK
    # a lifetime out of range is a state error, but not of the id map
    lf = run.st.lifetimes[1].cpu().numpy()
    occ1 = np.nonzero(run.st.slot_table[1].cpu().numpy() >= 0)[0]
    run.st.lifetimes[1, int(occ1[0])] = W.lifetime_L + 1
    assert run.ctx.validate_state(run.st.slot_table, run.st.lifetimes) == avsg.ERR_STATE
    assert run.ctx.rebuild_index(run.st.slot_table) == avsg.OK
    run.st.lifetimes[1, int(occ1[0])] = int(lf[occ1[0]])
    # an id held by two slots breaks both
    st = run.st.slot_table[0].cpu().numpy()
    occ = np.nonzero(st >= 0)[0]
    run.st.slot_table[0, int(occ[1])] = int(st[occ[0]])
    assert run.ctx.validate_state(run.st.slot_table, run.st.lifetimes) == avsg.ERR_STATE
    assert run.ctx.rebuild_index(run.st.slot_table) == avsg.ERR_STATE
    # an id past the context as well
    run.st.slot_table[0, int(occ[1])] = W.n_entries
    assert run.ctx.rebuild_index(run.st.slot_table) == avsg.ERR_STATE
    run.close()


def test_not_pinned_rejected():
    import torch
    avsg = ensure_lib()
    say("[behaviour] not pinned")
    cfg = avsg.config_from_workload(W)
    ctx = avsg.Context(cfg)
    st = avsg.State(cfg)
    ctx.reset(st.slot_table, st.lifetimes)
    plain = np.zeros((W.units, W.n_entries, W.row_elems), np.uint16)
    sel = torch.from_numpy(tg.selections(W, steps=1)[0]).cuda()
    q = torch.from_numpy(tg.queries(W, 0).view(np.int16)).cuda()
    with pytest.raises(avsg.AvsgError) as e:
        ctx.step(sel, q, plain.ctypes.data, st.buf_kv, st.slot_table, st.lifetimes, st.out, st.stats)
    assert e.value.status == avsg.ERR_NOT_PINNED
    assert ctx.t == 0
    ctx.close()


def test_profile_events_per_stage():
    """Per-stage event timing: every profiled step reports its match_reserve,
    (absent) gather, attention and combine intervals; profiling does not
    change the results."""
    say("[behaviour] profile events")
    w = W.replace(k=500)   # two attention splits per (unit, token)
    sel = tg.selections(w)
    a, oa, _ = _run(w, sel, stop=3)
    run = Runner(w, host=a.host, track_buf=False)
    run.ctx.profile_begin(3)
    for t in range(3):
        run.gpu_step(sel[t], tg.queries(w, t))
    ms, n = run.ctx.profile_end()
    assert n == 3 and len(ms) == 4
    assert ms[0] > 0 and ms[2] > 0 and ms[3] > 0 and ms[1] >= 0
    assert run.ctx.attn_splits > 1
    assert np.array_equal(run.st.out.cpu().numpy(), oa[2])
    with pytest.raises(Exception):
        run.ctx.profile_end()   # not profiling any more
    run.close()
    a.close()


def test_profile_merge_baseline_phases():
    """The dual-pointer baseline reports the time of its sort and of its walk
    under profiling (both positive, walk and sort within the match stage);
    the hash modes report none; profiling it does not change its results."""
    say("[behaviour] profile merge phases")
    sel = tg.selections(W)
    a, oa, _ = _run(W, sel, stop=3)
    run = Runner(W, host=a.host, track_buf=False)
    run.ctx.set_match_mode(avsg_match_merge())
    run.ctx.profile_begin(3)
    for t in range(3):
        run.gpu_step(sel[t], tg.queries(W, t))
    ms, n = run.ctx.profile_end()
    sort_ms, walk_ms = run.ctx.profile_match_phases()
    assert n == 3 and sort_ms > 0 and walk_ms > 0
    assert sort_ms + walk_ms < ms[0]
    assert np.array_equal(run.st.out.cpu().numpy(), oa[2])
    run.ctx.set_match_mode(0)
    run.ctx.profile_begin(1)
    run.gpu_step(sel[3], tg.queries(W, 3))
    run.ctx.profile_end()
    assert run.ctx.profile_match_phases() == (0.0, 0.0)
    assert run.ctx.last_error() == 0
    run.close()
    a.close()


def avsg_match_merge():
    from device_buffer_reuse_amd import avsg
    return avsg.MATCH_MERGE


def test_new_entry_points_reject_bad_arguments():
    """Argument errors of the append, the variable-length step and the
    capacity call are reported synchronously and enqueue nothing."""
    import ctypes
    import torch
    avsg = ensure_lib()
    say("[behaviour] argument errors of append / varlen / capacity")
    cfg = avsg.config_from_workload(W)
    ctx = avsg.Context(cfg)
    st = avsg.State(cfg)
    ctx.reset(st.slot_table, st.lifetimes)
    host = avsg.HostBuffer((W.units, W.n_entries, W.row_elems))
    plain = np.zeros((W.units, W.n_entries, W.row_elems), np.uint16)
    new = torch.zeros((W.units, W.head_dim_qk + W.head_dim_v), dtype=torch.int16, device="cuda")
    pos = torch.zeros(W.batch, dtype=torch.int32, device="cuda")
    lib = avsg.load()
    # unpinned host memory, a misaligned token, null pointers
    assert lib.avsg_append(ctx.handle, new.data_ptr(), pos.data_ptr(), plain.ctypes.data,
                           st.buf_kv.data_ptr(), st.slot_table.data_ptr()) == avsg.ERR_NOT_PINNED
    assert lib.avsg_append(ctx.handle, new.data_ptr() + 2, pos.data_ptr(), host.ptr,
                           st.buf_kv.data_ptr(), st.slot_table.data_ptr()) == avsg.ERR_INVALID_ARG
    assert lib.avsg_append(ctx.handle, None, pos.data_ptr(), host.ptr, st.buf_kv.data_ptr(),
                           st.slot_table.data_ptr()) == avsg.ERR_INVALID_ARG
    # the variable-length step needs its length array
    sel = torch.from_numpy(tg.selections(W, steps=1)[0]).cuda()
    q = torch.from_numpy(tg.queries(W, 0).view(np.int16)).cuda()
    hs = st.stats.struct()
    assert lib.avsg_step_varlen(ctx.handle, sel.data_ptr(), None, q.data_ptr(), host.ptr,
                                st.buf_kv.data_ptr(), st.slot_table.data_ptr(),
                                st.lifetimes.data_ptr(), st.out.data_ptr(),
                                ctypes.byref(hs)) == avsg.ERR_INVALID_ARG
    assert lib.avsg_set_capacity(None, None) == avsg.ERR_INVALID_ARG
    assert ctx.t == 0
    assert ctx.last_error() == avsg.OK
    ctx.close()
    host.free()
