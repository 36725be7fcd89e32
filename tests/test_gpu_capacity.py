"""Per-unit buffer sizes (avsg_set_capacity) on the GPU vs the oracle,
through the C ABI.  Capacities change between steps: constant below S,
shrinking below the occupied slots (their entries are dropped), growing
again, and out of range or below |U| for one unit (a data error of that unit
only).  State, buffer bytes and attention must match the oracle."""
from __future__ import annotations

import numpy as np
import pytest

import tracegen as tg
from gpu_harness import Runner, say, ensure_lib

pytestmark = pytest.mark.gpu

CASES = {
    "token": tg.WORKLOADS[2].replace(batch=3, n_kv_heads=2, n_q_heads=8, n_entries=5003, k=300,
                                     n_slots=1000, steps=12),
    "mtp": tg.WORKLOADS[3].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=5003, k=300,
                                   n_slots=700, steps=10),
    "lru_pages": tg.WORKLOADS[4].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=1001, k=37,
                                         n_slots=100, steps=14),
    "latent": tg.WORKLOADS[5].replace(batch=3, n_entries=5003, k=700, n_slots=1500, steps=8),
    "slots_16k": tg.WORKLOADS[2].replace(batch=1, n_kv_heads=2, n_q_heads=8, n_entries=40000,
                                         k=2000, n_slots=16384, steps=6),
}


def _caps(w, t, rng, union):
    """Step t's capacities: full, then random sizes between |U| and S, with a
    deep shrink (to |U|) on step 3 and back to S on step 5."""
    S = w.n_slots
    if t < 2:
        return np.full(w.units, S, np.int32)
    if t == 3:
        return union.astype(np.int32)
    if t == 5:
        return np.full(w.units, S, np.int32)
    return rng.integers(union, S + 1).astype(np.int32)


def _union_sizes(sel_t):
    return np.array([len(np.unique(sel_t[u])) for u in range(sel_t.shape[0])])


@pytest.mark.parametrize("name", list(CASES))
def test_capacity_parity(name):
    w = CASES[name]
    say("[capacity] %s units=%d S=%d" % (name, w.units, w.n_slots))
    sel = tg.selections(w)
    rng = np.random.default_rng(len(name))
    run = Runner(w)
    try:
        for t in range(w.steps):
            run.set_caps(_caps(w, t, rng, _union_sizes(sel[t])))
            run.step_and_compare(t, sel[t], tg.queries(w, t), check_buf=True)
            st = run.st.slot_table.cpu().numpy()
            for u in range(w.units):
                assert (st[u, run.caps[u]:] == -1).all()
        assert run.ctx.last_error() == 0
    finally:
        run.close()


@pytest.mark.parametrize("mode", ["merge", "hash_table"])
def test_capacity_match_modes(mode):
    avsg = ensure_lib()
    w = CASES["token"].replace(steps=7)
    say("[capacity] %s" % mode)
    sel = tg.selections(w)
    rng = np.random.default_rng(4)
    run = Runner(w)
    run.ctx.set_match_mode(avsg.MATCH_MERGE if mode == "merge" else avsg.MATCH_HASH_TABLE)
    try:
        for t in range(w.steps):
            run.set_caps(_caps(w, t, rng, _union_sizes(sel[t])))
            run.step_and_compare(t, sel[t], tg.queries(w, t), check_buf=True)
    finally:
        run.close()


def test_capacity_errors_are_unit_errors():
    avsg = ensure_lib()
    w = CASES["token"].replace(steps=5)
    say("[capacity] errors")
    sel = tg.selections(w)
    run = Runner(w)
    try:
        run.step_and_compare(0, sel[0], tg.queries(w, 0), check_buf=True)
        for t, bad, want in ((1, 0, avsg.ERR_RANGE), (2, w.n_slots + 1, avsg.ERR_RANGE),
                             (3, w.k - 1, avsg.ERR_CAPACITY), (4, w.k, avsg.OK)):
            caps = np.full(w.units, w.n_slots, np.int32)
            caps[1] = bad
            run.set_caps(caps)
            r, _ = run.step_and_compare(t, sel[t], tg.queries(w, t), check_buf=True)
            assert r["status"][1] == want and (np.delete(r["status"], 1) == 0).all()
            assert run.ctx.last_error() == want
        run.set_caps(None)
    finally:
        run.close()


def test_state_error_with_shrink_keeps_state():
    """A duplicated id of U in one unit while every unit's buffer shrinks:
    that unit reports a state error and keeps all of its slots, the ones
    past its size included (the error takes precedence over the shrink);
    the other units shrink and step as the oracle says."""
    avsg = ensure_lib()
    w = CASES["token"].replace(steps=3)
    say("[capacity] state error with a shrink")
    sel = tg.selections(w)
    run = Runner(w)
    try:
        for t in range(2):
            run.step_and_compare(t, sel[t], tg.queries(w, t), check_buf=True)
        bad = 1
        st = run.st.slot_table[bad].cpu().numpy()
        occ = np.nonzero(st >= 0)[0]
        cap = w.k + 10
        assert occ.max() >= cap, "an occupied slot past the new size"
        below = occ[occ < cap]
        x = int(np.intersect1d(st[below], sel[2][bad, 0])[0])
        other = int(below[st[below] != x][0])
        run.st.slot_table[bad, other] = x
        run.ob.slot_tok[bad, other] = x
        before = (run.st.slot_table[bad].cpu().numpy().copy(),
                  run.st.lifetimes[bad].cpu().numpy().copy())
        run.set_caps(np.full(w.units, cap, np.int32))
        r, _ = run.step_and_compare(2, sel[2], tg.queries(w, 2), check_buf=True)
        assert r["status"][bad] == avsg.ERR_STATE and (np.delete(r["status"], bad) == 0).all()
        assert np.array_equal(run.st.slot_table[bad].cpu().numpy(), before[0])
        assert np.array_equal(run.st.lifetimes[bad].cpu().numpy(), before[1])
        good = run.st.slot_table.cpu().numpy()[np.arange(w.units) != bad]
        assert (good[:, cap:] == -1).all()
        assert run.ctx.last_error() == avsg.ERR_STATE
        run.set_caps(None)
    finally:
        run.close()


def test_plan_then_step():
    """The planner's capacities for the next step's unions, then the step."""
    avsg = ensure_lib()
    from oracle.plan import plan_capacity
    w = CASES["token"].replace(steps=6)
    say("[capacity] planned")
    sel = tg.selections(w)
    run = Runner(w)
    reuse = np.zeros(w.units, np.int32)
    try:
        for t in range(w.steps):
            demand = _union_sizes(sel[t]).astype(np.int32)
            budget = int(demand.sum() + 0.3 * w.units * (w.n_slots - w.k))
            st, caps = avsg.avsg_plan_capacity(demand, reuse, budget, w.n_slots)
            assert st == avsg.OK
            assert np.array_equal(caps, plan_capacity(demand, reuse, budget, w.n_slots))
            run.set_caps(caps)
            r, _ = run.step_and_compare(t, sel[t], tg.queries(w, t), check_buf=True)
            reuse = r["n_hit"].astype(np.int32)
    finally:
        run.close()


def test_lengths_capacity_and_appends_together():
    """Variable list lengths, changing buffer sizes and appends interleaved
    over one trace, on paged entries under the LRU policy: every step's
    state, buffer bytes and attention against the oracle."""
    import torch
    from oracle import append as oapp
    w = CASES["lru_pages"].replace(steps=12)
    say("[capacity] lengths + sizes + appends")
    sel, lens = tg.shorten(tg.selections(w), 11, 1)
    rng = np.random.default_rng(12)
    run = Runner(w)
    try:
        for t in range(w.steps):
            caps = rng.integers(lens[t], w.n_slots + 1).astype(np.int32)
            if t == 6:
                caps = lens[t].astype(np.int32)   # shrink to the mandatory slots
            run.set_caps(caps)
            run.step_and_compare(t, sel[t], tg.queries(w, t), check_buf=True, lengths=lens[t])
            # every request appends a token into an entry its first head holds
            pos = np.array([sel[t, b * w.n_kv_heads, 0, 0] * w.tokens_per_entry + t % 16
                            for b in range(w.batch)], np.int32)
            x = rng.standard_normal((w.units, w.head_dim_qk + w.head_dim_v)).astype(np.float32)
            new = (x.view(np.uint32) >> 16).astype(np.uint16)
            ref_host = run.host.array.copy()
            oapp.append(w, ref_host, new, pos, run.ob.slot_tok, run.ob.buf)
            run.ctx.append(torch.from_numpy(new.view(np.int16)).cuda(), torch.from_numpy(pos).cuda(),
                           run.host, run.st.buf_kv, run.st.slot_table)
            torch.cuda.synchronize()
            assert np.array_equal(run.host.array, ref_host)
            assert np.array_equal(run.st.buf_kv.cpu().numpy().view(np.uint16), run.ob.buf)
        assert run.ctx.last_error() == 0
    finally:
        run.close()
        run.host.free()
