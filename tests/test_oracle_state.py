"""Pins of the oracle's slot-buffer state machine against things other than
itself: hand-worked traces, an independent brute-force replay, closed forms
and step invariants.  CPU only."""
from __future__ import annotations

import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st, HealthCheck

import oracle
import tracegen as tg
from bruteforce import BruteBuffer
from invariants import check_unit_step, check_buffer

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _parse_golden(path):
    cfg, steps = None, []
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        head, rest = line.split(" ", 1)
        if head == "config":
            cfg = {}
            for kv in rest.split():
                k, v = kv.split("=")
                cfg[k] = v if k == "policy" else int(v)
        elif head == "step":
            toks = rest.split()
            assert toks[0] == "sel"
            lists = [[int(x) for x in part.split()] for part in " ".join(toks[1:]).split("|")]
            steps.append({"sel": lists})
        elif head == "expect":
            d = steps[-1]
            words = rest.replace("|", " | ").split()
            i = 0
            while i < len(words):
                key = words[i]
                i += 1
                if key in ("hit", "slot"):
                    vals, cur = [], []
                    while i < len(words) and (words[i] == "|" or words[i].lstrip("-").isdigit()):
                        if words[i] == "|":
                            vals.append(cur)
                            cur = []
                        else:
                            cur.append(int(words[i]))
                        i += 1
                    vals.append(cur)
                    d[key] = vals
                else:
                    d[key] = int(words[i])
                    i += 1
        elif head == "state":
            words = rest.split()
            S = cfg["S"]
            assert words[0] == "tok" and words[S + 1] == "life"
            steps[-1]["tok"] = [int(x) for x in words[1:S + 1]]
            steps[-1]["life"] = [int(x) for x in words[S + 2:2 * S + 2]]
    return cfg, steps


@pytest.mark.parametrize("name", ["lifetime_s4.txt", "lru_b2_s3.txt", "mtp_s4.txt"])
def test_golden_hand_worked(name):
    cfg, steps = _parse_golden(os.path.join(GOLDEN, name))
    S = cfg["S"]
    tok = np.full(S, -1, np.int32)
    life = np.full(S, -1 if cfg["policy"] == "lru" else 0, np.int32)
    bb = BruteBuffer(S, cfg["N"], cfg["L"], cfg["B"], cfg["policy"])
    for t, d in enumerate(steps):
        sel = np.array(d["sel"], np.int32)
        st_, r = oracle.unit_step(S, cfg["N"], cfg["k"], cfg["policy"], cfg["L"], cfg["B"], t, sel,
                                  tok, life)
        assert st_ == oracle.OK
        assert r["hit_flag"].tolist() == d["hit"], (name, t)
        assert r["sel_slot"].tolist() == d["slot"], (name, t)
        assert (r["n_hit"], r["n_miss"], r["n_evict"]) == (d["n_hit"], d["n_miss"], d["n_evict"])
        assert tok.tolist() == d["tok"], (name, t)
        assert life.tolist() == d["life"], (name, t)
        # the brute force agrees with the hand-worked values too
        flags, slots, cnt = bb.step(d["sel"])
        assert [[int(x) for x in f] for f in flags] == d["hit"]
        assert slots == d["slot"]
        assert bb.tok == d["tok"] and bb.life_array() == d["life"]


def _random_trace(rng, S, N, k, T, steps, overlap):
    """Sorted random selections with some step-to-step overlap (test-local)."""
    out = []
    prev = None
    for t in range(steps):
        lists = []
        for j in range(T):
            if prev is not None and rng.random() < overlap:
                keep = rng.choice(prev, size=min(len(prev), k // 2), replace=False)
                rest = rng.choice(np.setdiff1d(np.arange(N), keep), size=k - keep.size, replace=False)
                lst = np.sort(np.concatenate([keep, rest]))
            else:
                lst = np.sort(rng.choice(N, size=k, replace=False))
            lists.append(lst.astype(np.int32))
        prev = lists[0]
        out.append(np.stack(lists))
    return out


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(seed=st.integers(0, 2**31 - 1), S=st.integers(4, 32), N=st.integers(8, 256),
       T=st.integers(1, 2), policy=st.sampled_from(["lifetime", "lru"]),
       L=st.integers(1, 6), B=st.integers(1, 6), W=st.integers(1, 4))
def test_oracle_matches_bruteforce(seed, S, N, T, policy, L, B, W):
    rng = np.random.default_rng(seed)
    k = int(rng.integers(1, max(2, min(S // T, N // 2)) + 1))
    k = max(1, min(k, S // T, N // 2))
    steps = 12
    trace = _random_trace(rng, S, N, k, T, steps, overlap=0.6)
    tok = np.full(S, -1, np.int32)
    life = np.full(S, -1 if policy == "lru" else 0, np.int32)
    bb = BruteBuffer(S, N, L, B, policy, W)
    for t, sel in enumerate(trace):
        st_, r = oracle.unit_step(S, N, k, policy, L, B, t, sel, tok, life, bucket_width=W)
        assert st_ == oracle.OK
        flags, slots, cnt = bb.step([list(map(int, l)) for l in sel])
        assert r["hit_flag"].astype(bool).tolist() == flags
        assert r["sel_slot"].tolist() == slots
        assert (r["n_hit"], r["n_miss"], r["n_evict"], r["n_union"]) == \
            (cnt["n_hit"], cnt["n_miss"], cnt["n_evict"], cnt["n_union"])
        assert tok.tolist() == bb.tok
        assert life.tolist() == bb.life_array()


def test_step0_closed_form():
    """Empty buffer: every entry misses and slot r takes the r-th smallest id."""
    S, N, k = 64, 1000, 40
    rng = np.random.default_rng(1)
    sel = np.sort(rng.choice(N, k, replace=False)).astype(np.int32)
    tok = np.full(S, -1, np.int32)
    life = np.zeros(S, np.int32)
    st_, r = oracle.unit_step(S, N, k, "lifetime", 5, 64, 0, sel, tok, life)
    assert st_ == 0 and r["n_miss"] == k and r["n_hit"] == 0 and r["n_evict"] == 0
    assert r["sel_slot"][0].tolist() == list(range(k))
    assert tok[:k].tolist() == sel.tolist() and (tok[k:] == -1).all()


@pytest.mark.parametrize("policy", ["lifetime", "lru"])
def test_repeat_selection_all_hits(policy):
    """Selecting the same set again hits fully and reserves nothing."""
    S, N, k = 32, 200, 16
    sel = np.arange(3, 3 + 2 * k, 2, dtype=np.int32)
    tok = np.full(S, -1, np.int32)
    life = np.full(S, -1 if policy == "lru" else 0, np.int32)
    oracle.unit_step(S, N, k, policy, 4, 64, 0, sel, tok, life)
    before = tok.copy()
    st_, r = oracle.unit_step(S, N, k, policy, 4, 64, 1, sel, tok, life)
    assert st_ == 0 and r["n_hit"] == k and r["n_miss"] == 0 and r["fill_slot"].size == 0
    assert np.array_equal(tok, before) and r["hit_flag"].all()


def test_lifetime_closed_form_age():
    """A slot filled at step t0 and never selected again has lifetime
    max(L - age, 0) until it is evicted."""
    S, N, L = 8, 100, 5
    tok = np.full(S, -1, np.int32)
    life = np.zeros(S, np.int32)
    oracle.unit_step(S, N, 1, "lifetime", L, 64, 0, np.array([7], np.int32), tok, life)
    s7 = int(np.nonzero(tok == 7)[0][0])
    for t in range(1, 7):   # 6 more steps with fresh ids, buffer never full
        oracle.unit_step(S, N, 1, "lifetime", L, 64, t, np.array([10 + t], np.int32), tok, life)
        assert life[s7] == max(L - t, 0)


def test_lifetime_L64_equals_lru_B64():
    """With bucket width one step, a 64-bucket LRU orders candidates exactly
    like lifetime management with L = 64 (life = 63 - bucket), so both
    policies produce the same slots on any trace."""
    w = tg.WORKLOADS[1].replace(n_slots=300, k=128, steps=40)
    sel = tg.selections(w)
    a = oracle.OracleBuffer(w.n_slots, w.n_entries, 1, w.k, "lifetime", 64, 64, 1)
    b = oracle.OracleBuffer(w.n_slots, w.n_entries, 1, w.k, "lru", 64, 64, 1)
    for t in range(w.steps):
        ra, rb = a.step(sel[t]), b.step(sel[t])
        assert np.array_equal(ra["sel_slot"], rb["sel_slot"])
        assert np.array_equal(a.slot_tok, b.slot_tok)
        assert ra["n_evict"][0] == rb["n_evict"][0]


def test_reset_every_step_all_miss():
    """Without reuse (buffer cleared before each step) every entry misses;
    the selections, and so the attention inputs, are unchanged."""
    w = tg.WORKLOADS[1]
    sel = tg.selections(w, steps=6)
    ob = oracle.OracleBuffer.for_workload(w)
    for t in range(6):
        ob.reset()
        r = ob.step(sel[t])
        assert r["n_hit"][0] == 0 and r["n_miss"][0] == w.k
        assert (ob.slot_tok[0][r["sel_slot"][0, 0]] == sel[t, 0, 0]).all()


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_invariants_on_workloads(cid):
    """I1-I9 on every step of each workload (first units only for size)."""
    w = tg.WORKLOADS[cid]
    nunits = min(w.units, 4)
    steps = min(w.steps, 48)
    sel = tg.selections(w, steps=steps)[:, :nunits]
    track = cid in (1, 2, 3)
    host = None
    if track:
        host = tg.fill_kv(w, units=nunits)
    ob = oracle.OracleBuffer.for_workload(w, track_buf=track, units=nunits)
    prev_union = [None] * nunits
    keep = int(np.floor(w.overlap * w.k + 0.5))
    for t in range(steps):
        ptok, plife = ob.slot_tok.copy(), ob.life.copy()
        r = ob.step(np.ascontiguousarray(sel[t]), host)
        for u in range(nunits):
            assert r["status"][u] == 0
            un = check_unit_step(sel[t, u], ptok[u], plife[u], ob.slot_tok[u], ob.life[u],
                                 r["hit_flag"][u], r["sel_slot"][u], r["n_hit"][u], r["n_miss"][u],
                                 r["n_evict"][u], w.lifetime_L, w.policy, t, prev_union[u],
                                 r["fill_slot"][u])
            if t > 0:
                # the generator keeps exactly round(f*k) of token 0's last list
                assert r["n_hit"][u] >= keep
            prev_union[u] = un
            if track:
                check_buffer(ob.buf[u], ob.slot_tok[u], host[u])


def _fresh(S, policy):
    return np.full(S, -1, np.int32), np.full(S, -1 if policy == "lru" else 0, np.int32)


@pytest.mark.parametrize("sel,code", [
    ([[3, 2, 9]], oracle.ERR_UNSORTED),
    ([[2, 2, 9]], oracle.ERR_UNSORTED),
    ([[1, 2, 16]], oracle.ERR_RANGE),
    ([[-1, 2, 9]], oracle.ERR_RANGE),
    ([[5, 3, 99]], oracle.ERR_RANGE),      # range wins over order
])
def test_errors_input(sel, code):
    S, N = 8, 16
    tok, life = _fresh(S, "lifetime")
    tok[0], life[0] = 4, 3
    t0, l0 = tok.copy(), life.copy()
    st_, r = oracle.unit_step(S, N, 3, "lifetime", 4, 64, 1, np.array(sel, np.int32), tok, life)
    assert st_ == code
    assert np.array_equal(tok, t0) and np.array_equal(life, l0)
    assert (r["sel_slot"] == -1).all() and not r["hit_flag"].any() and r["n_miss"] == 0


def test_error_capacity():
    S, N = 4, 32
    tok, life = _fresh(S, "lifetime")
    sel = np.array([[1, 2, 3], [4, 5, 6]], np.int32)   # union of 6 > 4 slots
    st_, r = oracle.unit_step(S, N, 3, "lifetime", 4, 64, 0, sel, tok, life)
    assert st_ == oracle.ERR_CAPACITY and (tok == -1).all()


@pytest.mark.parametrize("mut", ["dup_in_U", "tok_range", "life_range", "stamp_future"])
def test_error_state(mut):
    S, N = 6, 32
    pol = "lru" if mut == "stamp_future" else "lifetime"
    tok, life = _fresh(S, pol)
    oracle.unit_step(S, N, 3, pol, 4, 64, 0, np.array([[1, 5, 9]], np.int32), tok, life)
    if mut == "dup_in_U":
        tok[4] = 5
        life[4] = 1
    elif mut == "tok_range":
        tok[4] = 40
    elif mut == "life_range":
        life[0] = 9
    elif mut == "stamp_future":
        life[0] = 7
    t0, l0 = tok.copy(), life.copy()
    st_, r = oracle.unit_step(S, N, 3, pol, 4, 64, 1, np.array([[1, 5, 20]], np.int32), tok, life)
    assert st_ == oracle.ERR_STATE
    assert np.array_equal(tok, t0) and np.array_equal(life, l0)


def test_duplicate_outside_union_is_not_an_error():
    """A duplicated id that this step does not select does not change this
    step's result, so it is left to the explicit state validation."""
    S, N = 6, 32
    tok, life = _fresh(S, "lifetime")
    oracle.unit_step(S, N, 3, "lifetime", 4, 64, 0, np.array([[1, 5, 9]], np.int32), tok, life)
    tok[4], life[4] = 9, 1
    st_, _ = oracle.unit_step(S, N, 2, "lifetime", 4, 64, 1, np.array([[1, 5]], np.int32), tok, life)
    assert st_ == oracle.OK


@settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(seed=st.integers(0, 2**31 - 1), S=st.integers(4, 32), N=st.integers(8, 256),
       T=st.integers(1, 2), policy=st.sampled_from(["lifetime", "lru"]),
       L=st.integers(1, 6), B=st.integers(1, 6))
def test_oracle_variable_lengths_match_bruteforce(seed, S, N, T, policy, L, B):
    """Lists shorter than k (PSA abstract: per-token budgets instead of one
    fixed k): only the first len entries of each list count; the padding
    after them (here ids out of range and out of order) is ignored and its
    outputs stay slot -1, flag 0.  The brute-force replay sees only the
    shortened lists."""
    rng = np.random.default_rng(seed)
    k = max(1, min(int(rng.integers(1, max(2, S // T) + 1)), S // T, N // 2))
    trace = _random_trace(rng, S, N, k, T, 12, overlap=0.6)
    tok = np.full(S, -1, np.int32)
    life = np.full(S, -1 if policy == "lru" else 0, np.int32)
    bb = BruteBuffer(S, N, L, B, policy)
    for t, sel in enumerate(trace):
        lens = rng.integers(1, k + 1, size=T).astype(np.int32)
        padded = sel.copy()
        for j in range(T):
            padded[j, lens[j]:] = rng.integers(-5, N + 5, size=k - lens[j])
            # a shortened list keeps its first len ids (ascending)
        st_, r = oracle.unit_step(S, N, k, policy, L, B, t, padded, tok, life, lengths=lens)
        assert st_ == oracle.OK
        lists = [list(map(int, sel[j, :lens[j]])) for j in range(T)]
        flags, slots, cnt = bb.step(lists)
        for j in range(T):
            assert r["hit_flag"][j, :lens[j]].astype(bool).tolist() == flags[j]
            assert r["sel_slot"][j, :lens[j]].tolist() == slots[j]
            assert (r["sel_slot"][j, lens[j]:] == -1).all() and (r["hit_flag"][j, lens[j]:] == 0).all()
        assert (r["n_hit"], r["n_miss"], r["n_evict"], r["n_union"]) == \
            (cnt["n_hit"], cnt["n_miss"], cnt["n_evict"], cnt["n_union"])
        assert tok.tolist() == bb.tok
        assert life.tolist() == bb.life_array()


def test_oracle_length_out_of_range_is_an_error():
    S, N, k = 16, 100, 5
    sel = np.array([[3, 9, 20, 41, 77]], np.int32)
    for bad in (0, -1, k + 1):
        tok = np.full(S, -1, np.int32)
        life = np.zeros(S, np.int32)
        st_, r = oracle.unit_step(S, N, k, "lifetime", 4, 64, 0, sel, tok, life,
                                  lengths=np.array([bad]))
        assert st_ == oracle.ERR_RANGE
        assert (tok == -1).all() and (r["sel_slot"] == -1).all()
    # all k in use is the fixed-length step
    tok_a, life_a = np.full(S, -1, np.int32), np.zeros(S, np.int32)
    tok_b, life_b = np.full(S, -1, np.int32), np.zeros(S, np.int32)
    _, ra = oracle.unit_step(S, N, k, "lifetime", 4, 64, 0, sel, tok_a, life_a)
    _, rb = oracle.unit_step(S, N, k, "lifetime", 4, 64, 0, sel, tok_b, life_b,
                             lengths=np.array([k]))
    assert np.array_equal(tok_a, tok_b) and np.array_equal(ra["sel_slot"], rb["sel_slot"])


@settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(seed=st.integers(0, 2**31 - 1), S=st.integers(6, 32), N=st.integers(16, 256),
       policy=st.sampled_from(["lifetime", "lru"]), L=st.integers(1, 6), B=st.integers(1, 6))
def test_oracle_capacity_matches_bruteforce(seed, S, N, policy, L, B):
    """Per-unit capacity (Spin summary, section 2B: buffer elasticity): with
    capacity c the unit behaves as a buffer of c slots, slots past c stay
    empty, and a shrink empties the slots it removes before the step.  The
    brute-force replay runs on the first c slots, its tail emptied by hand."""
    rng = np.random.default_rng(seed)
    k = max(1, min(int(rng.integers(1, S // 2 + 1)), N // 2))
    trace = _random_trace(rng, S, N, k, 1, 14, overlap=0.6)
    tok = np.full(S, -1, np.int32)
    reset = -1 if policy == "lru" else 0
    life = np.full(S, reset, np.int32)
    bb = BruteBuffer(S, N, L, B, policy)
    for t, sel in enumerate(trace):
        cap = int(rng.integers(k, S + 1))
        for s in range(cap, S):
            bb.tok[s], bb.last[s] = -1, None
        bb.S = cap
        st_, r = oracle.unit_step(S, N, k, policy, L, B, t, sel, tok, life, cap=cap)
        assert st_ == oracle.OK
        flags, slots, cnt = bb.step([list(map(int, l)) for l in sel])
        assert r["hit_flag"].astype(bool).tolist() == flags
        assert r["sel_slot"].tolist() == slots
        assert (r["n_hit"], r["n_miss"], r["n_evict"]) == (cnt["n_hit"], cnt["n_miss"], cnt["n_evict"])
        assert tok[:cap].tolist() == bb.tok[:cap] and (tok[cap:] == -1).all()
        assert life[:cap].tolist() == bb.life_array() and (life[cap:] == reset).all()


def test_oracle_capacity_errors_change_nothing():
    S, N, k = 12, 100, 5
    sel = np.array([3, 9, 20, 41, 77], np.int32)
    tok = np.full(S, -1, np.int32)
    life = np.zeros(S, np.int32)
    oracle.unit_step(S, N, k, "lifetime", 4, 64, 0, sel, tok, life)
    before = (tok.copy(), life.copy())
    for cap, want in ((0, oracle.ERR_RANGE), (-1, oracle.ERR_RANGE), (S + 1, oracle.ERR_RANGE),
                      (4, oracle.ERR_CAPACITY)):
        st_, _ = oracle.unit_step(S, N, k, "lifetime", 4, 64, 1, sel, tok, life, cap=cap)
        assert st_ == want
        assert np.array_equal(tok, before[0]) and np.array_equal(life, before[1])
    # a constant capacity equal to S is the unsized step
    st_, r = oracle.unit_step(S, N, k, "lifetime", 4, 64, 1, sel, tok, life, cap=S)
    assert st_ == oracle.OK and r["n_hit"] == k


@pytest.mark.parametrize("policy", ["lifetime", "lru"])
def test_oracle_state_error_with_shrink_changes_nothing(policy):
    """A state error found while a smaller buffer size is set leaves every
    slot untouched, the ones past the size included: the error takes
    precedence over the shrink (an erroneous step changes no state)."""
    S, N = 8, 64
    life_occ = 3 if policy == "lifetime" else 0   # a valid lifetime / stamp at t = 1
    empty = 0 if policy == "lifetime" else -1
    # id 5 held by slots 1 and 5 (both below the size 6), slot 7 (past it) holds 20
    tok = np.array([1, 5, 9, -1, -1, 5, -1, 20], np.int32)
    life = np.array([life_occ, life_occ, life_occ, empty, empty, life_occ, empty, life_occ],
                    np.int32)
    before = (tok.copy(), life.copy())
    st_, r = oracle.unit_step(S, N, 3, policy, 4, 64, 1, np.array([[1, 5, 9]], np.int32), tok,
                              life, cap=6)
    assert st_ == oracle.ERR_STATE
    assert np.array_equal(tok, before[0]) and np.array_equal(life, before[1])
    assert (r["sel_slot"] == -1).all() and not r["hit_flag"].any() and r["n_miss"] == 0
    # the same state without the duplicate: the step runs and empties slot 7
    tok[5], life[5] = -1, empty
    st_, r = oracle.unit_step(S, N, 3, policy, 4, 64, 1, np.array([[1, 5, 9]], np.int32), tok,
                              life, cap=6)
    assert st_ == oracle.OK and r["n_hit"] == 3
    assert tok[7] == -1 and life[7] == empty


def test_plan_capacity_worked_example_and_invariants():
    from oracle.plan import plan_capacity
    # spare 6 shared 1 : 3 -> floor(6/4) = 1 and floor(18/4) = 4
    assert plan_capacity([2, 3], [0, 2], 11, 8).tolist() == [3, 7]
    # capped at S, and the plan that does not fit
    assert plan_capacity([2, 3], [0, 100], 40, 8).tolist() == [2, 8]
    assert plan_capacity([5, 6], [1, 1], 10, 8) is None
    rng = np.random.default_rng(0)
    for _ in range(200):
        n, S = int(rng.integers(1, 10)), int(rng.integers(1, 50))
        d = rng.integers(1, S + 1, n)
        r = rng.integers(0, 30, n)
        b = int(rng.integers(0, 2 * n * S))
        cap = plan_capacity(d, r, b, S)
        if d.sum() > b:
            assert cap is None
            continue
        assert (cap >= d).all() and (cap <= S).all() and cap.sum() <= b


def test_lru_bucket_width_worked_by_hand():
    """Buckets W = 3 steps wide, B = 3, at step t = 10: stamps 9, 7, 6, 3, 0
    are ages 0, 2, 3, 6, 9 past the last step, buckets 0, 0, 1, 2, 2 (9 // 3
    = 3 capped).  Slots 3 and 4 share the oldest bucket: slot 3 goes.  With
    one-step buckets (W = 1) slots 1..4 would all be in bucket 2 and slot 1
    would go."""
    sel = np.array([[11]], np.int32)
    for W, victim in ((3, 3), (1, 1)):
        tok = np.array([20, 21, 22, 23, 24], np.int32)
        life = np.array([9, 7, 6, 3, 0], np.int32)
        st_, r = oracle.unit_step(5, 30, 1, "lru", 4, 3, 10, sel, tok, life, bucket_width=W)
        assert st_ == oracle.OK and r["n_evict"] == 1
        assert r["sel_slot"][0, 0] == victim
        want = [20, 21, 22, 23, 24]
        want[victim] = 11
        assert tok.tolist() == want and life[victim] == 10
