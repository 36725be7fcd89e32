"""Pins of the oracle's two-level directory lookup and of its miss check
(a miss of an entry without a host row is a range error of the unit, found
after every other check, with the state untouched).  CPU only."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import directory as odir
from bruteforce import BruteBuffer
from directory_inputs import build_directory, permuted_pool


@pytest.mark.parametrize("seg", [1, 4, 16, 64])
def test_resolve_is_the_mapping(seg):
    rng = np.random.default_rng(seg)
    units, n, pool_rows = 3, 100, 500
    keys = [(u, e) for u in range(units) for e in range(n) if rng.random() < 0.4]
    rows = rng.choice(pool_rows, size=len(keys), replace=False)
    mapping = dict(zip(keys, (int(r) for r in rows)))
    top, segs = build_directory(mapping, units, n, seg, spare_segments=2)
    for u in range(units):
        for e in range(n):
            assert odir.resolve(top, segs, seg, pool_rows, u, e) == mapping.get((u, e), -1)
    # segments exist only where some entry is mapped (allocated on demand)
    used = {(u, e // seg) for (u, e) in mapping}
    assert (top >= 0).sum() == len(used) and len(segs) == len(used) + 2
    # a row outside the pool, or a segment index outside the segments, reads as unmapped
    u, e = keys[0]
    segs2 = segs.copy()
    segs2[top[u, e // seg], e % seg] = pool_rows
    assert odir.resolve(top, segs2, seg, pool_rows, u, e) == -1
    top2 = top.copy()
    top2[u, e // seg] = len(segs)
    assert odir.resolve(top2, segs, seg, pool_rows, u, e) == -1


def test_flat_view_of_a_permuted_pool():
    rng = np.random.default_rng(5)
    flat = rng.integers(0, 2**16, size=(2, 30, 8), dtype=np.uint16)
    pool, mapping = permuted_pool(flat, rng, extra_rows=7)
    top, segs = build_directory(mapping, 2, 30, 8)
    view, mapped = odir.flat_view(pool, top, segs, 8, 2, 30)
    assert mapped.all() and np.array_equal(view, flat)
    del mapping[(1, 17)]
    top, segs = build_directory(mapping, 2, 30, 8)
    view, mapped = odir.flat_view(pool, top, segs, 8, 2, 30)
    assert not mapped[1, 17] and mapped.sum() == 59 and (view[1, 17] == 0).all()


def _fresh(S, policy):
    return np.full(S, -1, np.int32), np.full(S, -1 if policy == "lru" else 0, np.int32)


@pytest.mark.parametrize("policy", ["lifetime", "lru"])
def test_unmapped_miss_is_a_range_error_and_changes_nothing(policy):
    S, N, k = 8, 64, 3
    tok, life = _fresh(S, policy)
    mapped = np.ones(N, bool)
    st_, _ = oracle.unit_step(S, N, k, policy, 4, 64, 0, np.array([[1, 5, 9]], np.int32), tok, life,
                              mapped=mapped)
    assert st_ == oracle.OK
    mapped[20] = False          # entry 20 has no host row
    before = (tok.copy(), life.copy())
    for cap in (None, 6):       # also while a smaller buffer size is set
        st_, r = oracle.unit_step(S, N, k, policy, 4, 64, 1, np.array([[1, 5, 20]], np.int32), tok,
                                  life, cap=cap, mapped=mapped)
        assert st_ == oracle.ERR_RANGE
        assert np.array_equal(tok, before[0]) and np.array_equal(life, before[1])
        assert (r["sel_slot"] == -1).all() and r["n_miss"] == 0
    # an unmapped entry that is resident hits: it needs no transfer
    mapped[5] = False
    st_, r = oracle.unit_step(S, N, k, policy, 4, 64, 1, np.array([[1, 5, 21]], np.int32), tok, life,
                              mapped=mapped)
    assert st_ == oracle.OK and r["hit_flag"].tolist() == [[1, 1, 0]]


def test_state_errors_come_before_the_directory_check():
    S, N, k = 8, 64, 3
    tok, life = _fresh(S, "lifetime")
    oracle.unit_step(S, N, k, "lifetime", 4, 64, 0, np.array([[1, 5, 9]], np.int32), tok, life)
    tok[4], life[4] = 5, 2      # id 5 held by two slots
    mapped = np.ones(N, bool)
    mapped[30] = False
    st_, _ = oracle.unit_step(S, N, k, "lifetime", 4, 64, 1, np.array([[1, 5, 30]], np.int32), tok,
                              life, mapped=mapped)
    assert st_ == oracle.ERR_STATE


def test_all_mapped_equals_no_directory_on_a_random_trace():
    rng = np.random.default_rng(9)
    S, N, k, steps = 16, 90, 6, 20
    a_tok, a_life = _fresh(S, "lru")
    b_tok, b_life = _fresh(S, "lru")
    bb = BruteBuffer(S, N, 4, 3, "lru")
    for t in range(steps):
        sel = np.sort(rng.choice(N, size=k, replace=False)).astype(np.int32)[None]
        sa, ra = oracle.unit_step(S, N, k, "lru", 4, 3, t, sel, a_tok, a_life)
        sb, rb = oracle.unit_step(S, N, k, "lru", 4, 3, t, sel, b_tok, b_life,
                                  mapped=np.ones(N, bool))
        flags, slots, _ = bb.step([list(map(int, sel[0]))])
        assert sa == sb == oracle.OK and rb["sel_slot"].tolist() == slots
        assert np.array_equal(a_tok, b_tok) and np.array_equal(a_life, b_life)
