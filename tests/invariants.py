"""Step invariants of the slot buffer (numpy, any size).

They follow from what the AVSG abstract (arxivdaily 2609.37538, abstract)
requires of the operator -- exact selections, hits reuse resident slots, only
misses are transferred -- and from the readings of lifetime and LRU
management.  `check_unit_step` raises AssertionError naming the invariant.
"""
from __future__ import annotations

import numpy as np


def check_unit_step(sel, prev_tok, prev_life, new_tok, new_life, hit_flag, sel_slot, n_hit, n_miss,
                    n_evict, L, policy, t, prev_union=None, fill_slot=None):
    sel = np.asarray(sel)
    union = np.unique(sel)
    prev_res = prev_tok[prev_tok >= 0]
    new_res = new_tok[new_tok >= 0]
    m = int(n_miss)
    # I1: hits + misses = |U|
    assert int(n_hit) + m == union.size, "I1"
    # I2: hits are exactly the union entries resident before the step
    assert int(n_hit) == np.intersect1d(union, prev_res).size, "I2"
    # I3: no id held by two slots
    assert np.unique(new_res).size == new_res.size, "I3"
    # I4: resident after = U plus the survivors of the resident before
    assert np.isin(union, new_res).all(), "I4 (U resident)"
    extra = np.setdiff1d(new_res, union)
    assert np.isin(extra, prev_res).all(), "I4 (nothing new outside U)"
    assert new_res.size == prev_res.size + m - int(n_evict), "I4 (count)"
    # I6: exactly m slots changed id, and they are the reserved ones
    changed = np.nonzero(new_tok != prev_tok)[0]
    assert changed.size == m, "I6"
    if fill_slot is not None:
        assert np.array_equal(np.sort(changed), np.sort(np.asarray(fill_slot)[:m])), "I6 (slots)"
    # I7: every slot of U carries lifetime L (or the current stamp)
    pos = np.nonzero(np.isin(new_tok, union))[0]
    want = t if policy == "lru" else L
    assert (new_life[pos] == want).all(), "I7"
    # I8: nothing evicted while an empty slot was available
    if int(n_evict) > 0:
        assert (new_tok >= 0).all(), "I8"
    # I9: the previous union was resident after its step, so it hits now
    if prev_union is not None:
        assert int(n_hit) >= np.intersect1d(union, prev_union).size, "I9"
    # per-(token, entry) outputs
    assert (new_tok[sel_slot] == sel).all(), "sel_slot"
    assert np.array_equal(hit_flag.astype(bool), np.isin(sel, prev_res)), "hit_flag"
    return union


def check_buffer(buf_unit, tok_unit, host_kv_unit):
    """I5: every occupied slot holds its entry's host row bit for bit."""
    occ = np.nonzero(tok_unit >= 0)[0]
    assert np.array_equal(buf_unit[occ], host_kv_unit[tok_unit[occ]]), "I5"
