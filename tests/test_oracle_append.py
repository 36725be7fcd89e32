"""Pins of the append (Offload) oracle against constructions written
independently of it.  CPU only.

* A page built by appending its tokens one at a time, in any order, equals the
  page built in one piece by numpy: the tokens' keys as a [P][d_qk] array,
  flattened, then their values as a [P][d_v] array, flattened.  A swapped key
  and value half, a wrong row stride or an off-by-one row fails it.
* Bytes outside the written token rows never change; a position outside the
  context is an error that writes nothing.
* Write-through: every occupied slot still holds an exact copy of its host row
  afterwards, and slots holding other entries are untouched.
* After an append, attention over a selection that contains the new token's
  entry equals attention over a dense per-token K/V tensor whose row at that
  position is the new token (written here by position, not by entry layout).
* Insertion (append_insert): victims worked by hand for both policies (one
  case where the oldest bucket and the oldest stamp disagree), write-through
  and refresh of a resident entry, the capacity, every error writing nothing,
  and on 600 random states the piecewise victim rule plus the step oracle
  hitting the inserted entry at the next step.
"""
from __future__ import annotations

import numpy as np
import pytest

import tracegen as tg
from oracle import append as oapp
from oracle import attention as oatt


def _w(latent=False, tpe=1, batch=2, Hkv=2, dqk=8, dv=8, N=12, S=5):
    if latent:
        return tg.WORKLOADS[5].replace(batch=batch, n_kv_heads=1, n_q_heads=4, head_dim_qk=dqk,
                                       head_dim_v=dv, n_entries=N, k=3, n_slots=S)
    return tg.WORKLOADS[4].replace(batch=batch, n_kv_heads=Hkv, n_q_heads=2 * Hkv, head_dim_qk=dqk,
                                   head_dim_v=dv, n_entries=N, tokens_per_entry=tpe, k=3,
                                   n_slots=S, policy="lifetime")


def _tok_elems(w):
    return w.head_dim_qk if w.latent else w.head_dim_qk + w.head_dim_v


@pytest.mark.parametrize("tpe", [1, 3, 16])
def test_page_assembled_by_appends_equals_numpy_layout(tpe):
    w = _w(tpe=tpe, batch=1, Hkv=1)
    rng = np.random.default_rng(tpe)
    host = np.zeros((w.units, w.n_entries, w.row_elems), np.uint16)
    e = 5
    K = rng.integers(1, 1 << 16, (tpe, w.head_dim_qk), dtype=np.uint16)
    V = rng.integers(1, 1 << 16, (tpe, w.head_dim_v), dtype=np.uint16)
    for r in rng.permutation(tpe):
        new = np.concatenate([K[r], V[r]])[None, :]
        st = oapp.append(w, host, new, np.array([e * tpe + r]))
        assert st[0] == 0
    expect = np.concatenate([K.reshape(-1), V.reshape(-1)])
    assert np.array_equal(host[0, e], expect)
    others = np.delete(host[0], e, axis=0)
    assert not others.any()


def test_latent_row_is_the_vector():
    w = _w(latent=True, dqk=12, dv=8)
    host = np.zeros((w.units, w.n_entries, w.row_elems), np.uint16)
    vec = np.arange(1, 13, dtype=np.uint16)
    new = np.stack([vec, vec + 100])
    oapp.append(w, host, new, np.array([3, 7]))
    assert np.array_equal(host[0, 3], vec) and np.array_equal(host[1, 7], vec + 100)
    assert np.count_nonzero(host) == 24


@pytest.mark.parametrize("latent,tpe", [(False, 1), (False, 4), (True, 1)])
def test_only_the_token_rows_change_and_range_errors_write_nothing(latent, tpe):
    w = _w(latent=latent, tpe=tpe, batch=3)
    rng = np.random.default_rng(11)
    host = rng.integers(0, 1 << 16, (w.units, w.n_entries, w.row_elems), dtype=np.uint16)
    before = host.copy()
    new = rng.integers(0, 1 << 16, (w.units, _tok_elems(w)), dtype=np.uint16)
    P, N = w.tokens_per_entry, w.n_entries
    pos = np.array([N * P - 1, N * P, -1])  # last position; two out of range
    st = oapp.append(w, host, new, pos)
    assert list(st) == [0, oapp.ERR_RANGE, oapp.ERR_RANGE]
    diff = np.argwhere(host != before)
    e, r = divmod(N * P - 1, P)
    per_unit = w.head_dim_qk if latent else w.head_dim_qk + w.head_dim_v
    # every changed element is in request 0's units, entry e (random data:
    # an element may be rewritten with its old value, so at most per_unit)
    assert all(u < w.n_kv_heads and ent == e for u, ent, _ in diff)
    assert len(diff) <= w.n_kv_heads * per_unit
    assert np.array_equal(host[w.n_kv_heads:], before[w.n_kv_heads:])


def test_write_through_keeps_exact_copies():
    w = _w(tpe=2, batch=2, Hkv=2, S=6)
    rng = np.random.default_rng(5)
    host = rng.integers(0, 1 << 16, (w.units, w.n_entries, w.row_elems), dtype=np.uint16)
    slot_tok = np.full((w.units, w.n_slots), -1, np.int32)
    for u in range(w.units):
        ids = rng.choice(w.n_entries, 4, replace=False)
        slot_tok[u, [0, 2, 3, 5]] = ids
    buf = np.zeros((w.units, w.n_slots, w.row_elems), np.uint16)
    for u in range(w.units):
        for s in range(w.n_slots):
            if slot_tok[u, s] >= 0:
                buf[u, s] = host[u, slot_tok[u, s]]
    buf_before = buf.copy()
    new = rng.integers(0, 1 << 16, (w.units, _tok_elems(w)), dtype=np.uint16)
    # request 0 appends into an entry resident in unit 0's slot 2, request 1
    # into an entry resident nowhere
    e0 = int(slot_tok[0, 2])
    free = sorted(set(range(w.n_entries)) - set(slot_tok[2:].ravel()))
    pos = np.array([e0 * 2 + 1, free[0] * 2])
    oapp.append(w, host, new, pos, slot_tok, buf)
    for u in range(w.units):
        for s in range(w.n_slots):
            if slot_tok[u, s] >= 0:
                assert np.array_equal(buf[u, s], host[u, slot_tok[u, s]])
    assert not np.array_equal(buf[0, 2], buf_before[0, 2])
    changed = {(u, s) for u, s, _ in np.argwhere(buf != buf_before)}
    assert all(slot_tok[u, s] == (e0 if u < 2 else free[0]) for u, s in changed)
    assert np.array_equal(buf[2:], buf_before[2:])


@pytest.mark.parametrize("latent,tpe", [(False, 1), (False, 4), (True, 1)])
def test_attention_after_append_equals_dense_by_position(latent, tpe):
    w = _w(latent=latent, tpe=tpe, batch=2, dqk=16, dv=8 if latent else 16, N=10)
    rng = np.random.default_rng(3)
    f32 = rng.standard_normal((w.units, w.n_entries, w.row_elems)).astype(np.float32)
    host = (f32.view(np.uint32) >> 16).astype(np.uint16)
    new = (rng.standard_normal((w.units, _tok_elems(w))).astype(np.float32).view(np.uint32)
           >> 16).astype(np.uint16)
    P = w.tokens_per_entry
    pos = np.array([7 * P + P - 1, 2 * P])
    # dense per-token K / V of the unmodified cache, then the new token
    # written at its position
    hk = oatt.bf16_to_f64(host)
    if latent:
        Kd, Vd = hk[..., :w.head_dim_qk].copy(), hk[..., :w.head_dim_v].copy()
    else:
        Kd = hk[..., :P * w.head_dim_qk].reshape(w.units, -1, w.head_dim_qk).copy()
        Vd = hk[..., P * w.head_dim_qk:].reshape(w.units, -1, w.head_dim_v).copy()
    nk = oatt.bf16_to_f64(new)
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            u = b * w.n_kv_heads + g
            Kd[u, pos[b]] = nk[u, :w.head_dim_qk]
            Vd[u, pos[b]] = nk[u, :w.head_dim_v] if latent else nk[u, w.head_dim_qk:]
    oapp.append(w, host, new, pos)
    q = (rng.standard_normal((w.batch, 1, w.n_q_heads, w.head_dim_qk)).astype(np.float32)
         .view(np.uint32) >> 16).astype(np.uint16)
    sel = np.zeros((w.units, 1, 3), np.int32)
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            sel[b * w.n_kv_heads + g, 0] = sorted({pos[b] // P, 0, 9} if pos[b] // P not in (0, 9)
                                                  else {pos[b] // P, 4, 9 if pos[b] // P != 9 else 5})
    got = oatt.attend(w.replace(n_q_tokens=1), q, host, sel)
    G = w.n_q_heads // w.n_kv_heads
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            u = b * w.n_kv_heads + g
            toks = np.concatenate([np.arange(e * P, (e + 1) * P) for e in sel[u, 0]])
            qq = oatt.bf16_to_f64(q[b, 0, g * G:(g + 1) * G])
            s = w.softmax_scale * qq @ Kd[u, toks].T
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            assert np.allclose(got[b, 0, g * G:(g + 1) * G], p @ Vd[u, toks], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# append_insert: the token's entry is also made resident, between steps.
# Expected victims below are worked by hand from the step's eviction order
# (empty slots first, then the lowest lifetime or the oldest bucket, then the
# lowest slot index); nothing ages.

def _one_unit(policy="lifetime", S=5, N=12, tpe=2, L=4, B=4, dqk=8, dv=8):
    w = tg.WORKLOADS[4].replace(batch=1, n_kv_heads=1, n_q_heads=2, head_dim_qk=dqk, head_dim_v=dv,
                                n_entries=N, tokens_per_entry=tpe, k=3, n_slots=S, policy=policy,
                                lifetime_L=L, n_buckets=B)
    rng = np.random.default_rng(S * 31 + N)
    host = rng.integers(0, 1 << 16, (1, N, w.row_elems), dtype=np.uint16)
    return w, host, rng


def _state(w, host, ids, life):
    slot_tok = np.array([ids], np.int32)
    lf = np.array([life], np.int32)
    buf = np.zeros((1, w.n_slots, w.row_elems), np.uint16)
    for s, x in enumerate(ids):
        if 0 <= x < w.n_entries:
            buf[0, s] = host[0, x]
    return slot_tok, lf, buf


def _insert(w, host, rng, slot_tok, lf, buf, e, t, r=1, caps=None, mapped=None):
    new = rng.integers(0, 1 << 16, (1, _tok_elems(w)), dtype=np.uint16)
    before = (host.copy(), slot_tok.copy(), lf.copy(), buf.copy())
    st = oapp.append_insert(w, host, new, np.array([e * w.tokens_per_entry + r]), slot_tok, lf, buf,
                            t, caps=caps, mapped=mapped)
    return int(st[0]), new, before


@pytest.mark.parametrize("ids,life,victim", [
    ([7, -1, 3, 9, -1], [2, 0, 4, 1, 0], 1),     # two empty slots: the lower one
    ([7, 2, 3, 9, 1], [2, 1, 4, 1, 3], 1),       # full: lifetime 1 at slots 1 and 3
    ([7, 2, 3, 9, 1], [0, 1, 0, 1, 3], 0),       # lifetime 0 is still resident, and first
])
def test_insert_lifetime_victims_worked_by_hand(ids, life, victim):
    w, host, rng = _one_unit()
    slot_tok, lf, buf = _state(w, host, ids, life)
    st, new, (h0, s0, l0, b0) = _insert(w, host, rng, slot_tok, lf, buf, e=5, t=3)
    assert st == 0
    exp_ids = list(ids)
    exp_ids[victim] = 5
    exp_life = list(life)
    exp_life[victim] = w.lifetime_L
    assert slot_tok[0].tolist() == exp_ids and lf[0].tolist() == exp_life
    # the slot holds the host row with the token written at row 1 of the page
    row = h0[0, 5].copy()
    row[1 * 8:2 * 8] = new[0, :8]
    row[2 * 8 + 1 * 8:2 * 8 + 2 * 8] = new[0, 8:]
    assert np.array_equal(host[0, 5], row) and np.array_equal(buf[0, victim], row)
    others = [s for s in range(w.n_slots) if s != victim]
    assert np.array_equal(buf[0, others], b0[0, others])


def test_insert_lru_takes_the_oldest_bucket_not_the_oldest_stamp():
    # t = 10, B = 4: stamps 9, 5, 3, 8 are buckets 0, 3, 3 (6 capped), 1.
    # Slots 1 and 2 share the oldest bucket; the lower index goes, although
    # slot 2's stamp is older (a global LRU would pick slot 2).
    w, host, rng = _one_unit(policy="lru", S=4, B=4)
    slot_tok, lf, buf = _state(w, host, [4, 6, 8, 10], [9, 5, 3, 8])
    st, _, _ = _insert(w, host, rng, slot_tok, lf, buf, e=2, t=10)
    assert st == 0
    assert slot_tok[0].tolist() == [4, 2, 8, 10]
    assert lf[0].tolist() == [9, 9, 3, 8]          # stamp t - 1: bucket 0 at step 10


def test_insert_into_resident_entry_writes_through_and_refreshes():
    w, host, rng = _one_unit(policy="lifetime", L=6)
    slot_tok, lf, buf = _state(w, host, [7, 5, 3, -1, 1], [2, 1, 6, 0, 0])
    st, new, (h0, s0, l0, b0) = _insert(w, host, rng, slot_tok, lf, buf, e=5, t=9, r=0)
    assert st == 0
    assert slot_tok[0].tolist() == [7, 5, 3, -1, 1]
    assert lf[0].tolist() == [2, 6, 6, 0, 0]
    assert np.array_equal(buf[0, 1], host[0, 5])
    assert not np.array_equal(buf[0, 1], b0[0, 1])
    assert np.array_equal(np.delete(buf[0], 1, axis=0), np.delete(b0[0], 1, axis=0))


def test_insert_applies_the_capacity():
    # cap 3 of 5: slots 3 and 4 are emptied; the entry, held only at slot 4,
    # is not in use there and takes a slot in [0, 3) (the lowest lifetime)
    w, host, rng = _one_unit(policy="lifetime")
    slot_tok, lf, buf = _state(w, host, [7, 2, 3, 9, 5], [3, 1, 2, 4, 4])
    st, _, _ = _insert(w, host, rng, slot_tok, lf, buf, e=5, t=4, caps=np.array([3]))
    assert st == 0
    assert slot_tok[0].tolist() == [7, 5, 3, -1, -1]
    assert lf[0].tolist() == [3, 4, 2, 0, 0]
    assert np.array_equal(buf[0, 1], host[0, 5])


@pytest.mark.parametrize("ids,life,caps,pos_entry,status", [
    ([7, 5, 3, 5, -1], [2, 1, 1, 1, 0], None, 5, 19),   # the entry in two slots
    ([7, 2, 3, 9, -1], [2, 5, 1, 1, 0], None, 5, 19),   # a lifetime above L = 4
    ([7, 2, 12, 9, -1], [2, 1, 1, 1, 0], None, 5, 19),  # an id outside [-1, N)
    ([7, 2, 3, 9, -1], [2, 1, 1, 1, 0], [0], 5, 17),    # capacity outside [1, S]
    ([7, 2, 3, 9, -1], [2, 1, 1, 1, 0], None, 12, 17),  # position outside the context
])
def test_insert_errors_write_nothing(ids, life, caps, pos_entry, status):
    w, host, rng = _one_unit(policy="lifetime")
    slot_tok, lf, buf = _state(w, host, ids, life)
    st, _, (h0, s0, l0, b0) = _insert(w, host, rng, slot_tok, lf, buf, e=pos_entry, t=5, r=0,
                                      caps=None if caps is None else np.array(caps))
    assert st == status
    for a, b in zip((host, slot_tok, lf, buf), (h0, s0, l0, b0)):
        assert np.array_equal(a, b)


def test_insert_before_the_first_lru_step_is_a_range_error():
    # no stamp t - 1 exists at t = 0: every unit writes nothing
    w, host, rng = _one_unit(policy="lru", S=4)
    slot_tok, lf, buf = _state(w, host, [-1] * 4, [-1] * 4)
    st, _, (h0, s0, l0, b0) = _insert(w, host, rng, slot_tok, lf, buf, e=3, t=0)
    assert st == oapp.ERR_RANGE
    for a, b in zip((host, slot_tok, lf, buf), (h0, s0, l0, b0)):
        assert np.array_equal(a, b)
    st, _, _ = _insert(w, host, rng, slot_tok, lf, buf, e=3, t=1)
    assert st == 0 and slot_tok[0].tolist() == [3, -1, -1, -1] and lf[0].tolist() == [0, -1, -1, -1]


def test_insert_of_an_unmapped_entry_is_a_range_error():
    w, host, rng = _one_unit()
    slot_tok, lf, buf = _state(w, host, [-1] * 5, [0] * 5)
    mapped = np.ones((1, w.n_entries), bool)
    mapped[0, 6] = False
    st, _, (h0, *_rest) = _insert(w, host, rng, slot_tok, lf, buf, e=6, t=1, mapped=mapped)
    assert st == oapp.ERR_RANGE and np.array_equal(host, h0) and (slot_tok == -1).all()


@pytest.mark.parametrize("policy", ["lifetime", "lru"])
def test_insert_on_random_states_against_the_rule_and_the_step(policy):
    """Random valid states: the victim equals the piecewise rule (the lowest
    empty slot if there is one; else, among the slots with the lowest
    lifetime or in the oldest bucket, the lowest index); afterwards the state
    is one the step oracle (pinned on its own) accepts, the entry is resident
    exactly once with an exact copy of its host row, and a step at t that
    selects it finds it as a hit."""
    import oracle
    rng = np.random.default_rng(8 if policy == "lru" else 9)
    S, N, L, B, t = 6, 10, 3, 3, 7
    for trial in range(300):
        w, host, _ = _one_unit(policy=policy, S=S, N=N, L=L, B=B, tpe=1)
        ids = [int(x) for x in rng.permutation(N)[:S]]
        for s in range(S):
            if rng.random() < 0.25:
                ids[s] = -1
        if policy == "lru":
            life = [int(rng.integers(0, t)) if x >= 0 else -1 for x in ids]
        else:
            life = [int(rng.integers(0, L + 1)) if x >= 0 else 0 for x in ids]
        slot_tok, lf, buf = _state(w, host, ids, life)
        e = int(rng.integers(0, N))
        st, _, (h0, s0, l0, b0) = _insert(w, host, rng, slot_tok, lf, buf, e=e, t=t, r=0)
        assert st == 0
        assert np.count_nonzero(slot_tok[0] == e) == 1
        s_e = int(np.nonzero(slot_tok[0] == e)[0][0])
        if e in ids:
            assert s_e == ids.index(e)
        else:
            empty = [s for s in range(S) if ids[s] < 0]
            if empty:
                want = empty[0]
            elif policy == "lru":
                bucket = [min(t - life[s] - 1, B - 1) for s in range(S)]
                want = bucket.index(max(bucket))
            else:
                want = life.index(min(life))
            assert s_e == want, (trial, ids, life, e)
        changed = [s for s in range(S) if (slot_tok[0, s], lf[0, s]) != (s0[0, s], l0[0, s])]
        assert set(changed) <= {s_e}
        for s in range(S):
            if slot_tok[0, s] >= 0:
                assert np.array_equal(buf[0, s], host[0, slot_tok[0, s]])
        sel = np.array([[e]], np.int32)
        stt, res = oracle.unit_step(S, N, 1, policy, L, B, t, sel, slot_tok[0].copy(),
                                    lf[0].copy())
        assert stt == 0 and res["hit_flag"][0, 0] == 1 and res["sel_slot"][0, 0] == s_e


def test_insert_keeps_every_unit_separate():
    # two requests, two heads each: every unit of a request inserts the same
    # entry into its own buffer; units of the other request are untouched
    w = _w(tpe=2, batch=2, Hkv=2, S=4).replace(lifetime_L=5)
    rng = np.random.default_rng(21)
    host = rng.integers(0, 1 << 16, (w.units, w.n_entries, w.row_elems), dtype=np.uint16)
    slot_tok = np.array([[1, 2, -1, -1], [3, -1, 4, -1], [5, 6, 7, 8], [9, 10, 11, 0]], np.int32)
    lf = np.array([[5, 5, 0, 0], [1, 0, 2, 0], [3, 2, 1, 4], [1, 1, 1, 1]], np.int32)
    buf = np.zeros((w.units, w.n_slots, w.row_elems), np.uint16)
    new = rng.integers(0, 1 << 16, (w.units, _tok_elems(w)), dtype=np.uint16)
    pos = np.array([9 * 2 + 1, 11 * 2])        # request 0: entry 9; request 1: entry 11
    st = oapp.append_insert(w, host, new, pos, slot_tok, lf, buf, t=2)
    assert st.tolist() == [0, 0, 0, 0]
    assert slot_tok.tolist() == [[1, 2, 9, -1], [3, 9, 4, -1], [5, 6, 11, 8], [9, 10, 11, 0]]
    assert lf.tolist() == [[5, 5, 5, 0], [1, 5, 2, 0], [3, 2, 5, 4], [1, 1, 5, 1]]


def test_insert_lru_bucket_width():
    # t = 10, W = 3, B = 3: stamps 9, 7, 6, 3 are buckets 0, 0, 1, 2: slot 3
    w, host, rng = _one_unit(policy="lru", S=4, B=3)
    w = w.replace(bucket_width=3)
    slot_tok, lf, buf = _state(w, host, [4, 6, 8, 10], [9, 7, 6, 3])
    st, _, _ = _insert(w, host, rng, slot_tok, lf, buf, e=2, t=10)
    assert st == 0 and slot_tok[0].tolist() == [4, 6, 8, 2] and lf[0].tolist() == [9, 7, 6, 9]
