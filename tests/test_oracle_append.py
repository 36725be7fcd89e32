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
