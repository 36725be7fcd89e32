"""Pins of the context-length reading (the last page of a context may be only
partly written), against constructions written independently of the oracle.
CPU only.

* Entries in a context: entry e holds positions [e P, (e + 1) P) and is in a
  context of n tokens when e P < n; the count is checked against brute force
  over every position.  A selected entry past it is a range error that leaves
  the state unchanged (hand-worked), as is a length outside [1, N P].
* Attention with context lengths equals softmax attention over a dense
  per-position K/V array restricted to the selected positions below the
  length (built here position by position from the row layout, not through
  the oracle's row reader), in both the numpy and the C oracle; rows past the
  context may hold NaN without effect; a length that ends on a page boundary
  equals attention over whole pages.
* A page assembled by appending its tokens one at a time, attended after each
  append with the context ending at the new token, equals dense attention
  over the positions written so far, while the page's unwritten rows hold NaN.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import tracegen as tg
from oracle import append as oapp
from oracle import attention as oatt


def _w(tpe=4, N=10, batch=2, Hkv=2, d=8, k=3, S=6, T=1):
    return tg.WORKLOADS[4].replace(batch=batch, n_kv_heads=Hkv, n_q_heads=2 * Hkv, head_dim_qk=d,
                                   head_dim_v=d, n_entries=N, tokens_per_entry=tpe, k=k,
                                   n_slots=S, policy="lifetime", lifetime_L=4, n_q_tokens=T)


@pytest.mark.parametrize("P", [1, 3, 16])
def test_context_entries_against_positions(P):
    N = 7
    for n in range(-1, N * P + 3):
        got = int(oracle.context_entries([n], P, N)[0])
        if 1 <= n <= N * P:
            want = len({pos // P for pos in range(n)})
        else:
            want = 0
        assert got == want, (P, n)


@pytest.mark.parametrize("ctx_len,sel,want", [
    (13, [1, 3], 0),      # entry 3 holds position 12 only: in the context
    (13, [1, 4], 17),     # entry 4 starts at 16: past the context
    (12, [1, 3], 17),     # entry 3 starts at 12 = the length
    (40, [2, 9], 0),      # the whole store
    (41, [2, 9], 17),     # a length past N P
    (0, [2, 9], 17),      # an empty context
    (13, [4, 1], 17),     # range before order: entry 4 is past the context
])
def test_selection_past_the_context_is_a_range_error(ctx_len, sel, want):
    w = _w(tpe=4, N=10, batch=1, Hkv=1, k=2)
    ob = oracle.OracleBuffer.for_workload(w)
    ob.step(np.array([[[0, 5]]], np.int32), ctx_len=np.array([40]), tokens_per_entry=4)
    snap = ob.snapshot()
    r = ob.step(np.array([[sel]], np.int32), ctx_len=np.array([ctx_len]), tokens_per_entry=4)
    assert int(r["status"][0]) == want
    if want:
        t, st, lf, _ = snap
        assert np.array_equal(ob.slot_tok, st) and np.array_equal(ob.life, lf)


def _dense(w, host):
    """Per-position K [units][N P][d] and V, written position by position
    from the row layout: position p is entry p // P, row p % P; its key at
    [r d, (r + 1) d) of the row, its value at [P d + r d, P d + (r + 1) d)."""
    P, d = w.tokens_per_entry, w.head_dim_qk
    n = w.n_entries * P
    K = np.empty((w.units, n, d))
    V = np.empty((w.units, n, d))
    for u in range(w.units):
        for p in range(n):
            e, r = divmod(p, P)
            K[u, p] = oatt.bf16_to_f64(host[u, e, r * d:(r + 1) * d])
            V[u, p] = oatt.bf16_to_f64(host[u, e, P * d + r * d:P * d + (r + 1) * d])
    return K, V


def _by_position(w, q, K, V, sel, ctx_len):
    G = w.n_q_heads // w.n_kv_heads
    P = w.tokens_per_entry
    out = np.zeros((w.batch, w.n_q_tokens, w.n_q_heads, w.head_dim_v))
    for u in range(w.units):
        b, g = divmod(u, w.n_kv_heads)
        for j in range(w.n_q_tokens):
            pos = [e * P + r for e in sel[u, j] for r in range(P) if e * P + r < ctx_len[b]]
            qq = oatt.bf16_to_f64(q[b, j, g * G:(g + 1) * G])
            s = w.softmax_scale * qq @ K[u, pos].T
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[b, j, g * G:(g + 1) * G] = (p / p.sum(axis=1, keepdims=True)) @ V[u, pos]
    return out


def _bits(rng, shape):
    return (rng.standard_normal(shape).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("tpe", [1, 3, 4])
def test_attention_with_context_lengths_equals_dense_by_position(tpe):
    w = _w(tpe=tpe, N=9, batch=2, Hkv=2, T=2)
    rng = np.random.default_rng(tpe)
    host = _bits(rng, (w.units, w.n_entries, w.row_elems))
    q = _bits(rng, (w.batch, w.n_q_tokens, w.n_q_heads, w.head_dim_qk))
    ctx_len = np.array([6 * tpe + max(tpe - 2, 1), 4 * tpe + 1], np.int32)
    last = (ctx_len - 1) // tpe          # the entry holding each context's last token
    sel = np.zeros((w.units, w.n_q_tokens, w.k), np.int32)
    for u in range(w.units):
        b = u // w.n_kv_heads
        for j in range(w.n_q_tokens):
            sel[u, j] = sorted({int(last[b]), j, 2 + j})
    assert (sel.max(axis=2) == last[np.arange(w.units) // w.n_kv_heads][:, None]).all()
    K, V = _dense(w, host)
    want = _by_position(w, q, K, V, sel, ctx_len)
    # rows of the last entries past each context hold NaN: they must not count
    for u in range(w.units):
        b = u // w.n_kv_heads
        for p in range(int(ctx_len[b]), (int(last[b]) + 1) * tpe):
            e, r = divmod(p, tpe)
            host[u, e, r * 8:(r + 1) * 8] = 0x7fc0
            host[u, e, tpe * 8 + r * 8:tpe * 8 + (r + 1) * 8] = 0x7fc0
    got_np = oatt.attend(w, q, host, sel, ctx_len=ctx_len)
    got_c = oatt.attend_native(w, q, host, sel, ctx_len=ctx_len)
    assert np.allclose(got_np, want, rtol=1e-12, atol=1e-12)
    assert np.allclose(got_c, want, rtol=1e-12, atol=1e-12)


def test_length_on_a_page_boundary_equals_whole_pages():
    w = _w(tpe=4, N=9)
    rng = np.random.default_rng(5)
    host = _bits(rng, (w.units, w.n_entries, w.row_elems))
    q = _bits(rng, (w.batch, 1, w.n_q_heads, w.head_dim_qk))
    sel = np.array([[[0, 3, 6]], [[1, 2, 6]], [[2, 5, 8]], [[0, 7, 8]]], np.int32)
    ctx_len = np.array([7 * 4, 9 * 4], np.int32)
    a = oatt.attend_native(w, q, host, sel, ctx_len=ctx_len)
    b = oatt.attend_native(w, q, host, sel)
    assert np.array_equal(a, b)


def test_page_assembled_by_appends_attended_as_it_grows():
    """Request 0 decodes positions 20..27 into page 5 (P = 4) and the next;
    after each append the context ends at the new token and attention over
    a selection holding the current page equals dense attention over the
    written positions.  The pages start as NaN."""
    w = _w(tpe=4, N=8, batch=1, Hkv=2)
    rng = np.random.default_rng(9)
    host = _bits(rng, (w.units, w.n_entries, w.row_elems))
    host[:, 5:] = 0x7fc0
    K, V = _dense(w, np.where(host == 0x7fc0, 0, host).astype(np.uint16))
    for p in range(20, 28):
        new = _bits(rng, (w.units, 16))
        assert (oapp.append(w, host, new, np.array([p])) == 0).all()
        for u in range(w.units):
            K[u, p] = oatt.bf16_to_f64(new[u, :8])
            V[u, p] = oatt.bf16_to_f64(new[u, 8:])
        e = p // 4
        sel = np.array([[[1, 3, e]], [[0, 2, e]]], np.int32)
        q = _bits(rng, (1, 1, w.n_q_heads, 8))
        ctx = np.array([p + 1], np.int32)
        want = _by_position(w, q, K, V, sel, ctx)
        for got in (oatt.attend(w, q, host, sel, ctx_len=ctx),
                    oatt.attend_native(w, q, host, sel, ctx_len=ctx)):
            assert np.isfinite(got).all()
            assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
