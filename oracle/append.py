"""ORACLE -- test infrastructure only (tests, the smoke check and the CPU leg
of the benchmark may use it; the product library never does).

Offload of a newly decoded token into the host KV store, written out as its
definition.  The Spin summary (gist.science 2604.26837, section 2A) names
Offload, placing KV data into memory, as one of the two system-managed
operations of the pipeline, over a page-based KV substrate; section 2B keeps
the physical pages per attention head.  The pages give no layout, so the
reading taken is the one the rest of this code base uses for a row:

  * split layout, an entry of P tokens: K[P][d_qk] followed by V[P][d_v];
    token r of the entry has its key at elements [r d_qk, (r + 1) d_qk) and
    its value at [P d_qk + r d_v, P d_qk + (r + 1) d_v);
  * latent layout (one token per entry): the whole row is the token's
    latent vector.

Token position p of a request lands in entry p // P, row p % P, for every KV
head of that request.  A device-buffer slot that holds the entry gets the same
bytes, so the buffer keeps exact copies of host rows (the AVSG abstract's
reuse is only valid for exact copies).  Slots, lifetimes and stamps do not
change: an append is not a selection.  A position outside [0, N P) is a range
error: that request writes nothing.

append_insert adds the optional second half of Offload: the token's entry is
also made resident in every unit of the request, between steps, so that the
next step finds it in the buffer.  The pages fix no rule for it; the reading
taken follows the step's own eviction order without ageing anyone:

  * the slots in use are [0, cap) (the unit's buffer size); slots past it are
    emptied, as the next step would empty them;
  * if a slot in use holds the entry it is written through and its keep-state
    refreshed (lifetime L; for bucketed LRU the stamp t - 1, i.e. bucket 0 at
    the coming step t);
  * otherwise the first slot in the order (occupied?, lifetime or minus
    bucket at step t, slot index) takes the entry, receives its whole host
    row with the token already written, and the fresh keep-state;
  * a unit whose slots in use are not a valid state (an id outside [-1, N),
    a lifetime outside [0, L] or stamp outside [0, t), the entry in two slots)
    writes nothing and reports a state error; a bad position or capacity, an
    entry without a host row, or (bucketed LRU) an insertion before the
    first step, when no stamp t - 1 exists, is a range error of the unit.
"""
from __future__ import annotations

import numpy as np

OK, ERR_RANGE, ERR_STATE = 0, 17, 19


def token_slices(latent: bool, tokens_per_entry: int, d_qk: int, d_v: int, r: int):
    """(row slice of the token's key, row slice of its value); the value
    slice is None in the latent layout (the row is one vector)."""
    if latent:
        return slice(0, d_qk), None
    P = tokens_per_entry
    return slice(r * d_qk, (r + 1) * d_qk), slice(P * d_qk + r * d_v, P * d_qk + (r + 1) * d_v)


def append(w, host_kv: np.ndarray, new_kv: np.ndarray, pos: np.ndarray,
           slot_tok: np.ndarray | None = None, buf: np.ndarray | None = None) -> np.ndarray:
    """Writes new_kv [units][tok_elems] (uint16 bf16 bits: K then V, or the
    latent vector) at token position pos[b] of every unit of request b, in
    host_kv [units][N][row] and in every slot of buf [units][S][row] whose
    slot_tok is that entry.  Returns the per-request status (0 or 17)."""
    P = w.tokens_per_entry
    N = w.n_entries
    d_qk, d_v = w.head_dim_qk, w.head_dim_v
    status = np.zeros(w.batch, dtype=np.int32)
    for b in range(w.batch):
        p = int(pos[b])
        if p < 0 or p >= N * P:
            status[b] = ERR_RANGE
            continue
        e, r = divmod(p, P)
        ks, vs = token_slices(w.latent, P, d_qk, d_v, r)
        for g in range(w.n_kv_heads):
            u = b * w.n_kv_heads + g
            rows = [host_kv[u, e]]
            if slot_tok is not None and buf is not None:
                for s in np.nonzero(slot_tok[u] == e)[0]:
                    rows.append(buf[u, s])
            for row in rows:
                row[ks] = new_kv[u, :d_qk]
                if vs is not None:
                    row[vs] = new_kv[u, d_qk:d_qk + d_v]
    return status


def _write_token(row, new_tok, latent, P, d_qk, d_v, r):
    ks, vs = token_slices(latent, P, d_qk, d_v, r)
    row[ks] = new_tok[:d_qk]
    if vs is not None:
        row[vs] = new_tok[d_qk:d_qk + d_v]


def append_insert(w, host_kv: np.ndarray, new_kv: np.ndarray, pos: np.ndarray,
                  slot_tok: np.ndarray, life: np.ndarray, buf: np.ndarray, t: int,
                  caps: np.ndarray | None = None, mapped: np.ndarray | None = None) -> np.ndarray:
    """append() plus insertion of the token's entry into each unit's buffer
    (slot_tok, life [units][S] int32 and buf [units][S][row] updated in
    place) before step t.  caps [units]: slots in use (None: all S);
    mapped [units][N] bool: entries with a host row (None: all).  Returns
    the per-unit status (0, 17 or 19)."""
    P, N, S = w.tokens_per_entry, w.n_entries, w.n_slots
    d_qk, d_v = w.head_dim_qk, w.head_dim_v
    lru = w.policy == "lru"
    L, B, W = w.lifetime_L, w.n_buckets, w.bucket_width
    fresh = t - 1 if lru else L
    empty_life = -1 if lru else 0
    status = np.zeros(w.units, dtype=np.int32)
    for u in range(w.units):
        b = u // w.n_kv_heads
        p = int(pos[b])
        cap = S if caps is None else int(caps[u])
        if p < 0 or p >= N * P or not 1 <= cap <= S or (lru and t < 1):
            status[u] = ERR_RANGE
            continue
        e, r = divmod(p, P)
        if mapped is not None and not mapped[u, e]:
            status[u] = ERR_RANGE
            continue
        ids, lv = slot_tok[u, :cap], life[u, :cap]
        occ = ids >= 0
        bad = ((ids < -1) | (ids >= N)).any()
        if lru:
            bad |= (occ & ((lv < 0) | (lv >= t))).any()
        else:
            bad |= (occ & ((lv < 0) | (lv > L))).any()
        bad |= np.count_nonzero(ids == e) > 1
        if bad:
            status[u] = ERR_STATE
            continue
        _write_token(host_kv[u, e], new_kv[u], w.latent, P, d_qk, d_v, r)
        slot_tok[u, cap:] = -1
        life[u, cap:] = empty_life
        held = np.nonzero(ids == e)[0]
        if held.size:
            s = int(held[0])
            _write_token(buf[u, s], new_kv[u], w.latent, P, d_qk, d_v, r)
        else:
            def order(s):
                if slot_tok[u, s] < 0:
                    return (0, 0, s)
                key = int(life[u, s]) if not lru else -min((t - int(life[u, s]) - 1) // W, B - 1)
                return (1, key, s)
            s = min(range(cap), key=order)
            slot_tok[u, s] = e
            buf[u, s] = host_kv[u, e]
        life[u, s] = fresh
    return status
