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
"""
from __future__ import annotations

import numpy as np

OK, ERR_RANGE = 0, 17


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
