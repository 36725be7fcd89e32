"""Inputs for tests of context lengths (a partly written last page): lists
clipped to each request's context, NaN in every token row past a context,
and starting lengths that leave room to grow by one token per step."""
from __future__ import annotations

import numpy as np

NAN = 0x7FC0     # bf16 quiet NaN


def clip_to_context(sel_t, w, ctx_len):
    """Each list keeps its first k - 1 ids below the entry holding the
    context's last token, gains that entry, and is filled up to k with the
    smallest ids not in it (ascending, distinct, all in the context)."""
    P, k = w.tokens_per_entry, w.k
    out = np.empty_like(sel_t)
    for u in range(w.units):
        last = (int(ctx_len[u // w.n_kv_heads]) - 1) // P
        for j in range(w.n_q_tokens):
            keep = [int(x) for x in sel_t[u, j] if x < last][:k - 1] + [last]
            fill = (x for x in range(last) if x not in set(keep))
            while len(keep) < k:
                keep.append(next(fill))
            out[u, j] = sorted(keep)
    return out


def start_lengths(w):
    P = w.tokens_per_entry
    base = w.n_entries - 2 - (w.steps + P - 1) // P
    return np.array([base * P + 1 + (b * (P - 1) if b < 2 else P // 2) for b in range(w.batch)],
                    np.int32)


def nan_past_context(host, w, ctx_len):
    """Token rows at positions from each context's length to the end of the
    store hold NaN (K and V halves; the whole row for one-token entries)."""
    P, d, dv = w.tokens_per_entry, w.head_dim_qk, w.head_dim_v
    for u in range(w.units):
        n = int(ctx_len[u // w.n_kv_heads])
        e0, r0 = divmod(n, P)
        if e0 >= w.n_entries:      # the context fills the store
            continue
        if P == 1:
            host[u, e0:] = NAN
            continue
        for r in range(r0, P):
            host[u, e0, r * d:(r + 1) * d] = NAN
            host[u, e0, P * d + r * dv:P * d + (r + 1) * dv] = NAN
        host[u, e0 + 1:] = NAN
