"""ORACLE -- test infrastructure only (tests, smoke check, CPU benchmark leg).

Decode attention restricted to the selected entries, in float64, written as
its definition.  The AVSG abstract (arxivdaily 2609.37538, abstract) states
that the operator preserves the exact token selections of dynamic sparse
attention, so the output of a step is plain softmax attention of each query
head over exactly the selected K/V rows; it never depends on which rows
happened to be resident.  This model therefore reads the rows straight from
the host KV, not from any buffer.

Readings where the pages are silent:
  - query head h uses KV head h // (Hq / Hkv) (consecutive groups);
  - a selected page contributes all of its tokens, unless a context length
    is given: token row t of entry e is position e P + t of its request, and
    rows at or past the length are not attended (the context's last page may
    be only partly written);
  - a latent row serves as the key (all head_dim_qk values) and its first
    head_dim_v values serve as the value;
  - a unit whose step failed validation produces zeros.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def unit_kv(w, host_kv_unit: np.ndarray, ids: np.ndarray):
    """K [n][dqk] and V [n][dv] (float64) of the selected entries of one unit;
    n = len(ids) * tokens_per_entry, tokens of a page in order."""
    rows = bf16_to_f64(host_kv_unit[np.asarray(ids)])          # [k][row_elems]
    if w.latent:
        return rows[:, :w.head_dim_qk], rows[:, :w.head_dim_v]
    tpe = w.tokens_per_entry
    K = rows[:, :tpe * w.head_dim_qk].reshape(-1, w.head_dim_qk)
    V = rows[:, tpe * w.head_dim_qk:].reshape(-1, w.head_dim_v)
    return K, V


def softmax_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """o[h] = sum_i softmax_i(scale * <q[h], K[i]>) V[i], for q [G][d]."""
    s = scale * (q @ K.T)                                        # [G][n]
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ V                                                 # [G][dv]


def in_context(w, ids, ctx_len) -> np.ndarray:
    """Mask over the token rows of the entries `ids` (in unit_kv's order):
    row t of entry e is position e P + t, kept when below ctx_len."""
    P = 1 if w.latent else w.tokens_per_entry
    pos = np.asarray(ids, dtype=np.int64)[:, None] * P + np.arange(P)[None, :]
    return (pos < ctx_len).reshape(-1)


def attend_unit(w, q_bits: np.ndarray, host_kv_unit: np.ndarray, sel_unit: np.ndarray, unit: int,
                token: int, heads=None, ctx_len=None) -> np.ndarray:
    """Output rows [G'][dv] of unit `unit`, query token `token`, for the query
    heads `heads` (default: all heads mapped to this unit's KV head), over
    the rows of the request's context when ctx_len (its length) is given."""
    G = w.n_q_heads // w.n_kv_heads
    b, g = divmod(unit, w.n_kv_heads)
    if heads is None:
        heads = range(g * G, (g + 1) * G)
    heads = list(heads)
    q = bf16_to_f64(q_bits[b, token, heads, :])                  # [G'][dqk]
    K, V = unit_kv(w, host_kv_unit, sel_unit[token])
    if ctx_len is not None:
        keep = in_context(w, sel_unit[token], ctx_len)
        K, V = K[keep], V[keep]
    return softmax_attention(q, K, V, w.softmax_scale)


def attend(w, q_bits: np.ndarray, host_kv: np.ndarray, sel: np.ndarray, status=None,
           units=None, lengths=None, ctx_len=None) -> np.ndarray:
    """float64 out [B][T][Hq][dv] for one step.  host_kv is [units][N][row]
    (uint16 bf16 bits), sel is [units][T][k], of which the first
    lengths[u][j] entries are in use (all when lengths is None); ctx_len
    [B]: context lengths in tokens (None: whole entries).  Units not in
    `units` are NaN; units with a nonzero status are zero."""
    out = np.full((w.batch, w.n_q_tokens, w.n_q_heads, w.head_dim_v), np.nan)
    G = w.n_q_heads // w.n_kv_heads
    for u in (range(w.units) if units is None else units):
        b, g = divmod(u, w.n_kv_heads)
        for j in range(w.n_q_tokens):
            if status is not None and status[u] != 0:
                out[b, j, g * G:(g + 1) * G] = 0.0
            else:
                su = sel[u] if lengths is None else [sel[u][jj][:lengths[u][jj]]
                                                     for jj in range(w.n_q_tokens)]
                out[b, j, g * G:(g + 1) * G] = attend_unit(
                    w, q_bits, host_kv[u], su, u, j,
                    ctx_len=None if ctx_len is None else int(ctx_len[b]))
    return out


def attend_native(w, q_bits: np.ndarray, host_kv: np.ndarray, sel: np.ndarray, status=None,
                  lengths=None, threads=None, ctx_len=None) -> np.ndarray:
    """The same attention as `attend`, computed by the oracle library's C
    loops in double precision (attention.c), with OpenMP over (unit, token,
    head); every unit is computed.  threads: OpenMP threads (None: leave the
    current setting)."""
    import ctypes
    from oracle import AttnCfg, _load, set_threads
    lib = _load()
    if threads is not None:
        set_threads(threads)
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    assert host_kv.dtype == np.uint16 and host_kv.flags.c_contiguous
    assert host_kv.shape == (w.units, w.n_entries, w.row_elems)
    assert sel.shape == (w.units, w.n_q_tokens, w.k)
    assert q_bits.shape == (w.batch, w.n_q_tokens, w.n_q_heads, w.head_dim_qk)
    ln = None if lengths is None else np.ascontiguousarray(lengths, dtype=np.int32).reshape(
        w.units, w.n_q_tokens)
    stt = None if status is None else np.ascontiguousarray(status, dtype=np.int32).reshape(w.units)
    cl = None if ctx_len is None else np.ascontiguousarray(ctx_len, dtype=np.int32).reshape(w.batch)
    out = np.empty((w.batch, w.n_q_tokens, w.n_q_heads, w.head_dim_v), np.float64)
    cfg = AttnCfg(w.batch, w.n_kv_heads, w.n_q_heads, w.n_q_tokens, w.head_dim_qk, w.head_dim_v,
                  1 if w.latent else 0, w.tokens_per_entry, w.n_entries, w.k,
                  float(w.softmax_scale))
    lib.oracle_attend(ctypes.byref(cfg), q_bits.ctypes.data, host_kv.ctypes.data, sel.ctypes.data,
                      None if ln is None else ln.ctypes.data, None if stt is None else stt.ctypes.data,
                      None if cl is None else cl.ctypes.data, out.ctypes.data)
    return out
