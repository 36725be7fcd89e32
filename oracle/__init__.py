"""ORACLE -- test infrastructure only.

A plain, slow CPU model of the decode-step hot path (slot-buffer matching,
reservation under lifetime or bucketed-LRU eviction, miss-only row transfer,
and attention over the selected entries).  Only the tests, the smoke check
and the CPU leg of the benchmark may import it; the product library never
does, and shares no code with it.

  avsg_oracle.c   the state machine of one step per unit (plain C, qsort and
                  a two-pointer merge), compiled with gcc on first use
  attention.c     float64 attention over the selected rows (plain C loops,
                  OpenMP over (unit, token, head)), in the same library
  attention.py    the same attention in numpy, and the wrapper of the C one

Parity pins: the state machine is checked against a separate brute-force
replay, hand-worked traces, closed forms and invariants; attention against
torch's scaled_dot_product_attention with a boolean mask and closed forms.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

from . import attention  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "avsg_oracle.c"), os.path.join(_HERE, "attention.c")]
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()

OK, ERR_UNSORTED, ERR_RANGE, ERR_CAPACITY, ERR_STATE = 0, 16, 17, 18, 19
LIFETIME, LRU = 0, 1


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc: -O2, no intrinsics, OpenMP over units."""
    if force or not os.path.exists(_LIB_PATH) or any(
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(s) for s in _SRCS):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11"] + _SRCS +
                              ["-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_slots", "n_entries", "n_tokens", "k", "policy", "lifetime_L", "n_buckets",
                 "bucket_width")]


class AttnCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "n_kv_heads", "n_q_heads", "n_tokens", "head_dim_qk", "head_dim_v",
                 "latent", "tokens_per_entry", "n_entries", "k")] + [("scale", ctypes.c_double)]


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            p = ctypes.c_void_p
            lib.oracle_unit_step.argtypes = ([ctypes.POINTER(_Cfg), ctypes.c_int64, p, p,
                                              ctypes.c_int32] + [p] * 8 + [ctypes.c_int32])
            lib.oracle_unit_step.restype = ctypes.c_int
            lib.oracle_step.argtypes = [ctypes.POINTER(_Cfg), ctypes.c_int64, ctypes.c_int64] + [p] * 13
            lib.oracle_step.restype = None
            lib.oracle_set_threads.argtypes = [ctypes.c_int]
            lib.oracle_set_threads.restype = None
            lib.oracle_attend.argtypes = [ctypes.POINTER(AttnCfg)] + [p] * 7
            lib.oracle_attend.restype = None
            _lib = lib
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags.c_contiguous
    return a.ctypes.data


def set_threads(n: int) -> None:
    """Threads of the OpenMP loops (state machine: over units; attention:
    over (unit, token, head))."""
    _load().oracle_set_threads(int(n))


class OracleBuffer:
    """Per-unit slot state and (optionally) the device buffer contents,
    advanced one decode step at a time.

    slot_tok [units][S] int32 (-1 = empty), life [units][S] int32 (lifetime,
    or last-selected step with -1 = never for the LRU policy), buf
    [units][S][row_elems] uint16 when `track_buf`.
    """

    def __init__(self, n_slots, n_entries, n_tokens, k, policy, lifetime_L, n_buckets, units,
                 row_elems=0, track_buf=False, bucket_width=1):
        self.cfg = _Cfg(n_slots, n_entries, n_tokens, k,
                        LRU if policy in ("lru", LRU) else LIFETIME, lifetime_L, n_buckets,
                        bucket_width)
        self.units = units
        self.row_elems = row_elems
        self.track_buf = track_buf
        self.reset()

    @classmethod
    def for_workload(cls, w, track_buf=False, units=None):
        return cls(w.n_slots, w.n_entries, w.n_q_tokens, w.k, w.policy, w.lifetime_L, w.n_buckets,
                   w.units if units is None else units, w.row_elems, track_buf, w.bucket_width)

    def reset(self):
        S = self.cfg.n_slots
        self.t = 0
        self.slot_tok = np.full((self.units, S), -1, dtype=np.int32)
        self.life = np.full((self.units, S), -1 if self.cfg.policy == LRU else 0, dtype=np.int32)
        self.buf = (np.zeros((self.units, S, self.row_elems), dtype=np.uint16)
                    if self.track_buf else None)

    def step(self, sel: np.ndarray, host_kv: np.ndarray | None = None,
             lengths: np.ndarray | None = None, caps: np.ndarray | None = None,
             mapped: np.ndarray | None = None, ctx_len: np.ndarray | None = None,
             tokens_per_entry: int = 1) -> dict:
        """Advance one step with selections sel [units][T][k], of which the
        first lengths[u][j] entries of each list are in use (all k when
        lengths is None), unit u using slots [0, caps[u]) (all S when caps
        is None; slots past it are emptied).  mapped [units][N] (bool):
        entries that have a host row (all when None); a miss without one is
        a range error of its unit.  ctx_len [batch]: context length of each
        request in tokens (None: every entry is in the context); entry e
        holds positions [e P, (e + 1) P), P = tokens_per_entry, and an id in
        use whose first position is at or past the length is a range error,
        as is a length outside [1, N P].  When the buffer is tracked,
        reserved slots receive host_kv[u][id] byte for byte."""
        c = self.cfg
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        assert sel.shape == (self.units, c.n_tokens, c.k)
        if lengths is not None:
            lengths = np.ascontiguousarray(lengths, dtype=np.int32).reshape(self.units, c.n_tokens)
        tk = c.n_tokens * c.k
        res = dict(
            hit_flag=np.zeros((self.units, c.n_tokens, c.k), dtype=np.uint8),
            sel_slot=np.zeros((self.units, c.n_tokens, c.k), dtype=np.int32),
            fill_slot=np.zeros((self.units, c.n_slots), dtype=np.int32),
            fill_id=np.zeros((self.units, c.n_slots), dtype=np.int32),
            counts=np.zeros((self.units, 4), dtype=np.int32),
            status=np.zeros(self.units, dtype=np.int32),
        )
        assert tk > 0
        if caps is not None:
            caps = np.ascontiguousarray(caps, dtype=np.int32).reshape(self.units)
        if mapped is not None:
            mapped = np.ascontiguousarray(mapped, dtype=np.uint8).reshape(self.units, c.n_entries)
        n_ctx = None
        if ctx_len is not None:
            n_ctx = context_entries(ctx_len, tokens_per_entry, c.n_entries)
            n_ctx = np.ascontiguousarray(np.repeat(n_ctx, self.units // len(n_ctx)), dtype=np.int32)
        _load().oracle_step(ctypes.byref(c), self.units, self.t, _p(sel),
                            None if lengths is None else _p(lengths),
                            None if caps is None else _p(caps), _p(self.slot_tok),
                            _p(self.life), _p(res["hit_flag"]), _p(res["sel_slot"]),
                            _p(res["fill_slot"]), _p(res["fill_id"]), _p(res["counts"]),
                            _p(res["status"]), None if mapped is None else _p(mapped),
                            None if n_ctx is None else _p(n_ctx))
        res["n_hit"] = res["counts"][:, 0].copy()
        res["n_miss"] = res["counts"][:, 1].copy()
        res["n_evict"] = res["counts"][:, 2].copy()
        res["n_union"] = res["counts"][:, 3].copy()
        if self.track_buf:
            assert host_kv is not None
            for u in range(self.units):
                m = res["n_miss"][u]
                if m:
                    self.buf[u, res["fill_slot"][u, :m]] = host_kv[u, res["fill_id"][u, :m]]
        self.t += 1
        return res

    def snapshot(self):
        return (self.t, self.slot_tok.copy(), self.life.copy(),
                None if self.buf is None else self.buf.copy())

    def restore(self, snap):
        self.t, st, lf, bf = snap
        self.slot_tok, self.life = st.copy(), lf.copy()
        self.buf = None if bf is None else bf.copy()


def context_entries(ctx_len, tokens_per_entry: int, n_entries: int) -> np.ndarray:
    """Entries holding tokens of each context: entry e holds positions
    [e P, (e + 1) P) and is in a context of length n when e P < n, so there
    are ceil(n / P) of them; 0 for a length outside [1, N P] (a range
    error)."""
    n = np.asarray(ctx_len, dtype=np.int64).reshape(-1)
    P = int(tokens_per_entry)
    ok = (n >= 1) & (n <= n_entries * P)
    return np.where(ok, (n + P - 1) // P, 0).astype(np.int32)


def unit_step(n_slots, n_entries, k, policy, lifetime_L, n_buckets, t, sel, slot_tok, life,
              lengths=None, cap=None, mapped=None, n_ctx=None, bucket_width=1):
    """Single-unit call for small hand-built cases: returns (status, result
    dict) and updates slot_tok / life (int32 arrays) in place.  lengths: the
    entries in use of each token's list (default: all k); cap: slots in use
    (default: all n_slots); mapped: [N] bool, entries with a host row
    (default: all); n_ctx: entries in the request's context (default: N);
    bucket_width: steps per LRU bucket."""
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    if sel.ndim == 1:
        sel = sel[None, :]
    T = sel.shape[0]
    cfg = _Cfg(n_slots, n_entries, T, k, LRU if policy in ("lru", LRU) else LIFETIME, lifetime_L,
               n_buckets, bucket_width)
    assert slot_tok.dtype == np.int32 and life.dtype == np.int32
    hit = np.zeros((T, k), np.uint8)
    ss = np.zeros((T, k), np.int32)
    fs = np.zeros(n_slots, np.int32)
    fi = np.zeros(n_slots, np.int32)
    cnt = np.zeros(4, np.int32)
    ln = None if lengths is None else np.ascontiguousarray(lengths, dtype=np.int32).reshape(T)
    mp = None if mapped is None else np.ascontiguousarray(mapped, dtype=np.uint8).reshape(n_entries)
    st = _load().oracle_unit_step(ctypes.byref(cfg), t, _p(sel), None if ln is None else _p(ln),
                                  n_slots if cap is None else int(cap), _p(slot_tok), _p(life), _p(hit),
                                  _p(ss), _p(fs), _p(fi), _p(cnt), None if mp is None else _p(mp),
                                  n_entries if n_ctx is None else int(n_ctx))
    m = int(cnt[1])
    return st, dict(hit_flag=hit, sel_slot=ss, fill_slot=fs[:m].copy(), fill_id=fi[:m].copy(),
                    n_hit=int(cnt[0]), n_miss=m, n_evict=int(cnt[2]), n_union=int(cnt[3]))
