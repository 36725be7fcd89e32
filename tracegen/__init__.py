"""Seeded synthetic workloads for the sparse-attention KV slot buffer.

This package generates inputs only: bf16 K/V rows for the host-resident KV
cache, bf16 queries and per-step top-k selections.  It contains none of the
buffer-management method (matching, eviction, gather, attention); the HIP path
and the CPU oracle both take its output as plain arrays.

The five workloads follow the shapes the AVSG abstract (arxivdaily 2609.37538,
abstract) and the Spin summary (gist.science 2604.26837, section 2B) describe:
GQA decode over token entries, multi-token prediction with one shared
reservation, 16-token head-wise pages under a 64-bucket LRU, and a single
latent KV head with 128 query heads.  The pages' own datasets are not
available; Zipf(1.1)-tailed selections with a fixed step-to-step overlap
stand in for them.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tracegen.c")
_LIB_PATH = os.path.join(_HERE, "libtracegen.so")
_lib = None
_lock = threading.Lock()

MODE_NATURAL, MODE_ALL_HIT, MODE_ALL_MISS, MODE_SKEWED = 0, 1, 2, 3
_MODES = {"natural": MODE_NATURAL, "allhit": MODE_ALL_HIT, "allmiss": MODE_ALL_MISS,
          "skewed": MODE_SKEWED}


def build(force: bool = False) -> str:
    """Compile libtracegen.so with gcc (OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", _SRC,
                               "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            i64, u64, p = ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p
            lib.tg_fill_kv_rows.argtypes = [u64, i64, i64, i64, i64, p]
            lib.tg_fill_kv.argtypes = [u64, i64, i64, i64, p]
            lib.tg_fill_q.argtypes = [u64, i64, i64, p]
            lib.tg_permutation.argtypes = [u64, i64, i64, p]
            lib.tg_selections.argtypes = [u64, i64, i64, i64, i64, i64, ctypes.c_double,
                                          ctypes.c_double, ctypes.c_double, ctypes.c_int, p]
            lib.tg_selections.restype = ctypes.c_int
            lib.tg_rnd.argtypes = [u64, u64]
            lib.tg_rnd.restype = u64
            lib.tg_key2.argtypes = [u64, u64, u64]
            lib.tg_key2.restype = u64
            _lib = lib
    return _lib


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape, policy and trace recipe of one workload."""
    name: str
    batch: int
    n_kv_heads: int
    n_q_heads: int
    n_q_tokens: int
    head_dim_qk: int
    head_dim_v: int
    latent: bool          # one row per token serves as K (all dims) and V (first head_dim_v dims)
    n_entries: int        # N: entries per unit in the host KV
    tokens_per_entry: int
    k: int                # selected entries per query token
    n_slots: int          # S: device buffer slots per unit
    policy: str           # "lifetime" or "lru"
    lifetime_L: int
    n_buckets: int
    steps: int
    overlap: float        # fraction of the previous selection kept
    overlap_shared: float  # MTP: fraction of token 0's selection in token j's
    zipf_s: float
    seed: int
    bucket_width: int = 1  # steps per LRU bucket

    @property
    def units(self) -> int:
        return self.batch * self.n_kv_heads

    @property
    def row_elems(self) -> int:
        if self.latent:
            return self.head_dim_qk
        return self.tokens_per_entry * (self.head_dim_qk + self.head_dim_v)

    @property
    def row_bytes(self) -> int:
        return 2 * self.row_elems

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim_qk))

    @property
    def entries_per_step(self) -> int:
        """Selected KV entries per decode step, counted in tokens."""
        return self.units * self.n_q_tokens * self.k * self.tokens_per_entry

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _wl(cid, name, **kw):
    base = dict(n_q_tokens=1, head_dim_qk=128, head_dim_v=128, latent=False, tokens_per_entry=1,
                policy="lifetime", lifetime_L=16, n_buckets=64, overlap_shared=0.0, zipf_s=1.1,
                seed=20261200 + cid)
    base.update(kw)
    return Workload(name=name, **base)


WORKLOADS = {
    1: _wl(1, "tiny", batch=1, n_kv_heads=1, n_q_heads=4, n_entries=4096, k=256, n_slots=512,
           lifetime_L=8, steps=32, overlap=0.8),
    2: _wl(2, "batch", batch=8, n_kv_heads=8, n_q_heads=32, n_entries=32768, k=2048,
           n_slots=8192, steps=64, overlap=0.9),
    3: _wl(3, "mtp", batch=8, n_kv_heads=8, n_q_heads=32, n_q_tokens=2, n_entries=32768, k=2048,
           n_slots=8192, steps=64, overlap=0.9, overlap_shared=0.7),
    4: _wl(4, "long", batch=32, n_kv_heads=8, n_q_heads=32, n_entries=8192, tokens_per_entry=16,
           k=128, n_slots=1024, policy="lru", steps=128, overlap=0.85),
    5: _wl(5, "mla", batch=64, n_kv_heads=1, n_q_heads=128, head_dim_qk=576, head_dim_v=512,
           latent=True, n_entries=131072, k=2048, n_slots=8192, steps=64, overlap=0.9),
}


def _ptr(a: np.ndarray) -> int:
    assert a.flags.c_contiguous
    return a.ctypes.data


def fill_kv(w: Workload, out: np.ndarray | None = None, unit0: int = 0, units: int | None = None):
    """bf16 bit patterns (uint16) of the host KV, [units][N][row_elems]."""
    lib = _load()
    units = w.units - unit0 if units is None else units
    shape = (units, w.n_entries, w.row_elems)
    if out is None:
        out = np.empty(shape, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.size == int(np.prod(shape))
    per = w.n_entries * w.row_elems
    base = _ptr(out)
    for i in range(units):
        lib.tg_fill_kv_rows(w.seed, unit0 + i, w.row_elems, 0, w.n_entries, base + 2 * i * per)
    return out


def fill_kv_rows(w: Workload, unit: int, row0: int, nrows: int) -> np.ndarray:
    """Rows [row0, row0+nrows) of one unit, identical to the same rows of fill_kv."""
    out = np.empty((nrows, w.row_elems), dtype=np.uint16)
    _load().tg_fill_kv_rows(w.seed, unit, w.row_elems, row0, nrows, _ptr(out))
    return out


def queries(w: Workload, step: int) -> np.ndarray:
    """bf16 bit patterns of step `step`'s queries, [batch][T][Hq][dqk]."""
    shape = (w.batch, w.n_q_tokens, w.n_q_heads, w.head_dim_qk)
    out = np.empty(shape, dtype=np.uint16)
    _load().tg_fill_q(w.seed, step, out.size, _ptr(out))
    return out


def selections(w: Workload, steps: int | None = None, mode: str = "natural") -> np.ndarray:
    """int32 [steps][units][T][k], each list strictly ascending in [0, N)."""
    steps = w.steps if steps is None else steps
    out = np.empty((steps, w.units, w.n_q_tokens, w.k), dtype=np.int32)
    rc = _load().tg_selections(w.seed, w.units, w.n_entries, w.k, w.n_q_tokens, steps, w.overlap,
                               w.overlap_shared, w.zipf_s, _MODES[mode], _ptr(out))
    if rc != 0:
        raise ValueError("selection recipe cannot be satisfied for %s" % (w.name,))
    return out


def shorten(sel: np.ndarray, seed: int, lo: int, hi: int | None = None,
            pad: int = -1) -> tuple[np.ndarray, np.ndarray]:
    """Variable-size selections from fixed-size ones: for every (step, unit,
    query token) a length drawn uniformly from [lo, hi] (hi defaults to k),
    and that many of the k entries, chosen uniformly (numpy generator seeded
    with `seed`), kept in ascending order at the front of the list; the
    positions after them hold `pad`.  Returns (lists [steps][units][T][k],
    lengths [steps][units] for one token, else [steps][units][T])."""
    steps, units, T, k = sel.shape
    hi = k if hi is None else hi
    rng = np.random.default_rng(seed)
    out = np.full_like(sel, pad)
    lens = rng.integers(lo, hi + 1, size=(steps, units, T)).astype(np.int32)
    for t in range(steps):
        for u in range(units):
            for j in range(T):
                n = int(lens[t, u, j])
                keep = np.sort(rng.choice(k, size=n, replace=False))
                out[t, u, j, :n] = sel[t, u, j, keep]
    return out, (lens[:, :, 0] if T == 1 else lens)


def permutation(w: Workload, unit: int) -> np.ndarray:
    out = np.empty(w.n_entries, dtype=np.int32)
    _load().tg_permutation(w.seed, unit, w.n_entries, _ptr(out))
    return out


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def splitmix_output(key: int, i: int) -> int:
    return int(_load().tg_rnd(key, i))
