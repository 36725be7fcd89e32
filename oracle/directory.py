"""ORACLE -- test infrastructure only (tests and the smoke check).

The two-level directory of the host KV pool (Spin summary, gist.science
2604.26837, section 2C: a small top-level directory on the GPU points to
second-level segments allocated on demand in CPU memory), written as its
definition: entry e of unit u lives at pool row

    segments[top[u][e // seg_entries]][e % seg_entries]

where a top-level value outside [0, len(segments)) means "no segment" and
a row outside [0, pool_rows) means "not mapped".
"""
from __future__ import annotations

import numpy as np


def resolve(top, segments, seg_entries: int, pool_rows: int, u: int, e: int) -> int:
    """Pool row of entry e of unit u, or -1 if the entry has none."""
    s = int(top[u][e // seg_entries])
    if s < 0 or s >= len(segments):
        return -1
    r = int(segments[s][e % seg_entries])
    return r if 0 <= r < pool_rows else -1


def flat_view(pool, top, segments, seg_entries: int, units: int, n_entries: int):
    """The pool seen through the directory as the flat host KV
    [units][n_entries][row] (zeros where unmapped) and the mapped mask
    [units][n_entries]."""
    flat = np.zeros((units, n_entries) + pool.shape[1:], dtype=pool.dtype)
    mapped = np.zeros((units, n_entries), dtype=bool)
    for u in range(units):
        for e in range(n_entries):
            r = resolve(top, segments, seg_entries, len(pool), u, e)
            if r >= 0:
                flat[u, e] = pool[r]
                mapped[u, e] = True
    return flat, mapped
