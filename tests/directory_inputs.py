"""Inputs for tests of the two-level host directory: a pool of host rows
and the directory that maps (unit, entry) to pool rows, built from a plain
{(unit, entry): pool row} mapping.  Segments are handed out in order of
first need, as an on-demand allocator would; the rest of a segment is -1."""
from __future__ import annotations

import numpy as np


def build_directory(mapping: dict, units: int, n_entries: int, seg_entries: int,
                    spare_segments: int = 0):
    """(top int32 [units][n_seg], segments int32 [n_segments][seg_entries])."""
    n_seg = -(-n_entries // seg_entries)
    top = np.full((units, n_seg), -1, np.int32)
    segs = []
    for (u, e) in sorted(mapping):
        s = e // seg_entries
        if top[u, s] < 0:
            top[u, s] = len(segs)
            segs.append(np.full(seg_entries, -1, np.int32))
        segs[top[u, s]][e % seg_entries] = mapping[(u, e)]
    segs += [np.full(seg_entries, -1, np.int32) for _ in range(spare_segments)]
    if not segs:
        segs = [np.full(seg_entries, -1, np.int32)]
    return top, np.stack(segs)


def permuted_pool(flat: np.ndarray, rng, extra_rows: int = 0, fill: int = 0x7FC0):
    """Every (unit, entry) row of flat [units][N][row] placed at a random
    row of a pool with extra_rows more rows (those hold `fill`, a bf16 NaN,
    so reading one of them shows).  Returns (pool, mapping)."""
    units, n, row = flat.shape
    rows = units * n + extra_rows
    perm = rng.permutation(rows)[:units * n]
    pool = np.full((rows, row), fill, flat.dtype)
    pool[perm] = flat.reshape(units * n, row)
    mapping = {(u, e): int(perm[u * n + e]) for u in range(units) for e in range(n)}
    return pool, mapping
