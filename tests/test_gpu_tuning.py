"""Results do not depend on how the work is cut: the same trace with other
attention split sizes (avsg_config.attn_split_rows) and other gather grids
(avsg_set_gather_workgroups, balanced transfer) gives bit-identical slot
state, hit statistics and buffer bytes, and attention within the oracle's
tolerance; the same settings twice give bit-identical outputs (nothing
depends on the order in which workgroups finish)."""
from __future__ import annotations

import numpy as np
import pytest

import tracegen as tg
from oracle import attention as oatt
from gpu_harness import check_attention, ensure_lib, say

pytestmark = pytest.mark.gpu

CASES = {
    "token": (tg.WORKLOADS[2].replace(batch=3, n_kv_heads=2, n_q_heads=8, n_entries=5003, k=300,
                                      n_slots=1000, steps=6), [0, 128, 64, 32]),
    "lru_pages": (tg.WORKLOADS[4].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=1001, k=37,
                                          n_slots=100, steps=6), [0, 128, 32]),
    "latent": (tg.WORKLOADS[5].replace(batch=2, n_entries=3001, k=700, n_slots=1500, steps=5),
               [0, 256, 96, 32]),
}


def _run(avsg, w, host, sel, split_rows, mode=0, grid=0):
    """Per step: (state and statistics as one tuple of arrays, outputs)."""
    import torch
    cfg = avsg.config_from_workload(w, attn_split_rows=split_rows)
    ctx = avsg.Context(cfg)
    ctx.set_transfer_mode(mode)
    if grid:
        ctx.set_gather_workgroups(grid)
    st = avsg.State(cfg)
    ctx.reset(st.slot_table, st.lifetimes)
    snaps, outs = [], []
    try:
        for t in range(w.steps):
            q = tg.queries(w, t)
            ctx.step(torch.from_numpy(sel[t]).cuda(), torch.from_numpy(q.view(np.int16)).cuda(), host,
                     st.buf_kv, st.slot_table, st.lifetimes, st.out, st.stats)
            torch.cuda.synchronize()
            snaps.append(tuple(x.cpu().numpy().copy() for x in (
                st.slot_table, st.lifetimes, st.buf_kv, st.stats.sel_slot, st.stats.hit_flag,
                st.stats.n_hit, st.stats.n_miss, st.stats.n_evict)))
            outs.append(st.out.cpu().numpy().copy())
        assert ctx.last_error() == 0
        splits = ctx.attn_splits
    finally:
        ctx.close()
    return snaps, outs, splits


@pytest.mark.parametrize("name", list(CASES))
def test_split_sizes_change_nothing_but_rounding(name):
    avsg = ensure_lib()
    w, split_list = CASES[name]
    sel = tg.selections(w)
    host = avsg.HostBuffer((w.units, w.n_entries, w.row_elems))
    tg.fill_kv(w, out=host.array)
    refs = [oatt.attend(w, tg.queries(w, t), host.array, sel[t]) for t in range(w.steps)]
    try:
        base = None
        for rows in split_list:
            snaps, outs, splits = _run(avsg, w, host, sel, rows)
            say("[tuning] %s split rows %d: %d splits" % (name, rows, splits))
            for t in range(w.steps):
                check_attention(outs[t], refs[t], "%s rows=%d t=%d" % (name, rows, t))
            if base is None:
                base = (snaps, outs)
                # the same cut twice: the same bits
                snaps2, outs2, _ = _run(avsg, w, host, sel, rows)
                for t in range(w.steps):
                    assert all(np.array_equal(a, b) for a, b in zip(snaps[t], snaps2[t])), t
                    assert np.array_equal(outs[t], outs2[t]), t
            else:
                for t in range(w.steps):
                    assert all(np.array_equal(a, b) for a, b in zip(base[0][t], snaps[t])), (rows, t)
    finally:
        host.free()


def test_gather_grids_change_nothing():
    avsg = ensure_lib()
    w, _ = CASES["token"]
    sel = tg.selections(w)
    host = avsg.HostBuffer((w.units, w.n_entries, w.row_elems))
    tg.fill_kv(w, out=host.array)
    try:
        base = None
        for grid in (0, 1, 7, 1000):
            snaps, outs, _ = _run(avsg, w, host, sel, 0, mode=avsg.TRANSFER_BALANCED, grid=grid)
            say("[tuning] gather grid %d" % grid)
            if base is None:
                base = (snaps, outs)
            else:
                for t in range(w.steps):
                    assert all(np.array_equal(a, b) for a, b in zip(base[0][t], snaps[t])), (grid, t)
                    assert np.array_equal(base[1][t], outs[t]), (grid, t)
        cfg = avsg.config_from_workload(w)
        ctx = avsg.Context(cfg)
        try:
            assert avsg.avsg_set_gather_workgroups(ctx.handle, -1) == avsg.ERR_INVALID_ARG
            assert avsg.avsg_set_gather_workgroups(ctx.handle, 65536) == avsg.ERR_INVALID_ARG
        finally:
            ctx.close()
    finally:
        host.free()
