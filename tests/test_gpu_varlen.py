"""Selections of a different size per unit (avsg_step_varlen) on the GPU vs
the oracle, through the C ABI: state bit-exact, buffer bytes bit-exact,
attention within tolerance, positions past a unit's length reported as
slot -1 / flag 0, and a length outside [1, k] reported as a range error of
that unit only."""
from __future__ import annotations

import numpy as np
import pytest

import tracegen as tg
from gpu_harness import Runner, say, ensure_lib

pytestmark = pytest.mark.gpu

CASES = {
    # lengths from 1 to k, splits of 256 rows partly or wholly unused
    "token": (tg.WORKLOADS[2].replace(batch=3, n_kv_heads=2, n_q_heads=8, n_entries=5003, k=700,
                                      n_slots=1500, steps=10), 1),
    "token_skewed": (tg.WORKLOADS[2].replace(batch=2, n_kv_heads=4, n_q_heads=16, n_entries=6000,
                                             k=1000, n_slots=2000, steps=8), 900),
    "page16": (tg.WORKLOADS[4].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=1001, k=37,
                                       n_slots=100, steps=12), 1),
    "page3": (tg.WORKLOADS[4].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=1000,
                                      tokens_per_entry=3, k=200, n_slots=400, steps=8), 1),
    "latent": (tg.WORKLOADS[5].replace(batch=3, n_entries=5003, k=1100, n_slots=2000, steps=6), 1),
    "tiny": (tg.WORKLOADS[1], 1),
}


def _trace(w, lo, seed):
    sel, lens = tg.shorten(tg.selections(w), seed, lo)
    if lo == 1:  # the extremes: one entry, and every entry
        lens[0, 0] = 1
        lens[min(1, w.steps - 1), -1] = w.k
        full = tg.selections(w)
        sel[min(1, w.steps - 1), -1, 0] = full[min(1, w.steps - 1), -1, 0]
        sel[0, 0, 0, 1:] = -1
    return sel, lens


@pytest.mark.parametrize("name", list(CASES))
def test_varlen_parity(name):
    w, lo = CASES[name]
    if lo > w.k:
        lo = w.k
    say("[varlen] %s units=%d k=%d" % (name, w.units, w.k))
    sel, lens = _trace(w, lo if name != "token_skewed" else 1, len(name))
    if name == "token_skewed":
        # one long list per step among short ones
        lens[:] = np.minimum(lens, 40)
        lens[:, 3] = w.k
        full = tg.selections(w)
        sel[:, 3] = full[:, 3]
    run = Runner(w)
    try:
        for t in range(w.steps):
            run.step_and_compare(t, sel[t], tg.queries(w, t), check_buf=True, lengths=lens[t])
        assert run.ctx.last_error() == 0
    finally:
        run.close()


@pytest.mark.parametrize("mode", ["merge", "hash_table", "transfer1", "transfer2", "transfer3"])
def test_varlen_modes(mode):
    avsg = ensure_lib()
    w, _ = CASES["token"]
    w = w.replace(steps=5)
    say("[varlen] modes %s" % mode)
    sel, lens = _trace(w, 1, 7)
    run = Runner(w, mode=int(mode[-1]) if mode.startswith("transfer") else None)
    if mode == "merge":
        run.ctx.set_match_mode(avsg.MATCH_MERGE)
    elif mode == "hash_table":
        run.ctx.set_match_mode(avsg.MATCH_HASH_TABLE)
    try:
        for t in range(w.steps):
            run.step_and_compare(t, sel[t], tg.queries(w, t), check_buf=True, lengths=lens[t])
    finally:
        run.close()


def test_varlen_bad_length_is_a_unit_error():
    avsg = ensure_lib()
    w, _ = CASES["token"]
    w = w.replace(steps=4)
    say("[varlen] bad length")
    sel, lens = _trace(w, 1, 3)
    run = Runner(w)
    try:
        run.step_and_compare(0, sel[0], tg.queries(w, 0), check_buf=True, lengths=lens[0])
        for t, bad in ((1, 0), (2, w.k + 1), (3, -7)):
            ln = lens[t].copy()
            ln[2] = bad
            r, _ = run.step_and_compare(t, sel[t], tg.queries(w, t), check_buf=True, lengths=ln)
            assert r["status"][2] == avsg.ERR_RANGE and (r["status"][np.arange(w.units) != 2] == 0).all()
            assert run.ctx.last_error() == avsg.ERR_RANGE
    finally:
        run.close()


MTP_CASES = {
    "mtp": tg.WORKLOADS[3].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=5003, k=300,
                                   n_slots=700, steps=10),
    "mtp_pages": tg.WORKLOADS[3].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=1001,
                                         tokens_per_entry=16, k=37, n_slots=100, steps=10),
    "mla_mtp": tg.WORKLOADS[5].replace(batch=2, n_q_tokens=2, overlap_shared=0.5, n_entries=5003,
                                       k=600, n_slots=1300, steps=6),
}


@pytest.mark.parametrize("name,mode", [(n, "hash") for n in MTP_CASES] +
                         [("mtp", "hash_table"), ("mtp", "merge")])
def test_varlen_two_tokens(name, mode):
    """Two query tokens with a length per token: the union is formed from
    the lists in use (direct-addressed, sorted-list and merge forms), a row
    is fetched by the first token whose list in use holds it, and each
    token attends over its own prefix."""
    avsg = ensure_lib()
    w = MTP_CASES[name]
    say("[varlen] two tokens %s %s" % (name, mode))
    sel, lens = tg.shorten(tg.selections(w), 21, 1)
    lens[0, 0] = [1, w.k]          # one entry beside a full list
    lens[1, -1] = [w.k, 1]
    full = tg.selections(w)
    sel[0, 0, 1] = full[0, 0, 1]
    sel[1, -1, 0] = full[1, -1, 0]
    run = Runner(w)
    if mode == "merge":
        run.ctx.set_match_mode(avsg.MATCH_MERGE)
    elif mode == "hash_table":
        run.ctx.set_match_mode(avsg.MATCH_HASH_TABLE)
    try:
        for t in range(w.steps):
            run.step_and_compare(t, sel[t], tg.queries(w, t), check_buf=True, lengths=lens[t])
        assert run.ctx.last_error() == 0
        # a bad length of either token is a range error of that unit
        ln = lens[w.steps - 1].copy()
        ln[1, 1] = w.k + 1
        r, _ = run.step_and_compare(w.steps, sel[w.steps - 1], tg.queries(w, w.steps - 1),
                                    check_buf=True, lengths=ln)
        assert r["status"][1] == avsg.ERR_RANGE
        assert run.ctx.last_error() == avsg.ERR_RANGE
    finally:
        run.close()


@pytest.mark.parametrize("cid", [2, 5])
def test_varlen_full_size(cid):
    """Full shapes with lengths from k/8 to k (PSA-style budgets): state
    bit-exact every step, attention of sampled units."""
    w = tg.WORKLOADS[cid]
    steps = 6
    say("[varlen-full] %s units=%d" % (w.name, w.units))
    sel, lens = tg.shorten(tg.selections(w, steps=steps), cid, w.k // 8)
    run = Runner(w, attn_units=[0, 7, w.units - 1])
    try:
        for t in range(steps):
            run.step_and_compare(t, sel[t], tg.queries(w, t), check_attn=(t % 2 == 1),
                                 lengths=lens[t])
        assert run.ctx.last_error() == 0
    finally:
        run.close()
