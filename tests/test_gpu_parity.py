"""HIP path vs oracle, element by element, through the C ABI.

State (slot tables, lifetimes / stamps, hit flags, slots, counts, buffer
bytes) must match bit for bit; attention within 2e-2 max abs and 1e-3
relative L1 per step."""
from __future__ import annotations

import numpy as np
import pytest

import tracegen as tg
from gpu_harness import Runner, say

pytestmark = pytest.mark.gpu

# Reduced shapes that span several tiles and end in ragged tails (k, S, N not
# multiples of 64/128/1024), plus the tiny workload at full size.
SMALL = {
    "tiny": tg.WORKLOADS[1],
    "batch_ragged": tg.WORKLOADS[2].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=5003,
                                            k=300, n_slots=1000, steps=14),
    "mtp_ragged": tg.WORKLOADS[3].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=5003,
                                          k=300, n_slots=700, steps=12),
    "long_ragged": tg.WORKLOADS[4].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=1001,
                                           k=37, n_slots=100, steps=40),
    "lru_small_b": tg.WORKLOADS[4].replace(batch=1, n_kv_heads=2, n_q_heads=4, n_entries=700,
                                           tokens_per_entry=1, k=50, n_slots=90, n_buckets=3,
                                           steps=30),
    "gqa8_L1": tg.WORKLOADS[2].replace(batch=1, n_kv_heads=2, n_q_heads=16, n_entries=3000,
                                       k=129, n_slots=300, lifetime_L=1, steps=10),
    "gqa1_k1": tg.WORKLOADS[2].replace(batch=3, n_kv_heads=1, n_q_heads=1, n_entries=64, k=1,
                                       n_slots=2, steps=10, overlap=0.0),
    "slots_16k": tg.WORKLOADS[2].replace(batch=1, n_kv_heads=2, n_q_heads=8, n_entries=40000,
                                         k=4000, n_slots=16384, steps=6),
    "mla_ragged": tg.WORKLOADS[5].replace(batch=3, n_entries=5003, k=700, n_slots=1500, steps=8),
    "mla_h64_short": tg.WORKLOADS[5].replace(batch=2, n_q_heads=64, n_entries=3000, k=45,
                                             n_slots=200, steps=8),
    "mla_mtp": tg.WORKLOADS[5].replace(batch=2, n_q_tokens=2, overlap_shared=0.5, n_entries=5003,
                                       k=600, n_slots=1300, steps=6),
}


# Edge shapes: k equal to the slot count, pages of 3 tokens whose rows straddle
# the 256-row attention splits, 32- and 256-token pages, the largest lifetime and
# bucket counts, 2 query heads per KV head, a single selected latent row, a
# latent head whose selection fits one split, and a context of 200000 ids.
EDGE = {
    "k_eq_S": tg.WORKLOADS[2].replace(batch=1, n_kv_heads=2, n_q_heads=8, n_entries=3000, k=200,
                                      n_slots=200, steps=8),
    "tpe3_straddle": tg.WORKLOADS[4].replace(batch=1, n_kv_heads=2, n_q_heads=8, n_entries=1000,
                                             tokens_per_entry=3, k=200, n_slots=400, steps=8),
    "tpe32": tg.WORKLOADS[4].replace(batch=1, n_kv_heads=2, n_q_heads=4, n_entries=300,
                                     tokens_per_entry=32, k=20, n_slots=40, steps=8),
    # the largest page the kernels take: 256 tokens (128 KiB rows), one page
    # per 256-row attention split
    "tpe256": tg.WORKLOADS[4].replace(batch=1, n_kv_heads=2, n_q_heads=4, n_entries=40,
                                      tokens_per_entry=256, k=6, n_slots=12, steps=8),
    "L126": tg.WORKLOADS[2].replace(batch=1, n_kv_heads=2, n_q_heads=8, n_entries=3000, k=150,
                                    n_slots=400, lifetime_L=126, steps=10),
    "B127": tg.WORKLOADS[4].replace(batch=1, n_kv_heads=2, n_q_heads=4, n_entries=2000,
                                    tokens_per_entry=1, k=100, n_slots=300, n_buckets=127, steps=12),
    "gqa2": tg.WORKLOADS[2].replace(batch=2, n_kv_heads=2, n_q_heads=4, n_entries=3000, k=333,
                                    n_slots=800, steps=8),
    "mla_k1": tg.WORKLOADS[5].replace(batch=2, n_entries=100, k=1, n_slots=4, steps=6, overlap=0.0),
    "mla_one_split": tg.WORKLOADS[5].replace(batch=2, n_entries=2000, k=300, n_slots=600, steps=6),
    # a context too large for direct addressing in LDS: the default match
    # takes the open-addressing hash table
    "big_context": tg.WORKLOADS[2].replace(batch=1, n_kv_heads=2, n_q_heads=8, n_entries=200000,
                                           k=200, n_slots=400, steps=8),
    # two-token reservations whose victims run past eviction bins 0..3 but
    # stay within bins 0..7 (lifetime 8, and 7 LRU buckets)
    "mtp_L8": tg.WORKLOADS[3].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=5003,
                                      k=300, n_slots=700, lifetime_L=8, steps=12),
    "mtp_lru_b7": tg.WORKLOADS[3].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=5003,
                                          k=300, n_slots=700, policy="lru", n_buckets=7,
                                          steps=12),
    # LRU buckets several steps wide: 3 steps (5 buckets, so ages past 14
    # share the oldest), 2 steps with two-token reservations, and 4-step
    # buckets of 16-token pages
    "lru_w3": tg.WORKLOADS[4].replace(batch=1, n_kv_heads=2, n_q_heads=4, n_entries=700,
                                      tokens_per_entry=1, k=50, n_slots=90, n_buckets=5,
                                      bucket_width=3, steps=30),
    "mtp_lru_w2": tg.WORKLOADS[3].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=5003,
                                          k=300, n_slots=700, policy="lru", n_buckets=7,
                                          bucket_width=2, steps=12),
    "pages_lru_w4": tg.WORKLOADS[4].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=1001,
                                            k=37, n_slots=100, n_buckets=3, bucket_width=4,
                                            steps=40),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_parity_edge(name):
    w = EDGE[name]
    say("[parity-edge] %s" % name)
    sel = tg.selections(w)
    run = Runner(w)
    try:
        for t in range(w.steps):
            run.step_and_compare(t, sel[t], tg.queries(w, t), check_buf=True)
    finally:
        run.close()


def test_parity_select_everything():
    """Every entry of the context selected every step (k = N = S): all misses
    on the first step, all hits afterwards."""
    w = tg.WORKLOADS[2].replace(batch=1, n_kv_heads=2, n_q_heads=8, n_entries=300, k=300,
                                n_slots=300, steps=5)
    say("[parity-edge] select everything")
    sel = np.broadcast_to(np.arange(w.k, dtype=np.int32), (w.steps, w.units, 1, w.k)).copy()
    run = Runner(w)
    try:
        for t in range(w.steps):
            r, _ = run.step_and_compare(t, sel[t], tg.queries(w, t), check_buf=True)
            if t == 0:
                assert (r["n_miss"] == w.k).all()
            else:
                assert (r["n_hit"] == w.k).all()
    finally:
        run.close()


@pytest.mark.parametrize("name", list(SMALL))
def test_parity_small(name):
    w = SMALL[name]
    say("[parity] %s units=%d k=%d S=%d T=%d" % (name, w.units, w.k, w.n_slots, w.n_q_tokens))
    sel = tg.selections(w)
    run = Runner(w)
    try:
        for t in range(w.steps):
            run.step_and_compare(t, sel[t], tg.queries(w, t), check_buf=True)
        assert run.ctx.last_error() == 0
    finally:
        run.close()


@pytest.mark.parametrize("name", ["batch_ragged", "mtp_ragged", "long_ragged", "mla_ragged"])
@pytest.mark.parametrize("transfer", [1, 2, 3])
def test_parity_transfer_modes(name, transfer):
    """The separate gather kernel (balanced shares, or one workgroup per unit)
    and the fused transfer forced into its gather-first form give the same
    state, buffer bytes and outputs as the oracle."""
    w = SMALL[name].replace(steps=6)
    say("[parity] %s transfer mode %d" % (name, transfer))
    sel = tg.selections(w)
    run = Runner(w, mode=transfer)
    try:
        for t in range(w.steps):
            run.step_and_compare(t, sel[t], tg.queries(w, t), check_buf=True)
    finally:
        run.close()


@pytest.mark.parametrize("mode", ["allhit", "allmiss"])
def test_parity_trace_modes(mode):
    w = SMALL["batch_ragged"].replace(n_entries=6000, steps=8)
    say("[parity] modes %s" % mode)
    sel = tg.selections(w, mode=mode)
    run = Runner(w)
    try:
        for t in range(w.steps):
            r, _ = run.step_and_compare(t, sel[t], tg.queries(w, t), check_buf=True)
            if mode == "allmiss":
                assert (r["n_hit"] == 0).all()
            elif t > 0:
                assert (r["n_miss"] == 0).all()
    finally:
        run.close()


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_parity_full_size(cid):
    """Full workload shapes, every step: all state bit-exact, attention of a
    sample of units against the oracle, buffer bytes at the end."""
    w = tg.WORKLOADS[cid]
    steps = w.steps
    say("[parity-full] %s units=%d steps=%d" % (w.name, w.units, steps))
    sel = tg.selections(w, steps=steps)
    rng = np.random.default_rng(cid)
    sample = sorted(rng.choice(w.units, size=min(6, w.units), replace=False).tolist())
    run = Runner(w, attn_units=sample)
    try:
        for t in range(steps):
            run.step_and_compare(t, sel[t], tg.queries(w, t), check_attn=(t % 4 == 0 or t == steps - 1))
        got = run.st.buf_kv.cpu().numpy().view(np.uint16)
        occ = run.ob.slot_tok >= 0
        assert np.array_equal(got[occ], run.ob.buf[occ])
        assert run.ctx.last_error() == 0
    finally:
        run.close()


def test_parity_full_size_wide_buckets():
    """The long-context workload at full size with LRU buckets 4 steps wide
    (64 of them), 64 steps: state bit-exact every step, attention of sampled
    units, buffer bytes at the end."""
    w = tg.WORKLOADS[4].replace(bucket_width=4, steps=64)
    say("[parity-full] %s buckets of 4 steps, units=%d steps=%d" % (w.name, w.units, w.steps))
    sel = tg.selections(w)
    rng = np.random.default_rng(44)
    sample = sorted(rng.choice(w.units, size=4, replace=False).tolist())
    run = Runner(w, attn_units=sample)
    try:
        for t in range(w.steps):
            run.step_and_compare(t, sel[t], tg.queries(w, t), check_attn=(t % 16 == 0))
        got = run.st.buf_kv.cpu().numpy().view(np.uint16)
        occ = run.ob.slot_tok >= 0
        assert np.array_equal(got[occ], run.ob.buf[occ])
        assert run.ctx.last_error() == 0
    finally:
        run.close()


def test_parity_full_size_small_buffer():
    """The long-context workload at full size with 384 slots per unit: the
    slots outside each union are few and young, so victims come from LRU
    buckets past the first eight bins (the general histogram and ranking);
    state bit-exact every step, attention of sampled units, buffer bytes."""
    w = tg.WORKLOADS[4].replace(n_slots=384, steps=48)
    say("[parity-full] %s 384 slots, units=%d steps=%d" % (w.name, w.units, w.steps))
    sel = tg.selections(w)
    rng = np.random.default_rng(45)
    sample = sorted(rng.choice(w.units, size=4, replace=False).tolist())
    run = Runner(w, attn_units=sample)
    try:
        for t in range(w.steps):
            run.step_and_compare(t, sel[t], tg.queries(w, t), check_attn=(t % 16 == 0))
        got = run.st.buf_kv.cpu().numpy().view(np.uint16)
        occ = run.ob.slot_tok >= 0
        assert np.array_equal(got[occ], run.ob.buf[occ])
        assert run.ctx.last_error() == 0
    finally:
        run.close()


def test_parity_full_size_hash_table():
    """The batch workload at full size, every step, matched by the
    open-addressing table at load factor 1/2 (its stated setting; the
    default mode direct-addresses this context): state bit-exact, attention
    of sampled units, buffer bytes at the end."""
    from gpu_harness import ensure_lib
    avsg = ensure_lib()
    w = tg.WORKLOADS[2]
    say("[parity-full] %s hash table, units=%d steps=%d" % (w.name, w.units, w.steps))
    sel = tg.selections(w)
    rng = np.random.default_rng(22)
    sample = sorted(rng.choice(w.units, size=6, replace=False).tolist())
    run = Runner(w, attn_units=sample)
    run.ctx.set_match_mode(avsg.MATCH_HASH_TABLE)
    try:
        for t in range(w.steps):
            run.step_and_compare(t, sel[t], tg.queries(w, t), check_attn=(t % 8 == 0))
        got = run.st.buf_kv.cpu().numpy().view(np.uint16)
        occ = run.ob.slot_tok >= 0
        assert np.array_equal(got[occ], run.ob.buf[occ])
        assert run.ctx.last_error() == 0
    finally:
        run.close()


@pytest.mark.parametrize("name", ["batch_ragged", "mtp_ragged", "lru_small_b", "tiny"])
@pytest.mark.parametrize("mode", ["merge", "hash_table"])
def test_parity_match_modes(name, mode):
    """The scalar dual-pointer matching baseline and the open-addressing hash
    table (which the default mode replaces by direct addressing on these
    small contexts) give the same state and outputs as the oracle."""
    from gpu_harness import ensure_lib
    avsg = ensure_lib()
    w = SMALL[name].replace(steps=min(SMALL[name].steps, 8))
    say("[parity] %s %s matching" % (name, mode))
    sel = tg.selections(w)
    run = Runner(w)
    run.ctx.set_match_mode(avsg.MATCH_MERGE if mode == "merge" else avsg.MATCH_HASH_TABLE)
    try:
        for t in range(w.steps):
            run.step_and_compare(t, sel[t], tg.queries(w, t), check_buf=True)
    finally:
        run.close()
