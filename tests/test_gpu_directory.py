"""The host KV reached through the two-level directory (avsg_set_host_directory)
on the GPU, against the oracle on the same data laid out flat.  The pool
holds every (unit, entry) row at a random place, with spare rows of bf16 NaN,
so a row read from the wrong place shows in the attention output; the buffer
bytes, the slot state and the attention must match the oracle's, in every
transfer mode.  Entries without a row are range errors of their unit when
they miss; appends write through the directory."""
from __future__ import annotations

import numpy as np
import pytest

import tracegen as tg
import oracle
from oracle import attention as oatt
from oracle import append as oapp
from gpu_harness import check_attention, ensure_lib, say
from directory_inputs import build_directory, permuted_pool
from context_inputs import clip_to_context, nan_past_context, start_lengths

pytestmark = pytest.mark.gpu

CASES = {
    "token": (tg.WORKLOADS[2].replace(batch=3, n_kv_heads=2, n_q_heads=8, n_entries=3001, k=300,
                                      n_slots=900, steps=8), 64),
    "mtp": (tg.WORKLOADS[3].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=3001, k=200,
                                    n_slots=700, steps=6), 16),
    "lru_pages": (tg.WORKLOADS[4].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=601, k=37,
                                          n_slots=100, steps=8), 4),
    "latent": (tg.WORKLOADS[5].replace(batch=2, n_entries=3001, k=600, n_slots=1500, steps=5), 256),
}


class DirRun:
    """GPU context reading a permuted pool through a directory, beside the
    oracle reading the flat rows."""

    def __init__(self, w, seg, rng, mapping_filter=None, mode=None, split_rows=0, prepare=None):
        import torch
        avsg = ensure_lib()
        self.avsg, self.torch, self.w, self.seg = avsg, torch, w, seg
        self.flat = tg.fill_kv(w)
        if prepare is not None:      # changes the rows before the pool is laid out
            prepare(self.flat)
        pool, mapping = permuted_pool(self.flat, rng, extra_rows=w.units * 3)
        if mapping_filter is not None:
            mapping = {key: r for key, r in mapping.items() if mapping_filter(*key)}
        self.mapping = mapping
        top, segs = build_directory(mapping, w.units, w.n_entries, seg, spare_segments=1)
        self.mapped = np.zeros((w.units, w.n_entries), bool)
        for (u, e) in mapping:
            self.mapped[u, e] = True
        self.pool = avsg.HostBuffer(pool.shape)
        self.pool.array[...] = pool
        self.segs = avsg.HostBuffer(segs.shape, dtype=np.int32)
        self.segs.array[...] = segs
        self.top = torch.from_numpy(top).cuda()
        self.cfg = avsg.config_from_workload(w, split_rows)
        self.ctx = avsg.Context(self.cfg)
        if mode is not None:
            self.ctx.set_transfer_mode(mode)
        self.ctx.set_host_directory(self.top, self.segs, seg, len(segs), len(pool))
        self.st = avsg.State(self.cfg)
        self.ctx.reset(self.st.slot_table, self.st.lifetimes)
        self.ob = oracle.OracleBuffer.for_workload(w, track_buf=True)

    def step(self, t, sel_t):
        torch, w, s = self.torch, self.w, self.st
        q = tg.queries(w, t)
        self.ctx.step(torch.from_numpy(np.ascontiguousarray(sel_t)).cuda(),
                      torch.from_numpy(q.view(np.int16)).cuda(), self.pool, s.buf_kv,
                      s.slot_table, s.lifetimes, s.out, s.stats)
        torch.cuda.synchronize()
        r = self.ob.step(sel_t, self.flat, mapped=self.mapped)
        what = "t=%d" % t
        assert np.array_equal(s.slot_table.cpu().numpy(), self.ob.slot_tok), what
        assert np.array_equal(s.lifetimes.cpu().numpy(), self.ob.life), what
        assert np.array_equal(s.stats.sel_slot.cpu().numpy(), r["sel_slot"]), what
        assert np.array_equal(s.stats.hit_flag.cpu().numpy(), r["hit_flag"]), what
        assert np.array_equal(s.stats.n_miss.cpu().numpy(), r["n_miss"]), what
        assert np.array_equal(s.stats.unit_status.cpu().numpy(), r["status"]), what
        assert np.array_equal(s.buf_kv.cpu().numpy().view(np.uint16), self.ob.buf), what
        ref = oatt.attend(w, q, self.flat, sel_t, r["status"])
        check_attention(s.out.cpu().numpy(), ref, what)
        return r

    def close(self):
        self.ctx.close()
        self.pool.free()
        self.segs.free()


@pytest.mark.parametrize("name", list(CASES))
def test_directory_parity(name):
    w, seg = CASES[name]
    say("[directory] %s seg=%d units=%d" % (name, seg, w.units))
    sel = tg.selections(w)
    run = DirRun(w, seg, np.random.default_rng(len(name)))
    try:
        for t in range(w.steps):
            r = run.step(t, sel[t])
            assert (r["status"] == 0).all()
        assert run.ctx.last_error() == 0
    finally:
        run.close()


@pytest.mark.parametrize("mode", [1, 2, 3])
def test_directory_transfer_modes(mode):
    w, seg = CASES["token"]
    w = w.replace(steps=5)
    say("[directory] transfer mode %d" % mode)
    sel = tg.selections(w)
    run = DirRun(w, seg, np.random.default_rng(40 + mode), mode=mode)
    try:
        for t in range(w.steps):
            run.step(t, sel[t])
        assert run.ctx.last_error() == 0
    finally:
        run.close()


def test_unmapped_misses_are_unit_errors():
    """Unit 1 lacks rows for a few entries: a step where one of them misses
    is a range error of unit 1 alone, which keeps its state."""
    avsg = ensure_lib()
    w, seg = CASES["token"]
    w = w.replace(steps=8)
    sel = tg.selections(w)
    holes = set(int(x) for x in np.unique(sel[3:, 1]))   # selected from step 3 on
    holes = set(sorted(holes - set(int(x) for x in np.unique(sel[:3, 1])))[:3])
    say("[directory] unmapped entries %s" % sorted(holes))
    run = DirRun(w, seg, np.random.default_rng(77), mapping_filter=lambda u, e: not (u == 1 and e in holes))
    errors = 0
    try:
        for t in range(w.steps):
            before = run.st.slot_table[1].cpu().numpy().copy()
            r = run.step(t, sel[t])
            assert (np.delete(r["status"], 1) == 0).all()
            if r["status"][1] != 0:
                assert r["status"][1] == avsg.ERR_RANGE
                assert np.array_equal(run.st.slot_table[1].cpu().numpy(), before)
                errors += 1
        assert errors > 0
        assert run.ctx.last_error() == avsg.ERR_RANGE
    finally:
        run.close()


def test_append_through_the_directory():
    import torch
    avsg = ensure_lib()
    w, seg = CASES["lru_pages"]
    say("[directory] append")
    sel = tg.selections(w)
    run = DirRun(w, seg, np.random.default_rng(91),
                 mapping_filter=lambda u, e: not (u == w.units - 1 and e == 599))
    rng = np.random.default_rng(3)
    try:
        for t in range(4):
            run.step(t, sel[t])
            pos = np.array([sel[t, b * w.n_kv_heads, 0, 0] * w.tokens_per_entry + t
                            for b in range(w.batch)], np.int32)
            x = rng.standard_normal((w.units, w.head_dim_qk + w.head_dim_v)).astype(np.float32)
            new = (x.view(np.uint32) >> 16).astype(np.uint16)
            oapp.append(w, run.flat, new, pos, run.ob.slot_tok, run.ob.buf)
            run.ctx.append(torch.from_numpy(new.view(np.int16)).cuda(), torch.from_numpy(pos).cuda(),
                           run.pool, run.st.buf_kv, run.st.slot_table)
            torch.cuda.synchronize()
            for (u, e), row in run.mapping.items():
                assert np.array_equal(run.pool.array[row], run.flat[u, e]), (u, e)
            assert np.array_equal(run.st.buf_kv.cpu().numpy().view(np.uint16), run.ob.buf)
        assert run.ctx.last_error() == 0
        # an append to an entry without a row writes nothing and is a range error
        snapshot = run.pool.array.copy()
        pos = np.zeros(w.batch, np.int32)
        pos[-1] = 599 * w.tokens_per_entry
        new = np.ones((w.units, w.head_dim_qk + w.head_dim_v), np.uint16)
        run.ctx.append(torch.from_numpy(new.view(np.int16)).cuda(), torch.from_numpy(pos).cuda(),
                       run.pool, run.st.buf_kv, run.st.slot_table)
        torch.cuda.synchronize()
        assert run.ctx.last_error() == avsg.ERR_RANGE
        changed = np.nonzero((run.pool.array != snapshot).any(axis=1))[0]
        last = w.units - w.n_kv_heads          # first unit of the last request
        want = {run.mapping[(u, 0)] for u in range(last)}
        want |= {run.mapping[(u, 599)] for u in range(last, w.units - 1)}
        assert set(changed.tolist()) == want   # the last unit's entry 599 has no row
    finally:
        run.close()


def test_append_insert_through_the_directory():
    """Insertion reads the entry's whole row from its pool row; a unit whose
    entry has no row writes nothing (a range error of that unit alone)."""
    import torch
    avsg = ensure_lib()
    w, seg = CASES["lru_pages"]
    say("[directory] append with insertion")
    sel = tg.selections(w)
    hole = (w.units - 1, 599)
    run = DirRun(w, seg, np.random.default_rng(92), mapping_filter=lambda u, e: (u, e) != hole)
    rng = np.random.default_rng(4)
    try:
        for t in range(5):
            run.step(t, sel[t])
            # even steps: the first selected entry; odd: an unselected one
            ent = [int(sel[t, b * w.n_kv_heads, 0, 0]) if t % 2 == 0 else 590 + b
                   for b in range(w.batch)]
            pos = np.array([e * w.tokens_per_entry + t for e in ent], np.int32)
            x = rng.standard_normal((w.units, w.head_dim_qk + w.head_dim_v)).astype(np.float32)
            new = (x.view(np.uint32) >> 16).astype(np.uint16)
            st = oapp.append_insert(w, run.flat, new, pos, run.ob.slot_tok, run.ob.life, run.ob.buf,
                                    run.ob.t, mapped=run.mapped)
            assert (st == 0).all()
            run.ctx.append_insert(torch.from_numpy(new.view(np.int16)).cuda(),
                                  torch.from_numpy(pos).cuda(), run.pool, run.st.buf_kv,
                                  run.st.slot_table, run.st.lifetimes)
            torch.cuda.synchronize()
            for (u, e), row in run.mapping.items():
                assert np.array_equal(run.pool.array[row], run.flat[u, e]), (u, e)
            assert np.array_equal(run.st.slot_table.cpu().numpy(), run.ob.slot_tok)
            assert np.array_equal(run.st.lifetimes.cpu().numpy(), run.ob.life)
            assert np.array_equal(run.st.buf_kv.cpu().numpy().view(np.uint16), run.ob.buf)
        assert run.ctx.last_error() == 0
        # the last request inserts entry 599: its last unit has no row for it
        pos = np.full(w.batch, 3 * w.tokens_per_entry, np.int32)
        pos[-1] = 599 * w.tokens_per_entry
        new = np.ones((w.units, w.head_dim_qk + w.head_dim_v), np.uint16)
        st = oapp.append_insert(w, run.flat, new, pos, run.ob.slot_tok, run.ob.life, run.ob.buf,
                                run.ob.t, mapped=run.mapped)
        assert st.tolist() == [0] * (w.units - 1) + [oapp.ERR_RANGE]
        run.ctx.append_insert(torch.from_numpy(new.view(np.int16)).cuda(),
                              torch.from_numpy(pos).cuda(), run.pool, run.st.buf_kv,
                              run.st.slot_table, run.st.lifetimes)
        torch.cuda.synchronize()
        assert run.ctx.last_error() == avsg.ERR_RANGE
        for (u, e), row in run.mapping.items():
            assert np.array_equal(run.pool.array[row], run.flat[u, e]), (u, e)
        assert np.array_equal(run.st.slot_table.cpu().numpy(), run.ob.slot_tok)
        assert np.array_equal(run.st.lifetimes.cpu().numpy(), run.ob.life)
        assert np.array_equal(run.st.buf_kv.cpu().numpy().view(np.uint16), run.ob.buf)
        run.step(5, sel[5])
    finally:
        run.close()


def test_directory_bad_arguments():
    import torch
    avsg = ensure_lib()
    w, _ = CASES["token"]
    cfg = avsg.config_from_workload(w)
    ctx = avsg.Context(cfg)
    top = torch.zeros((w.units, 64), dtype=torch.int32, device="cuda")
    segs = avsg.HostBuffer((2, 64), dtype=np.int32)
    try:
        for seg, nseg, rows in ((48, 2, 10), (0, 2, 10), (64, 0, 10), (64, 2, 0), (64, 2, 2**31)):
            st = avsg.avsg_set_host_directory(ctx.handle, top.data_ptr(), segs.ptr, seg, nseg, rows)
            assert st == avsg.ERR_INVALID_ARG, (seg, nseg, rows)
        unpinned = np.zeros((2, 64), np.int32)
        st = avsg.avsg_set_host_directory(ctx.handle, top.data_ptr(), unpinned.ctypes.data, 64, 2, 10)
        assert st == avsg.ERR_NOT_PINNED
        assert avsg.avsg_set_host_directory(ctx.handle, top.data_ptr(), segs.ptr, 64, 2, 10) == avsg.OK
        assert avsg.avsg_set_host_directory(ctx.handle, None, None, 0, 0, 0) == avsg.OK
    finally:
        ctx.close()
        segs.free()


def test_directory_full_size_long_context():
    """The long-context workload at full size (256 units, 8192 pages of
    8 KiB each) with its host rows reached through a directory of 256-entry
    segments: state every step, attention on sampled units."""
    import torch
    avsg = ensure_lib()
    w = tg.WORKLOADS[4]
    seg, steps = 256, 24
    say("[directory] full size long, %d steps" % steps)
    n_seg = -(-w.n_entries // seg)
    host = avsg.HostBuffer((w.units, w.n_entries, w.row_elems))
    tg.fill_kv(w, out=host.array)
    # pool = the same rows; entry e of unit u at pool row u * N + e, one
    # segment per (unit, range of 256 entries), numbered in reverse so the
    # top level is not the identity
    segs = avsg.HostBuffer((w.units * n_seg, seg), dtype=np.int32)
    order = np.arange(w.units * n_seg)[::-1].reshape(w.units, n_seg).astype(np.int32)
    for u in range(w.units):
        for s in range(n_seg):
            segs.array[order[u, s]] = u * w.n_entries + s * seg + np.arange(seg)
    top = torch.from_numpy(order.copy()).cuda()
    cfg = avsg.config_from_workload(w)
    ctx = avsg.Context(cfg)
    ctx.set_host_directory(top, segs, seg, w.units * n_seg, w.units * w.n_entries)
    st = avsg.State(cfg)
    ctx.reset(st.slot_table, st.lifetimes)
    ob = oracle.OracleBuffer.for_workload(w)
    sel = tg.selections(w, steps=steps)
    units = [0, 37, 128, 255]
    try:
        for t in range(steps):
            q = tg.queries(w, t)
            ctx.step(torch.from_numpy(sel[t]).cuda(), torch.from_numpy(q.view(np.int16)).cuda(),
                     host.ptr, st.buf_kv, st.slot_table, st.lifetimes, st.out, st.stats)
            torch.cuda.synchronize()
            r = ob.step(sel[t])
            assert np.array_equal(st.slot_table.cpu().numpy(), ob.slot_tok), t
            assert np.array_equal(st.lifetimes.cpu().numpy(), ob.life), t
            assert np.array_equal(st.stats.sel_slot.cpu().numpy(), r["sel_slot"]), t
            if t in (0, steps - 1):
                ref = oatt.attend(w, q, host.array, sel[t], r["status"], units=units)
                check_attention(st.out.cpu().numpy(), ref, "t=%d" % t)
        assert ctx.last_error() == 0
    finally:
        ctx.close()
        host.free()
        segs.free()


COMBINED = {
    "token": (tg.WORKLOADS[2].replace(batch=3, n_kv_heads=2, n_q_heads=8, n_entries=3001, k=300,
                                      n_slots=900, steps=10), 64),
    "mtp_lru": (tg.WORKLOADS[3].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=3001, k=200,
                                        n_slots=700, steps=8, policy="lru", n_buckets=5), 16),
    "latent": (tg.WORKLOADS[5].replace(batch=2, n_entries=3001, k=600, n_slots=1500, steps=6), 256),
}


@pytest.mark.parametrize("name", list(COMBINED))
def test_lengths_sizes_and_directory_together(name):
    """Variable-length lists, a buffer size per unit that shrinks and grows
    between steps, and host rows reached through the directory, all in one
    trace: state, flags, slots, buffer bytes and attention against the
    oracle given the same lengths, sizes and flat rows."""
    w, seg = COMBINED[name]
    say("[directory] lengths + sizes + directory: %s" % name)
    rng = np.random.default_rng(97 + len(name))
    sel_full = tg.selections(w)
    sel, lens = tg.shorten(sel_full, seed=31 + len(name), lo=max(1, w.k // 8))
    lens = lens.reshape(w.steps, w.units, w.n_q_tokens)
    run = DirRun(w, seg, rng)
    torch = run.torch
    try:
        for t in range(w.steps):
            # sizes at least the union of this step's lists in use
            need = np.array([len(np.unique(np.concatenate(
                [sel[t, u, j, :lens[t, u, j]] for j in range(w.n_q_tokens)])))
                for u in range(w.units)], np.int32)
            caps = np.minimum(w.n_slots, need + rng.integers(0, w.n_slots // 2, size=w.units)).astype(np.int32)
            cap_dev = torch.from_numpy(caps).cuda()
            run.ctx.set_capacity(cap_dev)
            q = tg.queries(w, t)
            s = run.st
            ln_dev = torch.from_numpy(np.ascontiguousarray(lens[t].reshape(-1))).cuda()
            run.ctx.step(torch.from_numpy(np.ascontiguousarray(sel[t])).cuda(),
                         torch.from_numpy(q.view(np.int16)).cuda(), run.pool, s.buf_kv,
                         s.slot_table, s.lifetimes, s.out, s.stats, sel_len=ln_dev)
            torch.cuda.synchronize()
            r = run.ob.step(sel[t], run.flat, lengths=lens[t], caps=caps, mapped=run.mapped)
            what = "%s t=%d" % (name, t)
            assert (r["status"] == 0).all(), what
            assert np.array_equal(s.slot_table.cpu().numpy(), run.ob.slot_tok), what
            assert np.array_equal(s.lifetimes.cpu().numpy(), run.ob.life), what
            assert np.array_equal(s.stats.sel_slot.cpu().numpy(), r["sel_slot"]), what
            assert np.array_equal(s.stats.hit_flag.cpu().numpy(), r["hit_flag"]), what
            assert np.array_equal(s.stats.n_miss.cpu().numpy(), r["n_miss"]), what
            assert np.array_equal(s.stats.n_evict.cpu().numpy(), r["n_evict"]), what
            occ = run.ob.slot_tok >= 0
            assert np.array_equal(s.buf_kv.cpu().numpy().view(np.uint16)[occ], run.ob.buf[occ]), what
            ref = oatt.attend(w, q, run.flat, sel[t], r["status"], lengths=lens[t])
            check_attention(s.out.cpu().numpy(), ref, what)
        assert run.ctx.last_error() == 0
    finally:
        run.close()


EVERYTHING = {
    "pages16_lru": (tg.WORKLOADS[4].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=301, k=37,
                                            n_slots=100, steps=12, n_buckets=5), 16, 0),
    "pages3_lifetime": (tg.WORKLOADS[4].replace(batch=3, n_kv_heads=2, n_q_heads=8, n_entries=400,
                                                tokens_per_entry=3, k=11, n_slots=40, steps=10,
                                                policy="lifetime", lifetime_L=4), 8, 32),
}


@pytest.mark.parametrize("name", list(EVERYTHING))
def test_every_option_together(name):
    """Context lengths with a partly written last page (rows past each
    context hold NaN), list lengths whose last entry in use is that page,
    buffer sizes that change every step, host rows through the directory,
    and an insertion of each new token's entry after every step: state,
    flags, buffer bytes, host rows and attention against the oracle."""
    w, seg, split_rows = EVERYTHING[name]
    P = w.tokens_per_entry
    say("[everything] %s" % name)
    rng = np.random.default_rng(5 + len(name))
    ctx_len = start_lengths(w)
    run = DirRun(w, seg, rng, split_rows=split_rows,
                 prepare=lambda flat: nan_past_context(flat, w, ctx_len))
    torch = run.torch
    sel_full = tg.selections(w)
    _, lens = tg.shorten(sel_full, seed=7, lo=max(2, w.k // 4))
    lens = lens.reshape(w.steps, w.units, w.n_q_tokens)
    ob = run.ob
    try:
        for t in range(w.steps):
            sel_t = clip_to_context(sel_full[t], w, ctx_len)
            for u in range(w.units):           # the page with the context's end is in use
                last = (int(ctx_len[u // w.n_kv_heads]) - 1) // P
                for j in range(w.n_q_tokens):
                    sel_t[u, j, lens[t, u, j] - 1] = last
            need = np.array([len(np.unique(np.concatenate(
                [sel_t[u, j, :lens[t, u, j]] for j in range(w.n_q_tokens)])))
                for u in range(w.units)], np.int32)
            caps = np.minimum(w.n_slots, need + rng.integers(0, w.n_slots // 2, size=w.units))
            caps = caps.astype(np.int32)
            cap_dev = torch.from_numpy(caps).cuda()
            ctx_dev = torch.from_numpy(ctx_len).cuda()
            run.ctx.set_capacity(cap_dev)
            run.ctx.set_context_lengths(ctx_dev)
            q = tg.queries(w, t)
            s = run.st
            ln_dev = torch.from_numpy(np.ascontiguousarray(lens[t].reshape(-1))).cuda()
            run.ctx.step(torch.from_numpy(np.ascontiguousarray(sel_t)).cuda(),
                         torch.from_numpy(q.view(np.int16)).cuda(), run.pool, s.buf_kv,
                         s.slot_table, s.lifetimes, s.out, s.stats, sel_len=ln_dev)
            torch.cuda.synchronize()
            r = ob.step(sel_t, run.flat, lengths=lens[t], caps=caps, mapped=run.mapped,
                        ctx_len=ctx_len, tokens_per_entry=P)
            what = "%s t=%d" % (name, t)
            assert (r["status"] == 0).all(), what
            assert np.array_equal(s.slot_table.cpu().numpy(), ob.slot_tok), what
            assert np.array_equal(s.lifetimes.cpu().numpy(), ob.life), what
            assert np.array_equal(s.stats.sel_slot.cpu().numpy(), r["sel_slot"]), what
            assert np.array_equal(s.stats.hit_flag.cpu().numpy(), r["hit_flag"]), what
            assert np.array_equal(s.buf_kv.cpu().numpy().view(np.uint16), ob.buf), what
            ref = oatt.attend(w, q, run.flat, sel_t, r["status"], lengths=lens[t], ctx_len=ctx_len)
            check_attention(s.out.cpu().numpy(), ref, what)
            # the new token at position ctx_len, its entry made resident
            x = rng.standard_normal((w.units, w.head_dim_qk + w.head_dim_v)).astype(np.float32)
            new = (x.view(np.uint32) >> 16).astype(np.uint16)
            st = oapp.append_insert(w, run.flat, new, ctx_len, ob.slot_tok, ob.life, ob.buf, ob.t,
                                    caps=caps, mapped=run.mapped)
            assert (st == 0).all(), what
            run.ctx.append_insert(torch.from_numpy(new.view(np.int16)).cuda(), ctx_dev, run.pool,
                                  s.buf_kv, s.slot_table, s.lifetimes)
            torch.cuda.synchronize()
            for (u, e), row in run.mapping.items():
                assert np.array_equal(run.pool.array[row], run.flat[u, e]), (what, u, e)
            assert np.array_equal(s.slot_table.cpu().numpy(), ob.slot_tok), what
            assert np.array_equal(s.lifetimes.cpu().numpy(), ob.life), what
            assert np.array_equal(s.buf_kv.cpu().numpy().view(np.uint16), ob.buf), what
            ctx_len = ctx_len + 1
        assert run.ctx.last_error() == 0
    finally:
        run.close()
