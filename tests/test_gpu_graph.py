"""Steps captured in a HIP graph and replayed (through torch.cuda.graph on
the context's stream), against the oracle.

The step counter lives in the workspace and the match kernel advances it, so
a replayed step uses the right step number: with bucketed LRU every stamp and
bucket depends on it.  One step runs eagerly, one is captured, and each
replay reads the next step's selections and queries from the same device
buffers, which are refilled between replays by ordinary copies; every
replay's state, flags, buffer bytes and attention must match the oracle's
step, and the counter must have advanced once per replay."""
from __future__ import annotations

import numpy as np
import pytest

import tracegen as tg
import oracle
from oracle import attention as oatt
from gpu_harness import check_attention, ensure_lib, say
from context_inputs import clip_to_context, nan_past_context

pytestmark = pytest.mark.gpu

CASES = {
    "tokens_lifetime": tg.WORKLOADS[2].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=3001,
                                               k=300, n_slots=700, steps=8),
    "pages_lru": tg.WORKLOADS[4].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=601, k=37,
                                         n_slots=100, n_buckets=5, steps=10),
    "mtp_lru": tg.WORKLOADS[3].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=3001, k=200,
                                       n_slots=600, policy="lru", n_buckets=6, steps=8),
    "latent": tg.WORKLOADS[5].replace(batch=2, n_entries=3001, k=600, n_slots=1500, steps=6),
}


@pytest.mark.parametrize("name", list(CASES))
def test_captured_step_replays(name):
    import torch
    avsg = ensure_lib()
    w = CASES[name]
    say("[graph] %s policy=%s" % (name, w.policy))
    cfg = avsg.config_from_workload(w)
    stream = torch.cuda.Stream()
    ctx = avsg.Context(cfg, stream=stream)
    st = avsg.State(cfg)
    host = avsg.HostBuffer((w.units, w.n_entries, w.row_elems))
    tg.fill_kv(w, out=host.array)
    ob = oracle.OracleBuffer.for_workload(w, track_buf=True)
    sel = tg.selections(w)
    sel_dev = torch.empty(sel[0].shape, dtype=torch.int32, device="cuda")
    q_dev = torch.empty((w.batch, w.n_q_tokens, w.n_q_heads, w.head_dim_qk), dtype=torch.int16,
                        device="cuda")

    def load(t):
        with torch.cuda.stream(stream):
            sel_dev.copy_(torch.from_numpy(np.ascontiguousarray(sel[t])))
            q_dev.copy_(torch.from_numpy(tg.queries(w, t).view(np.int16)))

    def step():
        ctx.step(sel_dev, q_dev, host, st.buf_kv, st.slot_table, st.lifetimes, st.out, st.stats)

    def compare(t):
        torch.cuda.synchronize()
        r = ob.step(sel[t], host.array)
        what = "%s t=%d" % (name, t)
        assert np.array_equal(st.slot_table.cpu().numpy(), ob.slot_tok), what
        assert np.array_equal(st.lifetimes.cpu().numpy(), ob.life), what
        assert np.array_equal(st.stats.sel_slot.cpu().numpy(), r["sel_slot"]), what
        assert np.array_equal(st.stats.hit_flag.cpu().numpy(), r["hit_flag"]), what
        assert np.array_equal(st.stats.n_miss.cpu().numpy(), r["n_miss"]), what
        assert np.array_equal(st.buf_kv.cpu().numpy().view(np.uint16), ob.buf), what
        ref = oatt.attend(w, tg.queries(w, t), host.array, sel[t], r["status"])
        check_attention(st.out.cpu().numpy(), ref, what)
        assert ctx.t == t + 1, what

    try:
        with torch.cuda.stream(stream):
            ctx.reset(st.slot_table, st.lifetimes)
        load(0)
        with torch.cuda.stream(stream):
            step()
        compare(0)
        graph = torch.cuda.CUDAGraph()
        load(1)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            step()                       # recorded, not run
        assert ctx.t == 1
        for t in range(1, w.steps):
            load(t)
            with torch.cuda.stream(stream):
                graph.replay()
            compare(t)
        assert ctx.last_error() == avsg.OK
    finally:
        ctx.close()
        host.free()


def test_captured_step_reads_settings_at_replay():
    """The context keeps its buffer sizes and context lengths by pointer: a
    captured step reads the arrays' contents when it is replayed.  Both are
    rewritten before every replay (contexts grow by one token per step and
    end inside a page; sizes change), against the oracle given the same."""
    import torch
    avsg = ensure_lib()
    w = CASES["pages_lru"].replace(steps=12)
    P = w.tokens_per_entry
    say("[graph] settings read at replay")
    cfg = avsg.config_from_workload(w)
    stream = torch.cuda.Stream()
    ctx = avsg.Context(cfg, stream=stream)
    st = avsg.State(cfg)
    host = avsg.HostBuffer((w.units, w.n_entries, w.row_elems))
    tg.fill_kv(w, out=host.array)
    ctx_len = np.array([(w.n_entries - 4) * P + 3, (w.n_entries - 4) * P + 9], np.int32)
    nan_past_context(host.array, w, ctx_len)
    ob = oracle.OracleBuffer.for_workload(w, track_buf=True)
    rng = np.random.default_rng(12)
    sel = tg.selections(w)
    sel_dev = torch.empty(sel[0].shape, dtype=torch.int32, device="cuda")
    q_dev = torch.empty((w.batch, 1, w.n_q_heads, w.head_dim_qk), dtype=torch.int16, device="cuda")
    cap_dev = torch.empty(w.units, dtype=torch.int32, device="cuda")
    len_dev = torch.empty(w.batch, dtype=torch.int32, device="cuda")
    ctx.set_capacity(cap_dev)
    ctx.set_context_lengths(len_dev)
    try:
        with torch.cuda.stream(stream):
            ctx.reset(st.slot_table, st.lifetimes)
        graph = None
        for t in range(w.steps):
            sel_t = clip_to_context(sel[t], w, ctx_len)
            caps = np.minimum(w.n_slots, w.k + rng.integers(0, w.n_slots, size=w.units)).astype(np.int32)
            with torch.cuda.stream(stream):
                sel_dev.copy_(torch.from_numpy(sel_t))
                q_dev.copy_(torch.from_numpy(tg.queries(w, t).view(np.int16)))
                cap_dev.copy_(torch.from_numpy(caps))
                len_dev.copy_(torch.from_numpy(ctx_len))
            torch.cuda.synchronize()
            if t == 0:
                with torch.cuda.stream(stream):
                    ctx.step(sel_dev, q_dev, host, st.buf_kv, st.slot_table, st.lifetimes, st.out,
                             st.stats)
            else:
                if graph is None:
                    graph = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(graph, stream=stream):
                        ctx.step(sel_dev, q_dev, host, st.buf_kv, st.slot_table, st.lifetimes,
                                 st.out, st.stats)
                with torch.cuda.stream(stream):
                    graph.replay()
            torch.cuda.synchronize()
            r = ob.step(sel_t, host.array, caps=caps, ctx_len=ctx_len, tokens_per_entry=P)
            what = "t=%d" % t
            assert (r["status"] == 0).all(), what
            assert np.array_equal(st.slot_table.cpu().numpy(), ob.slot_tok), what
            assert np.array_equal(st.lifetimes.cpu().numpy(), ob.life), what
            assert np.array_equal(st.buf_kv.cpu().numpy().view(np.uint16), ob.buf), what
            ref = oatt.attend(w, tg.queries(w, t), host.array, sel_t, r["status"], ctx_len=ctx_len)
            check_attention(st.out.cpu().numpy(), ref, what)
            assert ctx.t == t + 1, what
            ctx_len = ctx_len + 1
        assert ctx.last_error() == avsg.OK
    finally:
        ctx.close()
        host.free()
