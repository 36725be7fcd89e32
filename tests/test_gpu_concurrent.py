"""Several contexts on one GPU: each keeps its own workspace, state and step
counter, so contexts of different layouts stepped in turn on one stream, or
stepped concurrently on two streams, each match their own oracle step by
step (state bit for bit, attention within the parity tolerance)."""
from __future__ import annotations

import numpy as np
import pytest

import tracegen as tg
from gpu_harness import Runner, say

pytestmark = pytest.mark.gpu

SPLIT = tg.WORKLOADS[2].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=5003, k=300,
                                n_slots=1000, steps=10)
LATENT = tg.WORKLOADS[5].replace(batch=3, n_entries=5003, k=700, n_slots=1500, steps=10)
PAGED_LRU = tg.WORKLOADS[4].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=1001, k=37,
                                    n_slots=100, steps=10)


def test_contexts_of_different_layouts_interleave():
    """A split-layout lifetime context, a latent one and a paged bucketed-LRU
    one, created together and stepped in turn on the same stream."""
    say("[concurrent] three layouts interleaved")
    ws = [SPLIT, LATENT, PAGED_LRU]
    runs = [Runner(w) for w in ws]
    sels = [tg.selections(w) for w in ws]
    for t in range(min(w.steps for w in ws)):
        for run, w, sel in zip(runs, ws, sels):
            run.step_and_compare(t, sel[t], tg.queries(w, t), check_buf=True)
    for run, w in zip(runs, ws):
        assert run.ctx.t == min(x.steps for x in ws)
        assert run.ctx.last_error() == 0
        run.close()


def test_contexts_on_two_streams():
    """Two contexts on two streams, each step of both enqueued before the
    device synchronizes, so their kernels may run at the same time."""
    import torch
    say("[concurrent] two streams")
    s2 = torch.cuda.Stream()
    a = Runner(SPLIT)
    with torch.cuda.stream(s2):
        b = Runner(LATENT)
    torch.cuda.synchronize()
    sa, sb = tg.selections(SPLIT), tg.selections(LATENT)
    for t in range(min(SPLIT.steps, LATENT.steps)):
        qa, qb = tg.queries(SPLIT, t), tg.queries(LATENT, t)
        # inputs on the device before either stream's kernels read them
        dev = [(torch.from_numpy(np.ascontiguousarray(s[t])).cuda(),
                torch.from_numpy(q.view(np.int16)).cuda()) for s, q in ((sa, qa), (sb, qb))]
        torch.cuda.synchronize()
        for run, (sel_d, q_d) in zip((a, b), dev):
            run.ctx.step(sel_d, q_d, run.host, run.st.buf_kv, run.st.slot_table, run.st.lifetimes,
                         run.st.out, run.st.stats)
        torch.cuda.synchronize()
        a.compare(t, sa[t], qa, check_buf=True)
        b.compare(t, sb[t], qb, check_buf=True)
    assert a.ctx.last_error() == 0 and b.ctx.last_error() == 0
    a.close()
    b.close()


def test_context_moves_to_another_stream():
    """A context's later calls go to the stream avsg_set_stream names: steps
    continue there, with the step counter kept in the workspace."""
    import torch
    say("[concurrent] set_stream")
    w = PAGED_LRU
    run = Runner(w)
    sel = tg.selections(w)
    half = w.steps // 2
    for t in range(half):
        run.step_and_compare(t, sel[t], tg.queries(w, t), check_buf=True)
    s2 = torch.cuda.Stream()
    run.ctx.set_stream(s2)
    for t in range(half, w.steps):
        q = tg.queries(w, t)
        sel_d = torch.from_numpy(np.ascontiguousarray(sel[t])).cuda()
        q_d = torch.from_numpy(q.view(np.int16)).cuda()
        torch.cuda.synchronize()   # inputs in place before s2's kernels read them
        run.ctx.step(sel_d, q_d, run.host, run.st.buf_kv, run.st.slot_table, run.st.lifetimes,
                     run.st.out, run.st.stats)
        s2.synchronize()
        run.compare(t, sel[t], q, check_buf=True)
    assert run.ctx.t == w.steps
    assert run.ctx.last_error() == 0
    run.close()
