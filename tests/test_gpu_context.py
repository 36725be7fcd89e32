"""Context lengths on the GPU (avsg_set_context_lengths) against the oracle,
through the C ABI: the last page of each context is only partly written, and
grows by one appended token per step.

The rows of every page past each context hold bf16 NaN in host memory until
a token is appended there, so a row attended past the context, or a masked
row whose value still reaches the output, shows as a non-finite output.  Every
list holds the page with the context's end.  Buffer bytes (whole rows,
NaN included), slot state and attention must match the oracle's after every
step, in each transfer mode, with split sizes that put the context's end
inside a split, at a split boundary and past a split's start (a split of
masked rows only)."""
from __future__ import annotations

import numpy as np
import pytest

import tracegen as tg
from gpu_harness import Runner, say
from context_inputs import clip_to_context, nan_past_context, start_lengths
from oracle import append as oapp

pytestmark = pytest.mark.gpu


CASES = {
    # name: (workload, attention split rows (0: the library's), transfer mode)
    "pages16": (tg.WORKLOADS[4].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=301, k=37,
                                        n_slots=100, steps=20), 0, None),
    "pages3_split32": (tg.WORKLOADS[4].replace(batch=3, n_kv_heads=2, n_q_heads=8, n_entries=400,
                                               tokens_per_entry=3, k=11, n_slots=40, steps=10,
                                               policy="lifetime", lifetime_L=4), 32, None),
    "pages16_mtp": (tg.WORKLOADS[3].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=300,
                                            tokens_per_entry=16, k=40, n_slots=120, steps=18), 0,
                    None),
    "pages16_gather_first": (tg.WORKLOADS[4].replace(batch=2, n_kv_heads=2, n_q_heads=8,
                                                     n_entries=301, k=37, n_slots=100, steps=12),
                             64, 3),
    "pages3_gather_first": (tg.WORKLOADS[4].replace(batch=3, n_kv_heads=2, n_q_heads=8,
                                                    n_entries=400, tokens_per_entry=3, k=11,
                                                    n_slots=40, steps=10), 32, 3),
    "pages16_balanced": (tg.WORKLOADS[4].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=301,
                                                 k=37, n_slots=100, steps=12), 0, 1),
    "tokens": (tg.WORKLOADS[2].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=3001, k=300,
                                       n_slots=700, steps=8), 0, None),
}


def _tokens(w, rng):
    x = rng.standard_normal((w.units, w.head_dim_qk + w.head_dim_v)).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("name", list(CASES))
def test_partial_last_page_grows_by_appends(name):
    from device_buffer_reuse_amd import avsg
    w, split_rows, mode = CASES[name]
    P, N = w.tokens_per_entry, w.n_entries
    say("[context] %s units=%d P=%d split_rows=%d mode=%s" % (name, w.units, P, split_rows, mode))
    sel = tg.selections(w)
    rng = np.random.default_rng(len(name))
    run = Runner(w, mode=mode, split_rows=split_rows)
    # contexts end early enough to grow for every step: one token into a
    # page for request 0, the last token of a page for request 1, mid-page
    # after that
    ctx_len = start_lengths(w)
    nan_past_context(run.host.array, w, ctx_len)
    torch = run.torch
    try:
        for t in range(w.steps):
            run.set_ctx_len(ctx_len)
            s_t = clip_to_context(sel[t], w, ctx_len)
            r, _ = run.step_and_compare(t, s_t, tg.queries(w, t), check_buf=True)
            assert (r["status"] == 0).all()
            # the new token of every request goes to position ctx_len (into
            # the resident last page, or the first row of the next one)
            new = _tokens(w, rng)
            ref_host = run.host.array.copy()
            st = oapp.append(w, ref_host, new, ctx_len, run.ob.slot_tok, run.ob.buf)
            assert (st == 0).all()
            run.ctx.append(torch.from_numpy(new.view(np.int16)).cuda(),
                           torch.from_numpy(ctx_len).cuda(), run.host, run.st.buf_kv,
                           run.st.slot_table)
            torch.cuda.synchronize()
            assert np.array_equal(run.host.array, ref_host), "host t=%d" % t
            assert np.array_equal(run.st.buf_kv.cpu().numpy().view(np.uint16), run.ob.buf), \
                "buf after append t=%d" % t
            ctx_len = ctx_len + 1
        assert run.ctx.last_error() == avsg.OK
    finally:
        run.close()
        run.host.free()


def test_selection_past_the_context_is_a_unit_range_error():
    from device_buffer_reuse_amd import avsg
    w, _, _ = CASES["pages16"]
    P, N = w.tokens_per_entry, w.n_entries
    say("[context] range errors")
    sel = tg.selections(w)
    run = Runner(w)
    try:
        ctx_len = np.array([(N - 3) * P + 5, (N - 3) * P + 9], np.int32)
        run.set_ctx_len(ctx_len)
        nan_past_context(run.host.array, w, ctx_len)
        s0 = clip_to_context(sel[0], w, ctx_len)
        run.step_and_compare(0, s0, tg.queries(w, 0), check_buf=True)
        # unit 1 selects the entry after its context's last one; request 1's
        # length is 0 (outside [1, N P]) for step 2
        s1 = clip_to_context(sel[1], w, ctx_len)
        s1[1, 0, -1] = N - 2
        before = run.st.slot_table.cpu().numpy().copy()
        r, _ = run.step_and_compare(1, s1, tg.queries(w, 1), check_buf=True)
        assert r["status"].tolist() == [0, avsg.ERR_RANGE, 0, 0]
        assert np.array_equal(run.st.slot_table[1].cpu().numpy(), before[1])
        assert run.ctx.last_error() == avsg.ERR_RANGE
        bad = ctx_len.copy()
        bad[1] = 0
        run.set_ctx_len(bad)
        r, _ = run.step_and_compare(2, clip_to_context(sel[2], w, ctx_len), tg.queries(w, 2),
                                    check_buf=True)
        assert r["status"].tolist() == [0, 0, avsg.ERR_RANGE, avsg.ERR_RANGE]
        assert run.ctx.last_error() == avsg.ERR_RANGE
        run.set_ctx_len(None)
        run.step_and_compare(3, sel[3], tg.queries(w, 3), check_buf=True)
        assert run.ctx.last_error() == avsg.OK
    finally:
        run.close()
        run.host.free()


def test_partial_pages_full_size_long_context():
    """The long-context workload at full size, in the launch configuration
    the benchmark times: every request's context ends inside its last page
    (a different row per request), which every list selects; state compared
    whole, attention on the first and last units."""
    from device_buffer_reuse_amd import avsg
    w = tg.WORKLOADS[4]
    P, N = w.tokens_per_entry, w.n_entries
    steps = 5
    say("[context-full] %s units=%d" % (w.name, w.units))
    sel = tg.selections(w, steps=steps)
    run = Runner(w, attn_units=[0, 1, w.units - 1])
    try:
        ctx_len = np.array([(N - 1) * P + 1 + (b % P) for b in range(w.batch)], np.int32)
        nan_past_context(run.host.array, w, ctx_len)
        run.set_ctx_len(ctx_len)
        for t in range(steps):
            r, _ = run.step_and_compare(t, clip_to_context(sel[t], w, ctx_len), tg.queries(w, t),
                                        check_attn=(t >= steps - 2))
            assert (r["status"] == 0).all()
        assert run.ctx.last_error() == avsg.OK
    finally:
        run.close()
        run.host.free()
