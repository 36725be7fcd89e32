"""Seeded random configurations, every option at once, against the oracle.

Each case draws a layout (split with 1, 3 or 16 tokens per entry, or
latent), one or two query tokens, a policy with its lifetime or bucket count
and bucket width, and the sizes; each step then draws list lengths, buffer
sizes and (for pages) a context that ends inside the last selected page, and
after each step the new token is appended, with insertion on odd steps.
State, flags, buffer bytes, host rows and attention must match the oracle's
after every step and every append."""
from __future__ import annotations

import numpy as np
import pytest

import tracegen as tg
from gpu_harness import Runner, say
from oracle import append as oapp
from context_inputs import clip_to_context

pytestmark = pytest.mark.gpu

SEEDS = list(range(256))


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    layout = ["split1", "split3", "split16", "latent"][seed % 4]
    T = int(rng.integers(1, 3))
    lru = bool(rng.integers(0, 2))
    kw = dict(policy="lru" if lru else "lifetime", lifetime_L=int(rng.integers(1, 12)),
              n_buckets=int(rng.integers(1, 9)), bucket_width=int(rng.choice([1, 1, 2, 5])),
              steps=int(rng.integers(4, 8)), n_q_tokens=T, seed=5000 + seed,
              overlap=float(rng.choice([0.5, 0.8, 0.95])),
              overlap_shared=float(rng.choice([0.3, 0.7])) if T == 2 else 0.0)
    if layout == "latent":
        k = int(rng.integers(20, 400))
        w = tg.WORKLOADS[5].replace(batch=int(rng.integers(1, 4)),
                                    n_q_heads=int(rng.choice([64, 128])), k=k,
                                    n_entries=int(rng.integers(3 * k, 8 * k)),
                                    n_slots=int(rng.integers(T * k, 3 * T * k + 1)), **kw)
    else:
        tpe = {"split1": 1, "split3": 3, "split16": 16}[layout]
        Hkv = int(rng.integers(1, 4))
        G = int(rng.choice([1, 2, 4, 8]))
        k = int(rng.integers(8, 300 if tpe == 1 else 60))
        w = tg.WORKLOADS[4].replace(batch=int(rng.integers(1, 4)), n_kv_heads=Hkv,
                                    n_q_heads=Hkv * G, tokens_per_entry=tpe, k=k,
                                    n_entries=int(rng.integers(3 * k, 10 * k)),
                                    n_slots=int(rng.integers(T * k, 3 * T * k + 1)), **kw)
    return w, rng


@pytest.mark.parametrize("seed", SEEDS)
def test_random_configuration(seed):
    from device_buffer_reuse_amd import avsg
    w, rng = draw(seed)
    P = w.tokens_per_entry
    say("[random] seed=%d latent=%s P=%d T=%d units=%d k=%d N=%d S=%d policy=%s L=%d B=%d W=%d"
        % (seed, w.latent, P, w.n_q_tokens, w.units, w.k, w.n_entries, w.n_slots, w.policy,
           w.lifetime_L, w.n_buckets, w.bucket_width))
    split_rows = int(rng.choice([0, 32, 64])) if not w.latent else int(rng.choice([0, 64, 128]))
    run = Runner(w, split_rows=split_rows)
    torch = run.torch
    sel_full = tg.selections(w)
    _, lens = tg.shorten(sel_full, seed=seed, lo=max(1, w.k // 3))
    lens = lens.reshape(w.steps, w.units, w.n_q_tokens)
    use_ctx = P > 1 and bool(rng.integers(0, 2))
    ctx_len = np.array([(w.n_entries - 2 - w.steps) * P + 1 + int(rng.integers(0, P))
                        for _ in range(w.batch)], np.int32)
    try:
        for t in range(w.steps):
            sel_t = sel_full[t].copy()
            if use_ctx:
                run.set_ctx_len(ctx_len)
                sel_t = clip_to_context(sel_t, w, ctx_len)
                for u in range(w.units):
                    last = (int(ctx_len[u // w.n_kv_heads]) - 1) // P
                    for j in range(w.n_q_tokens):
                        sel_t[u, j, lens[t, u, j] - 1] = last
            need = np.array([len(np.unique(np.concatenate(
                [sel_t[u, j, :lens[t, u, j]] for j in range(w.n_q_tokens)])))
                for u in range(w.units)], np.int32)
            if rng.integers(0, 2):
                run.set_caps(np.minimum(w.n_slots, need + rng.integers(0, w.n_slots, size=w.units)))
            else:
                run.set_caps(None)
            r, _ = run.step_and_compare(t, sel_t, tg.queries(w, t), check_buf=True, lengths=lens[t])
            assert (r["status"] == 0).all(), r["status"]
            # the next token of every request (at its context length, or at a
            # random position), inserted on odd steps
            if use_ctx:
                pos = ctx_len.copy()
            else:
                pos = rng.integers(0, w.n_entries * P, size=w.batch).astype(np.int32)
            x = rng.standard_normal((w.units, w.head_dim_qk if w.latent else 2 * w.head_dim_qk))
            new = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
            ref_host = run.host.array.copy()
            insert = t % 2 == 1
            if insert:
                st = oapp.append_insert(w, ref_host, new, pos, run.ob.slot_tok, run.ob.life,
                                        run.ob.buf, run.ob.t, caps=getattr(run, "caps", None))
                run.ctx.append_insert(torch.from_numpy(new.view(np.int16)).cuda(),
                                      torch.from_numpy(pos).cuda(), run.host, run.st.buf_kv,
                                      run.st.slot_table, run.st.lifetimes)
            else:
                st = oapp.append(w, ref_host, new, pos, run.ob.slot_tok, run.ob.buf)
                run.ctx.append(torch.from_numpy(new.view(np.int16)).cuda(),
                               torch.from_numpy(pos).cuda(), run.host, run.st.buf_kv,
                               run.st.slot_table)
            torch.cuda.synchronize()
            what = "seed=%d t=%d %s" % (seed, t, "insert" if insert else "append")
            assert (st == 0).all(), what
            assert np.array_equal(run.host.array, ref_host), what
            assert np.array_equal(run.st.slot_table.cpu().numpy(), run.ob.slot_tok), what
            assert np.array_equal(run.st.lifetimes.cpu().numpy(), run.ob.life), what
            assert np.array_equal(run.st.buf_kv.cpu().numpy().view(np.uint16), run.ob.buf), what
            ctx_len = ctx_len + 1
        assert run.ctx.last_error() == avsg.OK
    finally:
        run.close()
        run.host.free()
