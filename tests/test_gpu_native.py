"""libavsg driven by a native program through its C ABI alone (HIP runtime
memory, plain pointers, HIP graph calls, no Python binding or torch), against
the oracle: bucketed LRU, three direct steps, then one step captured in a
graph and replayed for the rest.

tests/native/avsg_native_steps.cpp builds its inputs from closed formulas;
this test rebuilds the same inputs, runs the oracle on them and compares the
program's slot tables, lifetimes, hit counts and attention outputs."""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

import tracegen as tg
import oracle
from gpu_harness import check_attention, say
from oracle import attention as oatt

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "native", "avsg_native_steps")
W = tg.WORKLOADS[2].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_entries=1000, k=100,
                            n_slots=300, lifetime_L=3, policy="lru", n_buckets=8, steps=6)


def _bf16(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_native_caller_matches_oracle(tmp_path):
    from gpu_harness import ensure_lib
    ensure_lib()
    if not os.path.exists(BIN):
        from device_buffer_reuse_amd import build as hipbuild
        hipbuild.build_native_test()
    say("[native] C ABI caller")
    out_file = str(tmp_path / "native.bin")
    r = subprocess.run([BIN, out_file], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    w = W
    units, S, N, k, D = w.units, w.n_slots, w.n_entries, w.k, w.head_dim_qk
    Hq, B = w.n_q_heads, w.batch
    u_, e_, i_ = np.meshgrid(np.arange(units), np.arange(N), np.arange(2 * D), indexing="ij")
    host = _bf16(((u_ * 7 + e_ * 3 + i_) % 17 - 8) / 8.0)
    per_step = 2 * units * S + units + B * Hq * D
    data = np.fromfile(out_file, dtype=np.int32)
    assert data.size == w.steps * per_step
    ob = oracle.OracleBuffer.for_workload(w)
    for t in range(w.steps):
        chunk = data[t * per_step:(t + 1) * per_step]
        st = chunk[:units * S].reshape(units, S)
        lf = chunk[units * S:2 * units * S].reshape(units, S)
        nh = chunk[2 * units * S:2 * units * S + units]
        out = chunk[2 * units * S + units:].view(np.float32).reshape(B, 1, Hq, D)
        sel = np.stack([np.sort((np.arange(k) * 3 + t * 5 + u) % N) for u in range(units)])
        sel = sel.reshape(units, 1, k).astype(np.int32)
        b_, h_, i2 = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(D), indexing="ij")
        q = _bf16(((b_ * 5 + h_ * 11 + i2 + t) % 13 - 6) / 8.0).reshape(B, 1, Hq, D)
        res = ob.step(sel)
        assert np.array_equal(st, ob.slot_tok), "slot_table t=%d" % t
        assert np.array_equal(lf, ob.life), "lifetimes t=%d" % t
        assert np.array_equal(nh, res["n_hit"]), "n_hit t=%d" % t
        ref = oatt.attend(w, q, host, sel, res["status"])
        check_attention(out, ref, "native out t=%d" % t)
