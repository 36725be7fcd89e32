"""The oracle's C code built with the address and undefined-behaviour
sanitizers (gcc -fsanitize=address,undefined, every finding fatal) and run
on the hand-worked traces, on brute-force-checked micro-traces (buffer sizes
and data errors included) and on a small attention case.  The sanitized
program must exit cleanly and agree with the pins.  CPU only."""
from __future__ import annotations

import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

import oracle
from oracle import attention as oatt
from bruteforce import BruteBuffer
from test_oracle_state import GOLDEN, _parse_golden, _random_trace

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ODIR = os.path.join(ROOT, "oracle")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")


@pytest.fixture(scope="module")
def cli(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("asan") / "oracle_cli")
    srcs = [os.path.join(ODIR, f) for f in ("avsg_oracle.c", "attention.c", "oracle_cli.c")]
    subprocess.check_call(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fopenmp"] + srcs + ["-o", exe, "-lm"])
    return exe


def _run(exe, text):
    env = dict(os.environ, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="abort_on_error=0:halt_on_error=1:detect_leaks=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], input=text, capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "runtime error" not in r.stderr, r.stderr[-3000:]
    return r.stdout.split("\n")


def _state_run(exe, S, N, T, k, policy, L, B, steps):
    """steps: list of (t, cap, sel [T][k]); returns per step (status, counts,
    flags, slots, tok, life)."""
    words = ["state", S, N, T, k, 1 if policy == "lru" else 0, L, B, len(steps)]
    for t, cap, sel in steps:
        words += [t, cap] + [int(x) for x in np.asarray(sel).ravel()]
    lines = _run(exe, " ".join(str(x) for x in words) + "\n")
    out = []
    for i in range(len(steps)):
        head, fl, sl, tk, lf = lines[5 * i:5 * i + 5]
        h = [int(x) for x in head.split()]
        out.append((h[0], h[1:], [int(x) for x in fl.split()], [int(x) for x in sl.split()],
                    [int(x) for x in tk.split()], [int(x) for x in lf.split()]))
    return out


@pytest.mark.parametrize("name", ["lifetime_s4.txt", "lru_b2_s3.txt", "mtp_s4.txt"])
def test_sanitized_golden(cli, name):
    cfg, steps = _parse_golden(os.path.join(GOLDEN, name))
    T = len(steps[0]["sel"])
    res = _state_run(cli, cfg["S"], cfg["N"], T, cfg["k"], cfg["policy"], cfg["L"], cfg["B"],
                     [(t, -1, d["sel"]) for t, d in enumerate(steps)])
    for t, (d, (st, cnt, fl, sl, tok, life)) in enumerate(zip(steps, res)):
        assert st == oracle.OK
        assert fl == [x for row in d["hit"] for x in row], (name, t)
        assert sl == [x for row in d["slot"] for x in row], (name, t)
        assert cnt[:3] == [d["n_hit"], d["n_miss"], d["n_evict"]]
        assert tok == d["tok"] and life == d["life"], (name, t)


@pytest.mark.parametrize("seed", range(24))
def test_sanitized_matches_bruteforce(cli, seed):
    rng = np.random.default_rng(1000 + seed)
    S = int(rng.integers(4, 33))
    N = int(rng.integers(max(8, 2 * S), 257))
    T = int(rng.integers(1, 3))
    policy = "lru" if seed % 2 else "lifetime"
    L, B = int(rng.integers(1, 7)), int(rng.integers(1, 7))
    k = max(1, min(int(rng.integers(1, S // T + 1)), N // 2))
    trace = _random_trace(rng, S, N, k, T, 12, overlap=0.6)
    res = _state_run(cli, S, N, T, k, policy, L, B, [(t, -1, sel) for t, sel in enumerate(trace)])
    bb = BruteBuffer(S, N, L, B, policy)
    for t, (sel, (st, cnt, fl, sl, tok, life)) in enumerate(zip(trace, res)):
        assert st == oracle.OK
        flags, slots, c = bb.step([list(map(int, l)) for l in sel])
        assert fl == [int(x) for row in flags for x in row]
        assert sl == [x for row in slots for x in row]
        assert cnt == [c["n_hit"], c["n_miss"], c["n_evict"], c["n_union"]]
        assert tok == bb.tok and life == bb.life_array()


def test_sanitized_sizes_and_errors(cli):
    """Buffer sizes (shrink, grow) and every data error, against the
    unsanitized library on the same inputs."""
    S, N, k = 12, 100, 5
    lists = [[3, 9, 20, 41, 77], [3, 9, 21, 41, 80], [3, 9, 22, 42, 80], [1, 9, 22, 42, 80],
             [9, 3, 22, 42, 80], [1, 9, 22, 42, 100], [4, 9, 22, 42, 81], [5, 9, 22, 42, 82]]
    caps = [-1, 8, 6, 12, 7, 7, 4, 12]
    steps = [(t, c, np.array([l], np.int32)) for t, (l, c) in enumerate(zip(lists, caps))]
    res = _state_run(cli, S, N, 1, k, "lifetime", 3, 64, steps)
    tok = np.full(S, -1, np.int32)
    life = np.zeros(S, np.int32)
    for (t, c, sel), (st, cnt, fl, sl, tk, lf) in zip(steps, res):
        want, r = oracle.unit_step(S, N, k, "lifetime", 3, 64, t, sel, tok, life,
                                   cap=None if c < 0 else c)
        assert st == want
        assert fl == r["hit_flag"].ravel().tolist() and sl == r["sel_slot"].ravel().tolist()
        assert tk == tok.tolist() and lf == life.tolist()
    assert [r[0] for r in res] == [0, 0, 0, 0, oracle.ERR_UNSORTED, oracle.ERR_RANGE,
                                   oracle.ERR_CAPACITY, 0]


def test_sanitized_attention(cli):
    import tracegen as tg
    w = tg.WORKLOADS[1].replace(batch=2, n_kv_heads=2, n_q_heads=8, n_q_tokens=2, head_dim_qk=16,
                                head_dim_v=16, n_entries=30, tokens_per_entry=3, k=5, n_slots=10)
    rng = np.random.default_rng(5)
    bits = lambda x: (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    host = bits(rng.standard_normal((w.units, w.n_entries, w.row_elems)))
    q = bits(rng.standard_normal((w.batch, w.n_q_tokens, w.n_q_heads, w.head_dim_qk)))
    sel = np.stack([np.stack([np.sort(rng.choice(w.n_entries, w.k, replace=False))
                              for _ in range(w.n_q_tokens)]) for _ in range(w.units)]).astype(np.int32)
    status = np.array([0, 0, 17, 0], np.int32)
    hi, lo = struct.unpack("<II", struct.pack("<d", w.softmax_scale))[::-1]
    words = ["attn", w.batch, w.n_kv_heads, w.n_q_heads, w.n_q_tokens, w.head_dim_qk,
             w.head_dim_v, 0, w.tokens_per_entry, w.n_entries, w.k, hi, lo]
    text = " ".join(str(x) for x in words) + "\n" + " ".join(
        " ".join(str(int(v)) for v in a.ravel()) for a in (q, host, sel, status)) + "\n"
    got = np.array([float(x) for x in _run(cli, text)[0].split()]).reshape(
        w.batch, w.n_q_tokens, w.n_q_heads, w.head_dim_v)
    ref = oatt.attend(w, q, host, sel, status)
    assert np.abs(got - ref).max() <= 1e-13
    assert (got[1, :, :4] == 0).all()   # unit 2 = request 1, KV head 0 failed
