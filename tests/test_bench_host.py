"""Host-side accounting of bench.py: algorithmic bytes and flops per step,
union sizes, and the lookup of the committed HBM counter summary (which
must refuse counters taken on a different kernel source)."""
from __future__ import annotations

import os
import shutil

import numpy as np
import pytest

import bench
import tracegen as tg


def test_attention_bytes_of_the_batch_workload():
    # 64 units x 2048 selected tokens, each a 512-byte row (128 bf16 of K,
    # 128 of V) plus its 4-byte slot; 8 requests x 32 heads of bf16 queries
    # (128 values) and fp32 outputs (128 values)
    w = tg.WORKLOADS[2]
    rows = 64 * 2048 * (512 + 4)
    qo = 8 * 32 * (128 * 2 + 128 * 4)
    assert bench.attn_bytes(w) == rows + qo == 67829760


def test_attention_bytes_of_the_latent_and_paged_workloads():
    # latent: a 1152-byte row (576 bf16) per token, queries of 576, outputs of 512
    w = tg.WORKLOADS[5]
    assert bench.attn_bytes(w) == 64 * 2048 * (1152 + 4) + 64 * 128 * (576 * 2 + 512 * 4)
    # pages of 16 tokens: one 8 KiB row per selected page
    w = tg.WORKLOADS[4]
    assert bench.attn_bytes(w) == 256 * 128 * (16 * 512 + 4) + 32 * 32 * (128 * 2 + 128 * 4)


def test_two_token_steps_count_the_union_once():
    w = tg.WORKLOADS[3]
    full = bench.attn_bytes(w)
    union = bench.attn_bytes(w, union_entries=64 * 2662)
    row = 512 + 4
    assert full - union == (64 * 2 * 2048 - 64 * 2662) * row


def test_union_entries_against_sets():
    rng = np.random.default_rng(3)
    sel = np.sort(rng.integers(0, 50, size=(4, 3, 2, 10)), axis=-1).astype(np.int32)
    want = np.mean([sum(len(set(sel[t, u].ravel().tolist())) for u in range(3)) for t in range(4)])
    assert bench.union_entries(sel) == pytest.approx(want)


def test_flops_of_the_latent_workload():
    # 2 flops per multiply-add, 128 heads x 2048 tokens x (576 + 512) per request
    w = tg.WORKLOADS[5]
    assert bench.attn_flops(w) == 2 * 64 * 128 * 2048 * (576 + 512)
    assert abs(bench.attn_flops(w) / 1e9 - 36.5) < 0.05


def test_match_bytes_of_the_batch_workload():
    # selections read (4 B), slot table read and lifetimes read + written
    # (3 x 4 B per slot), hit flag + slot written (5 B per selected entry),
    # and per miss its slot id and its (slot, id) list entry
    w = tg.WORKLOADS[2]
    tk = 64 * 2048
    assert bench.match_bytes(w, 0) == tk * 4 + 64 * 8192 * 12 + tk * 5 == 7471104
    assert bench.match_bytes(w, 100) - bench.match_bytes(w, 0) == 100 * 12


def test_counter_summary_is_read_for_the_current_source():
    for kernel in ("attention", "match_reserve"):
        for trace in ("allhit", "natural"):
            v = bench.counter_traffic(kernel, trace)
            assert isinstance(v, int) and v > 0, (kernel, trace)
    # the attention reads at least its algorithmic bytes
    assert bench.counter_traffic("attention", "allhit") >= bench.attn_bytes(tg.WORKLOADS[2])
    assert bench.counter_traffic("combine", "allhit") is None
    assert bench.counter_traffic("attention", "skewed") is None


def test_counter_summary_is_refused_after_a_source_change(tmp_path, monkeypatch):
    root = tmp_path / "repo"
    (root / "profiles").mkdir(parents=True)
    shutil.copy(os.path.join(bench.ROOT, "profiles", "counters_batch.md"), root / "profiles")
    shutil.copytree(os.path.join(bench.ROOT, "device_buffer_reuse_amd", "csrc"),
                    root / "device_buffer_reuse_amd" / "csrc")
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench.counter_traffic("attention", "allhit") is not None
    src = root / "device_buffer_reuse_amd" / "csrc" / "attn_split.hip"
    src.write_text(src.read_text() + "\n// changed\n")
    assert bench.counter_traffic("attention", "allhit") is None
    # the other kernel's counters stay valid
    assert bench.counter_traffic("match_reserve", "allhit") is not None


def test_step_roofline_takes_the_larger_time():
    # 80 MB over 8 TB/s = 10 us of HBM, 0.64 MB over 64 GB/s = 10 us of link:
    # a tie counts as host-link; a 20 us step reaches half of it
    r = bench.step_roofline(70e6, 10e6, 0.64e6, True, 20e-6)
    assert r["t_hbm_us"] == 10.0 and r["t_link_us"] == 10.0
    assert r["bound"] == "host-link" and r["frac"] == 0.5
    # a separate gather reads the missed rows back: host bytes count on HBM too
    r = bench.step_roofline(70e6, 10e6, 8e6, False, 250e-6)
    assert r["hbm_bytes"] == 88000000 and r["t_hbm_us"] == 11.0
    assert r["bound"] == "host-link" and r["t_link_us"] == 125.0 and r["frac"] == 0.5
    # no host traffic: HBM-bound
    r = bench.step_roofline(70e6, 10e6, 0, True, 40e-6)
    assert r["bound"] == "hbm" and r["frac"] == 0.25
