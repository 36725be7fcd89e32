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


def _counters_file(root, kernels):
    """A counter summary in the committed format, for the long workload."""
    import json
    body = {"calibration": {"fetch_scale": 2.0, "write_scale": 1.0}, "kernels": kernels}
    (root / "profiles").mkdir(parents=True, exist_ok=True)
    (root / "profiles" / "counters_long.md").write_text(
        "# counters\n\n```json\n" + json.dumps(body, indent=1) + "\n```\n")


def _copy_sources(root):
    shutil.copytree(os.path.join(bench.ROOT, "device_buffer_reuse_amd", "csrc"),
                    root / "device_buffer_reuse_amd" / "csrc")


def test_counter_summary_is_read_for_the_current_source(tmp_path, monkeypatch):
    root = tmp_path / "repo"
    _copy_sources(root)
    monkeypatch.setattr(bench, "ROOT", str(root))
    name = bench.KERNEL_SOURCES["attention"][4]
    _counters_file(root, {name: {"source_sha256_16": bench.kernel_source_hash(name),
                                 "read_bytes_natural": 300, "write_bytes_natural": 40,
                                 "read_bytes_allhit": 200, "write_bytes_allhit": 4}})
    assert bench.counter_traffic("attention", "natural", 4) == 340
    assert bench.counter_traffic("attention", "allhit", 4) == 204
    assert bench.counter_traffic("attention", "skewed", 4) is None
    assert bench.counter_traffic("combine", "natural", 4) is None
    assert bench.counter_traffic("match_reserve", "natural", 4) is None


def test_counter_summary_is_refused_after_a_source_change(tmp_path, monkeypatch):
    root = tmp_path / "repo"
    _copy_sources(root)
    monkeypatch.setattr(bench, "ROOT", str(root))
    att, mr = bench.KERNEL_SOURCES["attention"][4], bench.KERNEL_SOURCES["match_reserve"][4]
    _counters_file(root, {n: {"source_sha256_16": bench.kernel_source_hash(n),
                              "read_bytes_natural": 10, "write_bytes_natural": 1} for n in (att, mr)})
    assert bench.counter_traffic("attention", "natural", 4) == 11
    src = root / "device_buffer_reuse_amd" / "csrc" / "attn_split.hip"
    src.write_text(src.read_text() + "\n// changed\n")
    assert bench.counter_traffic("attention", "natural", 4) is None
    # the other kernel's counters stay valid
    assert bench.counter_traffic("match_reserve", "natural", 4) == 11


def test_committed_counter_summaries_parse():
    """Every committed counter summary holds a JSON block with per-kernel
    source hashes and byte counts."""
    import glob
    import json
    import re
    for path in glob.glob(os.path.join(bench.ROOT, "profiles", "counters_*.md")):
        m = re.search(r"```json\n(.*?)```", open(path).read(), re.S)
        if not m:
            continue
        data = json.loads(m.group(1))
        for name, k in data["kernels"].items():
            assert len(k["source_sha256_16"]) == 16, (path, name)
            assert any(key.startswith("read_bytes_") for key in k), (path, name)


def test_dominant_roofline_picks_the_longest_kernel_and_its_resource():
    w = tg.WORKLOADS[4]
    use = bench.kernel_use(w, miss_per_step=2000, union_per_step=256 * 128, fused=True)
    per = {"match_reserve": 6.0, "gather": 0.0, "attention": 300.0, "combine": 4.0}
    r = bench.dominant_roofline(use, per)
    assert r["kernel"] == "attention" and r["bound"] == "host-link"
    host = 2000 * w.row_bytes
    assert r["achieved"] == round(host / 300e-6 / 1e9, 2) and r["frac"] == round(host / 300e-6 / 64e9, 4)
    # all hits: no host bytes, the attention is HBM-bound
    use = bench.kernel_use(w, miss_per_step=0, union_per_step=256 * 128, fused=True)
    r = bench.dominant_roofline(use, {"match_reserve": 6.0, "gather": 0.0, "attention": 50.0,
                                      "combine": 4.0})
    assert r["bound"] == "hbm" and r["per_step_work"] == bench.attn_bytes(w)
    # the latent attention's flops are priced at the bf16 matrix-core peak
    t = bench.kernel_table(bench.kernel_use(tg.WORKLOADS[5], 0, 64 * 2048, True),
                           {"match_reserve": 10.0, "gather": 0.0, "attention": 50.0,
                            "combine": 10.0}, True)
    assert t["attention"]["flop_frac"] == round(bench.attn_flops(tg.WORKLOADS[5]) / 50e-6 / 2.5e15, 4)
    assert "gather" not in t


def test_bench_arguments_default_to_the_long_context_workload():
    a = bench.parse([])
    assert a.workload == 4 and a.passes >= 5 and a.fill >= 64 and a.gpus == 1


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


def test_metadata_bytes_of_the_directory():
    # 256 units of 8192 entries: a flat int32 table is 8 MiB of HBM, the
    # top level of 256-entry segments 32 KiB; the segments (host) hold the rows
    m = bench.metadata_bytes(256, 8192, 256)
    assert m["flat_table_hbm_bytes"] == 4 * 256 * 8192 == 8388608
    assert m["top_level_hbm_bytes"] == 4 * 256 * 32 and m["segments_host_bytes"] == 8388608
    assert m["hbm_ratio"] == 256.0
    # a context that is not a whole number of segments rounds the top level up
    m = bench.metadata_bytes(2, 1000, 256)
    assert m["top_level_hbm_bytes"] == 4 * 2 * 4 and m["segments_host_bytes"] == 4 * 2 * 4 * 256
