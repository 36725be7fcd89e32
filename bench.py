#!/usr/bin/env python3
"""Decode-step benchmark of the HBM slot buffer on one MI355X.

One step = one avsg_step over all units of a workload: match + reserve,
miss-only transfer from pinned host memory, split-k attention, merge of the
splits.  The headline workload is the long-context one (32 requests x 8 KV
heads x 32 query heads, head_dim 128, context 131072 tokens in 16-token
head-wise pages, 128 pages selected per step, 1024-page buffer per (request,
head), bucketed LRU with 64 buckets, 85% step-to-step overlap plus a Zipf(1.1)
tail); every other workload gets an object of its own in the same line.

Timing protocol, per workload and trace: a pass resets the buffer
(avsg_reset), runs `--fill` + `--warmup` steps untimed (the fill brings the
buffer to its steady state: every workload's miss rate is flat from about
step 64 on), then times exactly `--steps` steps between two HIP events on the
library's stream.  `--warmup-passes` untimed passes come first, then
`--passes` timed passes; the reported step time is their median.  Per-kernel
times come from further passes with the library's per-stage HIP events, and
the hit statistics from one more pass.  Inputs (selections, queries) are in
HBM before the timed region; the KV cache is in pinned host memory, which is
the method's premise, so host transfers of misses are part of every step.

Prints one JSON line.  `roofline` names the dominant kernel of the headline
step and the resource it uses most: the host link (PCIe 5.0 x16, 64 GB/s),
HBM (8 TB/s) or the bf16 matrix cores (2.5 PFLOP/s dense).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
HOST_LINK_GBS = 64.0        # PCIe 5.0 x16, one direction
MFMA_BF16_TFLOPS = 2500.0   # dense bf16 matrix cores (both attention kernels run on them)
HEADLINE = 4                # the long-context workload
Q_SETS = 32                 # distinct query sets, step t uses set t % Q_SETS
STAGES = ("match_reserve", "gather", "attention", "combine")


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64, help="timed steps per pass")
    ap.add_argument("--warmup", type=int, default=8, help="untimed steps after the fill")
    ap.add_argument("--fill", type=int, default=96,
                    help="untimed steps that bring the buffer to its steady state")
    ap.add_argument("--passes", type=int, default=5, help="timed passes (median reported)")
    ap.add_argument("--warmup-passes", type=int, default=3)
    ap.add_argument("--workload", type=int, default=HEADLINE, help="1..5 (tracegen.WORKLOADS)")
    ap.add_argument("--others", default="1,2,3,5",
                    help="workloads measured besides the headline one ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-extra", action="store_true",
                    help="headline trace only: no all-hit / all-miss, other workloads or extras")
    ap.add_argument("--trace", default="natural", choices=["natural", "allhit", "allmiss", "skewed"],
                    help="selection trace of the headline steps (default natural)")
    ap.add_argument("--transfer", type=int, default=0,
                    help="0 fused (default), 1 balanced gather kernel, 2 per-unit gather kernel, "
                         "3 fused, gather-first")
    ap.add_argument("--ablations", action="store_true",
                    help="also compare transfer modes on a skewed-miss trace and hash vs "
                         "dual-pointer matching (batch workload)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain device copy of known size (for counter scaling)")
    ap.add_argument("--buffer-sweep", default="",
                    help="comma-separated slot counts: the headline trace at each buffer size")
    return ap.parse_args(argv)


class Bench:
    """Context, device state, pinned host KV and queries of one workload."""

    def __init__(self, w):
        import torch
        import tracegen as tg
        from device_buffer_reuse_amd import avsg
        self.torch, self.tg, self.avsg, self.w = torch, tg, avsg, w
        self.lib = avsg.load()
        self.cfg = avsg.config_from_workload(w)
        self.ctx = avsg.Context(self.cfg)
        self.st = avsg.State(self.cfg)
        self.host = avsg.HostBuffer((w.units, w.n_entries, w.row_elems))
        tg.fill_kv(w, out=self.host.array)
        q = np.stack([tg.queries(w, t) for t in range(Q_SETS)])
        self.q_dev = torch.from_numpy(q.view(np.int16)).cuda()
        self.hs = self.st.stats.struct()
        self.sel_np = self.sel_dev = self.len_np = self.len_dev = None

    def close(self):
        self.ctx.close()
        self.host.free()

    def resize(self, n_slots):
        """A new context and device state with n_slots slots per unit, over
        the same host KV and queries (the selection trace does not depend on
        the buffer size)."""
        self.ctx.close()
        self.w = self.w.replace(n_slots=n_slots)
        self.cfg = self.avsg.config_from_workload(self.w)
        self.ctx = self.avsg.Context(self.cfg)
        self.st = self.avsg.State(self.cfg)
        self.hs = self.st.stats.struct()

    def load_trace(self, mode, steps):
        self.len_np = self.len_dev = None
        self.sel_np = self.tg.selections(self.w, steps=steps, mode=mode)
        self.sel_dev = self.torch.from_numpy(self.sel_np).cuda()

    def load_varlen(self, steps, lo):
        """The natural trace with a list length per (step, unit) drawn from
        [lo, k] (PSA-style budgets); the following runs use avsg_step_varlen."""
        sel, lens = self.tg.shorten(self.tg.selections(self.w, steps=steps), 5, lo)
        self.sel_np, self.len_np = sel, lens
        self.sel_dev = self.torch.from_numpy(sel).cuda()
        self.len_dev = self.torch.from_numpy(lens).cuda()

    def reset(self):
        self.ctx.reset(self.st.slot_table, self.st.lifetimes)

    def run(self, t0, t1, stats=None):
        import ctypes
        lib, h, s = self.lib, self.ctx.handle, self.st
        hsp = ctypes.byref(self.hs)
        sel0, selb = self.sel_dev.data_ptr(), self.sel_dev[0].numel() * 4
        q0, qb = self.q_dev.data_ptr(), self.q_dev[0].numel() * 2
        args = (self.host.ptr, s.buf_kv.data_ptr(), s.slot_table.data_ptr(), s.lifetimes.data_ptr(),
                s.out.data_ptr())
        lens = self.len_dev
        for t in range(t0, t1):
            if lens is not None:
                rc = lib.avsg_step_varlen(h, sel0 + t * selb, lens.data_ptr() + t * lens[0].numel() * 4,
                                          q0 + (t % Q_SETS) * qb, *args, hsp)
            else:
                rc = lib.avsg_step(h, sel0 + t * selb, q0 + (t % Q_SETS) * qb, *args, hsp)
            if rc != 0:
                raise self.avsg.AvsgError(rc, "avsg_step")
            if stats is not None:
                stats[0] += s.stats.n_hit
                stats[1] += s.stats.n_miss

    def one_pass(self, t0, t1, profile=False):
        """Reset, steps [0, t0) untimed, steps [t0, t1) timed: (ms, per-stage
        ms or None).  The events are on torch's current stream, which is the
        context's stream."""
        torch = self.torch
        self.reset()
        self.run(0, t0)
        if profile:
            self.ctx.profile_begin(t1 - t0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        self.run(t0, t1)
        e1.record()
        torch.cuda.synchronize()
        kern = None
        if profile:
            kern, n = self.ctx.profile_end()
            assert n == t1 - t0
        return e0.elapsed_time(e1), kern

    def passes(self, t0, t1, warm, timed, profiled=3):
        """Median step ms over `timed` passes (after `warm` untimed ones), the
        per-pass step ms, and the median per-stage us from `profiled` passes
        with the library's stage events."""
        for _ in range(warm):
            self.one_pass(t0, t1)
        n = t1 - t0
        per_pass = [self.one_pass(t0, t1)[0] / n for _ in range(timed)]
        stage = [self.one_pass(t0, t1, profile=True)[1] for _ in range(profiled)]
        kern = {name: statistics.median(s[i] for s in stage) / n * 1e3
                for i, name in enumerate(STAGES)}
        return statistics.median(per_pass), per_pass, kern

    def window_counts(self, t0, t1):
        """Hits and misses summed over the steps [t0, t1) of the loaded trace."""
        torch = self.torch
        self.reset()
        self.run(0, t0)
        acc = [torch.zeros(self.w.units, dtype=torch.int64, device="cuda") for _ in range(2)]
        self.run(t0, t1, stats=acc)
        return int(acc[0].sum()), int(acc[1].sum())


def attn_bytes(w, union_entries=None):
    """Algorithmic bytes of the attention of one step: the selected K/V rows,
    the slot list, the queries and the fp32 outputs.  With two query tokens
    in the split layout the rows of the union are read once (union_entries:
    the union's entries summed over units)."""
    row = w.tokens_per_entry * (w.head_dim_qk + (0 if w.latent else w.head_dim_v)) * 2
    entries = w.units * w.n_q_tokens * w.k
    if union_entries is not None and w.n_q_tokens > 1 and not w.latent:
        entries = union_entries
    return entries * (row + 4) + w.batch * w.n_q_tokens * w.n_q_heads * (
        w.head_dim_qk * 2 + w.head_dim_v * 4)


def union_entries(sel):
    """Entries of the union of each unit's query tokens, summed over units,
    averaged over the steps of sel [steps][units][T][k]."""
    return float(np.mean([sum(len(np.unique(sel[t, u])) for u in range(sel.shape[1]))
                          for t in range(sel.shape[0])]))


def attn_flops(w):
    return 2 * w.batch * w.n_q_tokens * w.n_q_heads * w.k * w.tokens_per_entry * (w.head_dim_qk +
                                                                                  w.head_dim_v)


def match_bytes(w, misses_per_step):
    """Algorithmic bytes of one match_reserve launch: selections, the slot
    table read, lifetimes read and written, hit flags and slots written, the
    reserved slots' ids and the miss list."""
    tk = w.units * w.n_q_tokens * w.k
    return tk * 4 + w.units * w.n_slots * 4 * 3 + tk * 5 + misses_per_step * (4 + 8)


def step_roofline(attn_b, match_b, host_b, fused, t_step):
    """The whole step against its roofline: the larger of its algorithmic HBM
    time and its host-link time, over the measured step time t_step (s).
    HBM: the attention's bytes (hits read, missed rows written into their
    slots, which the fused transfer never reads back; metadata, queries and
    outputs) and match_reserve's; a separate gather also reads the missed
    rows back (host_b more)."""
    step_hbm = attn_b + match_b + (0.0 if fused else host_b)
    t_hbm, t_link = step_hbm / (HBM_PEAK_GBS * 1e9), host_b / (HOST_LINK_GBS * 1e9)
    return {"hbm_bytes": int(step_hbm), "host_bytes": int(host_b),
            "t_hbm_us": round(t_hbm * 1e6, 2), "t_link_us": round(t_link * 1e6, 2),
            "bound": "host-link" if t_link >= t_hbm else "hbm",
            "frac": round(max(t_hbm, t_link) / t_step, 4)}


PEAKS = {"hbm": (HBM_PEAK_GBS, "GB/s", 1e9), "host": (HOST_LINK_GBS, "GB/s", 1e9),
         "flop": (MFMA_BF16_TFLOPS, "TFLOP/s", 1e12)}
BOUND_NAMES = {"hbm": "hbm", "host": "host-link", "flop": "mfma"}


def kernel_use(w, miss_per_step, union_per_step, fused):
    """Algorithmic work of one step per kernel: HBM bytes, host-link bytes
    and flops."""
    host_b = miss_per_step * w.row_bytes
    ab = attn_bytes(w, union_per_step)
    return {
        "match_reserve": {"hbm": match_bytes(w, miss_per_step), "host": 0.0, "flop": 0.0},
        "gather": {"hbm": 0.0 if fused else host_b, "host": 0.0 if fused else host_b, "flop": 0.0},
        "attention": {"hbm": ab + (host_b if fused else 0.0), "host": host_b if fused else 0.0,
                      "flop": float(attn_flops(w))},
        # the merge of the split partials: no algorithmic bytes of its own
        # (the outputs are counted with the attention)
        "combine": {"hbm": 0.0, "host": 0.0, "flop": 0.0},
    }


def kernel_table(use, per_us, fused):
    """Per kernel: its time and every resource's achieved rate and fraction."""
    kernels = {}
    for name, u in use.items():
        if name == "gather" and fused:
            continue   # not launched: the fused transfer runs inside the attention
        t = per_us[name] * 1e-6
        d = {"us": round(per_us[name], 2)}
        for res, (pk, unit, scale) in PEAKS.items():
            if u[res] > 0 and t > 0:
                ach = u[res] / t / scale
                d[res + "_" + unit] = round(ach, 2)
                d[res + "_frac"] = round(ach / pk, 4)
        kernels[name] = d
    return kernels


def dominant_roofline(use, per_us):
    """The longest kernel with algorithmic work of its own, against the
    resource it uses most: achieved = its algorithmic per-step work over its
    per-step time."""
    dom = max((n for n in per_us if any(v > 0 for v in use[n].values())), key=per_us.get)
    du, t = use[dom], per_us[dom] * 1e-6
    best = max((r for r in ("hbm", "host", "flop") if du[r] > 0),
               key=lambda r: du[r] / t / PEAKS[r][2] / PEAKS[r][0])
    pk, unit, scale = PEAKS[best]
    ach = du[best] / t / scale
    return {"bound": BOUND_NAMES[best], "achieved": round(ach, 2), "peak": pk, "unit": unit,
            "frac": round(ach / pk, 4), "kernel": dom, "per_step_work": du[best],
            "kernel_us": round(per_us[dom], 2)}


# kernel (as rocprofv3 names it) that carries each stage of a workload's step
KERNEL_SOURCES = {"attention": {2: "attn_split_kernel<4, false>", 3: "attn_split_kernel<4, false>",
                                4: "attn_split_kernel<4, true>", 5: "attn_latent_kernel<8>"},
                  "match_reserve": {2: "match_reserve_kernel<8>", 3: "match_reserve_kernel<8>",
                                    4: "match_reserve_kernel<1>", 5: "match_reserve_kernel<8>"}}
KERNEL_FILES = {"attn_split_kernel": "attn_split.hip", "attn_latent_kernel": "attn_latent.hip",
                "match_reserve_kernel": "match_reserve.hip", "attn_combine_kernel": "attn_combine.hip",
                "attn_combine_latent_kernel": "attn_combine.hip"}


def kernel_source_hash(name, root=None):
    """sha256 (16 hex) of the source file of a kernel plus avsg_internal.h."""
    import hashlib
    root = ROOT if root is None else root
    h = hashlib.sha256()
    for f in (KERNEL_FILES[name.split("<")[0]], "avsg_internal.h"):
        h.update(open(os.path.join(root, "device_buffer_reuse_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def counter_traffic(kernel, trace, workload=HEADLINE):
    """HBM bytes per launch (reads + writes) of `kernel` on `workload` from
    the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary
    (profiles/counters_<name>.md), scaled by the plain-copy calibration; None
    if the summary lacks that trace or the kernel's source changed since the
    counters were taken."""
    import re
    import tracegen as tg
    name = KERNEL_SOURCES.get(kernel, {}).get(workload)
    path = os.path.join(ROOT, "profiles", "counters_%s.md" % tg.WORKLOADS[workload].name)
    if name is None or not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)```", open(path).read(), re.S)
    if not m:
        return None
    k = json.loads(m.group(1))["kernels"].get(name)
    if not k or kernel_source_hash(name) != k["source_sha256_16"]:
        return None
    r, wr = k.get("read_bytes_" + trace), k.get("write_bytes_" + trace)
    if r is None or wr is None:
        return None
    return int(r + wr)


def measure(b, mode, t0, K, warm, timed, fused=True):
    """One trace of the loaded workload: the median step time over `timed`
    passes, per-stage times, hit statistics and the roofline of every
    kernel; the trace is generated for t0 + K steps."""
    w = b.w
    b.load_trace(mode, t0 + K)
    ms, per_pass, per = b.passes(t0, t0 + K, warm, timed)
    n_hit, n_miss = b.window_counts(t0, t0 + K)
    miss_ps, union_ps = n_miss / K, (n_hit + n_miss) / K
    use = kernel_use(w, miss_ps, union_ps, fused)
    res = {"trace": mode, "timed_steps": [t0, t0 + K - 1], "passes": timed,
           "ms_per_step": round(ms, 5), "ms_per_step_passes": [round(x, 5) for x in per_pass],
           "steps_per_s": round(1e3 / ms, 2),
           "entries_per_s": round(w.entries_per_step / (ms * 1e-3), 1),
           "hit_rate": round(n_hit / max(n_hit + n_miss, 1), 5),
           "miss_rows_per_step": round(miss_ps, 1),
           "host_bytes_per_step": int(miss_ps * w.row_bytes),
           "union_per_step": round(union_ps, 1),
           "kernels": kernel_table(use, per, fused),
           "roofline": dominant_roofline(use, per),
           "step_roofline": step_roofline(attn_bytes(w, union_ps),
                                          match_bytes(w, miss_ps), miss_ps * w.row_bytes, fused,
                                          ms * 1e-3)}
    step_hbm = attn_bytes(w, union_ps) + match_bytes(w, miss_ps)
    res["step_hbm_frac"] = round(step_hbm / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    res["step_host_link_frac"] = round(miss_ps * w.row_bytes / (ms * 1e-3) / 1e9 / HOST_LINK_GBS, 4)
    assert b.ctx.last_error() == 0
    return res


def measure_workload(b, a, traces=("natural", "allhit", "allmiss")):
    """The natural trace after the fill, all-hit (step 0 fills, every later
    step repeats it) and all-miss (disjoint windows) traces of one workload."""
    out = {}
    fused = a.transfer in (0, 3)
    for mode in traces:
        if mode == "natural":
            t0, K = a.fill + a.warmup, a.steps
        elif mode == "allhit":
            t0, K = 1 + a.warmup, min(a.steps, 64)
        else:
            t0, K = 4 + a.warmup, min(a.steps, 32)
        out[mode] = measure(b, mode, t0, K, a.warmup_passes, a.passes, fused)
    return out


def brief(r):
    """The fields of a trace measurement kept in a per-workload object."""
    keep = ("ms_per_step", "steps_per_s", "entries_per_s", "hit_rate", "host_bytes_per_step",
            "step_hbm_frac", "step_host_link_frac", "roofline", "kernels")
    return {k: r[k] for k in keep}


def buffer_sweep(b, a, sizes):
    """The headline workload's natural trace with the buffer at each size
    (slots per unit): hit rate, host bytes and time per step.  Each size gets
    its own fill phase before the timed window."""
    out = {}
    for S in sizes:
        b.resize(S)
        r = measure(b, "natural", a.fill + a.warmup, a.steps, a.warmup_passes, a.passes, True)
        out[str(S)] = {"hbm_buffer_bytes": b.w.units * S * b.w.row_bytes,
                       "ms_per_step": r["ms_per_step"], "hit_rate": r["hit_rate"],
                       "host_bytes_per_step": r["host_bytes_per_step"],
                       "entries_per_s": r["entries_per_s"],
                       "attention_us": r["kernels"]["attention"]["us"],
                       "match_reserve_us": r["kernels"]["match_reserve"]["us"]}
    return out


def ablations(a):
    """Comparisons the AVSG abstract reports, reproduced in kind on this GPU
    on the batch workload: (1) transfers spread over all workgroups vs
    assigned per unit, on a trace where every 8th unit misses everything and
    the others hit everything; (2) vectorised hash matching vs the scalar
    dual-pointer baseline (kernel time of match_reserve on the natural
    trace)."""
    import tracegen as tg
    w = tg.WORKLOADS[2]
    b = Bench(w)
    n = min(a.steps, 32)
    out, skew = {}, {}
    b.load_trace("skewed", n + 2)
    for mode, name in ((0, "fused"), (1, "balanced"), (2, "per-unit")):
        b.ctx.set_transfer_mode(mode)
        ms, kern = b.one_pass(2, n + 2, profile=True)
        units_missing = (w.units + 7) // 8
        host_b = units_missing * w.n_q_tokens * w.k * w.row_bytes
        kt = kern[2] if mode == 0 else kern[1]
        skew[name] = {"ms_per_step": round(ms / n, 4),
                      "transfer_kernel_us": round(kt / n * 1e3, 2),
                      "effective_host_GB/s": round(host_b / (kt / n * 1e-3) / 1e9, 2)}
    b.ctx.set_transfer_mode(0)
    out["skewed_transfer"] = skew
    match = {}
    b.load_trace("natural", a.fill + n)
    for mode, name in ((0, "hash"), (2, "hash_table"), (1, "dual_pointer")):
        b.ctx.set_match_mode(mode)
        ms, kern = b.one_pass(a.fill, a.fill + n, profile=True)
        match[name] = {"match_reserve_us": round(kern[0] / n * 1e3, 2),
                       "ms_per_step": round(ms / n, 4)}
        if mode == 1:
            # the baseline's two phases, from the kernel's own clock
            sort_ms, walk_ms = b.ctx.profile_match_phases()
            match[name]["sort_us"] = round(sort_ms / n * 1e3, 2)
            match[name]["walk_us"] = round(walk_ms / n * 1e3, 2)
    b.ctx.set_match_mode(0)
    dp = match["dual_pointer"]
    match["speedup"] = round(dp["match_reserve_us"] / match["hash"]["match_reserve_us"], 2)
    # as if the residents were kept sorted across steps: the baseline's
    # kernel time without its per-step sort
    match["speedup_without_sort"] = round(
        (dp["match_reserve_us"] - dp["sort_us"]) / match["hash"]["match_reserve_us"], 2)
    out["matching"] = match
    assert b.ctx.last_error() == 0
    b.close()
    return out


def graph_replay(b, a, t0, K):
    """Per-step time of steps [t0, t0 + K) replayed from one captured graph,
    against the same steps run eagerly, on the natural trace; the final
    slot state of a replayed pass must equal an eager pass's."""
    import ctypes
    torch = b.torch
    b.load_trace("natural", t0 + K)
    cap_stream = torch.cuda.Stream()
    default = b.ctx.stream

    def use(stream):
        st = b.avsg.avsg_set_stream(b.ctx.handle, stream.cuda_stream)
        assert st == 0
    # an eager pass for reference
    b.reset()
    b.run(0, t0 + K)
    torch.cuda.synchronize()
    ref = (b.st.slot_table.clone(), b.st.lifetimes.clone())
    # capture on a side stream (nothing runs while capturing)
    b.reset()
    b.run(0, t0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    use(cap_stream)
    try:
        with torch.cuda.graph(graph, stream=cap_stream):
            b.run(t0, t0 + K)
    finally:
        use(default)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per_pass = []
    for i in range(1 + a.passes):
        b.reset()
        b.run(0, t0)
        torch.cuda.synchronize()
        with torch.cuda.stream(cap_stream):
            e0.record()
            graph.replay()
            e1.record()
        torch.cuda.synchronize()
        if i:
            per_pass.append(e0.elapsed_time(e1) / K)
    assert torch.equal(b.st.slot_table, ref[0]) and torch.equal(b.st.lifetimes, ref[1])
    assert b.ctx.t == t0 + K
    assert b.ctx.last_error() == 0
    del graph
    ms_e = statistics.median([b.one_pass(t0, t0 + K)[0] / K for _ in range(a.passes)])
    return {"steps": K, "passes": a.passes, "ms_per_step": round(statistics.median(per_pass), 4),
            "eager_ms_per_step": round(ms_e, 4),
            "state_equals_eager": True}


def extras(b, a):
    """Variable list lengths, planned buffer sizes and the append on the
    headline workload; the box's plain copy, pinned memcpy and GEMM rates."""
    torch, w = b.torch, b.w
    out = {}
    t0, K = a.fill + a.warmup, min(a.steps, 64)
    # selections of a different size per list (PSA-style budgets, lengths
    # uniform in [k/8, k])
    b.load_varlen(t0 + K, max(1, w.k // 8))
    ms_v, _, kv = b.passes(t0, t0 + K, 1, a.passes)
    vh, vm = b.window_counts(t0, t0 + K)
    ent_v = float(b.len_np[t0:t0 + K].sum()) * w.tokens_per_entry / K
    hb_v = vm / K * w.row_bytes
    out["varlen"] = {
        "steps": K, "lengths": "uniform in [k/8, k] per list and step, a random subset of the "
                               "natural trace's list",
        "ms_per_step": round(ms_v, 4), "entries_per_step": round(ent_v, 1),
        "entries_per_s": round(ent_v / (ms_v * 1e-3), 1),
        "hit_rate": round(vh / max(vh + vm, 1), 5), "host_bytes_per_step": int(hb_v),
        "attention_us": round(kv["attention"], 2),
        "attention_host_GB/s": round(hb_v / (kv["attention"] * 1e-6) / 1e9, 2),
        "match_reserve_us": round(kv["match_reserve"], 2)}
    assert b.ctx.last_error() == 0
    # buffer sizes from the planner: every unit's union is mandatory, and a
    # quarter of the remaining slots (units x (S - |U|)) is shared by reuse
    # measured over the steps before the timed window
    b.load_trace("natural", t0 + K)
    b.reset()
    accw = [torch.zeros(w.units, dtype=torch.int64, device="cuda") for _ in range(2)]
    b.run(0, t0, stats=accw)
    ucap = min(w.n_q_tokens * w.k, w.n_slots)
    demand = np.full(w.units, ucap, np.int32)
    reuse = np.minimum(accw[0].cpu().numpy(), 2**31 - 1).astype(np.int32)
    budget = int(demand.sum() + 0.25 * w.units * (w.n_slots - ucap))
    pst, caps = b.avsg.avsg_plan_capacity(demand, reuse, budget, w.n_slots)
    assert pst == 0
    cap_dev = torch.from_numpy(caps).cuda()
    b.ctx.set_capacity(cap_dev)
    # the planned sizes apply from the start of each pass
    per_pass = [b.one_pass(t0, t0 + K)[0] / K for _ in range(a.passes)]
    ch, cm = b.window_counts(t0, t0 + K)
    b.ctx.set_capacity(None)
    assert b.ctx.last_error() == 0
    out["capacity"] = {
        "steps": K, "budget_slots": budget, "full_slots": w.units * w.n_slots,
        "caps_min_max": [int(caps.min()), int(caps.max())],
        "ms_per_step": round(statistics.median(per_pass), 4),
        "hit_rate": round(ch / max(ch + cm, 1), 5),
        "host_bytes_per_step": int(cm / K * w.row_bytes)}
    # context lengths ending inside each request's last page, which every
    # list selects (its last id becomes N - 1, the largest): the attention
    # masks that page's rows past the length
    if w.tokens_per_entry > 1:
        b.load_trace("natural", t0 + K)
        b.sel_np[..., -1] = w.n_entries - 1
        b.sel_dev = torch.from_numpy(b.sel_np).cuda()
        P = w.tokens_per_entry
        cl = torch.tensor([(w.n_entries - 1) * P + 1 + (r % (P - 1)) for r in range(w.batch)],
                          dtype=torch.int32, device="cuda")
        b.ctx.set_context_lengths(cl)
        ms_c, _, kc = b.passes(t0, t0 + K, 1, a.passes)
        b.ctx.set_context_lengths(None)
        ms_f, _, kf = b.passes(t0, t0 + K, 1, a.passes)
        assert b.ctx.last_error() == 0
        out["context_lengths"] = {
            "steps": K, "lists": "natural trace, last id of every list replaced by N - 1",
            "lengths": "(N - 1) P + 1 + (b mod (P - 1)) per request b: 1 to P - 1 rows of the "
                       "last page attended",
            "ms_per_step": round(ms_c, 4), "attention_us": round(kc["attention"], 2),
            "whole_pages_ms_per_step": round(ms_f, 4),
            "whole_pages_attention_us": round(kf["attention"], 2)}
    # the timed window captured once in a HIP graph (K steps, each reading
    # its own selections and queries) and replayed per pass, after the reset
    # and the fill steps run eagerly; the step counter lives in the
    # workspace, so the replayed steps stamp the right step numbers
    try:
        out["graph_replay"] = graph_replay(b, a, t0, K)
    except Exception as e:  # reported in the line; the other figures stand
        out["graph_replay"] = {"error": "%s: %s" % (type(e).__name__, e)}
        torch.cuda.synchronize()
    # the host KV reached through the two-level directory (256-entry
    # segments in pinned host memory, the top level in HBM), over the same
    # rows: entry e of unit u at pool row u * N + e
    out["host_directory"] = host_directory(b, a, t0, K)
    # Offload of the new token (append): every unit writes one token row into
    # host memory, and into its slot where the entry is resident
    na = 64
    tok_elems = w.head_dim_qk if w.latent else w.head_dim_qk + w.head_dim_v
    rng = np.random.default_rng(1)
    newkv = torch.from_numpy((rng.standard_normal((w.units, tok_elems)).astype(np.float32)
                              .view(np.uint32) >> 16).astype(np.int16)).cuda()
    ent = b.sel_np[-1][::w.n_kv_heads, 0, 0].astype(np.int64)   # resident in unit b*Hkv
    pos = torch.from_numpy((ent * w.tokens_per_entry).astype(np.int32)).cuda()
    st = b.st
    for _ in range(4):
        b.ctx.append(newkv, pos, b.host, st.buf_kv, st.slot_table)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(na):
        b.ctx.append(newkv, pos, b.host, st.buf_kv, st.slot_table)
    e1.record()
    torch.cuda.synchronize()
    assert b.ctx.last_error() == 0
    out["append"] = {"us": round(e0.elapsed_time(e1) / na * 1e3, 2),
                     "host_write_bytes": w.units * tok_elems * 2,
                     "slot_table_bytes_read": w.units * w.n_slots * 4}
    # append with insertion: (a) into the resident entries above (write
    # through, keep-state refreshed); (b) into entries no slot holds
    for _ in range(4):
        b.ctx.append_insert(newkv, pos, b.host, st.buf_kv, st.slot_table, st.lifetimes)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(na):
        b.ctx.append_insert(newkv, pos, b.host, st.buf_kv, st.slot_table, st.lifetimes)
    e1.record()
    torch.cuda.synchronize()
    us_res = e0.elapsed_time(e1) / na * 1e3
    # (b) from an emptied buffer at step 1: call i puts entry i of every unit
    # into slot i (empty slots go first), each unit copying the whole row
    b.reset()
    b.ctx.t = 1
    pos_miss = [torch.full((w.batch,), i * w.tokens_per_entry, dtype=torch.int32, device="cuda")
                for i in range(na)]
    torch.cuda.synchronize()
    e0.record()
    for i in range(na):
        b.ctx.append_insert(newkv, pos_miss[i], b.host, st.buf_kv, st.slot_table, st.lifetimes)
    e1.record()
    torch.cuda.synchronize()
    assert (st.slot_table[:, :na].cpu().numpy() == np.arange(na)).all()
    us_miss = e0.elapsed_time(e1) / na * 1e3
    assert b.ctx.last_error() == 0
    out["append_insert"] = {
        "resident_us": round(us_res, 2), "insert_us": round(us_miss, 2),
        "insert_host_read_bytes": w.units * (w.row_bytes - tok_elems * 2),
        "insert_host_GB/s": round(w.units * (w.row_bytes - tok_elems * 2) / (us_miss * 1e-6) / 1e9, 2)}
    # pinned hipMemcpy host->device peak, for context
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8).pin_memory()
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(4):
        dst.copy_(src, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    out["pinned_memcpy_h2d_GB/s"] = round(4 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9, 2)
    del src, dst
    # a plain device-to-device copy of 1 GiB: HBM bytes read + written
    xa = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    xb = torch.empty_like(xa)
    xb.copy_(xa)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(4):
        xb.copy_(xa)
    e1.record()
    torch.cuda.synchronize()
    out["hbm_copy_GB/s"] = round(4 * 2 * xa.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del xa, xb
    # a plain library bf16 GEMM (8192^3, contiguous operands): the matrix
    # cores' reachable rate beside the 2.5 PFLOP/s dense specification
    ga = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16).contiguous()
    gb = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16).contiguous()
    gc = torch.mm(ga, gb)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(8):
        torch.mm(ga, gb, out=gc)
    e1.record()
    torch.cuda.synchronize()
    out["gemm_bf16_TFLOP/s"] = round(8 * 2 * 8192.0 ** 3 / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    del ga, gb, gc
    return out


DIR_SEG = 256   # entries per second-level segment of the host directory


def metadata_bytes(units, n_entries, seg=DIR_SEG):
    """Bytes of the host-row metadata of a context of n_entries entries per
    unit: a flat table in HBM (one int32 pool row per entry) against the two
    levels (an int32 segment index per `seg` entries in HBM, the int32 rows
    of the segments in host memory)."""
    n_seg = -(-n_entries // seg)
    return {"entries_per_unit": n_entries, "flat_table_hbm_bytes": 4 * units * n_entries,
            "top_level_hbm_bytes": 4 * units * n_seg, "segments_host_bytes": 4 * units * n_seg * seg,
            "hbm_ratio": round(n_entries / n_seg, 1)}


def host_directory(b, a, t0, K):
    """The natural trace with host rows reached through the two-level
    directory, and its metadata sizes against a flat table."""
    torch, w, avsg = b.torch, b.w, b.avsg
    n_seg = -(-w.n_entries // DIR_SEG)
    segs = avsg.HostBuffer((w.units * n_seg, DIR_SEG), dtype=np.int32)
    rows = np.arange(w.units * n_seg * DIR_SEG, dtype=np.int64).reshape(w.units, n_seg * DIR_SEG)
    rows = rows - np.arange(w.units)[:, None] * (n_seg * DIR_SEG - w.n_entries)   # u * N + e
    rows[:, w.n_entries:] = -1
    segs.array[...] = rows.reshape(w.units * n_seg, DIR_SEG).astype(np.int32)
    top = torch.arange(w.units * n_seg, dtype=torch.int32, device="cuda").reshape(w.units, n_seg)
    b.ctx.set_host_directory(top, segs, DIR_SEG, w.units * n_seg, w.units * w.n_entries)
    b.load_trace("natural", t0 + K)
    ms, _, kern = b.passes(t0, t0 + K, 1, a.passes)
    b.ctx.set_host_directory(None, None, 0, 0, 0)
    assert b.ctx.last_error() == 0
    segs.free()
    ctx_tokens = [32768, 131072, 1 << 20]
    return {"seg_entries": DIR_SEG, "ms_per_step": round(ms, 5),
            "match_reserve_us": round(kern["match_reserve"], 2),
            "attention_us": round(kern["attention"], 2),
            "metadata": metadata_bytes(w.units, w.n_entries),
            "metadata_by_context_tokens": {
                str(n): metadata_bytes(w.units, -(-n // w.tokens_per_entry)) for n in ctx_tokens}}


def cpu_baseline(w, host_kv, t_start, seconds, threads=1):
    """The oracle (C state machine + float64 attention) on the same workload
    and the same pinned host KV, from step t_start on, until `seconds` have
    elapsed, with `threads` threads (OpenMP over units in the state machine,
    over (unit, token, head) in the attention)."""
    import tracegen as tg
    import oracle
    from oracle import attention as oatt
    oracle.set_threads(threads)
    steps_needed = t_start + 400  # the time bound ends the sample first
    sel = tg.selections(w, steps=steps_needed)
    ob = oracle.OracleBuffer.for_workload(w)
    for t in range(t_start):
        ob.step(sel[t])
    done, t0, t_state = 0, time.perf_counter(), 0.0
    t = t_start
    while time.perf_counter() - t0 < seconds and t < steps_needed:
        ts = time.perf_counter()
        r = ob.step(sel[t])
        t_state += time.perf_counter() - ts
        oatt.attend_native(w, tg.queries(w, t % Q_SETS), host_kv, sel[t], r["status"], threads=threads)
        done += 1
        t += 1
    el = time.perf_counter() - t0
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": done * w.entries_per_step / el, "unit": "entries/s", "cores": threads,
            "kind": "oracle", "steps_per_s": done / el,
            "state_only_value": done * w.entries_per_step / t_state,
            "state_only_steps_per_s": done / t_state,
            "cpu_model": cpu,
            "sample": "%d decode steps (t=%d..%d) of the %s workload, all %d units: C state "
                      "machine + C float64 attention, %s" % (
                          done, t_start, t_start + done - 1, w.name, w.units,
                          "one thread" if threads == 1 else "%d threads" % threads)}


def config_of(w, a):
    return {"workload": w.name, "requests": w.batch, "kv_heads": w.n_kv_heads,
            "q_heads": w.n_q_heads, "q_tokens": w.n_q_tokens, "head_dim_qk": w.head_dim_qk,
            "head_dim_v": w.head_dim_v, "context_entries": w.n_entries,
            "tokens_per_entry": w.tokens_per_entry,
            "context_tokens": w.n_entries * w.tokens_per_entry, "k": w.k, "slots": w.n_slots,
            "policy": w.policy, "lifetime_L": w.lifetime_L, "buckets": w.n_buckets,
            "bucket_width_steps": w.bucket_width,
            "trace": ("natural: %.0f%% overlap + Zipf(%.1f) tail" % (100 * w.overlap, w.zipf_s)
                      if a.trace == "natural" else a.trace),
            "transfer": ["fused", "balanced", "per-unit", "fused-gather-first"][a.transfer],
            "entries_per_step": w.entries_per_step, "fill_steps": a.fill}


def main(argv=None):
    a = parse(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus > 1 or world > 1:
        print("bench.py measures one GPU: the slot buffer's units are independent and the library "
              "runs on a single MI355X; --gpus %d is not supported" % max(a.gpus, world),
              file=sys.stderr)
        sys.exit(2)
    import torch
    import tracegen as tg
    from device_buffer_reuse_amd import avsg
    avsg.load()   # raises if the HIP library is not built
    w = tg.WORKLOADS[a.workload]
    W, K = a.warmup, a.steps
    b = Bench(w)
    b.ctx.set_transfer_mode(a.transfer)
    fused = a.transfer in (0, 3)

    # ---- the headline trace: value, kernels, roofline
    t0 = (a.fill + W) if a.trace == "natural" else (1 + W if a.trace == "allhit" else 4 + W)
    head = measure(b, a.trace, t0, K, a.warmup_passes, a.passes, fused)
    roof = dict(head["roofline"])
    roof["traffic"] = (counter_traffic(roof["kernel"], a.trace, a.workload)
                       if a.transfer == 0 else None)

    line = {
        "metric": "decode steps/s & selected KV entries/s; % HBM and host-link roofline",
        "value": head["entries_per_s"], "unit": "entries/s",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": head["ms_per_step"],
        "steps_per_s": head["steps_per_s"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": config_of(w, a),
        "timing": "median of %d passes (after %d untimed), each: avsg_reset, %d untimed steps "
                  "(fill %d + warmup %d), then %d timed steps t=%d..%d" % (
                      a.passes, a.warmup_passes, t0, a.fill if a.trace == "natural" else 0, W, K,
                      t0, t0 + K - 1),
        "ms_per_step_passes": head["ms_per_step_passes"],
        "hit_rate": head["hit_rate"],
        "miss_rows_per_step": head["miss_rows_per_step"],
        "host_bytes_per_step": head["host_bytes_per_step"],
        "union_per_step": head["union_per_step"],
        "kernels": head["kernels"],
        "roofline": roof,
        "step_roofline": head["step_roofline"],
    }
    if not a.no_extra:
        if a.trace == "natural":
            rest = measure_workload(b, a, ("allhit", "allmiss"))
            line["all_hit"] = brief(rest["allhit"])
            line["all_miss"] = brief(rest["allmiss"])
        line.update(extras(b, a))
    if a.buffer_sweep:
        line["buffer_sweep"] = buffer_sweep(b, a, [int(x) for x in a.buffer_sweep.split(",")])
    if a.ablations:
        line["ablations"] = ablations(a)
    if a.calibrate_copy:
        x = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            torch.mul(x, 1.0, out=y)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = {"read": x.numel() * 4, "write": y.numel() * 4}
    if not a.no_cpu_baseline:
        # the oracle reads the same pinned host KV the GPU steps read
        line["cpu_baseline"] = cpu_baseline(w, b.host.array, a.fill + W, a.cpu_seconds)
        nthr = len(os.sched_getaffinity(0))
        if nthr > 1:
            line["cpu_baseline_all_threads"] = cpu_baseline(w, b.host.array, a.fill + W,
                                                            a.cpu_seconds, nthr)
    b.close()
    del b
    if not a.no_extra and a.others.strip():
        line["workloads"] = {}
        for cid in [int(x) for x in a.others.split(",") if x.strip()]:
            if cid == a.workload:
                continue
            wo = tg.WORKLOADS[cid]
            bo = Bench(wo)
            bo.ctx.set_transfer_mode(a.transfer)
            r = measure_workload(bo, a)
            line["workloads"][wo.name] = {"config": config_of(wo, a)}
            line["workloads"][wo.name].update({m: brief(v) for m, v in r.items()})
            bo.close()
            del bo
            torch.cuda.empty_cache()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
