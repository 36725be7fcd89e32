#!/usr/bin/env python3
"""Decode-step benchmark of the HBM slot buffer on one MI355X.

One step = one avsg_step over all units of the workload: match + reserve,
miss-only gather from pinned host memory, split-k attention.  The default
workload is the batch one (8 requests x 8 KV heads x 32 query heads,
head_dim 128, context 32768, k = 2048, 8192 slots per unit, lifetime L = 16)
on its natural trace (90% overlap + Zipf(1.1) tail), with `--warmup` untimed
steps, then exactly `--steps` timed steps.  Inputs (selections, queries) are
resident in HBM before the timed region; the KV cache is in pinned host
memory, which is the method's premise.

Prints one JSON line (rank 0).  Extra fields: per-kernel event times, hit
rate and host bytes per step, the all-hit and all-miss traces, and the CPU
oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
HOST_LINK_GBS = 64.0        # PCIe 5.0 x16, one direction
MFMA_BF16_TFLOPS = 2500.0   # dense bf16 matrix cores
FP32_VALU_TFLOPS = 157.3    # fp32 vector ALU


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--workload", type=int, default=2, help="1..5 (tracegen.WORKLOADS)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-extra", action="store_true", help="skip all-hit / all-miss passes")
    ap.add_argument("--trace", default="natural", choices=["natural", "allhit", "allmiss", "skewed"],
                    help="selection trace of the timed steps (default natural)")
    ap.add_argument("--transfer", type=int, default=0,
                    help="0 fused (default), 1 balanced gather kernel, 2 per-unit gather kernel, "
                         "3 fused, gather-first")
    ap.add_argument("--ablations", action="store_true",
                    help="also compare transfer modes on a skewed-miss trace and hash vs "
                         "dual-pointer matching")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain device copy of known size (for counter scaling)")
    return ap.parse_args()


class Bench:
    def __init__(self, w, total_steps):
        import torch
        import tracegen as tg
        from device_buffer_reuse_amd import avsg, build as hipbuild
        if not os.path.exists(avsg.LIB_PATH):
            hipbuild.build()
        self.torch, self.tg, self.avsg, self.w = torch, tg, avsg, w
        self.cfg = avsg.config_from_workload(w)
        self.ctx = avsg.Context(self.cfg)
        self.st = avsg.State(self.cfg)
        self.host = avsg.HostBuffer((w.units, w.n_entries, w.row_elems))
        tg.fill_kv(w, out=self.host.array)
        self.total = total_steps
        q = np.stack([tg.queries(w, t) for t in range(total_steps)])
        self.q_dev = torch.from_numpy(q.view(np.int16)).cuda()
        self.hs = self.st.stats.struct()
        self.lib = avsg.load()

    def load_trace(self, mode, steps):
        self.len_dev = None
        sel = self.tg.selections(self.w, steps=steps, mode=mode)
        self.sel_np = sel
        self.sel_dev = self.torch.from_numpy(sel).cuda()

    def reset(self):
        self.ctx.reset(self.st.slot_table, self.st.lifetimes)

    def load_varlen(self, steps, lo):
        """The natural trace with a list length per (step, unit) drawn from
        [lo, k] (PSA-style budgets); the following runs use avsg_step_varlen."""
        sel, lens = self.tg.shorten(self.tg.selections(self.w, steps=steps), 5, lo)
        self.sel_np = sel
        self.sel_dev = self.torch.from_numpy(sel).cuda()
        self.len_np = lens
        self.len_dev = self.torch.from_numpy(lens).cuda()

    def run(self, t0, t1, stats=None):
        lib, h, s = self.lib, self.ctx.handle, self.st
        import ctypes
        hsp = ctypes.byref(self.hs)
        sel0, selb = self.sel_dev.data_ptr(), self.sel_dev[0].numel() * 4
        q0, qb = self.q_dev.data_ptr(), self.q_dev[0].numel() * 2
        args = (self.host.ptr, s.buf_kv.data_ptr(), s.slot_table.data_ptr(), s.lifetimes.data_ptr(),
                s.out.data_ptr())
        lens = getattr(self, "len_dev", None)
        for t in range(t0, t1):
            if lens is not None:
                rc = lib.avsg_step_varlen(h, sel0 + t * selb, lens.data_ptr() + t * lens[0].numel() * 4,
                                          q0 + (t % self.total) * qb, *args, hsp)
            else:
                rc = lib.avsg_step(h, sel0 + t * selb, q0 + (t % self.total) * qb, *args, hsp)
            if rc != 0:
                raise self.avsg.AvsgError(rc, "avsg_step")
            if stats is not None:
                stats[0] += s.stats.n_hit
                stats[1] += s.stats.n_miss

    def timed(self, t0, t1, profile=False):
        torch = self.torch
        if profile:
            self.ctx.profile_begin(t1 - t0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        self.run(t0, t1)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        kern = None
        if profile:
            kern, n = self.ctx.profile_end()
            assert n == t1 - t0
        return ms, kern


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


KERNEL_SOURCES = {"attention": ("attn_split_kernel<4>", ["attn_split.hip", "avsg_internal.h"]),
                  "match_reserve": ("match_reserve_kernel<8>", ["match_reserve.hip", "avsg_internal.h"])}


def counter_traffic(kernel, trace):
    """HBM bytes per launch (reads + writes) of `kernel` from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary of the batch workload, scaled by
    the plain-copy calibration; None if the summary lacks that trace or the
    kernel's source changed since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "counters_batch.md")
    if kernel not in KERNEL_SOURCES or not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)```", open(path).read(), re.S)
    if not m:
        return None
    data = json.loads(m.group(1))
    name, files = KERNEL_SOURCES[kernel]
    k = data["kernels"].get(name)
    if not k:
        return None
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "device_buffer_reuse_amd", "csrc", f), "rb").read())
    if h.hexdigest()[:16] != k["source_sha256_16"]:
        return None
    r, wr = k.get("read_bytes_" + trace), k.get("write_bytes_" + trace)
    if r is None or wr is None:
        return None
    return int(r + wr)


def ablations(b, w, n):
    """Comparisons the AVSG abstract reports, reproduced in kind on this GPU:
    (1) transfers spread over all workgroups vs assigned per unit, on a trace
    where every 8th unit misses everything and the others hit everything;
    (2) vectorised hash matching vs the scalar dual-pointer baseline (kernel
    time of match_reserve on the natural trace)."""
    out = {}
    skew = {}
    b.load_trace("skewed", n + 2)
    for mode, name in ((0, "fused"), (1, "balanced"), (2, "per-unit")):
        b.ctx.set_transfer_mode(mode)
        b.reset()
        b.run(0, 2)
        ms, kern = b.timed(2, n + 2, profile=True)
        units_missing = (w.units + 7) // 8
        host_b = units_missing * w.n_q_tokens * w.k * w.row_bytes
        kt = kern[2] if mode == 0 else kern[1]
        skew[name] = {"ms_per_step": round(ms / n, 4),
                      "transfer_kernel_us": round(kt / n * 1e3, 2),
                      "effective_host_GB/s": round(host_b / (kt / n * 1e-3) / 1e9, 2)}
    b.ctx.set_transfer_mode(0)
    out["skewed_transfer"] = skew
    match = {}
    b.load_trace("natural", n + 16)
    for mode, name in ((0, "hash"), (2, "hash_table"), (1, "dual_pointer")):
        b.ctx.set_match_mode(mode)
        b.reset()
        b.run(0, 16)
        ms, kern = b.timed(16, n + 16, profile=True)
        match[name] = {"match_reserve_us": round(kern[0] / n * 1e3, 2),
                       "ms_per_step": round(ms / n, 4)}
    b.ctx.set_match_mode(0)
    match["speedup"] = round(match["dual_pointer"]["match_reserve_us"] /
                             match["hash"]["match_reserve_us"], 2)
    out["matching"] = match
    assert b.ctx.last_error() == 0
    return out


def cpu_baseline(w, t_start, seconds, threads=1):
    """The oracle (state machine + float64 attention) on the same workload,
    from step t_start on, until `seconds` have elapsed, with `threads`
    threads (the state machine's OpenMP loop over units and numpy's BLAS)."""
    import tracegen as tg
    import oracle
    from oracle import attention as oatt
    from threadpoolctl import threadpool_limits
    lim = threadpool_limits(threads)
    oracle.set_threads(threads)
    steps_needed = t_start + 192  # the time bound ends the sample first
    sel = tg.selections(w, steps=steps_needed)
    host = tg.fill_kv(w)
    ob = oracle.OracleBuffer.for_workload(w)
    for t in range(t_start):
        ob.step(sel[t])
    done, t0, t_state = 0, time.perf_counter(), 0.0
    t = t_start
    while time.perf_counter() - t0 < seconds and t < steps_needed:
        ts = time.perf_counter()
        r = ob.step(sel[t])
        t_state += time.perf_counter() - ts
        oatt.attend(w, tg.queries(w, t), host, sel[t], r["status"])
        done += 1
        t += 1
    el = time.perf_counter() - t0
    del lim
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": done * w.entries_per_step / el, "unit": "entries/s", "cores": threads,
            "kind": "oracle",
            "state_only_value": done * w.entries_per_step / t_state,
            "cpu_model": cpu,
            "sample": "%d decode steps (t=%d..%d) of the same workload, all %d units: C state "
                      "machine + float64 numpy attention, %s" % (
                          done, t_start, t_start + done - 1, w.units,
                          "one thread" if threads == 1 else "%d threads" % threads)}


def main():
    a = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus > 1 or world > 1:
        print("bench.py measures one GPU: the slot buffer's units are independent and the library "
              "runs on a single MI355X; --gpus %d is not supported" % max(a.gpus, world),
              file=sys.stderr)
        sys.exit(2)
    import torch
    import tracegen as tg
    w = tg.WORKLOADS[a.workload]
    W, K = a.warmup, a.steps
    total = W + K
    b = Bench(w, total)
    entries = w.entries_per_step
    row_bytes = w.row_bytes

    b.ctx.set_transfer_mode(a.transfer)
    # ---- the timed trace (natural by default): value
    b.load_trace(a.trace, total)
    b.reset()
    b.run(0, W)
    ms, _ = b.timed(W, W + K)
    assert b.ctx.last_error() == 0

    # ---- same steps again with per-kernel events, plus hit statistics
    b.reset()
    b.run(0, W)
    _, kern = b.timed(W, W + K, profile=True)
    b.reset()
    b.run(0, W)
    acc = [torch.zeros(w.units, dtype=torch.int64, device="cuda") for _ in range(2)]
    b.run(W, W + K, stats=acc)
    n_hit, n_miss = int(acc[0].sum()), int(acc[1].sum())
    miss_per_step = n_miss / K
    union_per_step = (n_hit + n_miss) / K

    per = {"match_reserve": kern[0] / K, "gather": kern[1] / K, "attention": kern[2] / K,
           "combine": kern[3] / K}
    fused = a.transfer in (0, 3)
    host_b = miss_per_step * row_bytes          # bytes over the host link per step
    ab = attn_bytes(w, union_per_step)
    # per kernel: algorithmic bytes (HBM / host link) and flops of one launch
    use = {
        "match_reserve": {"hbm": match_bytes(w, miss_per_step), "host": 0.0, "flop": 0.0},
        "gather": {"hbm": 0.0 if fused else host_b, "host": 0.0 if fused else host_b, "flop": 0.0},
        "attention": {"hbm": ab + (host_b if fused else 0.0), "host": host_b if fused else 0.0,
                      "flop": float(attn_flops(w))},
        # the merge of the split partials: no algorithmic bytes of its own
        # (the outputs are counted with the attention)
        "combine": {"hbm": 0.0, "host": 0.0, "flop": 0.0},
    }
    peaks = {"hbm": (HBM_PEAK_GBS, "GB/s", 1e9), "host": (HOST_LINK_GBS, "GB/s", 1e9),
             "flop": (MFMA_BF16_TFLOPS if w.latent else FP32_VALU_TFLOPS, "TFLOP/s", 1e12)}
    kernels = {}
    for name, u in use.items():
        if name == "gather" and fused:
            continue   # not launched: the fused transfer runs inside the attention
        t = per[name] * 1e-3
        d = {"us": round(per[name] * 1e3, 2)}
        for res, (pk, unit, scale) in peaks.items():
            if u[res] > 0 and t > 0:
                ach = u[res] / t / scale
                d[res + "_" + unit] = round(ach, 2)
                d[res + "_frac"] = round(ach / pk, 4)
        kernels[name] = d
    # the longest kernel among those with algorithmic work of their own
    dominant = max((n for n in per if any(v > 0 for v in use[n].values())), key=per.get)
    du = use[dominant]
    best = max((r for r in ("hbm", "host", "flop") if du[r] > 0),
               key=lambda r: du[r] / (per[dominant] * 1e-3) / peaks[r][2] / peaks[r][0])
    pk, unit, scale = peaks[best]
    ach = du[best] / (per[dominant] * 1e-3) / scale
    roof = {"bound": {"hbm": "hbm", "host": "host-link",
                      "flop": "mfma" if w.latent else "alu"}[best],
            "achieved": round(ach, 2), "peak": pk, "unit": unit, "frac": round(ach / pk, 4),
            "traffic": (counter_traffic(dominant, a.trace)
                        if w.name == "batch" and a.transfer == 0 else None),
            "kernel": dominant,
            "per_launch": int(du[best]) if best != "flop" else du[best]}

    step_roof = step_roofline(ab, match_bytes(w, miss_per_step), host_b, fused, ms / K * 1e-3)

    extra = {}
    if not a.no_extra:
        # all-hit: step 0 fills the buffer, later steps reuse every entry
        nh = min(K, 64)
        b.load_trace("allhit", nh + 1)
        # the step time comes from a pass without per-kernel events (their
        # records between launches add gaps); the kernel times from a second
        b.reset()
        b.run(0, 1)
        ms_h, _ = b.timed(1, nh + 1)
        b.reset()
        b.run(0, 1)
        _, kh = b.timed(1, nh + 1, profile=True)
        ab_h = attn_bytes(w, union_entries(b.sel_np[1:]))
        step_bytes = ab_h + match_bytes(w, 0)
        extra["all_hit"] = {
            "steps": nh, "ms_per_step": round(ms_h / nh, 4),
            "step_hbm_GB/s": round(step_bytes / (ms_h / nh * 1e-3) / 1e9, 1),
            "step_hbm_frac": round(step_bytes / (ms_h / nh * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "attention_us": round(kh[2] / nh * 1e3, 2),
            "attention_hbm_frac": round(ab_h / (kh[2] / nh * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "combine_us": round(kh[3] / nh * 1e3, 2),
            "match_reserve_us": round(kh[0] / nh * 1e3, 2)}
        # all-miss: disjoint windows, every entry crosses the host link
        nm = min(K, 32)
        b.load_trace("allmiss", nm + 4)
        b.reset()
        b.run(0, 4)
        ms_m, _ = b.timed(4, nm + 4)
        b.reset()
        b.run(0, 4)
        _, km = b.timed(4, nm + 4, profile=True)
        mb = w.units * w.n_q_tokens * w.k * row_bytes
        kt = km[2] if fused else km[1]   # kernel that carries the host transfer
        extra["all_miss"] = {
            "steps": nm, "ms_per_step": round(ms_m / nm, 4),
            "host_bytes_per_step": mb,
            "step_host_GB/s": round(mb / (ms_m / nm * 1e-3) / 1e9, 2),
            "step_host_link_frac": round(mb / (ms_m / nm * 1e-3) / 1e9 / HOST_LINK_GBS, 4),
            "transfer_kernel": "attention" if fused else "gather",
            "transfer_kernel_us": round(kt / nm * 1e3, 2),
            "transfer_kernel_host_GB/s": round(mb / (kt / nm * 1e-3) / 1e9, 2),
            "transfer_kernel_host_link_frac": round(mb / (kt / nm * 1e-3) / 1e9 / HOST_LINK_GBS, 4)}
        assert b.ctx.last_error() == 0
        # selections of a different size per list (PSA-style budgets,
        # lengths uniform in [k/8, k])
        nv = min(K, 64)
        b.load_varlen(32 + nv, max(1, w.k // 8))
        b.reset()
        b.run(0, 32)
        ms_v, _ = b.timed(32, 32 + nv)
        b.reset()
        b.run(0, 32)
        _, kv = b.timed(32, 32 + nv, profile=True)
        b.reset()
        b.run(0, 32)
        accv = [torch.zeros(w.units, dtype=torch.int64, device="cuda") for _ in range(2)]
        b.run(32, 32 + nv, stats=accv)
        vh, vm = int(accv[0].sum()), int(accv[1].sum())
        ent_v = float(b.len_np[32:32 + nv].sum()) * w.tokens_per_entry / nv
        hb_v = vm / nv * row_bytes
        extra["varlen"] = {
            "steps": nv, "lengths": "uniform in [k/8, k] per list and step, a random "
                                    "subset of the natural trace's list",
            "ms_per_step": round(ms_v / nv, 4),
            "entries_per_step": round(ent_v, 1),
            "entries_per_s": round(ent_v / (ms_v / nv * 1e-3), 1),
            "hit_rate": round(vh / max(vh + vm, 1), 5),
            "host_bytes_per_step": int(hb_v),
            "attention_us": round(kv[2] / nv * 1e3, 2),
            "attention_host_GB/s": round(hb_v / (kv[2] / nv * 1e-3) / 1e9, 2),
            "match_reserve_us": round(kv[0] / nv * 1e3, 2)}
        assert b.ctx.last_error() == 0
        # buffer sizes from the planner: every unit's union is mandatory, and
        # a quarter of the remaining slots (units x (S - |U|)) is shared by
        # reuse measured over the warm-up steps; timed on the natural trace
        nc = min(K, 64)
        b.load_trace("natural", 32 + nc)
        b.reset()
        accw = [torch.zeros(w.units, dtype=torch.int64, device="cuda") for _ in range(2)]
        b.run(0, 32, stats=accw)
        ucap = min(w.n_q_tokens * w.k, w.n_slots)
        demand = np.full(w.units, ucap, np.int32)
        reuse = np.minimum(accw[0].cpu().numpy(), 2**31 - 1).astype(np.int32)
        budget = int(demand.sum() + 0.25 * w.units * (w.n_slots - ucap))
        pst, caps = b.avsg.avsg_plan_capacity(demand, reuse, budget, w.n_slots)
        assert pst == 0
        cap_dev = torch.from_numpy(caps).cuda()
        b.ctx.set_capacity(cap_dev)
        b.run(32, 33)   # the shrink step
        ms_c, _ = b.timed(33, 32 + nc)
        b.reset()
        b.run(0, 33)
        accc = [torch.zeros(w.units, dtype=torch.int64, device="cuda") for _ in range(2)]
        b.run(33, 32 + nc, stats=accc)
        b.ctx.set_capacity(None)
        assert b.ctx.last_error() == 0
        ch, cm = int(accc[0].sum()), int(accc[1].sum())
        extra["capacity"] = {
            "steps": nc - 1, "budget_slots": budget, "full_slots": w.units * w.n_slots,
            "caps_min_max": [int(caps.min()), int(caps.max())],
            "ms_per_step": round(ms_c / (nc - 1), 4),
            "hit_rate": round(ch / max(ch + cm, 1), 5),
            "host_bytes_per_step": int(cm / (nc - 1) * row_bytes)}
        # Offload of the new token (append): every unit writes one token row
        # into host memory, and into its slot where the entry is resident
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
        a_us = e0.elapsed_time(e1) / na * 1e3
        extra["append"] = {"us": round(a_us, 2), "host_write_bytes": w.units * tok_elems * 2,
                           "slot_table_bytes_read": w.units * w.n_slots * 4}
        # pinned hipMemcpy host->device peak, for context
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8).pin_memory()
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(4):
            dst.copy_(src, non_blocking=True)
        e1.record()
        torch.cuda.synchronize()
        extra["pinned_memcpy_h2d_GB/s"] = round(4 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9, 2)
        # a plain device-to-device copy of 1 GiB: HBM bytes read + written
        del src, dst
        xa = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        xb = torch.empty_like(xa)
        xb.copy_(xa)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(4):
            xb.copy_(xa)
        e1.record()
        torch.cuda.synchronize()
        extra["hbm_copy_GB/s"] = round(4 * 2 * xa.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
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
        extra["gemm_bf16_TFLOP/s"] = round(8 * 2 * 8192.0 ** 3 / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
        del ga, gb, gc
    if a.ablations:
        extra["ablations"] = ablations(b, w, min(K, 32))
    if a.calibrate_copy:
        x = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            torch.mul(x, 1.0, out=y)
        torch.cuda.synchronize()
        extra["copy_calibration_bytes"] = {"read": x.numel() * 4, "write": y.numel() * 4}

    value = K * entries / (ms * 1e-3)
    line = {
        "metric": "decode steps/s & selected KV entries/s; % HBM and host-link roofline",
        "value": round(value, 1), "unit": "entries/s",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(ms / K, 5),
        "steps_per_s": round(K / (ms * 1e-3), 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "requests": w.batch, "kv_heads": w.n_kv_heads,
                   "q_heads": w.n_q_heads, "q_tokens": w.n_q_tokens, "head_dim_qk": w.head_dim_qk,
                   "head_dim_v": w.head_dim_v, "context_entries": w.n_entries,
                   "tokens_per_entry": w.tokens_per_entry, "k": w.k, "slots": w.n_slots,
                   "policy": w.policy, "lifetime_L": w.lifetime_L, "buckets": w.n_buckets,
                   "trace": ("natural: %.0f%% overlap + Zipf(%.1f) tail" % (100 * w.overlap, w.zipf_s)
                             if a.trace == "natural" else a.trace),
                   "transfer": ["fused", "balanced", "per-unit", "fused-gather-first"][a.transfer],
                   "entries_per_step": entries},
        "hit_rate": round(n_hit / max(n_hit + n_miss, 1), 5),
        "miss_rows_per_step": round(miss_per_step, 1),
        "host_bytes_per_step": int(miss_per_step * row_bytes),
        "union_per_step": round(union_per_step, 1),
        "kernels": kernels,
        "roofline": roof,
        "step_roofline": step_roof,
    }
    line.update(extra)
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, W, a.cpu_seconds)
        # the same oracle on every host thread the process may use
        nthr = len(os.sched_getaffinity(0))
        if nthr > 1:
            line["cpu_baseline_all_threads"] = cpu_baseline(w, W, a.cpu_seconds, nthr)
    print(json.dumps(line), flush=True)
    b.ctx.close()
    b.host.free()


if __name__ == "__main__":
    main()
