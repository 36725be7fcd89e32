"""Python binding of libavsg (ctypes): argument marshalling only.

Every function named avsg_* mirrors the C function of the same name in
include/avsg.h; pointers are passed as integers (torch tensors' data_ptr()).
`Context` bundles a context handle, its workspace and its stream for torch
callers.  Every step of the decode hot path runs in the HIP kernels of
libavsg.so; this module never computes any part of it, and raises if the
library is missing.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libavsg.so")

OK, ERR_INVALID_ARG, ERR_NOT_PINNED, ERR_HIP, ERR_UNSUPPORTED = 0, 1, 2, 3, 4
ERR_UNSORTED, ERR_RANGE, ERR_CAPACITY, ERR_STATE = 16, 17, 18, 19
KV_SPLIT, KV_LATENT = 0, 1
POLICY_LIFETIME, POLICY_BUCKET_LRU = 0, 1
HOST_COHERENT = 1
TRANSFER_FUSED, TRANSFER_BALANCED, TRANSFER_PER_UNIT, TRANSFER_FUSED_GATHER_FIRST = 0, 1, 2, 3
MATCH_HASH, MATCH_MERGE, MATCH_HASH_TABLE = 0, 1, 2

EXPORTED = ["avsg_check_config", "avsg_workspace_bytes", "avsg_create", "avsg_set_stream",
            "avsg_destroy", "avsg_reset", "avsg_step", "avsg_last_error", "avsg_validate_state",
            "avsg_get_step", "avsg_set_step", "avsg_host_alloc", "avsg_host_free",
            "avsg_status_string", "avsg_attn_splits", "avsg_profile_begin", "avsg_profile_end",
            "avsg_set_transfer_mode", "avsg_set_match_mode", "avsg_append", "avsg_append_insert",
            "avsg_rebuild_index", "avsg_step_varlen", "avsg_set_capacity",
            "avsg_plan_capacity", "avsg_step_static", "avsg_set_host_directory",
            "avsg_set_gather_workgroups", "avsg_profile_match_phases",
            "avsg_set_context_lengths"]
STATIC_SCRATCH_BYTES = 64 << 20   # AVSG_STATIC_SCRATCH_BYTES


class AvsgError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__("%s: %s (%d)" % (what, status_string(status), status))


class avsg_config(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_q_tokens", ctypes.c_int32),
                ("head_dim_qk", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
                ("kv_layout", ctypes.c_int32), ("n_entries", ctypes.c_int32),
                ("tokens_per_entry", ctypes.c_int32), ("k", ctypes.c_int32),
                ("n_slots", ctypes.c_int32), ("policy", ctypes.c_int32),
                ("lifetime_L", ctypes.c_int32), ("n_buckets", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("attn_split_rows", ctypes.c_int32),
                ("bucket_width", ctypes.c_int32)]


class avsg_hit_stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("hit_flag", "sel_slot", "n_hit", "n_miss", "n_evict", "unit_status")]


_lib = None


def load():
    """Load libavsg.so (built in-tree); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libavsg.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
    # torch carries its own copy of the HIP runtime under the same soname
    # (libamdhip64.so.7).  Loaded first, it is the copy libavsg binds to; were
    # libavsg loaded first, the process would hold two runtimes and the one
    # that initialises second finds no GPU.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    cfgp = ctypes.POINTER(avsg_config)
    sig = {
        "avsg_check_config": ([cfgp], i32),
        "avsg_workspace_bytes": ([cfgp], sz),
        "avsg_create": ([cfgp, p, p, sz, ctypes.POINTER(p)], i32),
        "avsg_set_stream": ([p, p], i32),
        "avsg_destroy": ([p], i32),
        "avsg_reset": ([p, p, p], i32),
        "avsg_step": ([p] * 8 + [ctypes.POINTER(avsg_hit_stats)], i32),
        "avsg_step_varlen": ([p] * 9 + [ctypes.POINTER(avsg_hit_stats)], i32),
        "avsg_step_static": ([cfgp, i64, p] + [p] * 7 + [ctypes.POINTER(avsg_hit_stats)], i32),
        "avsg_last_error": ([p], i32),
        "avsg_append": ([p] * 6, i32),
        "avsg_append_insert": ([p] * 7, i32),
        "avsg_validate_state": ([p, p, p], i32),
        "avsg_rebuild_index": ([p, p], i32),
        "avsg_set_capacity": ([p, p], i32),
        "avsg_set_context_lengths": ([p, p], i32),
        "avsg_set_host_directory": ([p, p, p, ctypes.c_int32, ctypes.c_int32, i64], i32),
        "avsg_plan_capacity": ([ctypes.c_int32, p, p, i64, ctypes.c_int32, p], i32),
        "avsg_get_step": ([p], i64),
        "avsg_set_step": ([p, i64], i32),
        "avsg_host_alloc": ([sz, ctypes.c_uint, ctypes.POINTER(p)], i32),
        "avsg_host_free": ([p], i32),
        "avsg_status_string": ([i32], ctypes.c_char_p),
        "avsg_attn_splits": ([p], ctypes.c_int32),
        "avsg_profile_begin": ([p, ctypes.c_int32], i32),
        "avsg_set_transfer_mode": ([p, ctypes.c_int32], i32),
        "avsg_set_gather_workgroups": ([p, ctypes.c_int32], i32),
        "avsg_set_match_mode": ([p, ctypes.c_int32], i32),
        "avsg_profile_end": ([p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)], i32),
        "avsg_profile_match_phases": ([p, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_double)], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


# ---------------------------------------------------------------- C mirrors

def status_string(s: int) -> str:
    return load().avsg_status_string(int(s)).decode()


def avsg_check_config(cfg: avsg_config) -> int:
    return load().avsg_check_config(ctypes.byref(cfg))


def avsg_workspace_bytes(cfg: avsg_config) -> int:
    return int(load().avsg_workspace_bytes(ctypes.byref(cfg)))


def avsg_create(cfg: avsg_config, stream: int, workspace: int, ws_bytes: int):
    h = ctypes.c_void_p()
    st = load().avsg_create(ctypes.byref(cfg), stream or None, workspace, ws_bytes, ctypes.byref(h))
    return st, h.value


def avsg_set_stream(ctx: int, stream: int) -> int:
    return load().avsg_set_stream(ctx, stream or None)


def avsg_destroy(ctx: int) -> int:
    return load().avsg_destroy(ctx)


def avsg_reset(ctx: int, slot_table: int, lifetimes: int) -> int:
    return load().avsg_reset(ctx, slot_table, lifetimes)


def avsg_step(ctx: int, sel_idx: int, q: int, host_kv: int, buf_kv: int, slot_table: int,
              lifetimes: int, out: int, hit_stats: avsg_hit_stats) -> int:
    return load().avsg_step(ctx, sel_idx, q, host_kv, buf_kv, slot_table, lifetimes, out,
                            ctypes.byref(hit_stats))


def avsg_step_varlen(ctx: int, sel_idx: int, sel_len: int, q: int, host_kv: int, buf_kv: int,
                     slot_table: int, lifetimes: int, out: int, hit_stats: avsg_hit_stats) -> int:
    return load().avsg_step_varlen(ctx, sel_idx, sel_len, q, host_kv, buf_kv, slot_table,
                                   lifetimes, out, ctypes.byref(hit_stats))


def avsg_step_static(cfg: avsg_config, t: int, stream: int, sel_idx: int, q: int, host_kv: int,
                     buf_kv: int, slot_table: int, lifetimes: int, out: int,
                     hit_stats: avsg_hit_stats) -> int:
    return load().avsg_step_static(ctypes.byref(cfg), t, stream or None, sel_idx, q, host_kv,
                                   buf_kv, slot_table, lifetimes, out, ctypes.byref(hit_stats))


def avsg_append(ctx: int, new_kv: int, pos: int, host_kv: int, buf_kv: int,
                slot_table: int) -> int:
    return load().avsg_append(ctx, new_kv, pos, host_kv, buf_kv, slot_table)


def avsg_append_insert(ctx: int, new_kv: int, pos: int, host_kv: int, buf_kv: int,
                       slot_table: int, lifetimes: int) -> int:
    return load().avsg_append_insert(ctx, new_kv, pos, host_kv, buf_kv, slot_table, lifetimes)


def avsg_last_error(ctx: int) -> int:
    return load().avsg_last_error(ctx)


def avsg_validate_state(ctx: int, slot_table: int, lifetimes: int) -> int:
    return load().avsg_validate_state(ctx, slot_table, lifetimes)


def avsg_rebuild_index(ctx: int, slot_table: int) -> int:
    return load().avsg_rebuild_index(ctx, slot_table)


def avsg_set_capacity(ctx: int, cap: int | None) -> int:
    return load().avsg_set_capacity(ctx, cap)


def avsg_set_context_lengths(ctx: int, ctx_len: int | None) -> int:
    return load().avsg_set_context_lengths(ctx, ctx_len)


def avsg_set_host_directory(ctx: int, top: int | None, segments: int | None, seg_entries: int,
                            n_segments: int, pool_rows: int) -> int:
    return load().avsg_set_host_directory(ctx, top, segments, seg_entries, n_segments, pool_rows)


def avsg_plan_capacity(demand: np.ndarray, reuse: np.ndarray, budget: int, n_slots: int):
    """Returns (status, cap int32 array)."""
    demand = np.ascontiguousarray(demand, dtype=np.int32)
    reuse = np.ascontiguousarray(reuse, dtype=np.int32)
    cap = np.zeros(demand.shape[0], dtype=np.int32)
    st = load().avsg_plan_capacity(int(demand.shape[0]), demand.ctypes.data, reuse.ctypes.data,
                                   int(budget), int(n_slots), cap.ctypes.data)
    return st, cap


def avsg_get_step(ctx: int) -> int:
    return int(load().avsg_get_step(ctx))


def avsg_set_step(ctx: int, t: int) -> int:
    return load().avsg_set_step(ctx, t)


def avsg_attn_splits(ctx: int) -> int:
    return int(load().avsg_attn_splits(ctx))


def avsg_set_transfer_mode(ctx: int, mode: int) -> int:
    return load().avsg_set_transfer_mode(ctx, mode)


def avsg_set_gather_workgroups(ctx: int, n: int) -> int:
    return load().avsg_set_gather_workgroups(ctx, n)


def avsg_set_match_mode(ctx: int, mode: int) -> int:
    return load().avsg_set_match_mode(ctx, mode)


def avsg_profile_begin(ctx: int, max_steps: int) -> int:
    return load().avsg_profile_begin(ctx, max_steps)


def avsg_profile_end(ctx: int):
    """Returns (status, [ms of match_reserve, gather, attention, combine], steps)."""
    ms = (ctypes.c_double * 4)()
    n = ctypes.c_int32()
    st = load().avsg_profile_end(ctx, ms, ctypes.byref(n))
    return st, [ms[0], ms[1], ms[2], ms[3]], n.value


def avsg_profile_match_phases(ctx: int):
    """Returns (status, sort ms, walk ms) of the dual-pointer baseline."""
    a, b = ctypes.c_double(), ctypes.c_double()
    st = load().avsg_profile_match_phases(ctx, ctypes.byref(a), ctypes.byref(b))
    return st, a.value, b.value


def avsg_host_alloc(nbytes: int, flags: int = 0):
    ptr = ctypes.c_void_p()
    st = load().avsg_host_alloc(nbytes, flags, ctypes.byref(ptr))
    return st, ptr.value


def avsg_host_free(ptr: int) -> int:
    return load().avsg_host_free(ptr)


# ---------------------------------------------------------------- conveniences

def config(batch, n_kv_heads, n_q_heads, n_q_tokens, head_dim_qk, head_dim_v, kv_layout,
           n_entries, tokens_per_entry, k, n_slots, policy, lifetime_L, n_buckets,
           softmax_scale, attn_split_rows=0, bucket_width=1) -> avsg_config:
    return avsg_config(batch, n_kv_heads, n_q_heads, n_q_tokens, head_dim_qk, head_dim_v,
                       kv_layout, n_entries, tokens_per_entry, k, n_slots, policy, lifetime_L,
                       n_buckets, softmax_scale, attn_split_rows, bucket_width)


def config_from_workload(w, attn_split_rows: int = 0) -> avsg_config:
    """avsg_config of a tracegen.Workload (shapes and policy only)."""
    return config(w.batch, w.n_kv_heads, w.n_q_heads, w.n_q_tokens, w.head_dim_qk, w.head_dim_v,
                  KV_LATENT if w.latent else KV_SPLIT, w.n_entries, w.tokens_per_entry, w.k,
                  w.n_slots, POLICY_BUCKET_LRU if w.policy == "lru" else POLICY_LIFETIME,
                  w.lifetime_L, w.n_buckets, w.softmax_scale, attn_split_rows, w.bucket_width)


# (address, ctypes buffer) of freed HostBuffers whose memory numpy arrays may
# still view: every array made from the buffer holds a reference to it
_pending_host_frees = []


def _release_host_memory():
    keep = []
    while _pending_host_frees:
        ptr, raw = _pending_host_frees.pop()
        # references: `raw` and getrefcount's argument
        if sys.getrefcount(raw) <= 2:
            avsg_host_free(ptr)
        else:
            keep.append((ptr, raw))
        del raw
    _pending_host_frees.extend(keep)


class HostBuffer:
    """Pinned, device-readable host memory from avsg_host_alloc, viewed as a
    numpy array (bf16 bit patterns as uint16 by default)."""

    def __init__(self, shape, dtype=np.uint16, flags: int = 0):
        self.shape = tuple(int(s) for s in shape)
        self.dtype = np.dtype(dtype)
        self.nbytes = int(np.prod(self.shape)) * self.dtype.itemsize
        st, ptr = avsg_host_alloc(self.nbytes, flags)
        if st != OK:
            raise AvsgError(st, "avsg_host_alloc(%d bytes)" % self.nbytes)
        self.ptr = ptr
        self._raw = (ctypes.c_char * self.nbytes).from_address(ptr)
        self.array = np.frombuffer(self._raw, dtype=self.dtype).reshape(self.shape)

    def free(self):
        """Returns the memory once no numpy view of it is left (a view kept
        elsewhere, e.g. by a traceback, would otherwise read freed memory);
        until then the release is retried by later calls."""
        if self.ptr:
            self.array = None
            _pending_host_frees.append((self.ptr, self._raw))
            self.ptr, self._raw = None, None
        _release_host_memory()

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


@dataclasses.dataclass
class HitStats:
    """Device tensors written by a step besides the attention output."""
    hit_flag: "object"     # uint8 [units][T][k]
    sel_slot: "object"     # int32 [units][T][k]
    n_hit: "object"        # int32 [units]
    n_miss: "object"
    n_evict: "object"
    unit_status: "object"  # int32 [units]

    @classmethod
    def empty(cls, units, T, k, device="cuda"):
        import torch
        z = lambda *s, dt=torch.int32: torch.zeros(*s, dtype=dt, device=device)
        return cls(z(units, T, k, dt=torch.uint8), z(units, T, k), z(units), z(units), z(units),
                   z(units))

    def struct(self) -> avsg_hit_stats:
        return avsg_hit_stats(self.hit_flag.data_ptr(), self.sel_slot.data_ptr(),
                              self.n_hit.data_ptr(), self.n_miss.data_ptr(),
                              self.n_evict.data_ptr(), self.unit_status.data_ptr())


class Context:
    """An avsg context with a torch-allocated workspace on the current device."""

    def __init__(self, cfg: avsg_config, stream=None):
        import torch
        self.cfg = cfg
        st = avsg_check_config(cfg)
        if st != OK:
            raise AvsgError(st, "avsg_check_config")
        self.ws_bytes = avsg_workspace_bytes(cfg)
        self.workspace = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device="cuda")
        base = self.workspace.data_ptr()
        self.ws_ptr = (base + 255) & ~255
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        st, h = avsg_create(cfg, self.stream.cuda_stream, self.ws_ptr, self.ws_bytes)
        if st != OK:
            raise AvsgError(st, "avsg_create")
        self.handle = h
        self.units = cfg.batch * cfg.n_kv_heads
        self._stats_struct = None

    def close(self):
        if getattr(self, "handle", None):
            avsg_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reset(self, slot_table, lifetimes):
        st = avsg_reset(self.handle, slot_table.data_ptr(), lifetimes.data_ptr())
        if st != OK:
            raise AvsgError(st, "avsg_reset")

    def step(self, sel_idx, q, host_kv, buf_kv, slot_table, lifetimes, out, stats: HitStats,
             sel_len=None):
        """host_kv: a HostBuffer or an integer address of pinned host memory;
        sel_len: optional device int32 [units] list lengths (avsg_step_varlen)."""
        hptr = host_kv.ptr if isinstance(host_kv, HostBuffer) else int(host_kv)
        if sel_len is None:
            st = avsg_step(self.handle, sel_idx.data_ptr(), q.data_ptr(), hptr, buf_kv.data_ptr(),
                           slot_table.data_ptr(), lifetimes.data_ptr(), out.data_ptr(),
                           stats.struct())
        else:
            st = avsg_step_varlen(self.handle, sel_idx.data_ptr(), sel_len.data_ptr(), q.data_ptr(),
                                  hptr, buf_kv.data_ptr(), slot_table.data_ptr(),
                                  lifetimes.data_ptr(), out.data_ptr(), stats.struct())
        if st != OK:
            raise AvsgError(st, "avsg_step_varlen" if sel_len is not None else "avsg_step")

    def append(self, new_kv, pos, host_kv, buf_kv, slot_table):
        """Offload of the new token: new_kv [batch][Hkv][tok_elems] (bf16 bits
        as int16), pos [batch] int32, both device tensors."""
        hptr = host_kv.ptr if isinstance(host_kv, HostBuffer) else int(host_kv)
        st = avsg_append(self.handle, new_kv.data_ptr(), pos.data_ptr(), hptr, buf_kv.data_ptr(),
                         slot_table.data_ptr())
        if st != OK:
            raise AvsgError(st, "avsg_append")

    def append_insert(self, new_kv, pos, host_kv, buf_kv, slot_table, lifetimes):
        """append() that also makes the token's entry resident in each unit's
        buffer before the coming step (slot_table, lifetimes in/out)."""
        hptr = host_kv.ptr if isinstance(host_kv, HostBuffer) else int(host_kv)
        st = avsg_append_insert(self.handle, new_kv.data_ptr(), pos.data_ptr(), hptr,
                                buf_kv.data_ptr(), slot_table.data_ptr(), lifetimes.data_ptr())
        if st != OK:
            raise AvsgError(st, "avsg_append_insert")

    def last_error(self) -> int:
        return avsg_last_error(self.handle)

    def validate_state(self, slot_table, lifetimes) -> int:
        return avsg_validate_state(self.handle, slot_table.data_ptr(), lifetimes.data_ptr())

    def set_capacity(self, cap):
        """cap: device int32 tensor [units] (kept alive by the caller), or None."""
        self._cap = cap
        st = avsg_set_capacity(self.handle, None if cap is None else cap.data_ptr())
        if st != OK:
            raise AvsgError(st, "avsg_set_capacity")

    def set_context_lengths(self, ctx_len):
        """ctx_len: device int32 tensor [batch] of context lengths in tokens
        (kept alive by the caller), or None: whole entries."""
        self._ctx_len = ctx_len
        st = avsg_set_context_lengths(self.handle, None if ctx_len is None else ctx_len.data_ptr())
        if st != OK:
            raise AvsgError(st, "avsg_set_context_lengths")

    def set_host_directory(self, top, segments, seg_entries: int, n_segments: int, pool_rows: int):
        """top: device int32 tensor [units][n_seg] (kept alive by the caller),
        segments: a HostBuffer of int32 [n_segments][seg_entries]; top=None
        returns to the flat host KV."""
        self._dir = (top, segments)
        st = avsg_set_host_directory(self.handle, None if top is None else top.data_ptr(),
                                     None if top is None else segments.ptr, seg_entries,
                                     n_segments, pool_rows)
        if st != OK:
            raise AvsgError(st, "avsg_set_host_directory")

    def rebuild_index(self, slot_table) -> int:
        return avsg_rebuild_index(self.handle, slot_table.data_ptr())

    @property
    def t(self) -> int:
        return avsg_get_step(self.handle)

    @t.setter
    def t(self, value: int):
        st = avsg_set_step(self.handle, value)
        if st != OK:
            raise AvsgError(st, "avsg_set_step")

    def set_stream(self, stream):
        """Later calls enqueue on `stream` (a torch.cuda.Stream)."""
        st = avsg_set_stream(self.handle, stream.cuda_stream)
        if st != OK:
            raise AvsgError(st, "avsg_set_stream")
        self.stream = stream

    def set_transfer_mode(self, mode: int):
        st = avsg_set_transfer_mode(self.handle, mode)
        if st != OK:
            raise AvsgError(st, "avsg_set_transfer_mode")

    def set_gather_workgroups(self, n: int):
        st = avsg_set_gather_workgroups(self.handle, n)
        if st != OK:
            raise AvsgError(st, "avsg_set_gather_workgroups")

    def set_match_mode(self, mode: int):
        st = avsg_set_match_mode(self.handle, mode)
        if st != OK:
            raise AvsgError(st, "avsg_set_match_mode")

    def profile_begin(self, max_steps: int):
        st = avsg_profile_begin(self.handle, max_steps)
        if st != OK:
            raise AvsgError(st, "avsg_profile_begin")

    def profile_end(self):
        """(per-stage summed ms [match_reserve, gather, attention, combine], steps)"""
        st, ms, n = avsg_profile_end(self.handle)
        if st != OK:
            raise AvsgError(st, "avsg_profile_end")
        return ms, n

    def profile_match_phases(self):
        """(sort ms, walk ms) of the dual-pointer baseline in the last profile"""
        st, a, b = avsg_profile_match_phases(self.handle)
        if st != OK:
            raise AvsgError(st, "avsg_profile_match_phases")
        return a, b

    @property
    def attn_splits(self) -> int:
        return avsg_attn_splits(self.handle)


class State:
    """Caller-owned device state and outputs for one workload (torch tensors)."""

    def __init__(self, cfg: avsg_config, device="cuda"):
        import torch
        units = cfg.batch * cfg.n_kv_heads
        row = cfg.head_dim_qk if cfg.kv_layout == KV_LATENT else \
            cfg.tokens_per_entry * (cfg.head_dim_qk + cfg.head_dim_v)
        self.units, self.row_elems = units, row
        self.slot_table = torch.full((units, cfg.n_slots), -1, dtype=torch.int32, device=device)
        self.lifetimes = torch.zeros((units, cfg.n_slots), dtype=torch.int32, device=device)
        self.buf_kv = torch.zeros((units, cfg.n_slots, row), dtype=torch.int16, device=device)
        self.out = torch.zeros((cfg.batch, cfg.n_q_tokens, cfg.n_q_heads, cfg.head_dim_v),
                               dtype=torch.float32, device=device)
        self.stats = HitStats.empty(units, cfg.n_q_tokens, cfg.k, device)
