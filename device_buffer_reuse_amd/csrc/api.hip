// Host side of the libavsg C ABI: configuration checks, workspace layout,
// stream-ordered launches of the step kernels, error words and pinned memory.
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "avsg_internal.h"

struct avsg_ctx {
  avsg_config cfg;
  avsg::WsLayout ws;
  avsg::Derived d;
  hipStream_t stream;
  int device;
  int num_cus;
  int gather_grid;
  char* workspace;
  int64_t t;                     // the step of a caller-counted call (host_step)
  bool host_step;                // the caller passes the step (avsg_step_static); else the
                                 // counter lives in the workspace
  int32_t transfer_mode;         // avsg_transfer_mode
  int32_t match_mode;            // avsg_match_mode
  const int32_t* cap;            // device [units] buffer size of each unit, or null (S)
  const int32_t* ctx_len;        // device [batch] context length in tokens, or null (N * tpe)
  avsg::HostDir dir;             // two-level host directory (null top: flat host KV)
  int lds_max;
  hipEvent_t* prof_events;       // kProfMarks per profiled step, or null
  int32_t prof_max, prof_used;
  double prof_sort_ms, prof_walk_ms;  // merge baseline's phases in the last profile
};

namespace avsg {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// profiling events per step: before match_reserve, then after match_reserve,
// gather, attention and combine
constexpr int kProfMarks = 5;

static int32_t next_pow2(int64_t x) {
  int32_t c = 64;
  while (c < x) c <<= 1;
  return c;
}

constexpr size_t kMRLdsLimit = 160 * 1024;

// dynamic LDS of match_reserve: table, bucket counters, U and its slots,
// per-wave bin counts and offsets, bin starts, scratch, miss list, and for
// two tokens the union map and duplicate counts
static size_t mr_lds_bytes(const avsg_config& c, const WsLayout& ws, const Derived& d) {
  const int64_t tk = (int64_t)c.n_q_tokens * c.k;
  const int64_t ints = 2 * (int64_t)ws.ucap + ws.table_cap + ws.table_cap / 4 +
                       2 * 16 * (int64_t)d.nbins + d.nbins + 192 +
                       (c.n_q_tokens > 1 ? tk : ws.ucap) + (c.n_q_tokens > 1 ? tk + c.k + 1 : 0);
  return 4 * (size_t)ints;
}

bool layout_for(const avsg_config& c, WsLayout* ws, Derived* d) {
  d->units = c.batch * c.n_kv_heads;
  d->G = c.n_q_heads / c.n_kv_heads;
  d->row_elems = c.kv_layout == AVSG_KV_LATENT
                     ? c.head_dim_qk
                     : c.tokens_per_entry * (c.head_dim_qk + c.head_dim_v);
  d->nbins = c.policy == AVSG_POLICY_BUCKET_LRU ? c.n_buckets + 1 : c.lifetime_L + 2;
  const int64_t tk = (int64_t)c.n_q_tokens * c.k;
  ws->ucap = (int32_t)(tk < c.n_slots ? tk : c.n_slots);
  // hash table of U: load factor <= 1/4 (overflowing 4-cell buckets are
  // rare, so almost every probe ends at its home bucket) where the LDS of
  // match_reserve allows, else <= 1/2
  ws->table_cap = next_pow2(4 * (int64_t)ws->ucap);
  if (mr_lds_bytes(c, *ws, *d) > kMRLdsLimit) ws->table_cap = next_pow2(2 * (int64_t)ws->ucap);
  d->log_table_cap = 0;
  while ((1 << d->log_table_cap) < ws->table_cap) ++d->log_table_cap;
  // ids of a small context are matched by direct addressing (a membership bit
  // and a rank base per 32 ids) when that takes no more LDS than the table
  {
    const int64_t words = (((int64_t)c.n_entries + 31) / 32 + 3) & ~(int64_t)3;
    // (two tokens: a third word array, token 0's membership)
    const int64_t arrays = c.n_q_tokens > 1 ? 3 : 2;
    d->direct_words =
        arrays * words <= (int64_t)ws->table_cap + ws->table_cap / 4 ? (int32_t)words : 0;
  }
  d->ubits = 1;
  while ((1 << d->ubits) < ws->ucap) ++d->ubits;
  const int64_t rows = (int64_t)c.k * c.tokens_per_entry;
  if (c.attn_split_rows > 0) {
    ws->split_rows = c.attn_split_rows;
  } else if (c.kv_layout == AVSG_KV_LATENT) {
    ws->split_rows = 512;  // 4 splits: one 8-wave workgroup per CU for 64 requests
  } else {
    ws->split_rows = 256;  // one workgroup of the split-layout attention
  }
  ws->nsplit = (int32_t)((rows + ws->split_rows - 1) / ws->split_rows);
  const int64_t T = c.n_q_tokens;
  size_t off = 0;
  ws->unit_status = off; off = align256(off + 4 * (size_t)d->units);
  ws->miss_count = off;  off = align256(off + 4 * (size_t)d->units);
  ws->misses = off;      off = align256(off + 8 * (size_t)d->units * ws->ucap);
  ws->fetch = off;       off = align256(off + (size_t)d->units * tk);
  ws->host_row = off;    off = align256(off + 4 * (size_t)d->units * tk);
  ws->err_word = off;    off = align256(off + 8);
  ws->step = off;        off = align256(off + 8);
  ws->phase_clk = off;   off = align256(off + 3 * 8);
  ws->partials = off;
  const size_t part_bytes = c.kv_layout == AVSG_KV_LATENT
                                ? latent_partial_bytes(c.n_q_heads, c.head_dim_v)
                                : 4 * partial_stride(c.n_q_heads / c.n_kv_heads, c.head_dim_v);
  off = align256(off + (size_t)d->units * T * ws->nsplit * part_bytes);
  ws->total = off;
  d->mr_lds = mr_lds_bytes(c, *ws, *d);
  d->merge_pow2 = 64;
  while (d->merge_pow2 < c.n_slots) d->merge_pow2 <<= 1;
  // merge baseline: the table at load factor <= 1/2 (it only validates and
  // hashes the selection), then one spare word, the sorted (id, slot) pairs
  // and slot -> union index
  WsLayout wm = *ws;
  wm.table_cap = next_pow2(2 * (int64_t)ws->ucap);
  d->table_cap_half = wm.table_cap;
  d->log_table_cap_half = 0;
  while ((1 << d->log_table_cap_half) < wm.table_cap) ++d->log_table_cap_half;
  d->mr_lds_merge = mr_lds_bytes(c, wm, *d) + 4 + 8 * (size_t)d->merge_pow2 + 4 * (size_t)c.n_slots;
  return true;
}

// Workspace of avsg_step_static: device memory of the library itself, one
// copy per GPU (each device holds its own at its own address), kept until
// the process ends.  Host code never uses this name as an address: it takes
// each device's address from hipGetSymbolAddress once (device_setup).
constexpr size_t kStaticScratchBytes = AVSG_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
struct DeviceInfo {
  int num_cus;
  int lds_max;          // dynamic LDS a kernel of this device may be launched with
  void* scratch_ptr;    // this device's copy of `scratch`
};
static std::mutex g_dev_mutex;
static bool g_dev_ready[kMaxDevices];
static DeviceInfo g_dev[kMaxDevices];

// Once per device, with that device current: its unit count and LDS limit,
// the LDS limits of the kernels that need more than the default (set to the
// device maximum, so contexts with different sizes never lower each
// other's), and the device address of the static workspace.
static avsg_status device_setup(int* dev_out, DeviceInfo* info) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return AVSG_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return AVSG_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_dev_mutex);
  if (!g_dev_ready[dev]) {
    DeviceInfo di{};
    void* ptr = nullptr;
    if (hipDeviceGetAttribute(&di.num_cus, hipDeviceAttributeMultiprocessorCount, dev) !=
            hipSuccess ||
        hipDeviceGetAttribute(&di.lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
            hipSuccess ||
        match_reserve_set_lds((size_t)di.lds_max) != hipSuccess ||
        attn_latent_set_lds() != hipSuccess ||
        hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return AVSG_ERR_HIP;
    }
    di.scratch_ptr = ptr;
    g_dev[dev] = di;
    g_dev_ready[dev] = true;
  }
  *dev_out = dev;
  *info = g_dev[dev];
  return AVSG_OK;
}

// The separate gather kernel keeps the prefix of all units' miss counts in
// the default LDS of a workgroup.
static bool gather_fits(int units) { return 4 * ((size_t)units + 1) <= 64 * 1024; }

}  // namespace avsg

using namespace avsg;

static avsg_status check_config_impl(const avsg_config* c) {
  if (!c) return AVSG_ERR_INVALID_ARG;
  if (c->batch < 1 || c->n_kv_heads < 1 || c->n_q_heads < 1 || c->n_q_tokens < 1 ||
      c->head_dim_qk < 1 || c->head_dim_v < 1 || c->n_entries < 1 || c->tokens_per_entry < 1 ||
      c->k < 1 || c->n_slots < 1)
    return AVSG_ERR_INVALID_ARG;
  if (c->n_q_heads % c->n_kv_heads != 0) return AVSG_ERR_INVALID_ARG;
  if (c->k > c->n_slots || c->k > c->n_entries) return AVSG_ERR_INVALID_ARG;
  if (c->policy != AVSG_POLICY_LIFETIME && c->policy != AVSG_POLICY_BUCKET_LRU)
    return AVSG_ERR_INVALID_ARG;
  if (c->lifetime_L < 1 || c->n_buckets < 1) return AVSG_ERR_INVALID_ARG;
  // eviction bins (empty + lifetimes 0..L, or empty + buckets) must fit 128
  if (c->policy == AVSG_POLICY_LIFETIME && c->lifetime_L > 126) return AVSG_ERR_UNSUPPORTED;
  if (c->policy == AVSG_POLICY_BUCKET_LRU && c->n_buckets > 127) return AVSG_ERR_UNSUPPORTED;
  if (c->kv_layout != AVSG_KV_SPLIT && c->kv_layout != AVSG_KV_LATENT) return AVSG_ERR_INVALID_ARG;
  if (c->bucket_width < 0 || c->bucket_width > (1 << 30)) return AVSG_ERR_INVALID_ARG;
  if (c->attn_split_rows != 0 &&
      (c->attn_split_rows < 32 || c->attn_split_rows % 32 != 0 ||
       c->attn_split_rows > (c->kv_layout == AVSG_KV_LATENT ? 512 : 256)))
    return AVSG_ERR_INVALID_ARG;
  if (!(c->softmax_scale > 0.f)) return AVSG_ERR_INVALID_ARG;
  if ((int64_t)c->batch * c->n_kv_heads > (1 << 20)) return AVSG_ERR_UNSUPPORTED;
  if (c->n_q_tokens > 2) return AVSG_ERR_UNSUPPORTED;
  if (c->n_slots > kMRThreads * kMaxSlotsPerLane) return AVSG_ERR_UNSUPPORTED;
  if (c->n_slots >= kMissFlag || c->n_entries >= (1 << 30)) return AVSG_ERR_UNSUPPORTED;
  if (c->kv_layout == AVSG_KV_SPLIT) {
    const int G = c->n_q_heads / c->n_kv_heads;
    if (c->head_dim_qk != 128 || c->head_dim_v != 128) return AVSG_ERR_UNSUPPORTED;
    if (G != 1 && G != 2 && G != 4 && G != 8) return AVSG_ERR_UNSUPPORTED;
    // entry of a token row by multiply-high: exact while rows * tpe < 2^32
    if (c->tokens_per_entry > 256) return AVSG_ERR_UNSUPPORTED;
  } else {
    if (c->tokens_per_entry != 1 || c->n_kv_heads != 1) return AVSG_ERR_INVALID_ARG;
    if (c->head_dim_qk != 576 || c->head_dim_v != 512) return AVSG_ERR_UNSUPPORTED;
    if (c->n_q_heads != 64 && c->n_q_heads != 128) return AVSG_ERR_UNSUPPORTED;
  }
  WsLayout ws;
  Derived d;
  layout_for(*c, &ws, &d);
  if (d.mr_lds > kMRLdsLimit) return AVSG_ERR_UNSUPPORTED;
  // a hash cell packs (id << ubits | union index) with the top bit clear
  if ((int64_t)c->n_entries > ((int64_t)1 << (31 - d.ubits))) return AVSG_ERR_UNSUPPORTED;
  // gather addresses rows with 32-bit piece indices
  const int64_t row16 = (int64_t)d.row_elems * 2 / 16;
  if ((int64_t)d.row_elems * 2 % 16 != 0) return AVSG_ERR_UNSUPPORTED;
  if ((int64_t)d.units * ws.ucap * row16 >= ((int64_t)1 << 32)) return AVSG_ERR_UNSUPPORTED;
  return AVSG_OK;
}

extern "C" {

avsg_status avsg_check_config(const avsg_config* cfg) { return check_config_impl(cfg); }

size_t avsg_workspace_bytes(const avsg_config* cfg) {
  if (check_config_impl(cfg) != AVSG_OK) return 0;
  WsLayout ws;
  Derived d;
  layout_for(*cfg, &ws, &d);
  return ws.total;
}

const char* avsg_status_string(avsg_status s) {
  switch (s) {
    case AVSG_OK: return "ok";
    case AVSG_ERR_INVALID_ARG: return "invalid argument";
    case AVSG_ERR_NOT_PINNED: return "host_kv is not pinned device-mapped host memory";
    case AVSG_ERR_HIP: return "HIP runtime error";
    case AVSG_ERR_UNSUPPORTED: return "configuration not supported by the library's kernels";
    case AVSG_ERR_UNSORTED: return "selection not strictly ascending";
    case AVSG_ERR_RANGE: return "selected id out of range";
    case AVSG_ERR_CAPACITY: return "selection union exceeds buffer slots";
    case AVSG_ERR_STATE: return "invalid buffer state";
  }
  return "unknown status";
}

avsg_status avsg_create(const avsg_config* cfg, void* stream, void* workspace, size_t ws_bytes,
                        avsg_ctx** out) {
  if (!out) return AVSG_ERR_INVALID_ARG;
  *out = nullptr;
  avsg_status st = check_config_impl(cfg);
  if (st != AVSG_OK) return st;
  if (!workspace || ((uintptr_t)workspace & 255)) return AVSG_ERR_INVALID_ARG;
  avsg_ctx* c = new (std::nothrow) avsg_ctx();
  if (!c) return AVSG_ERR_INVALID_ARG;
  c->cfg = *cfg;
  layout_for(*cfg, &c->ws, &c->d);
  if (ws_bytes < c->ws.total) { delete c; return AVSG_ERR_INVALID_ARG; }
  DeviceInfo di;
  st = device_setup(&c->device, &di);
  if (st != AVSG_OK) { delete c; return st; }
  c->num_cus = di.num_cus;
  const int lds_max = di.lds_max;
  if ((int64_t)c->d.mr_lds > lds_max) { delete c; return AVSG_ERR_UNSUPPORTED; }
  c->gather_grid = c->num_cus * 2;
  c->stream = (hipStream_t)stream;
  c->workspace = (char*)workspace;
  c->t = 0;
  c->host_step = false;
  c->cap = nullptr;
  c->prof_events = nullptr;
  c->prof_max = c->prof_used = 0;
  c->prof_sort_ms = c->prof_walk_ms = 0.0;
  c->transfer_mode = AVSG_TRANSFER_FUSED;
  c->match_mode = AVSG_MATCH_HASH;
  c->lds_max = lds_max;
  // zero the library-owned workspace words (status, counts, error)
  if (launch_fill_i32((int32_t*)c->workspace, 0, c->ws.partials / 4, c->stream) != hipSuccess) {
    delete c;
    return AVSG_ERR_HIP;
  }
  *out = c;
  return AVSG_OK;
}

avsg_status avsg_set_transfer_mode(avsg_ctx* ctx, int32_t mode) {
  if (!ctx || mode < AVSG_TRANSFER_FUSED || mode > AVSG_TRANSFER_FUSED_GATHER_FIRST)
    return AVSG_ERR_INVALID_ARG;
  if ((mode == AVSG_TRANSFER_BALANCED || mode == AVSG_TRANSFER_PER_UNIT) && !gather_fits(ctx->d.units))
    return AVSG_ERR_UNSUPPORTED;
  ctx->transfer_mode = mode;
  return AVSG_OK;
}

avsg_status avsg_set_match_mode(avsg_ctx* ctx, int32_t mode) {
  if (!ctx || (mode != AVSG_MATCH_HASH && mode != AVSG_MATCH_MERGE && mode != AVSG_MATCH_HASH_TABLE))
    return AVSG_ERR_INVALID_ARG;
  // (the kernel's LDS limit is the device maximum, set once per device)
  if (mode == AVSG_MATCH_MERGE && (int64_t)ctx->d.mr_lds_merge > ctx->lds_max)
    return AVSG_ERR_UNSUPPORTED;
  ctx->match_mode = mode;
  return AVSG_OK;
}

avsg_status avsg_set_stream(avsg_ctx* ctx, void* stream) {
  if (!ctx) return AVSG_ERR_INVALID_ARG;
  ctx->stream = (hipStream_t)stream;
  return AVSG_OK;
}

static void destroy_prof_events(avsg_ctx* ctx) {
  if (!ctx->prof_events) return;
  for (int32_t i = 0; i < kProfMarks * ctx->prof_max; ++i)
    if (ctx->prof_events[i]) (void)hipEventDestroy(ctx->prof_events[i]);
  free(ctx->prof_events);
  ctx->prof_events = nullptr;
  ctx->prof_max = ctx->prof_used = 0;
}

avsg_status avsg_profile_begin(avsg_ctx* ctx, int32_t max_steps) {
  if (!ctx || max_steps < 1 || ctx->prof_events) return AVSG_ERR_INVALID_ARG;
  ctx->prof_events = (hipEvent_t*)calloc(kProfMarks * (size_t)max_steps, sizeof(hipEvent_t));
  if (!ctx->prof_events) return AVSG_ERR_INVALID_ARG;
  ctx->prof_max = max_steps;
  ctx->prof_used = 0;
  ctx->prof_sort_ms = ctx->prof_walk_ms = 0.0;
  for (int32_t i = 0; i < kProfMarks * max_steps; ++i)
    if (hipEventCreate(&ctx->prof_events[i]) != hipSuccess) {
      destroy_prof_events(ctx);
      return AVSG_ERR_HIP;
    }
  // the merge baseline's phase clocks start from zero (a fill kernel, in
  // stream order with the steps)
  if (launch_fill_i32((int32_t*)(ctx->workspace + ctx->ws.phase_clk), 0, 6, ctx->stream) !=
      hipSuccess) {
    destroy_prof_events(ctx);
    return AVSG_ERR_HIP;
  }
  return AVSG_OK;
}

avsg_status avsg_profile_end(avsg_ctx* ctx, double* ms, int32_t* steps) {
  if (!ctx || !ms || !steps || !ctx->prof_events) return AVSG_ERR_INVALID_ARG;
  avsg_status st = AVSG_OK;
  for (int k = 0; k < kProfMarks - 1; ++k) ms[k] = 0.0;
  if (hipStreamSynchronize(ctx->stream) != hipSuccess) st = AVSG_ERR_HIP;
  for (int32_t i = 0; st == AVSG_OK && i < ctx->prof_used; ++i)
    for (int k = 0; k < kProfMarks - 1; ++k) {
      float x = 0.f;
      hipEvent_t* ev = ctx->prof_events + kProfMarks * i;
      if (hipEventElapsedTime(&x, ev[k], ev[k + 1]) != hipSuccess) {
        st = AVSG_ERR_HIP;
        break;
      }
      ms[k] += x;
    }
  unsigned long long clk[3] = {0, 0, 0};
  if (st == AVSG_OK &&
      (hipMemcpyAsync(clk, ctx->workspace + ctx->ws.phase_clk, sizeof(clk), hipMemcpyDeviceToHost,
                      ctx->stream) != hipSuccess ||
       hipStreamSynchronize(ctx->stream) != hipSuccess))
    st = AVSG_ERR_HIP;
  // the clocks are summed over units and steps (100 MHz); divided by the
  // number of units they give, summed over the profiled steps in that mode,
  // each step's mean over units (the units run concurrently)
  const double units = (double)ctx->d.units;
  ctx->prof_sort_ms = st == AVSG_OK ? (double)clk[0] * 1e-5 / units : 0.0;
  ctx->prof_walk_ms = st == AVSG_OK ? (double)clk[1] * 1e-5 / units : 0.0;
  *steps = ctx->prof_used;
  destroy_prof_events(ctx);
  return st;
}

avsg_status avsg_profile_match_phases(const avsg_ctx* ctx, double* sort_ms, double* walk_ms) {
  if (!ctx || !sort_ms || !walk_ms) return AVSG_ERR_INVALID_ARG;
  *sort_ms = ctx->prof_sort_ms;
  *walk_ms = ctx->prof_walk_ms;
  return AVSG_OK;
}

static inline void prof_mark(avsg_ctx* ctx, int k) {
  if (ctx->prof_events && ctx->prof_used < ctx->prof_max)
    (void)hipEventRecord(ctx->prof_events[kProfMarks * ctx->prof_used + k], ctx->stream);
}

avsg_status avsg_destroy(avsg_ctx* ctx) {
  if (ctx) destroy_prof_events(ctx);
  delete ctx;
  return AVSG_OK;
}

int64_t avsg_get_step(const avsg_ctx* ctx) {
  if (!ctx) return -1;
  int64_t t = -1;
  if (hipMemcpyAsync(&t, ctx->workspace + ctx->ws.step, sizeof(t), hipMemcpyDeviceToHost,
                     ctx->stream) != hipSuccess ||
      hipStreamSynchronize(ctx->stream) != hipSuccess) {
    (void)hipGetLastError();
    return -1;
  }
  return t;
}

avsg_status avsg_set_step(avsg_ctx* ctx, int64_t t) {
  if (!ctx || t < 0 || t > INT32_MAX) return AVSG_ERR_INVALID_ARG;
  return launch_set_step((int64_t*)(ctx->workspace + ctx->ws.step), t, ctx->stream) == hipSuccess
             ? AVSG_OK
             : AVSG_ERR_HIP;
}

int32_t avsg_attn_splits(const avsg_ctx* ctx) { return ctx ? ctx->ws.nsplit : 0; }

avsg_status avsg_set_gather_workgroups(avsg_ctx* ctx, int32_t n) {
  if (!ctx || n < 0 || n > 65535) return AVSG_ERR_INVALID_ARG;
  ctx->gather_grid = n == 0 ? ctx->num_cus * 2 : n;
  return AVSG_OK;
}

avsg_status avsg_reset(avsg_ctx* ctx, int32_t* slot_table, int32_t* lifetimes) {
  if (!ctx || !slot_table || !lifetimes) return AVSG_ERR_INVALID_ARG;
  const size_t n = (size_t)ctx->d.units * ctx->cfg.n_slots;
  const int32_t life0 = ctx->cfg.policy == AVSG_POLICY_BUCKET_LRU ? -1 : 0;
  if (launch_fill_i32(slot_table, -1, n, ctx->stream) != hipSuccess ||
      launch_fill_i32(lifetimes, life0, n, ctx->stream) != hipSuccess ||
      launch_fill_i32((int32_t*)(ctx->workspace + ctx->ws.err_word), 0, 2, ctx->stream) != hipSuccess ||
      launch_fill_i32((int32_t*)(ctx->workspace + ctx->ws.step), 0, 2, ctx->stream) != hipSuccess)
    return AVSG_ERR_HIP;
  return AVSG_OK;
}

// The device-visible address of pinned host memory, looked up on every call
// (a buffer freed and allocated again may come back at the same host address
// with a different mapping).
static avsg_status device_view_of_pinned(const void* host, const void** dev) {
  hipPointerAttribute_t attr;
  memset(&attr, 0, sizeof(attr));
  if (hipPointerGetAttributes(&attr, host) != hipSuccess) {
    (void)hipGetLastError();
    return AVSG_ERR_NOT_PINNED;
  }
  if (attr.type != hipMemoryTypeHost || attr.devicePointer == nullptr) return AVSG_ERR_NOT_PINNED;
  *dev = attr.devicePointer;
  return AVSG_OK;
}

// A roctx range over the host-side enqueue of one call (a step or an
// append), so a trace with markers shows each call's kernels under its name.
struct RoctxRange {
  explicit RoctxRange(const char* name) { roctxRangePushA(name); }
  ~RoctxRange() { roctxRangePop(); }
};

static avsg_status step_impl(avsg_ctx* ctx, const int32_t* sel_idx, const int32_t* sel_len,
                             const uint16_t* q, const uint16_t* host_kv, uint16_t* buf_kv,
                             int32_t* slot_table, int32_t* lifetimes, float* out,
                             const avsg_hit_stats* hs) {
  RoctxRange range(sel_len ? "avsg_step_varlen" : "avsg_step");
  if (!ctx || !sel_idx || !q || !host_kv || !buf_kv || !slot_table || !lifetimes || !out || !hs ||
      !hs->hit_flag || !hs->sel_slot || !hs->n_hit || !hs->n_miss || !hs->n_evict)
    return AVSG_ERR_INVALID_ARG;
  // the kernels move rows, queries and outputs in 16-byte pieces
  if (((uintptr_t)q | (uintptr_t)host_kv | (uintptr_t)buf_kv | (uintptr_t)out) & 15)
    return AVSG_ERR_INVALID_ARG;
  const void* host_dev = nullptr;
  avsg_status st = device_view_of_pinned(host_kv, &host_dev);
  if (st != AVSG_OK) return st;
  const avsg_config& c = ctx->cfg;
  const bool fused = ctx->transfer_mode == AVSG_TRANSFER_FUSED ||
                     ctx->transfer_mode == AVSG_TRANSFER_FUSED_GATHER_FIRST;
  // checked before anything is launched: slots are never reserved for rows
  // that no kernel would copy
  if (!fused && !gather_fits(ctx->d.units)) return AVSG_ERR_UNSUPPORTED;
  char* ws = ctx->workspace;
  int32_t* unit_status = (int32_t*)(ws + ctx->ws.unit_status);
  int32_t* miss_count = (int32_t*)(ws + ctx->ws.miss_count);
  int2* misses = (int2*)(ws + ctx->ws.misses);

  MatchReserveParams mp;
  mp.sel = sel_idx;
  mp.sel_len = sel_len;
  mp.cap = ctx->cap;
  mp.ctx_len = ctx->ctx_len;
  mp.slot_table = slot_table;
  mp.lifetimes = lifetimes;
  mp.hit_flag = hs->hit_flag;
  mp.sel_slot = hs->sel_slot;
  mp.n_hit = hs->n_hit;
  mp.n_miss = hs->n_miss;
  mp.n_evict = hs->n_evict;
  mp.user_status = hs->unit_status;
  mp.unit_status = unit_status;
  mp.miss_count = miss_count;
  mp.misses = misses;
  mp.fetch = (uint8_t*)(ws + ctx->ws.fetch);
  mp.err_word = (uint32_t*)(ws + ctx->ws.err_word);
  mp.step = ctx->host_step ? nullptr : (int64_t*)(ws + ctx->ws.step);
  mp.t = ctx->t;
  mp.S = c.n_slots;
  mp.N = c.n_entries;
  mp.T = c.n_q_tokens;
  mp.k = c.k;
  mp.ucap = ctx->ws.ucap;
  const bool merge = ctx->match_mode == AVSG_MATCH_MERGE;
  // the table-only mode runs at load factor <= 1/2 (the setting the batch
  // workload states), in the LDS sized for the default mode's larger table
  const bool half = merge || ctx->match_mode == AVSG_MATCH_HASH_TABLE;
  mp.table_cap = half ? ctx->d.table_cap_half : ctx->ws.table_cap;
  mp.log_table_cap = half ? ctx->d.log_table_cap_half : ctx->d.log_table_cap;
  mp.ubits = ctx->d.ubits;
  mp.policy = c.policy;
  mp.L = c.lifetime_L;
  mp.B = c.n_buckets;
  mp.nbins = ctx->d.nbins;
  mp.Hkv = c.n_kv_heads;
  mp.tpe = c.tokens_per_entry;
  mp.W = c.bucket_width > 1 ? c.bucket_width : 1;
  mp.match_mode = ctx->match_mode;
  mp.merge_pow2 = ctx->d.merge_pow2;
  mp.direct_words = ctx->match_mode == AVSG_MATCH_HASH ? ctx->d.direct_words : 0;
  mp.dir = ctx->dir;
  mp.host_row = (int32_t*)(ws + ctx->ws.host_row);
  mp.phase_clk = (merge && ctx->prof_events && ctx->prof_used < ctx->prof_max)
                     ? (unsigned long long*)(ws + ctx->ws.phase_clk)
                     : nullptr;
  prof_mark(ctx, 0);
  const size_t mr_lds = merge ? ctx->d.mr_lds_merge : ctx->d.mr_lds;
  if (launch_match_reserve(mp, ctx->d.units, mr_lds, ctx->stream) != hipSuccess)
    return AVSG_ERR_HIP;
  prof_mark(ctx, 1);

  GatherParams gp;
  gp.misses = misses;
  gp.miss_count = miss_count;
  gp.host_kv = (const uint4*)host_dev;
  gp.buf_kv = (uint4*)buf_kv;
  gp.N = c.n_entries;
  gp.S = c.n_slots;
  gp.units = ctx->d.units;
  gp.ucap = ctx->ws.ucap;
  gp.row16 = ctx->d.row_elems * 2 / 16;
  gp.per_unit = ctx->transfer_mode == AVSG_TRANSFER_PER_UNIT;
  gp.pooled = ctx->dir.top != nullptr;
  if (!fused &&
      launch_gather(gp, gp.per_unit ? ctx->d.units : ctx->gather_grid, ctx->stream) != hipSuccess)
    return AVSG_ERR_HIP;
  prof_mark(ctx, 2);

  AttnParams ap;
  ap.sel_slot = hs->sel_slot;
  ap.sel_len = sel_len;
  ap.sel = sel_idx;
  ap.ctx_len = ctx->ctx_len;
  ap.step = ctx->host_step ? nullptr : (int64_t*)(ws + ctx->ws.step);
  ap.fetch = fused ? (const uint8_t*)(ws + ctx->ws.fetch) : nullptr;
  ap.host_row = ctx->dir.top ? (const int32_t*)(ws + ctx->ws.host_row) : nullptr;
  ap.host_kv = (const uint16_t*)host_dev;
  ap.N = c.n_entries;
  ap.token = 0;
  ap.gather_first = ctx->transfer_mode == AVSG_TRANSFER_FUSED_GATHER_FIRST ? 1 : 0;
  ap.unit_status = unit_status;
  ap.q = q;
  ap.buf_kv = buf_kv;
  ap.out = out;
  ap.partials = (float*)(ws + ctx->ws.partials);
  ap.S = c.n_slots;
  ap.units = ctx->d.units;
  ap.Hkv = c.n_kv_heads;
  ap.Hq = c.n_q_heads;
  ap.T = c.n_q_tokens;
  ap.k = c.k;
  ap.tpe = c.tokens_per_entry;
  ap.row_elems = ctx->d.row_elems;
  ap.nsplit = ctx->ws.nsplit;
  ap.split_rows = ctx->ws.split_rows;
  ap.scale_log2e = c.softmax_scale * 1.4426950408889634f;
  hipError_t e = c.kv_layout == AVSG_KV_LATENT
                     ? launch_attn_latent(ap, c.head_dim_qk, c.head_dim_v, ctx->stream)
                     : launch_attn_split(ap, ctx->d.G, ctx->stream);
  if (e != hipSuccess) return AVSG_ERR_HIP;
  prof_mark(ctx, 3);
  if (ap.nsplit > 1) {
    const int G = c.n_q_heads / (c.kv_layout == AVSG_KV_LATENT ? 1 : c.n_kv_heads);
    if (launch_attn_combine(ap, G, c.head_dim_v, c.kv_layout == AVSG_KV_LATENT, ctx->stream) !=
        hipSuccess)
      return AVSG_ERR_HIP;
  }
  prof_mark(ctx, 4);
  if (ctx->prof_events && ctx->prof_used < ctx->prof_max) ctx->prof_used += 1;
  return AVSG_OK;
}

avsg_status avsg_step(avsg_ctx* ctx, const int32_t* sel_idx, const uint16_t* q,
                      const uint16_t* host_kv, uint16_t* buf_kv, int32_t* slot_table,
                      int32_t* lifetimes, float* out, const avsg_hit_stats* hs) {
  return step_impl(ctx, sel_idx, nullptr, q, host_kv, buf_kv, slot_table, lifetimes, out, hs);
}

avsg_status avsg_step_varlen(avsg_ctx* ctx, const int32_t* sel_idx, const int32_t* sel_len,
                             const uint16_t* q, const uint16_t* host_kv, uint16_t* buf_kv,
                             int32_t* slot_table, int32_t* lifetimes, float* out,
                             const avsg_hit_stats* hs) {
  if (!sel_len) return AVSG_ERR_INVALID_ARG;
  return step_impl(ctx, sel_idx, sel_len, q, host_kv, buf_kv, slot_table, lifetimes, out, hs);
}

avsg_status avsg_step_static(const avsg_config* cfg, int64_t t, void* stream,
                             const int32_t* sel_idx, const uint16_t* q, const uint16_t* host_kv,
                             uint16_t* buf_kv, int32_t* slot_table, int32_t* lifetimes, float* out,
                             const avsg_hit_stats* hs) {
  avsg_status st = check_config_impl(cfg);
  if (st != AVSG_OK) return st;
  if (t < 0 || t > INT32_MAX || !hs || !hs->unit_status) return AVSG_ERR_INVALID_ARG;
  // the context lives on this stack frame: nothing is allocated
  avsg_ctx c{};
  c.cfg = *cfg;
  layout_for(*cfg, &c.ws, &c.d);
  if (c.ws.total > kStaticScratchBytes) return AVSG_ERR_UNSUPPORTED;
  DeviceInfo di;
  st = device_setup(&c.device, &di);
  if (st != AVSG_OK) return st;
  if ((int64_t)c.d.mr_lds > di.lds_max) return AVSG_ERR_UNSUPPORTED;
  c.num_cus = di.num_cus;
  c.lds_max = di.lds_max;
  c.gather_grid = di.num_cus * 2;
  c.stream = (hipStream_t)stream;
  c.workspace = (char*)di.scratch_ptr;
  c.t = t;
  c.host_step = true;
  c.transfer_mode = AVSG_TRANSFER_FUSED;
  c.match_mode = AVSG_MATCH_HASH;
  // the step's words that accumulate (the error bits) start at zero: the
  // array keeps whatever the previous call on this device left
  if (launch_fill_i32((int32_t*)(c.workspace + c.ws.err_word), 0, 2, c.stream) != hipSuccess)
    return AVSG_ERR_HIP;
  return step_impl(&c, sel_idx, nullptr, q, host_kv, buf_kv, slot_table, lifetimes, out, hs);
}

static avsg_status status_from_bits(uint32_t bits) {
  if (bits & (1u << (AVSG_ERR_RANGE - 16))) return AVSG_ERR_RANGE;
  if (bits & (1u << (AVSG_ERR_UNSORTED - 16))) return AVSG_ERR_UNSORTED;
  if (bits & (1u << (AVSG_ERR_CAPACITY - 16))) return AVSG_ERR_CAPACITY;
  if (bits & (1u << (AVSG_ERR_STATE - 16))) return AVSG_ERR_STATE;
  return AVSG_OK;
}

avsg_status avsg_last_error(avsg_ctx* ctx) {
  if (!ctx) return AVSG_ERR_INVALID_ARG;
  uint32_t bits = 0;
  uint32_t* dev = (uint32_t*)(ctx->workspace + ctx->ws.err_word);
  if (hipMemcpyAsync(&bits, dev, 4, hipMemcpyDeviceToHost, ctx->stream) != hipSuccess ||
      hipStreamSynchronize(ctx->stream) != hipSuccess)
    return AVSG_ERR_HIP;
  if (launch_fill_i32((int32_t*)dev, 0, 1, ctx->stream) != hipSuccess) return AVSG_ERR_HIP;
  return status_from_bits(bits);
}

// Derives the id -> slot map of every unit from slot_table in LDS (and checks
// lifetimes when given); syncs.  AVSG_ERR_STATE if any unit's map is invalid.
static avsg_status check_state(avsg_ctx* ctx, const int32_t* slot_table, const int32_t* lifetimes) {
  uint32_t* word = (uint32_t*)(ctx->workspace + ctx->ws.err_word) + 1;
  if (launch_fill_i32((int32_t*)word, 0, 1, ctx->stream) != hipSuccess) return AVSG_ERR_HIP;
  const avsg_config& c = ctx->cfg;
  // the step the stamps must precede (a syncing call: read from the workspace)
  const int64_t t = lifetimes ? avsg_get_step(ctx) : 0;
  if (t < 0) return AVSG_ERR_HIP;
  if (launch_validate(slot_table, lifetimes, ctx->d.units, c.n_slots, c.n_entries, c.policy,
                      c.lifetime_L, t, word, ctx->stream) != hipSuccess)
    return AVSG_ERR_HIP;
  uint32_t bits = 0;
  if (hipMemcpyAsync(&bits, word, 4, hipMemcpyDeviceToHost, ctx->stream) != hipSuccess ||
      hipStreamSynchronize(ctx->stream) != hipSuccess)
    return AVSG_ERR_HIP;
  return bits ? AVSG_ERR_STATE : AVSG_OK;
}

avsg_status avsg_rebuild_index(avsg_ctx* ctx, const int32_t* slot_table) {
  if (!ctx || !slot_table) return AVSG_ERR_INVALID_ARG;
  return check_state(ctx, slot_table, nullptr);
}

avsg_status avsg_validate_state(avsg_ctx* ctx, const int32_t* slot_table, const int32_t* lifetimes) {
  if (!ctx || !slot_table || !lifetimes) return AVSG_ERR_INVALID_ARG;
  return check_state(ctx, slot_table, lifetimes);
}
avsg_status avsg_set_capacity(avsg_ctx* ctx, const int32_t* cap) {
  if (!ctx) return AVSG_ERR_INVALID_ARG;
  ctx->cap = cap;
  return AVSG_OK;
}

avsg_status avsg_set_context_lengths(avsg_ctx* ctx, const int32_t* ctx_len) {
  if (!ctx) return AVSG_ERR_INVALID_ARG;
  ctx->ctx_len = ctx_len;
  return AVSG_OK;
}

avsg_status avsg_set_host_directory(avsg_ctx* ctx, const int32_t* top, const int32_t* segments,
                                    int32_t seg_entries, int32_t n_segments, int64_t pool_rows) {
  if (!ctx) return AVSG_ERR_INVALID_ARG;
  if (!top) {  // back to the flat host KV
    ctx->dir = HostDir{};
    return AVSG_OK;
  }
  if (!segments || seg_entries < 1 || seg_entries > (1 << 20) ||
      (seg_entries & (seg_entries - 1)) != 0 || n_segments < 1 || pool_rows < 1 ||
      pool_rows > INT32_MAX || ((int64_t)n_segments << 20) > ((int64_t)1 << 40))
    return AVSG_ERR_INVALID_ARG;
  const void* seg_dev = nullptr;
  avsg_status st = device_view_of_pinned(segments, &seg_dev);
  if (st != AVSG_OK) return st;
  HostDir d{};
  d.top = top;
  d.segments = (const int32_t*)seg_dev;
  while ((1 << d.seg_log2) < seg_entries) ++d.seg_log2;
  d.n_seg = (int32_t)(((int64_t)ctx->cfg.n_entries + seg_entries - 1) / seg_entries);
  d.n_segments = n_segments;
  d.pool_rows = pool_rows;
  ctx->dir = d;
  return AVSG_OK;
}

avsg_status avsg_plan_capacity(int32_t units, const int32_t* demand, const int32_t* reuse,
                               int64_t budget, int32_t n_slots, int32_t* cap) {
  if (units < 1 || !demand || !reuse || !cap || n_slots < 1) return AVSG_ERR_INVALID_ARG;
  int64_t mandatory = 0, weights = 0;
  for (int32_t u = 0; u < units; ++u) {
    if (demand[u] < 1 || demand[u] > n_slots || reuse[u] < 0) return AVSG_ERR_INVALID_ARG;
    mandatory += demand[u];
    weights += (int64_t)reuse[u] + 1;
  }
  if (mandatory > budget) return AVSG_ERR_CAPACITY;
  const __int128 spare = budget - mandatory;
  for (int32_t u = 0; u < units; ++u) {
    const __int128 extra = spare * ((int64_t)reuse[u] + 1) / weights;
    const __int128 c = (__int128)demand[u] + extra;
    cap[u] = c < (__int128)n_slots ? (int32_t)c : n_slots;
  }
  return AVSG_OK;
}

static avsg_status enqueue_append(avsg_ctx* ctx, const uint16_t* new_kv, const int32_t* pos,
                                  uint16_t* host_kv, uint16_t* buf_kv, const int32_t* slot_table,
                                  int32_t* lifetimes, bool insert) {
  if (!ctx || !new_kv || !pos || !host_kv || !buf_kv || !slot_table) return AVSG_ERR_INVALID_ARG;
  if (insert && !lifetimes) return AVSG_ERR_INVALID_ARG;
  if (((uintptr_t)new_kv | (uintptr_t)host_kv | (uintptr_t)buf_kv) & 15)
    return AVSG_ERR_INVALID_ARG;
  const avsg_config& c = ctx->cfg;
  const bool lru = c.policy == AVSG_POLICY_BUCKET_LRU;
  const void* host_dev = nullptr;
  avsg_status st = device_view_of_pinned(host_kv, &host_dev);
  if (st != AVSG_OK) return st;
  AppendParams ap;
  ap.new_kv = new_kv;
  ap.pos = pos;
  ap.host_kv = (uint16_t*)host_dev;
  ap.buf_kv = buf_kv;
  ap.slot_table = const_cast<int32_t*>(slot_table);  // written only when inserting
  ap.lifetimes = insert ? lifetimes : nullptr;
  ap.cap = insert ? ctx->cap : nullptr;
  ap.err_word = (uint32_t*)(ctx->workspace + ctx->ws.err_word);
  ap.dir = ctx->dir;
  ap.step = (const int64_t*)(ctx->workspace + ctx->ws.step);
  ap.Hkv = c.n_kv_heads;
  ap.N = c.n_entries;
  ap.S = c.n_slots;
  ap.tpe = c.tokens_per_entry;
  ap.row_elems = ctx->d.row_elems;
  ap.latent = c.kv_layout == AVSG_KV_LATENT ? 1 : 0;
  ap.dqk = c.head_dim_qk;
  ap.dv = c.head_dim_v;
  ap.tok_elems = ap.latent ? c.head_dim_qk : c.head_dim_qk + c.head_dim_v;
  ap.insert = insert ? 1 : 0;
  ap.lru = lru ? 1 : 0;
  ap.L = c.lifetime_L;
  ap.B = c.n_buckets;
  ap.W = c.bucket_width > 1 ? c.bucket_width : 1;
  return launch_append(ap, ctx->d.units, ctx->stream) == hipSuccess ? AVSG_OK : AVSG_ERR_HIP;
}

avsg_status avsg_append(avsg_ctx* ctx, const uint16_t* new_kv, const int32_t* pos,
                        uint16_t* host_kv, uint16_t* buf_kv, const int32_t* slot_table) {
  RoctxRange range("avsg_append");
  return enqueue_append(ctx, new_kv, pos, host_kv, buf_kv, slot_table, nullptr, false);
}

avsg_status avsg_append_insert(avsg_ctx* ctx, const uint16_t* new_kv, const int32_t* pos,
                               uint16_t* host_kv, uint16_t* buf_kv, int32_t* slot_table,
                               int32_t* lifetimes) {
  RoctxRange range("avsg_append_insert");
  return enqueue_append(ctx, new_kv, pos, host_kv, buf_kv, slot_table, lifetimes, true);
}

avsg_status avsg_host_alloc(size_t bytes, unsigned flags, void** host_ptr) {
  if (!host_ptr || bytes == 0) return AVSG_ERR_INVALID_ARG;
  *host_ptr = nullptr;
  unsigned f = hipHostMallocMapped | hipHostMallocPortable |
               ((flags & AVSG_HOST_COHERENT) ? hipHostMallocCoherent : hipHostMallocNonCoherent);
  if (hipHostMalloc(host_ptr, bytes, f) != hipSuccess) {
    (void)hipGetLastError();
    *host_ptr = nullptr;
    return AVSG_ERR_HIP;
  }
  return AVSG_OK;
}

avsg_status avsg_host_free(void* host_ptr) {
  if (!host_ptr) return AVSG_ERR_INVALID_ARG;
  return hipHostFree(host_ptr) == hipSuccess ? AVSG_OK : AVSG_ERR_HIP;
}

}  // extern "C"

namespace avsg {

__global__ void fill_i32_kernel(int32_t* p, int32_t v, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ void set_step_kernel(int64_t* step, int64_t t) { step[0] = t; }

hipError_t launch_set_step(int64_t* step, int64_t t, hipStream_t s) {
  hipLaunchKernelGGL(set_step_kernel, dim3(1), dim3(1), 0, s, step, t);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int32_t v, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

}  // namespace avsg
