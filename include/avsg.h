/*
 * avsg.h -- C ABI of libavsg: an HBM slot buffer for dynamic sparse attention
 * decode over a host-offloaded KV cache, on one MI355X (gfx950).
 *
 * What one decode step computes (avsg_step) follows the AVSG abstract
 * (arxivdaily 2609.37538, abstract): the selected KV entries of each
 * (request, KV head) unit are matched against the entries already resident in
 * a device buffer by a vectorised hash match, slots are reserved for the
 * entries that need a host-to-device transfer, only those are transferred,
 * with the transfer split evenly over the GPU's compute units, lifetime-based
 * management keeps frequently selected entries resident across steps, and one
 * reservation serves every query token of a multi-token-prediction iteration.
 * The bucketed-LRU alternative and head-wise pages follow the Spin summary
 * (gist.science 2604.26837, section 2B).  Attention then runs over the
 * buffer's slots; because selections are exact, its result equals attention
 * over the selected entries read from host memory.
 *
 * Conventions
 *  - A unit is one (request, KV head): unit u = b * n_kv_heads + g.
 *  - An entry is one token (tokens_per_entry = 1) or one page of
 *    tokens_per_entry tokens.  Entries are identified by their position id in
 *    [0, n_entries) within their unit.
 *  - bf16 values are passed as their uint16_t bit patterns.
 *  - Every pointer documented as "device" must be device memory of the GPU the
 *    context was created on (hipMalloc / torch CUDA tensors); "host, pinned"
 *    means memory from avsg_host_alloc or hipHostMalloc.
 *  - The caller owns all memory.  The library owns only the context struct;
 *    the workspace belongs to the caller but its contents to the library, and
 *    it must stay allocated and untouched across steps.
 *  - All calls that enqueue GPU work are asynchronous and ordered on the
 *    context's stream; none waits for the GPU unless documented ("syncs").
 *  - Errors in the data (selections, buffer state) are found on the GPU:
 *    the affected unit keeps its state, its outputs are zero / -1, and the
 *    error is reported by avsg_last_error.  Nothing is dropped silently.
 *  - One context per stream; calls on one context are not thread-safe.
 */
#ifndef AVSG_H
#define AVSG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum avsg_status {
  AVSG_OK = 0,
  AVSG_ERR_INVALID_ARG = 1,  /* null pointer, bad config, workspace too small */
  AVSG_ERR_NOT_PINNED = 2,   /* host_kv is not pinned, device-mapped host memory */
  AVSG_ERR_HIP = 3,          /* a HIP runtime call failed */
  AVSG_ERR_UNSUPPORTED = 4,  /* config valid but outside the library's kernels */
  /* data errors, found on the GPU and reported by avsg_last_error */
  AVSG_ERR_UNSORTED = 16,    /* a token's selection is not strictly ascending */
  AVSG_ERR_RANGE = 17,       /* an id, length, size, position or context length out of range */
  AVSG_ERR_CAPACITY = 18,    /* the union of an iteration's selections exceeds n_slots */
  AVSG_ERR_STATE = 19        /* slot_table / lifetimes are not a valid buffer state */
} avsg_status;

typedef enum avsg_kv_layout {
  /* row of an entry = K[tokens_per_entry][head_dim_qk] then V[tokens_per_entry][head_dim_v] */
  AVSG_KV_SPLIT = 0,
  /* row of an entry = one latent vector of head_dim_qk values (one token);
   * the key is the whole row, the value its first head_dim_v values */
  AVSG_KV_LATENT = 1
} avsg_kv_layout;

typedef enum avsg_policy {
  /* Lifetime-based management (AVSG abstract).  A slot whose entry is selected
   * gets lifetime L; every other occupied slot loses one per step, floored at
   * 0; a slot at 0 stays resident and can still hit. */
  AVSG_POLICY_LIFETIME = 0,
  /* Bucketed LRU (Spin summary, section 2B): lifetimes[] holds the step of
   * last selection; the bucket of a slot is min(t - stamp - 1, n_buckets - 1)
   * with one-step buckets (bucket_width widens them) and older buckets are
   * evicted first.  Stamps are int32, so a context takes at most 2^31 steps
   * under this policy before avsg_reset (a later step's stamps fail
   * validation: AVSG_ERR_STATE). */
  AVSG_POLICY_BUCKET_LRU = 1
} avsg_policy;

typedef struct avsg_config {
  int32_t batch;             /* requests */
  int32_t n_kv_heads;        /* KV heads per request (1 for the latent layout) */
  int32_t n_q_heads;         /* query heads per request; head h reads KV head h / (n_q_heads / n_kv_heads) */
  int32_t n_q_tokens;        /* T: query tokens per iteration sharing one reservation (1 or 2) */
  int32_t head_dim_qk;       /* split layout: 128; latent layout: 576 */
  int32_t head_dim_v;        /* split layout: 128; latent layout: 512 */
  int32_t kv_layout;         /* avsg_kv_layout */
  int32_t n_entries;         /* N: entries per unit in host memory */
  int32_t tokens_per_entry;  /* 1 (token entries) .. 256 (pages); latent layout: 1 */
  int32_t k;                 /* entries selected per query token */
  int32_t n_slots;           /* S: buffer slots per unit */
  int32_t policy;            /* avsg_policy */
  int32_t lifetime_L;        /* L >= 1 (lifetime policy) */
  int32_t n_buckets;         /* B >= 1 (bucketed LRU) */
  float softmax_scale;       /* multiplies q.k before the softmax */
  /* token rows per attention workgroup (split-k): 0 = the library's choice
   * (256 for the split layout, 512 for the latent layout), else a multiple
   * of 32 in [32, 256] (split layout) or [32, 512] (latent layout).  Results
   * other than the attention output's rounding do not depend on it. */
  int32_t attn_split_rows;
  /* steps per bucket of the bucketed LRU (Spin summary, section 2B gives
   * recency buckets but not their width): the bucket of a slot is
   * min(floor((t - stamp - 1) / W), n_buckets - 1).  0 or 1: one step per
   * bucket; else W in [2, 2^30]. */
  int32_t bucket_width;
} avsg_config;

/* Per-step outputs besides the attention result; all device pointers. */
typedef struct avsg_hit_stats {
  uint8_t* hit_flag;     /* [units][T][k]: 1 if the entry was resident before this step */
  int32_t* sel_slot;     /* [units][T][k]: slot holding the entry after this step (-1 on error) */
  int32_t* n_hit;        /* [units]: entries of the union that were resident */
  int32_t* n_miss;       /* [units]: entries of the union transferred from host memory */
  int32_t* n_evict;      /* [units]: reserved slots that held another entry */
  int32_t* unit_status;  /* [units]: 0 or the avsg_status of that unit's data error; may be NULL */
} avsg_hit_stats;

typedef struct avsg_ctx avsg_ctx;

/* Checks a configuration on the host only (no GPU needed).  Returns AVSG_OK,
 * AVSG_ERR_INVALID_ARG (inconsistent values) or AVSG_ERR_UNSUPPORTED (a shape
 * the library's kernels do not handle). */
avsg_status avsg_check_config(const avsg_config* cfg);

/* Bytes of device workspace a context for cfg needs (0 if cfg is invalid).
 * Host only. */
size_t avsg_workspace_bytes(const avsg_config* cfg);

/* Creates a context on the current HIP device.  `stream` is a hipStream_t
 * (NULL = the null stream).  `workspace` is device memory of at least
 * avsg_workspace_bytes(cfg) bytes, 256-byte aligned, owned by the caller and
 * kept alive and untouched until avsg_destroy.  Initialising it is enqueued
 * on the stream.  The workspace holds the step counter (starting at 0), so a
 * step needs no host state: steps may be captured in a HIP graph and
 * replayed. */
avsg_status avsg_create(const avsg_config* cfg, void* stream, void* workspace, size_t ws_bytes,
                        avsg_ctx** out);

/* Changes the stream later calls enqueue on. */
avsg_status avsg_set_stream(avsg_ctx* ctx, void* stream);

/* Frees the context struct (not the caller's memory). Does not sync. */
avsg_status avsg_destroy(avsg_ctx* ctx);

/* Empties the buffer: slot_table[units][S] = -1, lifetimes[units][S] = 0
 * (lifetime policy) or -1 (LRU), step counter = 0, pending errors cleared.
 * Device pointers; enqueued on the stream. */
avsg_status avsg_reset(avsg_ctx* ctx, int32_t* slot_table, int32_t* lifetimes);

/* One decode step t (the context's counter in the workspace; the step's
 * kernels advance it by one on the GPU).  The context's settings apply:
 * buffer sizes (avsg_set_capacity), context lengths
 * (avsg_set_context_lengths), the host directory (avsg_set_host_directory),
 * the transfer and match modes.
 *   sel_idx    device, int32 [batch][n_kv_heads][T][k]: each token's selected
 *              entry ids, strictly ascending, in [0, N) (and inside the
 *              request's context when context lengths are set).  read only
 *   q          device, bf16 [batch][T][n_q_heads][head_dim_qk]     read only
 *   host_kv    host, pinned, bf16 [units][N][row]: the full KV cache, row as
 *              given by kv_layout.                                  read only
 *   buf_kv     device, bf16 [units][S][row]: the slot buffer.       in/out
 *   slot_table device, int32 [units][S]: id held by each slot, -1 = empty.
 *                                                                   in/out
 *   lifetimes  device, int32 [units][S]: lifetime, or stamp (LRU).   in/out
 *   out        device, fp32 [batch][T][n_q_heads][head_dim_v]: attention of
 *              each query head over its token's selected entries; 0 for a
 *              unit with a data error.                              written
 *   hit_stats  host struct of device pointers (see avsg_hit_stats). written
 * q, host_kv, buf_kv and out must be 16-byte aligned (rows, queries and
 * outputs move in 16-byte pieces).
 * Returns AVSG_ERR_INVALID_ARG for null or misaligned pointers,
 * AVSG_ERR_NOT_PINNED if host_kv is not device-accessible pinned host memory,
 * AVSG_ERR_HIP if a launch fails; data errors are reported later by
 * avsg_last_error.  Never waits for the GPU. */
avsg_status avsg_step(avsg_ctx* ctx, const int32_t* sel_idx, const uint16_t* q,
                      const uint16_t* host_kv, uint16_t* buf_kv, int32_t* slot_table,
                      int32_t* lifetimes, float* out, const avsg_hit_stats* hit_stats);

/* avsg_step with a selection length per list, for selections whose size
 * varies by request, head and query token (the PSA abstract: the KV budget
 * is adapted per token and layer to the attention weights instead of one
 * fixed k).
 *   sel_len    device, int32 [batch][n_kv_heads][T]: token j of unit u uses
 *              the first sel_len[u][j] ids of sel_idx[u][j] (strictly
 *              ascending, in [0, N)); the rest of its k positions are
 *              ignored, and their hit_flag, sel_slot outputs are 0 and -1.
 *                                                                  read only
 * All other arguments and results as avsg_step, with the union U formed
 * from the lists in use.  A length outside [1, k] is a data error of that
 * unit (AVSG_ERR_RANGE).  Attention splits past a list's length do no work,
 * so a long list is spread over as many workgroups as its rows need whatever
 * the other lists' lengths.  AVSG_ERR_INVALID_ARG if sel_len is null. */
avsg_status avsg_step_varlen(avsg_ctx* ctx, const int32_t* sel_idx, const int32_t* sel_len,
                             const uint16_t* q, const uint16_t* host_kv, uint16_t* buf_kv,
                             int32_t* slot_table, int32_t* lifetimes, float* out,
                             const avsg_hit_stats* hit_stats);

/* avsg_step for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): no
 * context and no caller workspace.  The step's scratch (per-unit status and
 * miss lists, fetch flags, error words, split partials) is a device array
 * inside the library, AVSG_STATIC_SCRATCH_BYTES per GPU, held by every GPU
 * the library runs on until the process ends; the call itself allocates
 * nothing (no hipMalloc, no host or device allocation by any library).
 *   cfg        host, the configuration (as avsg_create's)
 *   t          the decode step (the caller keeps the counter: 0 after an
 *              emptied buffer, then +1 per call), in [0, 2^31)
 *   stream     hipStream_t to enqueue on (NULL = the null stream), of the
 *              current device
 *   the rest   exactly as avsg_step, with the fused transfer, the hash
 *              match, all S slots, whole entries and a flat host KV (the
 *              context settings do not exist here); hit_stats->unit_status
 *              is required (it is where data errors are reported, per unit:
 *              there is no context to hold an error word for
 *              avsg_last_error).
 * Returns AVSG_ERR_UNSUPPORTED if the configuration's scratch exceeds
 * AVSG_STATIC_SCRATCH_BYTES (see avsg_workspace_bytes) and otherwise the
 * codes of avsg_check_config and avsg_step.  Results are bit-identical to
 * avsg_step's on the same inputs.  Every call on one GPU uses that GPU's one
 * array, which keeps the previous call's contents: calls that may overlap in
 * time on one GPU (other streams, other host threads) race, so serialise
 * them (one stream, or events).  The first call on a device also looks up
 * that device's copy of the array and sets the kernels' LDS limits. */
#define AVSG_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
avsg_status avsg_step_static(const avsg_config* cfg, int64_t t, void* stream,
                             const int32_t* sel_idx, const uint16_t* q, const uint16_t* host_kv,
                             uint16_t* buf_kv, int32_t* slot_table, int32_t* lifetimes, float* out,
                             const avsg_hit_stats* hit_stats);

/* Buffer size per unit (Spin summary, section 2B, buffer elasticity: each
 * request's device buffer is sized dynamically, mandatory pages for the
 * current step plus buffer pages kept for locality).  `cap` is a device
 * int32 array [batch][n_kv_heads] read by every later step when it runs
 * (update its contents between steps, stream-ordered), or NULL for S slots
 * each.  A step lets unit u use slots [0, cap[u]) only and empties the slots
 * at or past cap[u] (slot -1, lifetime 0 or stamp -1): shrinking a unit's
 * buffer drops the entries it held there, which stay exact in host memory.
 * cap[u] outside [1, S] is a range error and |U| > cap[u] a capacity error
 * of that unit (its state then stays untouched, as for every data error:
 * a step with any data error leaves the slots past cap[u] as they were).
 * The pointer is kept by the context; the caller owns the array. */
avsg_status avsg_set_capacity(avsg_ctx* ctx, const int32_t* cap);

/* Context length of each request, in tokens (page-based KV of the Spin
 * summary, sections 2A and 2B: decoded tokens are appended into the current
 * page, so the last page of a context may be only partly written).  Entry e
 * holds positions [e P, (e + 1) P), P = tokens_per_entry.  `ctx_len` is a
 * device int32 array [batch] read by every later step when it runs (update
 * it between steps, stream-ordered, e.g. after each avsg_append), or NULL:
 * every entry holds P tokens.  A step then attends, of each selected entry,
 * only the rows at positions below the length (what the other rows of the
 * last page hold never matters, NaN included); transfers still copy whole
 * rows, so the buffer keeps exact copies.  A selected id whose first position
 * is at or past the length is a range error of its unit, as is a length
 * outside [1, N P].  avsg_step_static takes no lengths.  The pointer is kept
 * by the context; the caller owns the array. */
avsg_status avsg_set_context_lengths(avsg_ctx* ctx, const int32_t* ctx_len);

/* Host KV through a two-level directory (Spin summary, section 2C:
 * hierarchical metadata; a small top-level directory on the GPU points to
 * second-level segments allocated on demand in CPU memory, so metadata
 * follows the mapped working set instead of the largest logical context, and
 * the latency-critical level stays on the GPU).  After this call host_kv
 * (of avsg_step, avsg_step_varlen and avsg_append) is a pool of pool_rows
 * rows [pool_rows][row], and entry e of unit u lives at pool row
 *   segments[top[u][e / seg_entries]][e % seg_entries]
 *   top        device, int32 [units][ceil(n_entries / seg_entries)]: the
 *              segment of each range of seg_entries entries, -1 = none.  The
 *              context keeps the pointer; contents are read by each step
 *              (update them between steps, stream-ordered).     read only
 *   segments   host, pinned (avsg_host_alloc), int32 [n_segments][seg_entries]:
 *              pool row of each entry, -1 = not mapped.  Kept by the
 *              context; read by the GPU during steps and appends.  read only
 *   seg_entries power of two in [1, 2^20]; n_segments >= 1; pool_rows in
 *              [1, 2^31).
 * Only missed entries are looked up (one top-level read in device memory and
 * one 4-byte read of host memory each, before any state changes): a selected
 * entry that misses and has no valid row (no segment, -1, or a row outside
 * the pool) is a range error of its unit (AVSG_ERR_RANGE, the unit's state
 * untouched); an entry still resident in the buffer hits without a lookup.
 * An append to an entry without a valid row writes nothing and raises
 * AVSG_ERR_RANGE.  top = NULL returns to the flat host KV [units][N][row].
 * Returns AVSG_ERR_INVALID_ARG for bad sizes, AVSG_ERR_NOT_PINNED if segments
 * is not pinned device-mapped host memory.  Not valid with avsg_step_static. */
avsg_status avsg_set_host_directory(avsg_ctx* ctx, const int32_t* top, const int32_t* segments,
                                    int32_t seg_entries, int32_t n_segments, int64_t pool_rows);

/* The capacity planner (host arrays, host only): gives each of `units`
 * units its mandatory slots demand[u] (the size of its next union, in
 * [1, n_slots]) and shares the rest of a slot budget over all units in
 * proportion to reuse[u] + 1 (reuse: the unit's recent hits, >= 0), rounded
 * down: cap[u] = min(n_slots, demand[u] + floor(spare * (reuse[u] + 1) /
 * sum(reuse + 1))), spare = budget - sum(demand).  The pages give no
 * formula; this is the plain reading of "mandatory plus buffer pages, with
 * throughput per request weighed against contention".  Returns
 * AVSG_ERR_CAPACITY if the mandatory slots exceed the budget (admit fewer
 * requests), AVSG_ERR_INVALID_ARG for null pointers or values out of range. */
avsg_status avsg_plan_capacity(int32_t units, const int32_t* demand, const int32_t* reuse,
                               int64_t budget, int32_t n_slots, int32_t* cap);

/* Offload of the newly decoded token (Spin summary, section 2A: Offload,
 * placing KV data into memory, is a system-managed operation over a
 * page-based KV substrate; section 2B: physical pages per attention head).
 * For every request b and KV head g, writes the token's key and value (latent
 * layout: its latent vector) at token position pos[b] of unit
 * u = b * n_kv_heads + g: entry e = pos[b] / tokens_per_entry, token row
 * r = pos[b] % tokens_per_entry.  Split layout: the key goes to elements
 * [r * head_dim_qk, +head_dim_qk) of the entry's row and the value to
 * [tokens_per_entry * head_dim_qk + r * head_dim_v, +head_dim_v); latent
 * layout: the whole row.  The bytes go to host_kv and, if entry e is resident
 * (a slot s with slot_table[s] == e), to buf_kv at slot s as well, so the
 * buffer keeps exact copies of host rows.  Slot table, lifetimes and the step
 * counter do not change (an append is not a selection).
 *   new_kv     device, bf16 [batch][n_kv_heads][tok_elems], tok_elems =
 *              head_dim_qk + head_dim_v (split: K then V) or head_dim_qk
 *              (latent).                                            read only
 *   pos        device, int32 [batch]: token position in
 *              [0, n_entries * tokens_per_entry).                   read only
 *   host_kv    host, pinned, bf16 [units][N][row] (as in avsg_step). written
 *   buf_kv     device, bf16 [units][S][row].                        in/out
 *   slot_table device, int32 [units][S].                            read only
 * new_kv, host_kv and buf_kv must be 16-byte aligned.  A request whose pos is
 * out of range writes nothing and raises AVSG_ERR_RANGE; a unit where more
 * than 32 slots hold the entry (an invalid state) writes nothing and raises
 * AVSG_ERR_STATE (both reported by avsg_last_error).  Returns
 * AVSG_ERR_INVALID_ARG, AVSG_ERR_NOT_PINNED or AVSG_ERR_HIP as avsg_step.
 * Stream-ordered with the steps; never waits for the GPU.  The host sees the
 * written bytes once the stream has been synchronised. */
avsg_status avsg_append(avsg_ctx* ctx, const uint16_t* new_kv, const int32_t* pos,
                        uint16_t* host_kv, uint16_t* buf_kv, const int32_t* slot_table);

/* Offload with insertion (Spin summary, section 2A: Offload places KV data
 * into memory; the rule for placing the entry in the buffer is this
 * library's, the step's own eviction order without ageing).  Does what
 * avsg_append does and also makes the token's entry resident, before the
 * coming step t (avsg_get_step), in every unit of the request:
 *   - the unit's slots in use are [0, cap) (avsg_set_capacity; all S by
 *     default); slots past it are emptied, as the coming step would do;
 *   - a slot in use holding the entry is written through and gets the fresh
 *     keep-state: lifetime L, or (bucketed LRU) stamp t - 1, which is bucket
 *     0 at step t;
 *   - otherwise the first slot in the order (empty first, then the lowest
 *     lifetime or the oldest bucket at step t, then the lowest index) takes
 *     the entry: slot_table and the keep-state as above, and buf_kv the
 *     entry's whole host row with the token written.
 * No other slot changes; the step counter does not advance.
 *   slot_table device, int32 [units][S].                            in/out
 *   lifetimes  device, int32 [units][S].                            in/out
 *   the rest   as avsg_append.
 * Per unit, a bad position, a capacity outside [1, S], an entry without a
 * host row or, under bucketed LRU, a call before the first step (t = 0: no
 * stamp t - 1 exists) is AVSG_ERR_RANGE, and slots in use that are not a
 * valid state (an id outside [-1, N), a lifetime outside [0, L] or stamp
 * outside [0, t) on an occupied slot, the entry in two slots) are
 * AVSG_ERR_STATE: that unit writes nothing (avsg_last_error reports it).
 * Returns AVSG_ERR_INVALID_ARG for a null lifetimes, else as avsg_append. */
avsg_status avsg_append_insert(avsg_ctx* ctx, const uint16_t* new_kv, const int32_t* pos,
                               uint16_t* host_kv, uint16_t* buf_kv, int32_t* slot_table,
                               int32_t* lifetimes);

/* Syncs the stream and returns the highest-precedence data error raised by
 * the steps and appends since the last call (RANGE, then UNSORTED, CAPACITY, STATE), or
 * AVSG_OK; then clears it. */
avsg_status avsg_last_error(avsg_ctx* ctx);

/* Full check of a buffer state (syncs): every id in [-1, N), no id held by
 * two slots, lifetimes in [0, L] (or stamps in [0, t)) for occupied slots.
 * Returns AVSG_OK or AVSG_ERR_STATE. */
avsg_status avsg_validate_state(avsg_ctx* ctx, const int32_t* slot_table, const int32_t* lifetimes);

/* No hash index persists between steps: every step derives the id -> slot
 * map of each unit afresh (in LDS) from the selection and slot_table, so a
 * buffer state restored from a checkpoint needs no index rebuild before it
 * is used.  This call derives the map once from slot_table alone and checks
 * that it is one: every id in [-1, N) and no id in two slots (syncs).
 * Returns AVSG_OK or AVSG_ERR_STATE. */
avsg_status avsg_rebuild_index(avsg_ctx* ctx, const int32_t* slot_table);

/* Step counter (decode step of the next avsg_step), for checkpoint/resume.
 * The counter lives in the workspace and every step advances it on the GPU,
 * so steps captured in a HIP graph and replayed keep counting.
 * avsg_get_step syncs the stream and returns it (-1 on error), so it cannot
 * be called while the stream is being captured; avsg_set_step sets it,
 * stream-ordered (capturable), t in [0, 2^31). */
int64_t avsg_get_step(const avsg_ctx* ctx);
avsg_status avsg_set_step(avsg_ctx* ctx, int64_t t);

/* Pinned host memory the GPU can read directly.  flags: 0 = default (non-
 * coherent, cacheable by the GPU), AVSG_HOST_COHERENT = fine-grained. */
#define AVSG_HOST_COHERENT 1u
avsg_status avsg_host_alloc(size_t bytes, unsigned flags, void** host_ptr);
avsg_status avsg_host_free(void* host_ptr);

/* Static string naming a status. */
const char* avsg_status_string(avsg_status s);

/* How missed rows reach the buffer.
 *  AVSG_TRANSFER_FUSED (default): the attention workgroup that consumes a
 *    missed row reads it from pinned host memory and stores it into its slot,
 *    so host transfers overlap the HBM reads of the hits; the rows are spread
 *    over all workgroups in selection order.  In the K/V split layout each
 *    workgroup either copies its missed rows with the tiles that hold them
 *    (when all workgroups are resident at once) or, when the grid runs in
 *    several rounds, has a second wave that gathers all of them into their
 *    slots while the first streams the tiles before the first missed row.
 *  AVSG_TRANSFER_BALANCED: a separate kernel copies the global list of missed
 *    rows, split into equal shares over all workgroups, before attention.
 *  AVSG_TRANSFER_PER_UNIT: like BALANCED, but each unit's rows are copied by
 *    one workgroup (request-level assignment; kept for comparison).
 *  AVSG_TRANSFER_FUSED_GATHER_FIRST: FUSED with the two-wave gather-first
 *    form in the split layout whatever the grid size (the latent layout: as
 *    FUSED).
 * Results are identical in every mode. */
typedef enum avsg_transfer_mode {
  AVSG_TRANSFER_FUSED = 0,
  AVSG_TRANSFER_BALANCED = 1,
  AVSG_TRANSFER_PER_UNIT = 2,
  AVSG_TRANSFER_FUSED_GATHER_FIRST = 3
} avsg_transfer_mode;
avsg_status avsg_set_transfer_mode(avsg_ctx* ctx, int32_t mode);

/* How the selection is matched against the resident ids.
 *  AVSG_MATCH_HASH (default): vectorised hash matching (AVSG abstract): the
 *    selection is entered into an LDS table keyed by id and every slot
 *    looks its resident id up, 64 lanes at a time.  When the context is
 *    small enough (n_entries / 16 words take no more LDS than the hash
 *    table), the table is direct-addressed: one membership bit per id and
 *    one rank base per 32 ids; otherwise it is the open-addressing table.
 *  AVSG_MATCH_MERGE: the scalar dual-pointer baseline the AVSG abstract
 *    compares against: the resident ids are sorted (bitonic sort in LDS) and
 *    one lane walks both sorted lists.  Kept for comparison; needs more LDS
 *    (AVSG_ERR_UNSUPPORTED if the device has too little).
 *  AVSG_MATCH_HASH_TABLE: AVSG_MATCH_HASH always in its open-addressing
 *    form, at load factor <= 1/2 (2|U| cells rounded up to a power of two,
 *    U the union of the step's lists; the default mode's table, used where
 *    direct addressing does not fit, takes 4|U| cells where LDS allows).
 * Results are identical in every mode. */
typedef enum avsg_match_mode {
  AVSG_MATCH_HASH = 0,
  AVSG_MATCH_MERGE = 1,
  AVSG_MATCH_HASH_TABLE = 2
} avsg_match_mode;
avsg_status avsg_set_match_mode(avsg_ctx* ctx, int32_t mode);

/* Number of split-k partitions the attention of one (unit, token) uses. */
int32_t avsg_attn_splits(const avsg_ctx* ctx);

/* Workgroups of the separate gather kernel (transfer modes BALANCED; the
 * list of missed rows is split into that many equal shares): 0 = the
 * library's choice (two per compute unit), else [1, 65535].  Results do not
 * depend on it. */
avsg_status avsg_set_gather_workgroups(avsg_ctx* ctx, int32_t n);

/* Per-kernel timing with HIP events on the context's stream (observability,
 * not part of the method).  avsg_profile_begin creates events for up to
 * max_steps later steps; each of those steps records an event before its
 * first kernel and after each of its four stages (match_reserve, gather,
 * attention, combine of the split partials; a stage a step does not run
 * measures as the gap between its neighbours).  avsg_profile_end syncs the
 * stream, writes the summed milliseconds of each stage to ms[0..3] and the
 * number of profiled steps to *steps, and destroys the events.  Returns
 * AVSG_ERR_INVALID_ARG if profiling is not in the expected state. */
avsg_status avsg_profile_begin(avsg_ctx* ctx, int32_t max_steps);
avsg_status avsg_profile_end(avsg_ctx* ctx, double* ms, int32_t* steps);

/* The two phases of the scalar dual-pointer baseline (AVSG_MATCH_MERGE; the
 * AVSG abstract compares its vectorised matching against scalar
 * dual-pointer matching) in the last profiling session that
 * avsg_profile_end closed: *sort_ms is the summed time of ordering the
 * resident ids (loading them and sorting (id, slot) pairs by id), *walk_ms
 * that of the one-lane walk over the sorted union and the sorted residents,
 * each the mean over units per profiled step (units run concurrently), from
 * the GPU's constant 100 MHz clock.  Both are 0 when no profiled step ran in
 * that mode.  The rest of the match kernel's time (validation, policy,
 * victims, reservation) is common to both modes.  Returns
 * AVSG_ERR_INVALID_ARG on a null argument. */
avsg_status avsg_profile_match_phases(const avsg_ctx* ctx, double* sort_ms, double* walk_ms);

#ifdef __cplusplus
}
#endif

#endif /* AVSG_H */
