// Internal declarations shared by the libavsg translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/avsg.h"

namespace avsg {

constexpr int kMRThreads = 1024;      // match_reserve: one workgroup per unit
constexpr int kMRWaves = kMRThreads / 64;
constexpr int kMaxSlotsPerLane = 16;  // => n_slots <= 16384
constexpr int kMissFlag = 1 << 30;    // marks a union entry that was a miss
constexpr int kAttnThreads = 256;
constexpr int kGatherThreads = 256;

// Layout of the caller's workspace (byte offsets, each 256-aligned).
struct WsLayout {
  size_t unit_status, miss_count, misses, fetch, host_row, err_word, step, phase_clk, partials,
      total;
  int32_t ucap;       // union capacity per unit = min(T*k, S)
  int32_t table_cap;  // hash table cells, power of two >= 2*ucap
  int32_t nsplit;     // attention splits per (unit, token)
  int32_t split_rows; // token rows per split
};

struct Derived {
  int32_t units, G, row_elems, nbins, log_table_cap, ubits;
  size_t mr_lds;        // dynamic LDS bytes of match_reserve
  size_t mr_lds_merge;  // the same with the merge baseline's sort buffers
  int32_t merge_pow2;
  // hash table at load factor <= 1/2 (2|U| cells, rounded up to a power of
  // two): the table-only matching mode and the merge baseline
  int32_t table_cap_half, log_table_cap_half;
  int32_t direct_words;  // membership words of the direct-address match (0: hash table)
};

bool layout_for(const avsg_config& c, WsLayout* ws, Derived* d);

// Floats of one split partial of a (unit, token): o[G][D], then m[G], l[G],
// padded to a multiple of 4 so that every partial starts 16-byte aligned.
inline __host__ __device__ size_t partial_stride(int G, int D) {
  return (size_t)G * D + (size_t)((2 * G + 3) & ~3);
}

// Two-level directory of the host KV pool: entry e of unit u is pool row
// segments[top[u][e >> seg_log2]][e & (2^seg_log2 - 1)] (-1: not mapped).
struct HostDir {
  const int32_t* top;       // device [units][n_seg]: segment index, -1 = none (null: flat host KV)
  const int32_t* segments;  // device-visible pinned host [n_segments][2^seg_log2]: pool row or -1
  int32_t seg_log2, n_seg, n_segments;
  int64_t pool_rows;
};

// Bytes of one split partial of the latent layout: o[G][D] normalized by the
// split's sum, as fp16, then m[G] and l[G] as fp32, padded to 16 bytes.
inline __host__ __device__ size_t latent_partial_bytes(int G, int D) {
  return ((size_t)G * D * 2 + (size_t)8 * G + 15) & ~(size_t)15;
}

struct MatchReserveParams {
  const int32_t* sel;     // [units][T][k]
  const int32_t* sel_len; // [units][T] entries in use of each token's list, or null: k
  const int32_t* cap;     // [units] slots in use of each unit's buffer, or null: S
  const int32_t* ctx_len; // [batch] context length in tokens, or null: every entry holds tokens
  int32_t* slot_table;    // [units][S]
  int32_t* lifetimes;     // [units][S]
  uint8_t* hit_flag;      // [units][T][k]
  int32_t* sel_slot;      // [units][T][k]
  int32_t* n_hit;
  int32_t* n_miss;
  int32_t* n_evict;
  int32_t* user_status;   // may be null
  int32_t* unit_status;   // workspace [units]
  int32_t* miss_count;    // workspace [units]
  int2* misses;           // workspace [units][ucap]: (slot, id) in miss order
  uint8_t* fetch;         // workspace [units][T][k]: row to transfer with this token
  uint32_t* err_word;
  // the decode step: the context's counter in the workspace; null: the value t
  const int64_t* step;
  int64_t t;
  int32_t S, N, T, k, ucap, table_cap, log_table_cap, ubits, policy, L, B, nbins;
  int32_t Hkv, tpe;       // KV heads per request, tokens per entry (context lengths)
  int32_t W;              // steps per LRU bucket (>= 1)
  int32_t match_mode;     // avsg_match_mode
  int32_t merge_pow2;     // power of two >= S (sort size of the merge baseline)
  int32_t direct_words;   // > 0: match through N-bit membership words and rank bases
                          // (this many words each, multiple of 4) instead of the hash table
  // host KV through a two-level directory (null dir_top: flat [units][N][row])
  HostDir dir;
  int32_t* host_row;      // workspace [units][T][k]: pool row of each fetched entry (directory)
  // merge baseline under profiling: summed 100 MHz clocks of its sort and
  // of its walk over all units, and the units counted (null: not recorded)
  unsigned long long* phase_clk;
};

struct GatherParams {
  const int2* misses;     // (slot, id), or (slot, pool row) with a host directory
  const int32_t* miss_count;
  const uint4* host_kv;   // device-visible address of the pinned host rows
  uint4* buf_kv;
  int64_t N, S;
  int32_t units, ucap, row16;
  int32_t per_unit;       // 1: workgroup u copies unit u's rows (request-level)
  int32_t pooled;         // 1: misses carry pool rows of one shared host array
};

struct AttnParams {
  const int32_t* sel_slot;    // [units][T][k]
  const int32_t* sel_len;     // [units][T] entries in use of each list, or null: k
  const int32_t* sel;         // [units][T][k] selected ids
  const int32_t* ctx_len;     // [batch] context length in tokens, or null: whole entries
  int64_t* step;              // the context's step counter: advanced once by the step's first
                              // launch (token 0, workgroup 0); null: not counted here
  const uint8_t* fetch;       // [units][T][k] or null: rows to read from host and store
  const int32_t* host_row;    // [units][T][k] pool row of each fetched entry, or null: flat
                              // host KV, row u * N + sel
  const uint16_t* host_kv;    // device-visible address of the pinned host rows
  int64_t N;
  const int32_t* unit_status; // [units]
  const uint16_t* q;          // [B][T][Hq][dqk]
  uint16_t* buf_kv;           // [units][S][row]
  float* out;                 // [B][T][Hq][dv]
  float* partials;            // [units*T][nsplit][partial_stride(G, dv)] floats, or (latent
                              // layout) [units*T][nsplit][latent_partial_bytes(G, dv)] bytes
  int64_t S;
  int32_t units, Hkv, Hq, T, k, tpe, row_elems, nsplit, split_rows;
  int32_t token;              // query token of this launch
  int32_t gather_first;       // split layout: fetch a split's missed entries before its tiles
                              // (1 forces it; the launcher also sets it for multi-round grids)
  float scale_log2e;
};

struct AppendParams {
  const uint16_t* new_kv;     // [units][tok_elems]: the token's K then V, or its latent vector
  const int32_t* pos;         // [batch]: token position of each request
  uint16_t* host_kv;          // device-visible address of the pinned host rows [units][N][row]
  uint16_t* buf_kv;           // [units][S][row]
  int32_t* slot_table;        // [units][S] (written only when inserting)
  int32_t* lifetimes;         // [units][S] (inserting only)
  const int32_t* cap;         // [units] slots in use, or null: all S (inserting only)
  uint32_t* err_word;
  HostDir dir;                // null dir.top: flat host KV
  const int64_t* step;        // the coming step, in the workspace (inserting only)
  int32_t Hkv, N, S, tpe, row_elems, tok_elems, dqk, dv, latent;
  int32_t insert, lru, L, B, W;  // insert: make the entry resident as well; W: steps per
                                 // LRU bucket
};

hipError_t launch_match_reserve(const MatchReserveParams& p, int units, size_t lds, hipStream_t s);
hipError_t launch_gather(const GatherParams& p, int grid, hipStream_t s);
hipError_t launch_attn_split(const AttnParams& p, int G, hipStream_t s);
hipError_t launch_attn_latent(const AttnParams& p, int dqk, int dv, hipStream_t s);
hipError_t launch_attn_combine(const AttnParams& p, int G, int D, bool latent, hipStream_t s);
hipError_t attn_latent_set_lds();
hipError_t launch_append(const AppendParams& p, int units, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int32_t v, size_t n, hipStream_t s);
hipError_t launch_validate(const int32_t* slot_table, const int32_t* lifetimes, int units, int S,
                           int N, int policy, int L, int64_t t, uint32_t* err, hipStream_t s);
hipError_t launch_set_step(int64_t* step, int64_t t, hipStream_t s);
hipError_t match_reserve_set_lds(size_t lds);

}  // namespace avsg
