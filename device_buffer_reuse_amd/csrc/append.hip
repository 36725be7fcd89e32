// Offload of a newly decoded token.  The Spin summary (gist.science
// 2604.26837, section 2A) lists Offload, placing KV data into memory, among
// the system-managed operations over a page-based KV substrate, and keeps the
// physical pages per attention head (section 2B).  Here the token's K and V
// (or its latent vector) are written into its row of the head-wise host
// store, and into the slot holding that entry if the entry is resident, so
// the device buffer keeps exact copies of host rows and later hits stay
// exact.  Slots, lifetimes and stamps are not touched.
//
// With insertion the entry is also made resident before the coming step, in
// each unit's slots in use: a slot holding it is written through and gets the
// fresh keep-state (lifetime L, or the stamp of the step before); otherwise
// the first slot of the step's eviction order (empty, then lowest lifetime or
// oldest bucket, then lowest index) takes it with the whole host row.  No
// other slot ages.  The victim is a block-wide minimum of packed keys.
//
// One workgroup per unit: the slot table is scanned for the entry (S int32
// reads, coalesced), then one lane per 16-byte piece of the token copies it
// to host memory and to each slot found.  With a two-level host directory
// (Spin summary, section 2C) the host row is the entry's pool row.
#include "avsg_internal.h"

namespace avsg {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kAppendThreads = 256;
constexpr int kMaxHolders = 32;  // slots recorded per entry (1 in a valid state)

// Eviction key of slot s for an insertion before step t, smaller = evicted
// first: (occupied, lifetime or minus bucket, slot index) packed into 64 bits
// (the key is biased by 256: lifetimes are at most 126, buckets at most 127).
__device__ inline uint64_t insert_key(int32_t id, int32_t lv, int s, int64_t t,
                                      const AppendParams& p) {
  if (id < 0) return (uint64_t)s;
  int64_t key = lv;
  if (p.lru) {
    int64_t bucket = (t - (int64_t)lv - 1) / p.W;
    bucket = bucket < 0 ? 0 : (bucket > p.B - 1 ? p.B - 1 : bucket);
    key = -bucket;
  }
  return (1ull << 48) | ((uint64_t)(key + 256) << 32) | (uint64_t)s;
}

__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendParams p) {
  __shared__ int32_t sHolder[kMaxHolders];
  __shared__ int32_t sCount;
  __shared__ int32_t sBad;
  __shared__ int32_t sCap;
  __shared__ int64_t sHostRow;
  __shared__ unsigned long long sBest;
  const int u = blockIdx.x;
  const int b = u / p.Hkv;
  const int tid = threadIdx.x;
  const int64_t pos = p.pos[b];
  if (pos < 0 || pos >= (int64_t)p.N * p.tpe) {
    if (tid == 0 && u == b * p.Hkv) atomicOr(p.err_word, 1u << (AVSG_ERR_RANGE - 16));
    return;
  }
  const int e = (int)(pos / p.tpe);
  const int r = (int)(pos - (int64_t)e * p.tpe);
  // the coming step (inserting): the context's counter in the workspace
  const int64_t t = p.insert ? p.step[0] : 0;
  if (tid == 0) {
    sCount = 0;
    sBad = 0;
    sBest = ~0ull;
    // the entry's host row: u * N + e, or its pool row through the two-level
    // directory (-1: not mapped, a range error of the unit)
    int64_t hrow = (int64_t)u * p.N + e;
    if (p.dir.top) {
      const int32_t seg = p.dir.top[(size_t)u * p.dir.n_seg + (e >> p.dir.seg_log2)];
      int32_t row = -1;
      if (seg >= 0 && seg < p.dir.n_segments)
        row = p.dir.segments[((size_t)seg << p.dir.seg_log2) + (e & ((1 << p.dir.seg_log2) - 1))];
      hrow = (row >= 0 && (int64_t)row < p.dir.pool_rows) ? row : -1;
    }
    // slots in use (inserting): [0, cap); a capacity outside [1, S] is a
    // range error of the unit
    int cap = p.S;
    if (p.insert && p.cap) {
      cap = p.cap[u];
      if (cap < 1 || cap > p.S) hrow = -1;
    }
    // a bucketed-LRU stamp of the step before the coming one needs a step
    // before it: an insertion before the first step is a range error
    if (p.insert && p.lru && t < 1) hrow = -1;
    sCap = cap;
    sHostRow = hrow;
  }
  __syncthreads();
  const int64_t hrow = sHostRow;
  if (hrow < 0) {
    if (tid == 0) atomicOr(p.err_word, 1u << (AVSG_ERR_RANGE - 16));
    return;
  }
  const int cap = sCap;
  int32_t* st = p.slot_table + (size_t)u * p.S;
  int32_t* lf = p.insert ? p.lifetimes + (size_t)u * p.S : nullptr;
  uint64_t best = ~0ull;
  int bad = 0;
  for (int s = tid; s < p.S; s += kAppendThreads) {
    const int32_t id = st[s];
    if (id == e && (!p.insert || s < cap)) {
      const int at = atomicAdd(&sCount, 1);
      if (at < kMaxHolders) sHolder[at] = s;
    }
    if (p.insert && s < cap) {
      // the slots in use must be a valid state: ids in [-1, N), lifetimes in
      // [0, L] or stamps in [0, t) for occupied slots
      if (id < -1 || id >= p.N) bad = 1;
      int32_t lv = 0;
      if (id >= 0) {
        lv = lf[s];
        if (lv < 0 || (p.lru ? (int64_t)lv >= t : lv > p.L)) bad = 1;
      }
      const uint64_t key = insert_key(id, lv, s, t, p);
      best = key < best ? key : best;
    }
  }
  if (p.insert) {
    if (bad) atomicOr(&sBad, 1);
    atomicMin(&sBest, (unsigned long long)best);
  }
  __syncthreads();
  const int holders = sCount;
  if (holders > (p.insert ? 1 : kMaxHolders) || sBad) {
    // more slots than a valid state allows hold the entry, or (inserting)
    // the slots in use are not a valid state: nothing is written
    if (tid == 0) atomicOr(p.err_word, 1u << (AVSG_ERR_STATE - 16));
    return;
  }
  // piece i of the token: key pieces first, then value pieces (split layout);
  // its offset in the row, in elements
  const int kp = p.dqk >> 3, vp = p.latent ? 0 : p.dv >> 3;
  const int64_t kbase = p.latent ? 0 : (int64_t)r * p.dqk;
  const int64_t vbase = (int64_t)p.tpe * p.dqk + (int64_t)r * p.dv;
  const uint16_t* tok = p.new_kv + (size_t)u * p.tok_elems;
  uint16_t* hrow_p = p.host_kv + (size_t)hrow * p.row_elems;
  if (p.insert) {
    // slots past the capacity are emptied (the coming step would empty them)
    for (int s = cap + tid; s < p.S; s += kAppendThreads) {
      st[s] = -1;
      lf[s] = p.lru ? -1 : 0;
    }
  }
  if (p.insert && holders == 0) {
    // the entry is not resident: the first slot of the eviction order takes
    // it and receives the whole host row, the token's pieces from new_kv
    const int v = (int)(sBest & 0xffffffffu);
    uint16_t* dst = p.buf_kv + ((size_t)u * p.S + v) * p.row_elems;
    const int pieces = p.row_elems >> 3;
    for (int j = tid; j < pieces; j += kAppendThreads) {
      const int64_t off = 8 * (int64_t)j;
      u32x4 x;
      if (off >= kbase && off < kbase + p.dqk) {
        x = *reinterpret_cast<const u32x4*>(tok + (off - kbase));
        *reinterpret_cast<u32x4*>(hrow_p + off) = x;
      } else if (vp && off >= vbase && off < vbase + p.dv) {
        x = *reinterpret_cast<const u32x4*>(tok + p.dqk + (off - vbase));
        *reinterpret_cast<u32x4*>(hrow_p + off) = x;
      } else {
        x = *reinterpret_cast<const u32x4*>(hrow_p + off);
      }
      *reinterpret_cast<u32x4*>(dst + off) = x;
    }
    if (tid == 0) {
      st[v] = e;
      lf[v] = p.lru ? (int32_t)(t - 1) : p.L;
    }
    return;
  }
  if (p.insert && tid == 0) lf[sHolder[0]] = p.lru ? (int32_t)(t - 1) : p.L;
  if (tid >= kp + vp) return;
  const int64_t off = tid < kp ? kbase + 8 * tid : vbase + 8 * (tid - kp);
  const u32x4 v = *reinterpret_cast<const u32x4*>(tok + 8 * tid);
  *reinterpret_cast<u32x4*>(hrow_p + off) = v;
  for (int h = 0; h < holders; ++h)
    *reinterpret_cast<u32x4*>(p.buf_kv + ((size_t)u * p.S + sHolder[h]) * p.row_elems + off) = v;
}

}  // namespace

hipError_t launch_append(const AppendParams& p, int units, hipStream_t s) {
  if (p.dqk % 8 != 0 || p.dv % 8 != 0 || (p.dqk >> 3) + (p.latent ? 0 : p.dv >> 3) > kAppendThreads)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)units), dim3(kAppendThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace avsg
