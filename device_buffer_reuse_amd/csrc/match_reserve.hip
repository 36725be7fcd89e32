// K1: match the selected entries of a unit against its slot buffer, update
// lifetimes / recency stamps, choose victims without a sort, reserve slots for
// the misses and list the misses for the gather.  One workgroup (16 waves)
// per (request, KV head) unit.
//
// Method (AVSG abstract, arxivdaily 2609.37538): a vectorised hash match finds
// reusable buffer slots and reserves slots for entries needing a transfer;
// lifetime-based management keeps frequently selected entries resident; one
// reservation is shared by all query tokens of an MTP iteration.  Bucketed LRU
// (Spin summary, gist.science 2604.26837, section 2B) groups slots by recency
// bucket so that eviction needs no global sort and runs in parallel.
//
// gfx950 mapping:
//  * The union U of the iteration's sorted selections is built in LDS (for
//    two tokens by a rank formula: each element's position in U is found by
//    binary search in the other list minus the duplicates before it).
//  * U is hashed into an LDS open-addressing table of 4-cell buckets
//    (multiplicative hash; load factor <= 1/4 where LDS allows, else <= 1/2,
//    and <= 1/2 in the table-only matching mode).  A cell packs (id << ubits
//    | union index) in 32 bits.  Insertion takes a position in the home bucket
//    from a per-bucket attempt counter (one LDS atomic; a full bucket sends
//    the entry on along its double-hashing sequence), so a counter of at
//    most 4 proves that an id absent from its home bucket is absent from the
//    table.  Every slot
//    of the buffer then probes its resident id, one slot per lane, 64 lanes
//    at a time: one 16-byte read fetches the home bucket, a second its
//    counter, and only the rare probe of an overflowed bucket reads on.
//    Hashing U rather than the slots keeps the table at 2-4|U| cells and turns
//    "is this slot a candidate" into the same probe.
//  * Victim selection is a stable counting selection: each candidate slot gets
//    a bin (empty first, then lifetime 0..L, or LRU bucket oldest-first).  A
//    histogram of the bins gives the threshold bin b* that holds the m-th
//    candidate: the counts of bins 0..7 per wave form a 128-word (bin, wave)
//    table that two chained wave scans turn into every (bin, wave) start, and
//    all bins are counted only if those eight hold fewer than m candidates.  Only
//    candidates in bins <= b* are ranked, inside their bin in slot order via
//    ballot/mbcnt per wave plus the (bin, wave) starts; the m first
//    candidates in (bin, slot) order are the victims.  No comparison sort, no
//    order-dependent atomics: the result is deterministic.
//  * The r-th miss in ascending id order takes the r-th victim, its row is
//    listed as (slot, id) for the gather kernel.
#include "avsg_internal.h"

namespace avsg {
namespace {

constexpr int kInvalid = -2;  // slot beyond S in this lane's range
constexpr int kDupFlag = 1 << 30;  // token-1 entry also selected by token 0

__device__ __forceinline__ uint32_t hash_id(int32_t id, int log_cap) {
  return ((uint32_t)id * 0x9E3779B1u) >> (32 - log_cap);
}
// Bucket step of an id (odd, so it visits every bucket of the power-of-two
// table): double hashing keeps overflow chains short, where stepping to the
// next bucket would let full buckets cluster.
__device__ __forceinline__ uint32_t hash_step(int32_t id, int log_cap) {
  return ((((uint32_t)id * 0x85EBCA77u) >> (34 - log_cap)) << 1) | 1u;
}

__device__ __forceinline__ int mbcnt64(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, BOUND_ZERO);
}

// Inclusive scan over the 64 lanes of a wave, on DPP only: shifts by 1, 2,
// 4, 8 inside each 16-lane row, then row 0's total into rows 1 and 3
// (row_bcast:15) and rows 0-1's total into rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_i<0x111, 0xF, true>(v);   // row_shr:1
  v += dpp_i<0x112, 0xF, true>(v);   // row_shr:2
  v += dpp_i<0x114, 0xF, true>(v);   // row_shr:4
  v += dpp_i<0x118, 0xF, true>(v);   // row_shr:8
  v += dpp_i<0x142, 0xA, false>(v);  // row_bcast:15 into rows 1, 3
  v += dpp_i<0x143, 0xC, false>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

__device__ __forceinline__ int wave_total(int v) {
  return __builtin_amdgcn_readlane(wave_incl_scan(v), 63);
}

// number of elements of the sorted array a[0..n) that are < x
__device__ __forceinline__ int lower_bound_lds(const int32_t* a, int n, int32_t x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

constexpr int32_t kEmpty = -1;  // a filled cell has its top bit clear

// Looks for x in one fetched bucket: returns the union index, -1 if the
// bucket has an empty cell (x is absent), or -2 if the search must go on.
__device__ __forceinline__ int bucket_check(const int4 c, int ubits, int32_t x) {
  const int umask = (1 << ubits) - 1;
  int found = -1;
  found = ((c.x >> ubits) == x) ? (c.x & umask) : found;
  found = ((c.y >> ubits) == x) ? (c.y & umask) : found;
  found = ((c.z >> ubits) == x) ? (c.z & umask) : found;
  found = ((c.w >> ubits) == x) ? (c.w & umask) : found;
  const int lo = min(min(c.x, c.y), min(c.z, c.w));  // -1 iff a cell is empty
  return (found >= 0 || lo < 0) ? found : -2;
}

// Inserts (x, i).  Each bucket of 4 cells has a counter of insertion
// attempts: the attempt that draws position 0..3 fills that cell (so a
// bucket's cells fill in order), later attempts move on along x's bucket
// sequence (home, home + step, ...).
// A counter <= 4 therefore means that no entry whose home is this bucket
// lives anywhere else.
// Union index of x in a fetched bucket, or -1.  A filled cell is (id <<
// ubits | index) with its top bit clear, so it holds x iff (cell ^ (x <<
// ubits)) < 2^ubits; an empty cell (-1) never passes for an id in range.
__device__ __forceinline__ int bucket_find(const int4 c, uint32_t xs, uint32_t lim, int umask) {
  const bool m0 = (uint32_t)(c.x ^ xs) < lim, m1 = (uint32_t)(c.y ^ xs) < lim;
  const bool m2 = (uint32_t)(c.z ^ xs) < lim, m3 = (uint32_t)(c.w ^ xs) < lim;
  const int v = m0 ? c.x : (m1 ? c.y : (m2 ? c.z : c.w));
  return (m0 | m1 | m2 | m3) ? (v & umask) : -1;
}

// Inserts cell v, trying buckets hb, hb + step, ... (bmask = buckets - 1).
__device__ __forceinline__ void hash_insert_at(int32_t* sHash, int32_t* sBcnt, uint32_t bmask,
                                               uint32_t hb, uint32_t step, int32_t v) {
  while (true) {
    const int pos = atomicAdd(&sBcnt[hb], 1);
    if (pos < 4) {
      sHash[hb * 4 + pos] = v;
      return;
    }
    hb = (hb + step) & bmask;
  }
}

__device__ __forceinline__ void hash_insert(int32_t* sHash, int32_t* sBcnt, int log_cap, int ubits,
                                            int32_t x, int32_t i) {
  const uint32_t bmask = ((1u << log_cap) >> 2) - 1;
  hash_insert_at(sHash, sBcnt, bmask, hash_id(x, log_cap) >> 2, hash_step(x, log_cap),
                 (x << ubits) | i);
}

enum { kFlagRange = 1, kFlagUnsorted = 2, kFlagCapacity = 4, kFlagState = 8 };

__device__ __forceinline__ int flags_to_status(int f) {
  if (f & kFlagRange) return AVSG_ERR_RANGE;
  if (f & kFlagUnsorted) return AVSG_ERR_UNSORTED;
  if (f & kFlagCapacity) return AVSG_ERR_CAPACITY;
  return AVSG_ERR_STATE;
}

// Exclusive scan of a 0/1 flag over the workgroup in thread order.
__device__ __forceinline__ int block_excl_scan_bit(bool v, int* sWs, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t m = __ballot(v);
  if (lane == 0) sWs[w] = __popcll(m);
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kMRWaves; ++i) {
    int x = sWs[i];
    pre += (i < w) ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return pre + mbcnt64(m);
}

// entry i of a unit's [T][k] selection array is in use: before end0 in the
// first list, or before end1 (= k + length) in the second
__device__ __forceinline__ bool in_use_at(int i, int k, int end0, int end1) {
  return i < k ? i < end0 : i < end1;
}

template <int MAXP>
__global__ __launch_bounds__(kMRThreads) void match_reserve_kernel(MatchReserveParams p) {
  extern __shared__ int32_t lds[];
  const int u = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int S = p.S, N = p.N, T = p.T, k = p.k, ucap = p.ucap, C = p.table_cap;
  // the decode step: the context's counter in the workspace (the step's
  // first attention launch advances it once this kernel has finished), or
  // the caller's value
  const int64_t step_t = p.step ? p.step[0] : p.t;
  // tks: stride of a unit's lists.  With a length array token j uses the
  // first sel_len[u][j] entries of its list (ka for token 0, kb for token 1;
  // a length outside [1, k] is a range error); tk: one token, the entries
  // in use; two tokens, the whole [2][k] array, of which the entries that
  // in_use_at() accepts are in use
  const int tks = T * k;
  const int len_in = p.sel_len ? p.sel_len[u * T] : k;
  const int len1_in = (T > 1 && p.sel_len) ? p.sel_len[u * T + 1] : k;
  const bool len_bad = len_in < 1 || len_in > k || len1_in < 1 || len1_in > k;
  const int ka = len_bad ? 1 : len_in, kb = len_bad ? 1 : len1_in;
  // slots in use: [0, cap) (the unit's buffer size; slots past it are
  // emptied by this step); a capacity outside [1, S] is a range error
  const int cap_in = p.cap ? p.cap[u] : S;
  const bool cap_bad = cap_in < 1 || cap_in > S;
  // entries of the request's context (entry e holds positions [e tpe,
  // (e + 1) tpe)): selected ids at or past them are out of range like ids
  // past N; a context length outside [1, N tpe] is a range error
  const int64_t ctx_in = p.ctx_len ? p.ctx_len[u / p.Hkv] : 1;
  const bool ctx_bad = ctx_in < 1 || ctx_in > (int64_t)N * p.tpe;
  const int lim = (p.ctx_len && !ctx_bad) ? (int)((ctx_in + p.tpe - 1) / p.tpe) : N;
  const int cap = cap_bad ? S : cap_in;
  const int nbins = p.nbins, tk = T == 1 ? ka : tks;
  // entry i of the [T][k] array is in use: one token, i < tk; two tokens,
  // i < ka in token 0's list or i - k < kb in token 1's
  const int live_end0 = T == 1 ? tk : ka, live_end1 = k + kb;
  const bool lru = p.policy == AVSG_POLICY_BUCKET_LRU;

  int32_t* sHash = lds;                      // [C] packed (id, union index) or -1
  int32_t* sBcnt = sHash + C;                // [C/4] insertion attempts per bucket
  int32_t* sU = sBcnt + (C >> 2);            // [ucap] union, ascending
  int32_t* sUslot = sU + ucap;               // [ucap] slot of each union entry (+ miss flag)
  int32_t* sCnt = sUslot + ucap;             // [16][nbins] per-wave candidates per bin
  int32_t* sOff = sCnt + kMRWaves * nbins;   // [16][nbins] first rank of (wave, bin)
  int32_t* sTot = sOff + kMRWaves * nbins;   // [nbins] -> exclusive bin starts
  int32_t* sMisc = sTot + nbins;             // [192]: 0 flags, 1 evictions, 16.. scan scratch,
                                             // 64.. per-lane sink of masked-off LDS atomics,
                                             // later the (bin, wave) victim-count table
  int32_t* sMiss = sMisc + 192;              // [max(ucap, T*k)]; T=2: first holds both lists
  int32_t* sMap = sMiss + (T > 1 ? tk : ucap);  // T=2: [T*k] union index per (token, entry)
  int32_t* sDup = sMap + (T > 1 ? tk : 0);      // T=2: [k+1] duplicates before each A index
  int32_t* sWs = sMisc + 16;
  int32_t* sSink = sMisc + 64;
  // direct-address form (dw > 0 words, in place of the hash table): bit x of
  // the membership words is set iff id x is in U, and the rank base of a word
  // is the union index of the first id of U in that word, so the union index
  // of a member x is base[x / 32] + (members of its word below x)
  const int dw = p.direct_words;
  uint32_t* sBits = reinterpret_cast<uint32_t*>(sHash);  // [dw] (two tokens: first token 1's ids)
  int32_t* sBase = sHash + dw;                            // [dw]
  uint32_t* sBitsA = sBits + 2 * dw;                      // [dw] two tokens: token 0's ids

  const int32_t* sel = p.sel + (size_t)u * tks;
  int32_t* slot_table = p.slot_table + (size_t)u * S;
  int32_t* lifetimes = p.lifetimes + (size_t)u * S;

  // ---- 0. issue the selection loads, then the loads of this lane's slots;
  //         the slots complete while the selection is validated and hashed
  int32_t* stage = (T > 1) ? sMiss : sU;  // T = 1: the list is U itself
  constexpr int kSelRegs = 4;
  int32_t selr[kSelRegs];
#pragma unroll
  for (int r = 0; r < kSelRegs; ++r) selr[r] = sel[min(tid + r * kMRThreads, tk - 1)];
  const int R = ((S + kMRThreads - 1) / kMRThreads) * 64;  // slots per wave, multiple of 64
  const int s0 = w * R, s1 = min(s0 + R, S);
  // every lane loads all its slots unconditionally (an index clamped into the
  // buffer), so the loads are in flight together; lanes past the wave's range
  // are marked invalid where the values are first used
  int tok[MAXP], lf[MAXP], bin[MAXP], rank[MAXP];
#pragma unroll
  for (int q = 0; q < MAXP; ++q) {
    const int s = min(s0 + q * 64 + lane, S - 1);
    tok[q] = slot_table[s];
    lf[q] = lifetimes[s];
  }
#pragma unroll
  for (int r = 0; r < kSelRegs; ++r) {
    const int i = tid + r * kMRThreads;
    if (i < tk) stage[i] = selr[r];
  }
  for (int i = tid + kSelRegs * kMRThreads; i < tk; i += kMRThreads) stage[i] = sel[i];
  if (tid < 192) sMisc[tid] = 0;
  if (dw > 0) {  // membership words 0 (dw is a multiple of 4); rank bases need no init
    int4* b4 = reinterpret_cast<int4*>(sBits);
    for (int i = tid; i < (dw >> 2); i += kMRThreads) b4[i] = make_int4(0, 0, 0, 0);
    int4* a4 = reinterpret_cast<int4*>(sBitsA);
    if (T > 1)
      for (int i = tid; i < (dw >> 2); i += kMRThreads) a4[i] = make_int4(0, 0, 0, 0);
  } else {  // table cells -1 and bucket counters 0, 16 bytes per store (C is a multiple of 64)
    int4* h4 = reinterpret_cast<int4*>(sHash);
    for (int i = tid; i < (C >> 2); i += kMRThreads) h4[i] = make_int4(-1, -1, -1, -1);
    int4* b4 = reinterpret_cast<int4*>(sBcnt);
    for (int i = tid; i < (C >> 4); i += kMRThreads) b4[i] = make_int4(0, 0, 0, 0);
  }
  for (int i = tid; i < ucap; i += kMRThreads) sUslot[i] = -1;
  __syncthreads();

  // ---- 1. validate each token's list: ids in range, strictly ascending.
  //         With one token the list is U, and valid ids are hashed in the
  //         same pass (the table is never used if a flag is raised).
  const int log_cap = p.log_table_cap, ubits = p.ubits;
  {
    int bad = 0;
    const uint32_t bmask = ((1u << log_cap) >> 2) - 1;
    // entries held in registers: the predecessor reads and the first
    // insertion attempts of all of them are issued together (a lane with
    // nothing to insert adds to its own sink word instead)
    int32_t prv[kSelRegs], pos[kSelRegs];
    uint32_t hb[kSelRegs];
#pragma unroll
    for (int r = 0; r < kSelRegs; ++r) prv[r] = stage[max(min(tid + r * kMRThreads, tk) - 1, 0)];
    if (T == 1 && dw > 0) {
#pragma unroll
      for (int r = 0; r < kSelRegs; ++r) {
        const int i = tid + r * kMRThreads;
        const int32_t x = selr[r];
        if (i < tk && x >= 0 && x < lim) {
          atomicOr(&sBits[x >> 5], 1u << (x & 31));
          if (i == 0 || (prv[r] >> 5) != (x >> 5)) sBase[x >> 5] = i;
        }
      }
    } else if (dw > 0) {  // two tokens: each list's membership bits
#pragma unroll
      for (int r = 0; r < kSelRegs; ++r) {
        const int i = tid + r * kMRThreads;
        const int32_t x = selr[r];
        if (i < tk && in_use_at(i, k, live_end0, live_end1) && x >= 0 && x < lim)
          atomicOr(&(i < k ? sBitsA : sBits)[x >> 5], 1u << (x & 31));
      }
    } else if (T == 1) {
#pragma unroll
      for (int r = 0; r < kSelRegs; ++r) {
        const int i = tid + r * kMRThreads;
        const int32_t x = selr[r];
        hb[r] = hash_id(x, log_cap) >> 2;
        pos[r] = atomicAdd((i < tk && x >= 0 && x < lim) ? &sBcnt[hb[r]] : &sSink[lane], 1);
      }
#pragma unroll
      for (int r = 0; r < kSelRegs; ++r) {
        const int i = tid + r * kMRThreads;
        const int32_t x = selr[r];
        if (i < tk && x >= 0 && x < lim) {
          const int32_t v = (x << ubits) | i;
          if (pos[r] < 4)
            sHash[hb[r] * 4 + pos[r]] = v;
          else
            hash_insert_at(sHash, sBcnt, bmask, (hb[r] + hash_step(x, log_cap)) & bmask,
                           hash_step(x, log_cap), v);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kSelRegs; ++r) {
      const int i = tid + r * kMRThreads;
      const int32_t x = selr[r];
      const bool in_use = i < tk && in_use_at(i, k, live_end0, live_end1), in_range = x >= 0 && x < lim;
      // a token's list starts at 0 and, for the second token, at k (T <= 2)
      bad |= (in_use && !in_range) ? kFlagRange : 0;
      bad |= (in_use && i != 0 && i != k && x <= prv[r]) ? kFlagUnsorted : 0;
    }
    if ((len_bad || cap_bad || ctx_bad) && tid == 0) bad |= kFlagRange;
    // one token: U is the list itself
    if (T == 1 && tk > cap && tid == 0) bad |= kFlagCapacity;
    for (int i = tid + kSelRegs * kMRThreads; i < tk; i += kMRThreads) {
      if (!in_use_at(i, k, live_end0, live_end1)) continue;
      const int32_t x = stage[i];
      const bool in_range = x >= 0 && x < lim;
      if (!in_range) bad |= kFlagRange;
      const int32_t xp = stage[i - 1];
      if (i != k && x <= xp) bad |= kFlagUnsorted;
      if (T == 1 && in_range && dw > 0) {
        atomicOr(&sBits[x >> 5], 1u << (x & 31));
        if ((xp >> 5) != (x >> 5)) sBase[x >> 5] = i;
      } else if (in_range && dw > 0) {
        atomicOr(&(i < k ? sBitsA : sBits)[x >> 5], 1u << (x & 31));
      } else if (T == 1 && in_range) {
        hash_insert(sHash, sBcnt, log_cap, ubits, x, i);
      }
    }
    if (bad) atomicOr(&sMisc[0], bad);
  }
  __syncthreads();

  // ---- 2. union U of the two lists (T = 2): position of each element =
  //         elements below it in both lists minus duplicates below it
  int nu = T == 1 ? tk : k;
  if (T > 1 && sMisc[0] == 0 && dw > 0) {
    // direct addressing: U's membership words are the two lists' words or'ed;
    // a block scan of their popcounts gives each word's rank base, the set
    // bits expand into the sorted U, and each (token, entry) finds its union
    // index from its word (a token-1 entry is a duplicate if token 0's bit
    // is set)
    int run = 0;
    for (int w0 = 0; w0 < dw; w0 += kMRThreads) {
      const int wi = w0 + tid;
      const uint32_t uw = wi < dw ? (sBitsA[wi] | sBits[wi]) : 0u;
      const int cnt = __popc(uw);
      const int inc = wave_incl_scan(cnt);
      if (lane == 63) sWs[w] = inc;
      __syncthreads();
      int pre = 0, tot = 0;
#pragma unroll
      for (int v = 0; v < kMRWaves; ++v) {
        const int x = sWs[v];
        pre += (v < w) ? x : 0;
        tot += x;
      }
      const int base = run + pre + inc - cnt;
      if (wi < dw) {
        sBits[wi] = uw;
        sBase[wi] = base;
      }
      if (base + cnt <= ucap) {  // a larger U is a capacity error (below)
        uint32_t rest = uw;
        for (int r = 0; rest != 0; ++r) {
          sU[base + r] = wi * 32 + __builtin_ctz(rest);
          rest &= rest - 1;
        }
      }
      run += tot;
      __syncthreads();  // sWs is reused; sBits and sBase are complete
    }
    nu = run;
    if (nu > cap) {
      if (tid == 0) sMisc[0] = kFlagCapacity;
    } else {
      for (int i = tid; i < tk; i += kMRThreads) {
        if (!in_use_at(i, k, live_end0, live_end1)) continue;
        const int32_t x = sMiss[i];
        const uint32_t word = sBits[x >> 5], bit = 1u << (x & 31);
        const int pos = sBase[x >> 5] + __popc(word & (bit - 1));
        const bool dup = i >= k && (sBitsA[x >> 5] & bit) != 0;
        sMap[i] = pos | (dup ? kDupFlag : 0);
      }
    }
    __syncthreads();
  } else if (T > 1 && sMisc[0] == 0) {
    // token 0's ka ids and token 1's kb ids, each sorted
    const int32_t* A = sMiss;
    const int32_t* Bl = sMiss + k;
    int run = 0;
    for (int c0 = 0; c0 < ka; c0 += kMRThreads) {
      const int i = c0 + tid;
      bool dup = false;
      if (i < ka) {
        const int lb = lower_bound_lds(Bl, kb, A[i]);
        dup = lb < kb && Bl[lb] == A[i];
      }
      int tot;
      const int pre = block_excl_scan_bit(dup, sWs, &tot);
      if (i < ka) sDup[i] = run + pre;
      run += tot;
    }
    if (tid == 0) sDup[ka] = run;
    __syncthreads();
    nu = ka + kb - sDup[ka];
    if (nu > cap) {
      if (tid == 0) sMisc[0] = kFlagCapacity;
    } else {
      for (int i = tid; i < ka; i += kMRThreads) {
        const int32_t a = A[i];
        const int pos = i + lower_bound_lds(Bl, kb, a) - sDup[i];
        sU[pos] = a;
        sMap[i] = pos;
      }
      for (int j = tid; j < kb; j += kMRThreads) {
        const int32_t b = Bl[j];
        const int la = lower_bound_lds(A, ka, b);
        const int pos = la + j - sDup[la];
        const bool dup = la < ka && A[la] == b;
        sU[pos] = b;  // a duplicate writes the same value at the same position
        sMap[k + j] = pos | (dup ? kDupFlag : 0);
      }
    }
    __syncthreads();
  }

  // ---- 3. hash U into the LDS table (two tokens; one token did it above)
  if (T > 1 && dw == 0) {
    if (sMisc[0] == 0) {
      for (int i = tid; i < nu; i += kMRThreads) hash_insert(sHash, sBcnt, log_cap, ubits, sU[i], i);
    }
    __syncthreads();
  }

  // ---- 4. every slot probes its resident id; state checks
  // slots at or past the capacity that hold something are emptied at the
  // end of the step (bit q); they take no part in it
  const int32_t life_empty = lru ? -1 : 0;
  uint32_t drop = 0;
  if (cap < S) {  // the whole workgroup: only a sized buffer empties slots
#pragma unroll
    for (int q = 0; q < MAXP; ++q) {
      const int s = s0 + q * 64 + lane;
      if (q * 64 < R && s < s1 && s >= cap && (tok[q] != -1 || lf[q] != life_empty))
        drop |= 1u << q;
    }
  }
  const int s_use = min(s1, cap);  // this wave's slots in use end here
#pragma unroll
  for (int q = 0; q < MAXP; ++q) {
    if (!(q * 64 < R && s0 + q * 64 + lane < s_use)) {
      tok[q] = kInvalid;
      lf[q] = 0;
    }
  }
  int hit_i[MAXP];
#pragma unroll
  for (int q = 0; q < MAXP; ++q) hit_i[q] = -1;
  if (sMisc[0] == 0 && p.match_mode == AVSG_MATCH_MERGE) {
    // comparison baseline: sort the resident (id, slot) pairs by id (bitonic,
    // in LDS), then one lane walks the sorted union and the sorted residents
    // with two pointers.  Same results as the hash probe.
    int bad = 0;
#pragma unroll
    for (int q = 0; q < MAXP; ++q) {
      const int32_t x = tok[q];
      bin[q] = kInvalid;
      hit_i[q] = -1;
      if (x == kInvalid) continue;
      bin[q] = 0;
      if (x < -1 || x >= N) {
        bad = 1;
      } else if (x >= 0) {
        const int32_t l = lf[q];
        if (!lru && (l < 0 || l > p.L)) bad = 1;
        if (lru && (l < 0 || (int64_t)l >= step_t)) bad = 1;
      }
    }
    const int P2 = p.merge_pow2;
    // [P2] pairs after the last array, rounded up to 8 bytes (one spare word)
    int2* sPair = reinterpret_cast<int2*>(
        (reinterpret_cast<uintptr_t>(sDup + (T > 1 ? k + 1 : 0)) + 7) & ~(uintptr_t)7);
    int32_t* sSlotU = reinterpret_cast<int32_t*>(sPair + P2);              // [S]
    // under profiling, thread 0 stamps the sort and the walk (100 MHz clock)
    const uint64_t c_sort0 = p.phase_clk ? __builtin_amdgcn_s_memrealtime() : 0;
    for (int i = tid; i < P2; i += kMRThreads) {
      const int32_t x = i < cap ? slot_table[i] : -1;
      sPair[i] = make_int2((x >= 0 && x < N) ? x : INT_MAX, i);
    }
    for (int i = tid; i < S; i += kMRThreads) sSlotU[i] = -1;
    __syncthreads();
    for (int k2 = 2; k2 <= P2; k2 <<= 1)
      for (int j2 = k2 >> 1; j2 > 0; j2 >>= 1) {
        for (int i = tid; i < P2; i += kMRThreads) {
          const int l = i ^ j2;
          if (l > i) {
            const int2 a = sPair[i], b = sPair[l];
            const bool up = (i & k2) == 0;
            const bool gt = a.x > b.x || (a.x == b.x && a.y > b.y);
            if (gt == up) {
              sPair[i] = b;
              sPair[l] = a;
            }
          }
        }
        __syncthreads();
      }
    const uint64_t c_sort1 = p.phase_clk ? __builtin_amdgcn_s_memrealtime() : 0;
    if (tid == 0) {
      int a = 0, b = 0, dup = 0;
      while (a < nu && b < P2 && sPair[b].x != INT_MAX) {
        const int32_t ua = sU[a], rb = sPair[b].x;
        if (ua < rb) {
          ++a;
        } else if (ua > rb) {
          ++b;
        } else {
          if (b + 1 < P2 && sPair[b + 1].x == ua) dup = 1;  // id of U held by two slots
          sUslot[a] = sPair[b].y;
          sSlotU[sPair[b].y] = a;
          ++a;
          ++b;
        }
      }
      if (dup) atomicOr(&sMisc[0], kFlagState);
    }
    __syncthreads();
    if (p.phase_clk && tid == 0) {
      const uint64_t c_walk1 = __builtin_amdgcn_s_memrealtime();
      atomicAdd(&p.phase_clk[0], (unsigned long long)(c_sort1 - c_sort0));
      atomicAdd(&p.phase_clk[1], (unsigned long long)(c_walk1 - c_sort1));
      atomicAdd(&p.phase_clk[2], 1ull);
    }
#pragma unroll
    for (int q = 0; q < MAXP; ++q) {
      if (bin[q] == kInvalid || tok[q] < 0) continue;
      const int i = sSlotU[s0 + q * 64 + lane];
      if (i >= 0) {
        hit_i[q] = i;
        bin[q] = -1;  // hit
      }
    }
    if (bad) atomicOr(&sMisc[0], kFlagState);
  } else if (sMisc[0] == 0 && dw > 0) {
    // direct-address membership: per slot one membership word and the rank
    // base of that word, the reads of a group of (up to) 8 slots issued
    // together; exact, so no probe reads on
    int bad = 0;
    constexpr int kGrp = MAXP < 8 ? MAXP : 8;
#pragma unroll
    for (int q0 = 0; q0 < MAXP; q0 += kGrp) {
      uint32_t wd[kGrp];
      int base[kGrp], res[kGrp], prev[kGrp];
#pragma unroll
      for (int qq = 0; qq < kGrp; ++qq) {
        const int q = q0 + qq;
        const int32_t x = tok[q], l = lf[q];
        const bool valid = x != kInvalid;
        const bool resident = x >= 0 && x < N;
        const bool bad_l = lru ? (l < 0 || (int64_t)l >= step_t) : (l < 0 || l > p.L);
        bad |= (valid && (x < -1 || x >= N)) | (resident && bad_l);
        bin[q] = valid ? 0 : kInvalid;
        const int wi = resident ? (x >> 5) : 0;
        wd[qq] = sBits[wi];
        base[qq] = sBase[wi];
      }
#pragma unroll
      for (int qq = 0; qq < kGrp; ++qq) {
        const int32_t x = tok[q0 + qq];
        const uint32_t bit = 1u << (x & 31);
        const bool member = x >= 0 && x < N && (wd[qq] & bit) != 0;
        res[qq] = member ? base[qq] + __popc(wd[qq] & (bit - 1)) : -1;
      }
      // hits record their slot; an id of U held by two slots is found by the
      // second exchange (a lane without a hit exchanges with its sink word)
#pragma unroll
      for (int qq = 0; qq < kGrp; ++qq)
        prev[qq] = atomicExch(res[qq] >= 0 ? &sUslot[res[qq]] : &sSink[lane],
                              s0 + (q0 + qq) * 64 + lane);
#pragma unroll
      for (int qq = 0; qq < kGrp; ++qq) {
        const bool hit = res[qq] >= 0;
        bad |= hit && prev[qq] != -1;
        hit_i[q0 + qq] = hit ? res[qq] : -1;
        bin[q0 + qq] = hit ? -1 : bin[q0 + qq];
      }
    }
    if (bad) atomicOr(&sMisc[0], kFlagState);
  } else if (sMisc[0] == 0) {
    int bad = 0;
    const int bmask = (C >> 2) - 1;
    const uint32_t lim = 1u << ubits;
    const int umask = (int)lim - 1;
    // state checks and the home bucket (cells and attempt counter) of every
    // probe of a group of (up to) 8 slots, all reads issued together; then
    // rounds in which every probe still open reads its next bucket
    constexpr int kGrp = MAXP < 8 ? MAXP : (MAXP > 8 ? 4 : 8);
#pragma unroll
    for (int q0 = 0; q0 < MAXP; q0 += kGrp) {
      int4 cb[kGrp];
      uint32_t hb[kGrp];
      int res[kGrp];  // union index, -1 absent, -2 searching, -3 home bucket full
      // branch-free: every lane reads a bucket (in range for any id), and
      // only lanes holding a resident id use it
#pragma unroll
      for (int qq = 0; qq < kGrp; ++qq) {
        const int q = q0 + qq;
        const int32_t x = tok[q], l = lf[q];
        const bool valid = x != kInvalid;
        const bool resident = x >= 0 && x < N;
        const bool bad_l = lru ? (l < 0 || (int64_t)l >= step_t) : (l < 0 || l > p.L);
        bad |= (valid && (x < -1 || x >= N)) | (resident && bad_l);
        bin[q] = valid ? 0 : kInvalid;
        hit_i[q] = -1;
        res[qq] = resident ? -2 : -1;
        hb[qq] = hash_id(x, log_cap) >> 2;
        cb[qq] = reinterpret_cast<const int4*>(sHash)[hb[qq]];
      }
      // home bucket: found there, or absent if the bucket has an empty cell;
      // a full home bucket without x needs its attempt counter
#pragma unroll
      for (int qq = 0; qq < kGrp; ++qq) {
        const int4 c = cb[qq];
        const int r = bucket_find(c, (uint32_t)tok[q0 + qq] << ubits, lim, umask);
        const bool full = min(min(c.x, c.y), min(c.z, c.w)) >= 0;
        res[qq] = res[qq] == -2 ? (r >= 0 ? r : (full ? -3 : -1)) : -1;
      }
      {  // counters of the (few) full home buckets: more than 4 attempts
         // means x may live further along its sequence
        bool any = false;
#pragma unroll
        for (int qq = 0; qq < kGrp; ++qq) any |= res[qq] == -3;
        if (__ballot(any)) {
          int hc[kGrp];
#pragma unroll
          for (int qq = 0; qq < kGrp; ++qq) hc[qq] = sBcnt[res[qq] == -3 ? hb[qq] : 0];
#pragma unroll
          for (int qq = 0; qq < kGrp; ++qq)
            if (res[qq] == -3) res[qq] = hc[qq] > 4 ? -2 : -1;
        }
      }
      while (true) {
        bool more = false;
#pragma unroll
        for (int qq = 0; qq < kGrp; ++qq) more |= res[qq] == -2;
        if (!__ballot(more)) break;
#pragma unroll
        for (int qq = 0; qq < kGrp; ++qq)
          if (res[qq] == -2) {
            hb[qq] = (hb[qq] + hash_step(tok[q0 + qq], log_cap)) & bmask;
            cb[qq] = reinterpret_cast<const int4*>(sHash)[hb[qq]];
          }
#pragma unroll
        for (int qq = 0; qq < kGrp; ++qq)
          if (res[qq] == -2) res[qq] = bucket_check(cb[qq], ubits, tok[q0 + qq]);
      }
      // hits record their slot; an id of U held by two slots is found by the
      // second exchange (the results are checked after all are issued)
      int prev[kGrp];
#pragma unroll
      for (int qq = 0; qq < kGrp; ++qq)
        prev[qq] = atomicExch(res[qq] >= 0 ? &sUslot[res[qq]] : &sSink[lane],
                              s0 + (q0 + qq) * 64 + lane);
#pragma unroll
      for (int qq = 0; qq < kGrp; ++qq) {
        const bool hit = res[qq] >= 0;
        bad |= hit && prev[qq] != -1;
        hit_i[q0 + qq] = hit ? res[qq] : -1;
        bin[q0 + qq] = hit ? -1 : bin[q0 + qq];
      }
    }
    if (bad) atomicOr(&sMisc[0], kFlagState);
  }
  {  // hits of this wave, summed into sMisc[2]: with every entry of U a hit
     // there are no misses to rank
    int nh = 0;
#pragma unroll
    for (int q = 0; q < MAXP; ++q) nh += __popcll(__ballot(hit_i[q] >= 0));
    if (lane == 0 && nh) atomicAdd(&sMisc[2], nh);
  }
  __syncthreads();

  // a data error: the unit keeps its state (nothing has been written to it)
  // and its outputs say so
  auto fail_unit = [&](int flags) {
    const int code = flags_to_status(flags);
    for (int i = tid; i < tks; i += kMRThreads) {
      p.sel_slot[(size_t)u * tks + i] = -1;
      p.hit_flag[(size_t)u * tks + i] = 0;
      p.fetch[(size_t)u * tks + i] = 0;
    }
    if (tid == 0) {
      p.n_hit[u] = 0;
      p.n_miss[u] = 0;
      p.n_evict[u] = 0;
      p.unit_status[u] = code;
      p.miss_count[u] = 0;
      if (p.user_status) p.user_status[u] = code;
      atomicOr(p.err_word, 1u << (code - 16));
    }
  };
  if (sMisc[0]) {
    fail_unit(sMisc[0]);
    return;
  }

  // ---- 5. policy update and eviction bins (registers, branch-free):
  //         hits take L (or the stamp t); other occupied slots decrement
  //         (lifetime) and get bin 1 + lifetime, or bin 1 + (B - 1 - bucket)
  //         (LRU, bucket = min((t - 1 - stamp) / W, B - 1)); empty slots keep
  //         bin 0
  if (!lru) {
#pragma unroll
    for (int q = 0; q < MAXP; ++q) {
      const int x = tok[q], l = lf[q];
      const bool hit = bin[q] == -1, occ = x >= 0;
      const int dec = max(l - 1, 0);
      lf[q] = hit ? p.L : (occ ? dec : l);
      bin[q] = (x == kInvalid || hit) ? bin[q] : (occ ? 1 + dec : 0);
    }
  } else {
    const int32_t t32 = (int32_t)step_t;  // stamps are int32 and below t
    const uint32_t W = (uint32_t)p.W;
#pragma unroll
    for (int q = 0; q < MAXP; ++q) {
      const int x = tok[q], l = lf[q];
      const bool hit = bin[q] == -1, occ = x >= 0;
      // steps since the last selection: in [0, 2^31) for a valid stamp (an
      // empty or padding slot's value is not used)
      uint32_t age = (uint32_t)t32 - 1u - (uint32_t)l;
      if (W > 1) age /= W;
      const int bucket = age < (uint32_t)(p.B - 1) ? (int)age : p.B - 1;
      lf[q] = hit ? t32 : l;
      bin[q] = (x == kInvalid || hit) ? bin[q] : (occ ? p.B - bucket : 0);
    }
  }

  // ---- 6. misses of U in ascending id order (two consecutive entries per
  //         thread, ranked by two ballots)
  int m = 0;
  const bool all_hit = sMisc[2] == nu;  // the same in every wave
  for (int c0 = 0; c0 < (all_hit ? 0 : nu); c0 += 2 * kMRThreads) {
    const int i0 = c0 + 2 * tid;
    const int v0 = sUslot[min(i0, nu - 1)], v1 = sUslot[min(i0 + 1, nu - 1)];
    const bool m0 = i0 < nu && v0 < 0;
    const bool m1 = i0 + 1 < nu && v1 < 0;
    const uint64_t b0 = __ballot(m0), b1 = __ballot(m1);
    if (lane == 0) sWs[w] = __popcll(b0) + __popcll(b1);
    __syncthreads();
    int pre = 0, tot = 0;
#pragma unroll
    for (int x = 0; x < kMRWaves; ++x) {
      const int v = sWs[x];
      pre += (x < w) ? v : 0;
      tot += v;
    }
    pre += mbcnt64(b0) + mbcnt64(b1);
    if (m0) sMiss[m + pre] = i0;
    if (m1) sMiss[m + pre + (m0 ? 1 : 0)] = i0 + 1;
    m += tot;
    // sWs is reused by the next round; after the last round, the barrier
    // that follows the bin histogram orders these stores before their reads
    if (c0 + 2 * kMRThreads < nu) __syncthreads();
  }

  // ---- 6b. with a host directory: the pool row of every miss, read
  //          through the two-level directory (top level in device memory,
  //          segment in pinned host memory) before anything is written; an
  //          entry without a row is a range error of the unit.  The probe's
  //          table is dead by now and holds the rows: sRowOf[r] for miss r,
  //          sURow[i] for union entry i.
  int32_t* sRowOf = lds;
  int32_t* sURow = lds + ucap;
  const bool dir = p.dir.top != nullptr;
  if (dir && m > 0) {  // (m is the same in every wave)
    __syncthreads();   // the miss list is complete
    const int32_t* top = p.dir.top + (size_t)u * p.dir.n_seg;
    const int lg = p.dir.seg_log2;
    const int32_t emask = (int32_t)((1u << lg) - 1);
    int bad = 0;
    constexpr int kDirGrp = 4;  // misses per thread whose reads are in flight together
    for (int r0 = 0; r0 < m; r0 += kDirGrp * kMRThreads) {
      int32_t idr[kDirGrp], seg[kDirGrp], row[kDirGrp];
#pragma unroll
      for (int g = 0; g < kDirGrp; ++g) {
        const int r = min(r0 + g * kMRThreads + tid, m - 1);
        idr[g] = sU[sMiss[r]];
        seg[g] = top[idr[g] >> lg];
      }
#pragma unroll
      for (int g = 0; g < kDirGrp; ++g) {
        const bool ok = seg[g] >= 0 && seg[g] < p.dir.n_segments;
        row[g] = p.dir.segments[((size_t)(ok ? seg[g] : 0) << lg) + (idr[g] & emask)];
        row[g] = ok ? row[g] : -1;
      }
#pragma unroll
      for (int g = 0; g < kDirGrp; ++g) {
        const int r = r0 + g * kMRThreads + tid;
        if (r < m) {
          bad |= row[g] < 0 || (int64_t)row[g] >= p.dir.pool_rows;
          sRowOf[r] = row[g];
        }
      }
    }
    if (bad) atomicOr(&sMisc[0], kFlagRange);
    __syncthreads();
    if (sMisc[0]) {
      fail_unit(sMisc[0]);
      return;
    }
  }

  // ---- 7. victims: the m first candidates in (bin, slot) order
  int ev = 0;
  bool changed[MAXP];
#pragma unroll
  for (int q = 0; q < MAXP; ++q) changed[q] = false;
  if (m > 0) {
    // per-wave counts of the candidates in bins 0..3 (one ballot per (bin,
    // slot group), counted on the scalar unit), published as a [bin][wave]
    // table of 64 words (the sink words, free after the probe); one read per
    // lane and one wave scan in (bin, wave) order then give every wave the
    // first rank of each of its bins.  If bins 0..3 hold fewer than m
    // candidates (a buffer turning over fast leaves the lowest lifetimes
    // empty), bins 4..7 are counted the same way into the next 64 words.
    int32_t* sC8 = sMisc + 64;
    int c8 = 0;  // lane b < 8: this wave's count of bin b
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      int cnt = 0;
#pragma unroll
      for (int q = 0; q < MAXP; ++q) cnt += __popcll(__ballot(bin[q] == b));
      c8 = lane == b ? cnt : c8;
    }
    if (lane < 4) sC8[lane * 16 + w] = c8;
    __syncthreads();
    const int c0 = sC8[lane];  // bin lane / 16, wave lane % 16
    const int inc0 = wave_incl_scan(c0);
    const int tot0 = __builtin_amdgcn_readlane(inc0, 63);
    int c1 = 0, inc1 = tot0;   // bins 4..7, counted only when needed
    if (tot0 < m) {  // the same in every wave
#pragma unroll
      for (int b = 4; b < 8; ++b) {
        int cnt = 0;
#pragma unroll
        for (int q = 0; q < MAXP; ++q) cnt += __popcll(__ballot(bin[q] == b));
        c8 = lane == b ? cnt : c8;
      }
      if (lane >= 4 && lane < 8) sC8[64 + (lane - 4) * 16 + w] = c8;
      __syncthreads();
      c1 = sC8[64 + lane];  // bin 4 + lane / 16, wave lane % 16
      inc1 = wave_incl_scan(c1) + tot0;
    }
    const bool fast = __builtin_amdgcn_readlane(inc1, 63) >= m;  // the same in every wave
    int bstar = nbins;
    int off[8] = {0, 0, 0, 0, 0, 0, 0, 0};  // fast: this wave's first rank in bins 0..7
    uint32_t nz = ~0u;  // fast: bins 0..7 in which this wave has candidates (bit b)
    uint64_t nz_lo = 0, nz_hi = 0;  // general: bins 0..63, 64..127 holding this wave's candidates
    if (fast) {
      const uint64_t r0 = __ballot((lane & 15) == 15 && inc0 >= m);
      const uint64_t r1 = __ballot((lane & 15) == 15 && inc1 >= m);
      bstar = r0 ? (__builtin_ctzll(r0) >> 4) : 4 + (__builtin_ctzll(r1) >> 4);
      const int ex0 = inc0 - c0, ex1 = inc1 - c1;
      const int wu = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        off[b] = __builtin_amdgcn_readlane(ex0, b * 16 + wu);
        off[4 + b] = __builtin_amdgcn_readlane(ex1, b * 16 + wu);
      }
      nz = (uint32_t)__ballot(lane < 8 && c8 != 0) | ~0xFFu;
    } else {
      // general: histogram of all bins (per wave, in LDS: the wave clears
      // its row, then one LDS add per candidate, in the wave's issue order),
      // the bin totals, their exclusive starts, b* and each wave's first
      // rank per bin; lane l covers bins l and l + 64 (nbins <= 128)
      int32_t* cnt_w = sCnt + w * nbins;
      if (lane < nbins) cnt_w[lane] = 0;
      if (lane + 64 < nbins) cnt_w[lane + 64] = 0;
#pragma unroll
      for (int q = 0; q < MAXP; ++q)
        if (bin[q] >= 0) atomicAdd(&cnt_w[bin[q]], 1);
      __syncthreads();
      int tot0 = 0, tot1 = 0, bef0 = 0, bef1 = 0, own0 = 0, own1 = 0;
      const int b0 = lane, b1 = lane + 64;
#pragma unroll
      for (int v = 0; v < kMRWaves; ++v) {
        const int c0v = b0 < nbins ? sCnt[v * nbins + b0] : 0;
        const int c1v = b1 < nbins ? sCnt[v * nbins + b1] : 0;
        tot0 += c0v;
        tot1 += c1v;
        bef0 += v < w ? c0v : 0;
        bef1 += v < w ? c1v : 0;
        own0 = v == w ? c0v : own0;
        own1 = v == w ? c1v : own1;
      }
      nz_lo = __ballot(own0 != 0);
      nz_hi = __ballot(own1 != 0);
      const int inc0 = wave_incl_scan(tot0);
      const int sum0 = __builtin_amdgcn_readlane(inc0, 63);
      const int inc1 = wave_incl_scan(tot1) + sum0;
      const int st0 = inc0 - tot0, st1 = inc1 - tot1;
      const uint64_t r0 = __ballot(b0 < nbins && st0 < m && st0 + tot0 >= m);
      const uint64_t r1 = __ballot(b1 < nbins && st1 < m && st1 + tot1 >= m);
      bstar = r0 ? __builtin_ctzll(r0) : 64 + __builtin_ctzll(r1);
      if (b0 < nbins) sOff[w * nbins + b0] = st0 + bef0;
      if (b1 < nbins) sOff[w * nbins + b1] = st1 + bef1;
    }
    // rank of each candidate in bins <= b* among the wave's candidates of
    // the same bin, in slot order (slot groups in order, lanes in order)
#pragma unroll
    for (int q = 0; q < MAXP; ++q) rank[q] = 0;
    auto rank_in_bin = [&](int b) {
      int run = 0;
#pragma unroll
      for (int q = 0; q < MAXP; ++q) {
        const uint64_t grp = __ballot(bin[q] == b);
        if (bin[q] == b) rank[q] = run + mbcnt64(grp);
        run += __popcll(grp);
      }
    };
    if (fast) {
      for (int b = 0; b <= bstar; ++b)
        if ((nz >> b) & 1) rank_in_bin(b);  // bins where the wave has candidates
    } else {
      // only the bins <= b* that hold candidates of this wave: with m
      // victims there are at most m of them besides b* itself
      uint64_t lo = nz_lo & (bstar >= 63 ? ~0ull : (2ull << bstar) - 1);
      uint64_t hi = bstar < 64 ? 0ull : nz_hi & (bstar >= 127 ? ~0ull : (2ull << (bstar - 64)) - 1);
      while (lo) {
        rank_in_bin(__builtin_ctzll(lo));
        lo &= lo - 1;
      }
      while (hi) {
        rank_in_bin(64 + __builtin_ctzll(hi));
        hi &= hi - 1;
      }
    }
    // rank[q] becomes the candidate's rank r among all candidates (m for
    // slots that are no candidates or lie beyond b*)
    if (fast) {
#pragma unroll
      for (int q = 0; q < MAXP; ++q) {
        const int b = bin[q];
        int o = off[0];
        o = b == 1 ? off[1] : o;
        o = b == 2 ? off[2] : o;
        o = b == 3 ? off[3] : o;
        if (bstar >= 4) {  // wave-uniform
#pragma unroll
          for (int bb = 4; bb < 8; ++bb) o = b == bb ? off[bb] : o;
        }
        rank[q] = (b >= 0 && b <= bstar) ? o + rank[q] : m;
      }
    } else {
#pragma unroll
      for (int q = 0; q < MAXP; ++q) {
        const int b = bin[q];
        const bool cand = b >= 0 && b <= bstar;
        const int o = sOff[w * nbins + (cand ? b : 0)];
        rank[q] = cand ? o + rank[q] : m;
      }
    }
    // the candidate of rank r < m takes the r-th miss; the reads of a group
    // of (up to) 8 slots are issued together (clamped for non-victims)
    int2* misses = p.misses + (size_t)u * ucap;
    constexpr int kGrp = MAXP < 8 ? MAXP : 8;
#pragma unroll
    for (int q0 = 0; q0 < MAXP; q0 += kGrp) {
      int r[kGrp], mi[kGrp], idv[kGrp], rowv[kGrp];
#pragma unroll
      for (int qq = 0; qq < kGrp; ++qq) r[qq] = rank[q0 + qq];
#pragma unroll
      for (int qq = 0; qq < kGrp; ++qq) mi[qq] = sMiss[min(r[qq], m - 1)];
#pragma unroll
      for (int qq = 0; qq < kGrp; ++qq) {
        idv[qq] = sU[mi[qq]];
        rowv[qq] = dir ? sRowOf[min(r[qq], m - 1)] : 0;
      }
#pragma unroll
      for (int qq = 0; qq < kGrp; ++qq) {
        const int q = q0 + qq;
        if (r[qq] < m) {
          const int s = s0 + q * 64 + lane;
          if (tok[q] >= 0) ++ev;
          tok[q] = idv[qq];
          lf[q] = lru ? (int32_t)step_t : p.L;
          changed[q] = true;
          sUslot[mi[qq]] = s | kMissFlag;
          if (dir) sURow[mi[qq]] = rowv[qq];
          // the transfer list: the row's id, or its pool row with a directory
          misses[r[qq]] = make_int2(s, dir ? rowv[qq] : idv[qq]);
        }
      }
    }
    ev = wave_total(ev);
    if (lane == 0 && ev) atomicAdd(&sMisc[1], ev);
    // the victims' union entries and the eviction count are read below; with
    // no miss (m is the same in every wave) nothing was written since the
    // probe's barrier, so only this branch needs one
    __syncthreads();
  }

  // ---- 8. per-(token, entry) outputs read off the union
  for (int i = tid; i < tk; i += kMRThreads) {
    if (T > 1 && !in_use_at(i, k, live_end0, live_end1)) {  // past a shortened list: no slot, no transfer
      p.sel_slot[(size_t)u * tks + i] = -1;
      p.hit_flag[(size_t)u * tks + i] = 0;
      p.fetch[(size_t)u * tks + i] = 0;
      continue;
    }
    const int mi = (T == 1) ? i : sMap[i];
    const int v = sUslot[mi & ~kDupFlag];
    const bool miss = (v & kMissFlag) != 0;
    p.sel_slot[(size_t)u * tks + i] = v & ~kMissFlag;
    p.hit_flag[(size_t)u * tks + i] = miss ? 0 : 1;
    // the row is transferred by the first token that selects it
    const bool fetch = miss && !(mi & kDupFlag);
    p.fetch[(size_t)u * tks + i] = fetch ? 1 : 0;
    if (dir) p.host_row[(size_t)u * tks + i] = fetch ? sURow[mi & ~kDupFlag] : -1;
  }
  // entries past a shortened list: no slot, no transfer
  for (int i = tk + tid; i < tks; i += kMRThreads) {
    p.sel_slot[(size_t)u * tks + i] = -1;
    p.hit_flag[(size_t)u * tks + i] = 0;
    p.fetch[(size_t)u * tks + i] = 0;
  }
  // ---- 9. write the new slot state back (registers only, after the
  //         outputs so that the stores overlap them)
#pragma unroll
  for (int q = 0; q < MAXP; ++q) {
    if (tok[q] == kInvalid) continue;
    const int s = s0 + q * 64 + lane;
    lifetimes[s] = lf[q];
    if (changed[q]) slot_table[s] = tok[q];
  }
  if (drop) {
#pragma unroll
    for (int q = 0; q < MAXP; ++q) {
      if ((drop >> q) & 1) {
        slot_table[s0 + q * 64 + lane] = -1;
        lifetimes[s0 + q * 64 + lane] = life_empty;
      }
    }
  }

  if (tid == 0) {
    p.n_hit[u] = nu - m;
    p.n_miss[u] = m;
    p.n_evict[u] = sMisc[1];
    p.unit_status[u] = 0;
    p.miss_count[u] = m;
    if (p.user_status) p.user_status[u] = 0;
  }
}

template <int MAXP>
hipError_t launch_mr(const MatchReserveParams& p, int units, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL(match_reserve_kernel<MAXP>, dim3(units), dim3(kMRThreads), lds, s, p);
  return hipGetLastError();
}

template <int MAXP>
hipError_t set_lds(size_t lds) {
  return hipFuncSetAttribute((const void*)match_reserve_kernel<MAXP>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

// ---- full state validation: ranges and duplicate ids over all slots
__global__ __launch_bounds__(kMRThreads) void validate_kernel(const int32_t* slot_table,
                                                              const int32_t* lifetimes, int S,
                                                              int N, int policy, int L, int64_t t,
                                                              int log_cap, uint32_t* err) {
  extern __shared__ int32_t tab[];
  const int u = blockIdx.x;
  const int C = 1 << log_cap;
  for (int i = threadIdx.x; i < C; i += kMRThreads) tab[i] = -1;
  __syncthreads();
  int bad = 0;
  for (int s = threadIdx.x; s < S; s += kMRThreads) {
    const int32_t x = slot_table[(size_t)u * S + s];
    if (x < -1 || x >= N) { bad = 1; continue; }
    if (x < 0) continue;
    if (lifetimes) {  // null: the id map alone
      const int32_t l = lifetimes[(size_t)u * S + s];
      if (policy == AVSG_POLICY_LIFETIME && (l < 0 || l > L)) bad = 1;
      if (policy == AVSG_POLICY_BUCKET_LRU && (l < 0 || (int64_t)l >= t)) bad = 1;
    }
    uint32_t h = hash_id(x, log_cap);
    while (true) {
      int prev = atomicCAS(&tab[h], -1, x);
      if (prev == -1) break;
      if (prev == x) { bad = 1; break; }
      h = (h + 1) & (C - 1);
    }
  }
  if (bad) atomicOr(err, 1u);
}

}  // namespace

hipError_t launch_match_reserve(const MatchReserveParams& p, int units, size_t lds, hipStream_t s) {
  const int per_lane = (p.S + kMRThreads - 1) / kMRThreads;
  if (per_lane <= 1) return launch_mr<1>(p, units, lds, s);
  if (per_lane <= 2) return launch_mr<2>(p, units, lds, s);
  if (per_lane <= 4) return launch_mr<4>(p, units, lds, s);
  if (per_lane <= 8) return launch_mr<8>(p, units, lds, s);
  return launch_mr<16>(p, units, lds, s);
}

hipError_t match_reserve_set_lds(size_t lds) {
  hipError_t e;
  if ((e = set_lds<1>(lds)) != hipSuccess) return e;
  if ((e = set_lds<2>(lds)) != hipSuccess) return e;
  if ((e = set_lds<4>(lds)) != hipSuccess) return e;
  if ((e = set_lds<8>(lds)) != hipSuccess) return e;
  return set_lds<16>(lds);
}

hipError_t launch_validate(const int32_t* slot_table, const int32_t* lifetimes, int units, int S,
                           int N, int policy, int L, int64_t t, uint32_t* err, hipStream_t s) {
  int log_cap = 6;
  while ((1 << log_cap) < 2 * S) ++log_cap;
  const size_t lds = sizeof(int32_t) << log_cap;
  hipError_t e = hipFuncSetAttribute((const void*)validate_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(validate_kernel, dim3(units), dim3(kMRThreads), lds, s, slot_table, lifetimes,
                     S, N, policy, L, t, log_cap, err);
  return hipGetLastError();
}

}  // namespace avsg
