// K3 + K4: split-k decode attention over the buffer slots of the selected
// entries (K/V split layout, grouped-query heads), then the merge of the
// splits.
//
// What it computes: for each unit, query token and query head of the unit,
// softmax(scale * q K^T) V over exactly the selected entries (all tokens of a
// selected page), reading every row from the slot that match_reserve assigned.
// The AVSG abstract (arxivdaily 2609.37538) requires the selections to stay
// exact, so this equals attention over the same rows read from host memory.
//
// gfx950 mapping (HBM-bound; the two contractions on MFMA):
//  * A workgroup is one wave and owns `split_rows` token rows of one (unit,
//    token): no barrier anywhere.  The rows stream through three LDS tiles of
//    32 rows (512 bytes each: K half, V half) by direct global-to-LDS copies
//    of 16 bytes per lane, 16 per tile: copy x reads rows 2x and 2x + 1, 16
//    lanes per 256-byte half row, so host memory is read in 256-byte runs
//    (shorter runs cost link efficiency).  The rows' source addresses are
//    computed once per tile into a small LDS table.  Inside a half row the
//    16-byte pieces are permuted by the row index (piece c at slot c ^ (row
//    mod 16)), which puts the 16 rows an MFMA operand reads in distinct LDS
//    banks.  Two tiles are in flight while one is used, and a vmcnt wait with
//    a constant count tells the wave that the tile it needs has landed.
//  * Scores are computed transposed, S^T = K Q^T, on v_mfma_f32_16x16x32_bf16
//    (M = 16 rows, N = the unit's G query heads padded to 16 columns, K = 32
//    dimensions, 4 steps).  In that result layout each lane owns one head's
//    column, so the online softmax reduces over 4 lanes with the gfx950 lane
//    swaps, and the probabilities are already the B operand of O^T = V^T P^T
//    (K = the tile's 32 rows).  V^T operands come from ds_read_b64_tr_b16,
//    the transposing LDS read, so V is never transposed in memory.  Padding
//    the heads wastes MFMA work, which is far from the bound; VALU work per
//    row is what limited the dot-product form of this kernel.
//  * P is split into bf16 hi + lo parts (two MFMAs on the same V fragment):
//    rounding P to bf16 alone would leave about 1e-3 relative error.
//  * Rows whose entry missed are copied from pinned host memory into the tile;
//    the lane that copied a piece then stores it from LDS into the entry's
//    slot, so the row crosses the host link once.  When the grid runs in
//    several rounds of resident workgroups, the workgroup has a second wave
//    instead, which copies all of the split's missed entries from host memory
//    into their slots (every host read in flight at once) while the first
//    wave streams the split's tiles from HBM in selection order; the first
//    wave waits (on an LDS flag) only at the first tile that holds a missed
//    row.  The host link then stays busy while tiles stream: with one wave
//    doing both, all resident workgroups fetched, then all streamed, in
//    lock-step rounds.
//  * All LDS reads of the tiles are inline assembly with waits tied to their
//    results: the compiler would otherwise order every LDS read after all
//    outstanding global-to-LDS copies.
//  * The reference maximum of the online softmax moves only when a tile
//    exceeds it by 2^8, so the accumulators are rescaled rarely; the result
//    does not depend on the reference chosen.
//  * Split partials (max, sum, o) go to the workspace and the combine kernel
//    merges them in split order, so the result does not depend on workgroup
//    timing.  (Merging inside the last workgroup of each (unit, token) needs
//    an agent-scope release in every workgroup, which writes back the XCD's
//    L2 each time and cost more than the extra launch.)
#include <mutex>
#include <type_traits>
#include <utility>

#include "avsg_internal.h"

namespace avsg {
namespace {

constexpr int kD = 128;                              // head dim of the split layout
constexpr int kChunk = 32;                           // token rows per LDS tile
constexpr int kCopies = kChunk * 4 * kD / 1024;      // 16 wave-wide copies of 1 KiB per tile
constexpr int kTileBytes = kCopies * 1024;           // 16 KiB
constexpr int kBufs = 3;                             // LDS tiles per workgroup
constexpr int kAhead = kBufs - 1;                    // tiles in flight beyond the one in use
static_assert(kAhead >= 1 && kAhead <= 3, "tile pipeline depth");
constexpr int kThreads = 64;                         // one wave per workgroup
constexpr int kSplitRows = 256;                      // token rows per workgroup
constexpr int kKSteps = kD / 32;                     // 4 MFMA k-steps for QK^T
constexpr int kDTiles = kD / 16;                     // 8 output tiles of 16 dimensions
constexpr int kGatherDepth = 4;                      // gather-first: host loads per lane per round

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void*)p;
}
template <int OFF>
__device__ __forceinline__ void ds_b128(u32x4& d, uint32_t a) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(d) : "v"(a), "n"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_tr(u32x2& d, uint32_t a) {
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(d) : "v"(a), "n"(OFF));
}
__device__ __forceinline__ void ds_b64(int2& d, uint32_t a) {
  asm volatile("ds_read_b64 %0, %1" : "=v"(d) : "v"(a));
}
__device__ __forceinline__ void ds_b32(int& d, uint32_t a) {
  asm volatile("ds_read_b32 %0, %1" : "=v"(d) : "v"(a));
}
template <int OFF>
__device__ __forceinline__ void ds_u64(uint64_t& d, uint32_t a) {
  asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(d) : "v"(a), "n"(OFF));
}
// LDS word read that completes before the next instruction (an LDS flag
// polled while global-to-LDS copies of other addresses are in flight)
__device__ __forceinline__ int ds_i32_now(uint32_t a) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
  return v;
}
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// max / sum over the four lanes l, l^16, l^32, l^48 (one head's column)
__device__ __forceinline__ float col_max(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float col_sum(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// GF (gather-first): two waves per workgroup, wave 1 fetching the split's
// missed entries into their slots while wave 0 computes; else one wave that
// copies missed rows from host memory into its tiles.
template <int G, bool GF>
__global__ __launch_bounds__(GF ? 2 * kThreads : kThreads)
__attribute__((amdgpu_waves_per_eu(1, 2))) void attn_split_kernel(AttnParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t sTile[];  // [kBufs][kTileBytes]
  __shared__ int2 sRow[kSplitRows];      // per entry of the split: (slot, host id or -1)
  __shared__ int32_t sHost[kSplitRows];  // entries to fetch (gather-first)
  __shared__ uint64_t sSrc[kBufs][kChunk];  // per tile row: source address
  __shared__ uint64_t sDst[kBufs][kChunk];  // per tile row: slot address (host rows)
  __shared__ int32_t sGathered;          // gather-first: wave 1 has stored every missed entry
  __shared__ int32_t sNHost;             // gather-first: entries to fetch

  // the context's step counter advances once per step, here: the match
  // kernel that read it has finished (a non-returning atomic: no wait)
  if (p.step && p.token == 0 && blockIdx.x == 0 && threadIdx.x == 0)
    __hip_atomic_fetch_add(p.step, (int64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int nsplit = p.nsplit;
  // workgroups are dealt to the 8 XCDs in turn (workgroup i on XCD i mod 8);
  // when the grid divides by 8, XCD x takes the x-th eighth of the (unit,
  // split) range, so every split of a unit runs behind the same L2 (a later
  // token's launch finds the rows an earlier one read or stored there)
  const int nb = (int)gridDim.x;
  const int bid = (nb & 7) == 0 ? (int)(blockIdx.x & 7) * (nb >> 3) + (int)(blockIdx.x >> 3)
                                : (int)blockIdx.x;
  const int u = bid / nsplit;
  const int sp = bid - u * nsplit;
  const int j = p.token;
  const int uj = u * p.T + j;
  const int b = u / p.Hkv, g = u - b * p.Hkv;
  const int lane = threadIdx.x & (kThreads - 1);
  const int wave = GF ? (int)(threadIdx.x / kThreads) : 0;  // GF: 0 computes, 1 fetches
  const int gq = lane >> 4, li = lane & 15;  // lane group (rows / dims), column (head)
  const int tpe = p.tpe;
  // a shortened list (length array): its first sel_len[u][j] entries; a
  // length outside [1, k] marks a unit whose step failed, whose workgroups
  // read at most k entries and then zero its outputs
  const int len = p.sel_len ? min(max(p.sel_len[uj], 1), p.k) : p.k;
  const int n_rows = len * tpe;
  const int r0 = sp * p.split_rows, r1 = min(r0 + p.split_rows, n_rows);
  if (r0 >= n_rows) return;  // a split past the list's end (merged as empty)
  float* orow = p.out + (((size_t)b * p.T + j) * p.Hq + g * G) * kD;
  const int e0 = r0 / tpe, e1 = (r1 - 1) / tpe + 1;
  const int ne = e1 - e0;  // entries of the split, <= kSplitRows
  // every global load of the prologue is issued before any is used: the
  // unit's status, the split's (slot, fetch flag, id) per entry (kEnt per
  // lane, indices clamped into the split) and this lane's Q operand: head li
  // (zero past the unit's G heads), dims 32 ks + 8 gq .. +8
  constexpr int kEnt = kSplitRows / kThreads;
  const int ustat = __builtin_nontemporal_load(p.unit_status + u);
  // with context lengths: the list's last id and the request's length (the
  // last entry may hold the context's end)
  const bool has_ctx = p.ctx_len != nullptr && tpe > 1;
  int ctx_last = 0, ctx_n = 0;
  if (has_ctx && wave == 0) {
    ctx_last = p.sel[(size_t)uj * p.k + len - 1];
    ctx_n = p.ctx_len[b];
  }
  int slot_v[kEnt], id_v[kEnt], fl_v[kEnt];
  // without fetch flags (rows already gathered) the flag loads read the
  // slot array instead and are ignored
  const bool has_fetch = p.fetch != nullptr;
  const uint8_t* fl_src = has_fetch ? p.fetch : reinterpret_cast<const uint8_t*>(p.sel_slot);
  // host row of a fetched entry: its id in the unit's part of a flat host KV,
  // or its pool row (host directory)
  const int32_t* id_src = p.host_row ? p.host_row : p.sel;
  bf16x8 qf[kKSteps];
  if (wave == 0) {  // (gather-first: wave 1 reads the split's entries from LDS)
#pragma unroll
    for (int k = 0; k < kEnt; ++k) {
      const size_t at = (size_t)uj * p.k + e0 + min(k * kThreads + lane, ne - 1);
      slot_v[k] = p.sel_slot[at];
      id_v[k] = id_src[at];
      fl_v[k] = fl_src[at];
    }
    const uint16_t* qrow =
        p.q + (((size_t)b * p.T + j) * p.Hq + g * G + (li < G ? li : 0)) * kD + 8 * gq;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 32 * ks);
      qf[ks] = __builtin_bit_cast(bf16x8, li < G ? v : u32x4{0, 0, 0, 0});
    }
  }
  // the loads stay above the status branch (one wait for all of them)
#pragma unroll
  for (int k = 0; k < kEnt; ++k) asm volatile("" ::"v"(slot_v[k]), "v"(id_v[k]), "v"(fl_v[k]));
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) asm volatile("" ::"v"(qf[ks]));
  asm volatile("" ::"v"(ctx_last), "v"(ctx_n));
  if (__builtin_amdgcn_readfirstlane(ustat) != 0) {  // the same in both waves
    if (nsplit == 1 && wave == 0)
      for (int idx = lane; idx < G * kD; idx += kThreads) orow[idx] = 0.f;
    return;
  }
  if (wave == 0) {
    int nhost = 0;  // entries of the split to fetch (gather-first)
#pragma unroll
    for (int k = 0; k < kEnt; ++k) {
      const int i = k * kThreads + lane;
      const bool fetch = has_fetch && i < ne && fl_v[k] != 0;
      if (i < ne) sRow[i] = make_int2(slot_v[k], fetch ? id_v[k] : -1);
      if (GF) {
        const uint64_t m = __builtin_amdgcn_ballot_w64(fetch);
        if (fetch)
          sHost[nhost + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] = i;
        nhost += __popcll(m);
      }
    }
    if (GF && lane == 0) {
      sNHost = nhost;
      sGathered = 0;
    }
  }
  __syncthreads();  // sRow, sHost, sNHost, sGathered
  // the queries are in registers before any copy is issued
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) asm volatile("" : "+v"(qf[ks]));

  // rows attended: [r0, rv1).  The list is ascending, so only its last entry
  // can hold the end of the request's context; that entry's rows at or past
  // the context length are masked like rows past the split (and a split
  // that lies wholly past it contributes nothing).  Those rows are still
  // staged, so that a row fetched from host memory reaches its slot whole.
  int rv1 = r1;
  if (has_ctx) {
    const int64_t in_ctx = (int64_t)__builtin_amdgcn_readfirstlane(ctx_n) -
                           (int64_t)__builtin_amdgcn_readfirstlane(ctx_last) * tpe;  // its rows inside
    const int keep = (int)max((int64_t)1, min((int64_t)tpe, in_ctx));
    rv1 = min(r1, (len - 1) * tpe + keep);
  }

  uint16_t* ubase = p.buf_kv + (size_t)u * p.S * p.row_elems;
  const uint16_t* hbase = p.host_kv + (p.host_row ? 0 : (size_t)u * p.N * p.row_elems);
  const int v_off = tpe * kD;  // elements from an entry's K rows to its V rows
  const uint32_t row_lds = lds_addr(sRow);
  const uint32_t tile_lds = lds_addr(sTile);

  // Gather-first, wave 1: the split's missed entries go from pinned host
  // memory into their slots, kGatherDepth 16-byte pieces per lane in flight
  // per round; once every store is complete, the flag tells wave 0 that the
  // tiles may copy those slots.  Wave 1 then exits.
  if (GF && wave == 1) {
    const int nhost = sNHost;
    const int pe = p.row_elems >> 3;  // 16-byte pieces per entry
    const int total = nhost * pe;
    const uint32_t host_lds = lds_addr(sHost);
    // per round: the entries of this lane's kGatherDepth pieces (LDS reads
    // in inline assembly, so that the compiler does not order them behind
    // the stores of the previous round), then the host loads and the slot
    // stores, each back to back.  Piece indices are clamped into the list: a lane past its
    // end re-reads the list's last piece and writes the same 16 bytes to the
    // same place as the lane that owns it, so no branch (and no wait per
    // store) is needed.
    for (int q0 = 0; q0 < total; q0 += kGatherDepth * kThreads) {
      int qv[kGatherDepth], ev[kGatherDepth];
      int2 rv[kGatherDepth];
#pragma unroll
      for (int bq = 0; bq < kGatherDepth; ++bq) {
        qv[bq] = min(q0 + bq * kThreads + lane, total - 1);
        ds_b32(ev[bq], host_lds + 4 * (qv[bq] / pe));
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int bq = 0; bq < kGatherDepth; ++bq) asm volatile("" : "+v"(ev[bq]));
#pragma unroll
      for (int bq = 0; bq < kGatherDepth; ++bq) ds_b64(rv[bq], row_lds + 8 * ev[bq]);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int bq = 0; bq < kGatherDepth; ++bq) asm volatile("" : "+v"(rv[bq]));
      u32x4 v[kGatherDepth];
#pragma unroll
      for (int bq = 0; bq < kGatherDepth; ++bq) {
        const int col = qv[bq] - (qv[bq] / pe) * pe;
        v[bq] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
            hbase + (size_t)(uint32_t)rv[bq].y * p.row_elems + col * 8));
      }
#pragma unroll
      for (int bq = 0; bq < kGatherDepth; ++bq) {
        const int col = qv[bq] - (qv[bq] / pe) * pe;
        *reinterpret_cast<u32x4*>(ubase + (size_t)(uint32_t)rv[bq].x * p.row_elems + col * 8) =
            v[bq];
      }
    }
    vm_wait<0>();  // the stores are complete (in L2) before the flag is raised
    if (lane == 0) __hip_atomic_store(&sGathered, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    return;
  }
  // gather-first, wave 0: the first tile that holds a missed row (ntiles if
  // none); the tiles before it are staged at once, and wave 1's flag is
  // awaited once, right before that tile is staged
  int t_miss = 1 << 30;
  if (GF) {
    const int nhost = sNHost;
    if (nhost > 0) {
      const int first_row = max((e0 + sHost[0]) * tpe - r0, 0);  // sHost is in entry order
      t_miss = first_row / kChunk;
    }
  }
  auto await_gathered = [&]() {
    // wave 1 raises the flag after its slot stores are complete; the tile
    // copies that follow are issued only after the raised flag has been read
    while (__builtin_amdgcn_readfirstlane(ds_i32_now(lds_addr(&sGathered))) == 0)
      __builtin_amdgcn_s_sleep(2);
  };

  // Entry of a row: r itself for token entries, else r / tpe by an exact
  // multiply-high with ceil(2^32 / tpe) (exact while r * tpe < 2^32).
  const uint32_t tpe_magic = tpe == 1 ? 0u : (uint32_t)((0x100000000ull + tpe - 1) / tpe);
  auto entry_of = [&](int r) -> int {
    return tpe == 1 ? r : (int)__umulhi((uint32_t)r, tpe_magic);
  };
  // LDS tile layout: piece c (16 bytes; 0..15 K half, 16..31 V half) of tile
  // row r sits at byte 512 r + 256 (c / 16) + 16 ((c % 16) ^ (r % 16)).  Copy
  // x fills bytes [1024 x, +1024): lane L takes half (L / 16) % 2 of row 2x +
  // L / 32, piece (L % 16) ^ (row % 16) of it.
  const uint32_t lane_c = (uint32_t)((lane & 15) ^ (lane >> 5));
  const uint32_t half_b = (uint32_t)(((lane >> 4) & 1) * v_off * 2);  // bytes to the V rows
  const uint32_t src_lds = lds_addr(sSrc) + 8 * (lane >> 5);
  const uint32_t dst_lds = lds_addr(sDst) + 8 * (lane >> 5);
  // Copies tile t into buffer `buf`.  Rows past the split repeat its last row
  // (their scores are masked), so every tile takes exactly kCopies copies.
  // Returns the tile rows that came from host memory (bit r, wave-uniform).
  auto stage = [&](int t, int buf) -> uint32_t {
    int ln = lane;
    asm volatile("" : "+v"(ln));  // recomputed per tile rather than held
    // lane l < 32: source (and slot) address of tile row l
    const int rr = r0 + t * kChunk + (ln & 31);
    const int r = min(rr, r1 - 1);
    const int e = entry_of(r);
    int2 ri;
    ds_b64(ri, row_lds + 8 * (e - e0));
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(ri)::"memory");
    // gather-first: every row is read from its slot (the tiles that hold a
    // missed row are staged only after wave 1 has stored all of them)
    const bool host = !GF && ri.y >= 0;
    const uint32_t in_entry = (uint32_t)((r - e * tpe) * kD);
    const uint16_t* src = (host ? hbase : ubase) +
                          (uint64_t)(uint32_t)(host ? ri.y : ri.x) * (uint32_t)p.row_elems + in_entry;
    if (ln < kChunk) {
      sSrc[buf][ln] = (uint64_t)(uintptr_t)src;
      sDst[buf][ln] = (uint64_t)(uintptr_t)(ubase + (uint64_t)(uint32_t)ri.x * (uint32_t)p.row_elems +
                                            in_entry);
    }
    const uint32_t hmask = (uint32_t)__builtin_amdgcn_ballot_w64(host && rr < r1 && ln < kChunk);
    asm volatile("" ::: "memory");  // the table stores above precede its reads
    uint64_t a[kCopies];
    const uint32_t sa = src_lds + buf * (kChunk * 8);
    static_for<0, kCopies>([&](auto x_) {
      constexpr int x = decltype(x_)::value;
      ds_u64<16 * x>(a[x], sa);
    });
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int x = 0; x < kCopies; ++x) asm volatile("" : "+v"(a[x]));
    uint8_t* tile = sTile + buf * kTileBytes;
#pragma unroll
    for (int x = 0; x < kCopies; ++x) {
      const uint8_t* srcx =
          reinterpret_cast<const uint8_t*>(a[x]) + half_b + 16 * (lane_c ^ ((2 * x) & 15));
      __builtin_amdgcn_global_load_lds(srcx, (lds_void*)(tile + x * 1024), 16, 0, 0);
    }
    return hmask;
  };
  // Stores the host rows of tile t (bit r of hmask) from LDS into their slots.
  auto write_back = [&](int t, int buf, uint32_t hmask) {
    if (hmask == 0) return;
    uint64_t a[kCopies];
    u32x4 d[kCopies];
    const uint32_t da = dst_lds + buf * (kChunk * 8);
    const uint32_t ta = tile_lds + buf * kTileBytes + lane * 16;
    static_for<0, kCopies>([&](auto x_) {
      constexpr int x = decltype(x_)::value;
      ds_u64<16 * x>(a[x], da);
      ds_b128<1024 * x>(d[x], ta);
    });
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int x = 0; x < kCopies; ++x) asm volatile("" : "+v"(a[x]), "+v"(d[x]));
#pragma unroll
    for (int x = 0; x < kCopies; ++x) {
      if ((hmask >> (2 * x + (lane >> 5))) & 1) {
        uint8_t* dst = reinterpret_cast<uint8_t*>(a[x]) + half_b + 16 * (lane_c ^ ((2 * x) & 15));
        *reinterpret_cast<u32x4*>(dst) = d[x];
      }
    }
  };

  // acc[t]: O^T[dims 16 t + 4 gq + i][head li], i = 0..3
  f32x4 acc[kDTiles];
#pragma unroll
  for (int t = 0; t < kDTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int ntiles = (r1 - r0 + kChunk - 1) / kChunk;
  // fmask[i]: the host rows of tile t + i
  uint32_t fmask[kAhead];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) {
    if (GF && i == t_miss) await_gathered();
    fmask[i] = i < ntiles ? stage(i, i) : 0u;
  }
  // per-lane operand addresses within a tile (rows 16..31: +8192): K row li,
  // dims 32 ks + 8 gq .. +8 (piece 4 ks + gq); V^T row R = 4 gq + li / 4, dims
  // 32 pr + 16 vb + 4 (li % 4) .. +4 (V piece 4 pr + 2 vb + (li % 4) / 2, byte
  // 8 (li % 2) of it)
  uint32_t k_off[kKSteps], v_off_l[kDTiles];
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) k_off[ks] = 512 * li + 16 * ((4 * ks + gq) ^ li);
  {
    const int R = 4 * gq + (li >> 2);
#pragma unroll
    for (int pr = 0; pr < kDTiles / 2; ++pr)
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
        v_off_l[2 * pr + vb] = 512 * R + 256 + 16 * ((4 * pr + 2 * vb + ((li & 3) >> 1)) ^ R) +
                               8 * (li & 1);
  }

  // one tile: wait for its copies, stage tile t + kAhead, compute
  auto tile_step = [&](int t) {
    const int buf = t % kBufs;
    // tile t has landed once only the copies of the later tiles in flight
    // (kCopies each) and later slot stores may still be outstanding
    const int later = min(kAhead - 1, ntiles - 1 - t);
    if (later <= 0) vm_wait<0>();
    else if (later == 1) vm_wait<kCopies>();
    else if (later == 2) vm_wait<2 * kCopies>();
    else vm_wait<3 * kCopies>();
    const uint32_t f_now = fmask[0];
#pragma unroll
    for (int i = 0; i + 1 < kAhead; ++i) fmask[i] = fmask[i + 1];
    fmask[kAhead - 1] = t + kAhead < ntiles ? stage(t + kAhead, (t + kAhead) % kBufs) : 0u;
    // slot stores of tile t's host rows, issued after the copies of tile
    // t + kAhead: the next tile's wait (its copies are older) does not wait
    // for them
    write_back(t, buf, f_now);

    const uint32_t tb = tile_lds + buf * kTileBytes;
    // rows of the tile at or past rv1 (when the context ends inside the
    // split) may hold anything, NaN included: their V halves are zeroed, so
    // that their zero probabilities give exact zeros in the MFMA (0 * NaN
    // would not); their scores, whatever K gives, are replaced by -inf
    // before the softmax.  After write_back's LDS reads, before the V reads
    // below.
    const int z0 = rv1 - (r0 + t * kChunk);
    if (rv1 < r1 && z0 < kChunk) {
      const u32x4 zero = {0u, 0u, 0u, 0u};
      const int zr = max(z0, 0);
      for (int i = lane; i < (kChunk - zr) * 16; i += kThreads) {
        const uint32_t a = tb + 512 * (zr + (i >> 4)) + 256 + 16 * (i & 15);
        asm volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(zero) : "memory");
      }
    }

    // S^T = K Q^T for rows 0..15 and 16..31 of the tile
    u32x4 kf0[kKSteps], kf1[kKSteps];
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      ds_b128<0>(kf0[ks], tb + k_off[ks]);
      ds_b128<8192>(kf1[ks], tb + k_off[ks]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(kf0[0]), "+v"(kf0[1]), "+v"(kf0[2]), "+v"(kf0[3]), "+v"(kf1[0]),
                   "+v"(kf1[1]), "+v"(kf1[2]), "+v"(kf1[3]));
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf0[ks]), qf[ks], s0,
                                                   0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf1[ks]), qf[ks], s1,
                                                   0, 0, 0);
    }
    // V^T operands of the first two output tiles, read while the softmax runs
    u32x2 vr[2][4];
    ds_tr<0>(vr[0][0], tb + v_off_l[0]);
    ds_tr<8192>(vr[0][1], tb + v_off_l[0]);
    ds_tr<0>(vr[0][2], tb + v_off_l[1]);
    ds_tr<8192>(vr[0][3], tb + v_off_l[1]);

    // lane owns head li: rows 4 gq + i (s0) and 16 + 4 gq + i (s1) of the tile
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = r0 + t * kChunk + 4 * gq + i, rb = ra + 16;
      sv[i] = ra < rv1 ? s0[i] * p.scale_log2e : -INFINITY;
      sv[4 + i] = rb < rv1 ? s1[i] * p.scale_log2e : -INFINITY;
    }
    float cm = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) cm = fmaxf(cm, sv[i]);
    cm = col_max(cm);
    const bool move = cm > m_run + 8.f;
    const float m_new = move ? cm : m_run;
    const float corr = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first tile
    float ps = 0.f;
    bf16x8 phi, plo;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float pv = __builtin_amdgcn_exp2f(sv[i] - m_new);
      ps += pv;
      const __bf16 hb = (__bf16)pv;
      phi[i] = hb;
      plo[i] = (__bf16)(pv - (float)hb);
    }
    l_run = l_run * corr + col_sum(ps);
    m_run = m_new;
    if (__builtin_amdgcn_ballot_w64(move)) {
#pragma unroll
      for (int d = 0; d < kDTiles; ++d) acc[d] *= corr;
    }

    // O^T += V^T P^T, output tiles in pairs.  k slot 8 gq + r is row 4 gq + r
    // for r < 4 and 16 + 4 gq + (r - 4) otherwise, matching the probabilities.
    static_for<0, kDTiles / 2>([&](auto pr_) {
      constexpr int pr = decltype(pr_)::value, st = pr & 1;
      if constexpr (pr + 1 < kDTiles / 2) {
        ds_tr<0>(vr[st ^ 1][0], tb + v_off_l[2 * pr + 2]);
        ds_tr<8192>(vr[st ^ 1][1], tb + v_off_l[2 * pr + 2]);
        ds_tr<0>(vr[st ^ 1][2], tb + v_off_l[2 * pr + 3]);
        ds_tr<8192>(vr[st ^ 1][3], tb + v_off_l[2 * pr + 3]);
        asm volatile("s_waitcnt lgkmcnt(4)"
                     : "+v"(vr[st][0]), "+v"(vr[st][1]), "+v"(vr[st][2]), "+v"(vr[st][3]));
      } else {
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(vr[st][0]), "+v"(vr[st][1]), "+v"(vr[st][2]), "+v"(vr[st][3]));
      }
      const u32x2 a2[2] = {vr[st][0], vr[st][1]}, b2[2] = {vr[st][2], vr[st][3]};
      const bf16x8 vta = __builtin_bit_cast(bf16x8, a2), vtb = __builtin_bit_cast(bf16x8, b2);
      acc[2 * pr] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vta, phi, acc[2 * pr], 0, 0, 0);
      acc[2 * pr + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vtb, phi, acc[2 * pr + 1], 0, 0, 0);
      acc[2 * pr] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vta, plo, acc[2 * pr], 0, 0, 0);
      acc[2 * pr + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vtb, plo, acc[2 * pr + 1], 0, 0, 0);
    });
  };
  int t = 0;
  if (GF) {
    // iterations that stage only tiles before t_miss, then the one wait
    // (when t_miss < kAhead it was taken before the first tiles were staged)
    for (const int t_end = min(ntiles, t_miss - kAhead); t < t_end; ++t) tile_step(t);
    if (t_miss >= kAhead && t_miss < ntiles) await_gathered();
  }
  for (; t < ntiles; ++t) tile_step(t);

  // lane holds O[head li][d = 16 t + 4 gq + i] (heads li < G are real)
  if (li >= G) return;
  if (rv1 <= r0) {
    // every row of the split is past the context: an empty partial
    // (maximum -inf, sum 0), which the merge weighs by zero
#pragma unroll
    for (int t = 0; t < kDTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    l_run = 0.f;
  }
  if (nsplit == 1) {
    const float inv = 1.f / l_run;
#pragma unroll
    for (int t = 0; t < kDTiles; ++t)
      *reinterpret_cast<f32x4*>(orow + (size_t)li * kD + 16 * t + 4 * gq) = acc[t] * inv;
    return;
  }
  const size_t part_stride = partial_stride(G, kD);
  float* part = p.partials + ((size_t)uj * nsplit + sp) * part_stride;
#pragma unroll
  for (int t = 0; t < kDTiles; ++t)
    *reinterpret_cast<f32x4*>(part + (size_t)li * kD + 16 * t + 4 * gq) = acc[t];
  if (gq == 0) {
    part[G * kD + li] = m_run;
    part[G * kD + G + li] = l_run;
  }
}

}  // namespace

// Workgroups of the one-wave form that device `dev` holds at once, per
// grouped-query width (index log2 G), computed once per device.
constexpr int kMaxDevices = 64;
static std::mutex g_resident_mutex;
static int g_resident[kMaxDevices][4];

template <int G>
static hipError_t resident_workgroups(int* out) {
  constexpr int gi = G == 1 ? 0 : (G == 2 ? 1 : (G == 4 ? 2 : 3));
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_resident_mutex);
  if (g_resident[dev][gi] == 0) {
    int cus = 0, per_cu = 0;
    hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_split_kernel<G, false>,
                                                       kThreads, kBufs * kTileBytes);
    if (e != hipSuccess) return e;
    g_resident[dev][gi] = cus * per_cu > 0 ? cus * per_cu : 1;
  }
  *out = g_resident[dev][gi];
  return hipSuccess;
}

template <int G>
static hipError_t launch_g(const AttnParams& p0, hipStream_t s) {
  // one launch per query token: a row that several tokens select is fetched
  // by the first of them, and later tokens read it from the buffer
  const dim3 grid((unsigned)(p0.units * p0.nsplit));
  int resident = 0;
  hipError_t e = resident_workgroups<G>(&resident);
  if (e != hipSuccess) return e;
  // the two-wave gather-first form when the grid runs in several rounds of
  // resident workgroups (or when asked for)
  const bool gf = p0.gather_first != 0 || (int64_t)grid.x > resident;
  AttnParams p = p0;
  for (int j = 0; j < p0.T; ++j) {
    p.token = j;
    if (gf)
      hipLaunchKernelGGL((attn_split_kernel<G, true>), grid, dim3(2 * kThreads), kBufs * kTileBytes,
                         s, p);
    else
      hipLaunchKernelGGL((attn_split_kernel<G, false>), grid, dim3(kThreads), kBufs * kTileBytes, s,
                         p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_attn_split(const AttnParams& p, int G, hipStream_t s) {
  if (p.split_rows > kSplitRows || p.split_rows % kChunk != 0) return hipErrorInvalidValue;
  switch (G) {
    case 1: return launch_g<1>(p, s);
    case 2: return launch_g<2>(p, s);
    case 4: return launch_g<4>(p, s);
    case 8: return launch_g<8>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace avsg
