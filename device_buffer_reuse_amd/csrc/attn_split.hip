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
// gfx950 mapping (HBM-bound, VALU):
//  * A workgroup (4 waves) owns `split_rows` token rows of one (unit, token).
//    The rows stream through three 16 KiB LDS tiles of 32 rows (K half and V
//    half of a row, 512 bytes) by direct global-to-LDS copies, 16 bytes per
//    lane and 4 copies per lane per tile; two tiles are in flight while one
//    is used.  Every wave issues the same number of copies, so a vmcnt wait
//    with a constant count tells it that its share of the tile it needs has
//    landed, and one barrier per tile publishes the tile.
//  * Rows whose entry missed are copied from pinned host memory into the tile;
//    the lane that copied a piece then stores it from LDS into the entry's
//    slot, so the row crosses the host link once.  When the grid runs in
//    several rounds of resident workgroups, a workgroup instead first copies
//    all of its split's missed entries from host memory into their slots
//    (every host read in flight at once) and then streams only from HBM.
//  * Each wave owns 8 rows of every tile, 16 lanes per row (16 bytes of the K
//    half and of the V half each).  q.k uses v_dot2_f32_bf16 on bf16 pairs
//    (products exact, fp32 sums) and four DPP steps inside the 16-lane row;
//    p * v accumulates in fp32.
//  * Each wave keeps its own online softmax per head (the reference maximum
//    moves only when a tile exceeds it by 2^8, so the accumulators are
//    rescaled rarely); the four waves merge once at the end of the split, in
//    wave order, so a tile needs no barrier beyond the one for its copies.
//  * All LDS reads of the tiles are inline assembly with waits tied to their
//    results: the compiler would otherwise order every LDS read after all
//    outstanding global-to-LDS copies.
//  * Split partials (max, sum, o) go to the workspace and the combine kernel
//    merges them in split order, so the result does not depend on workgroup
//    timing.  (Merging inside the last workgroup of each (unit, token) needs
//    an agent-scope release in every workgroup, which writes back the XCD's
//    L2 each time and cost more than the extra launch.)
#include <type_traits>
#include <utility>

#include "avsg_internal.h"

namespace avsg {
namespace {

constexpr int kD = 128;                              // head dim of the split layout
constexpr int kTileRows = 32;                        // token rows per LDS tile
constexpr int kRowBytes = 4 * kD;                    // K half + V half
constexpr int kTileBytes = kTileRows * kRowBytes;    // 16 KiB
constexpr int kBufs = 3;                             // LDS tiles per workgroup
constexpr int kAhead = kBufs - 1;                    // tiles in flight beyond the one in use
static_assert(kAhead >= 1 && kAhead <= 3, "tile pipeline depth");
constexpr int kWaves = kAttnThreads / 64;            // 4
constexpr int kCopies = kTileBytes / 16 / kAttnThreads;  // 4 per lane per tile
constexpr int kSplitRows = 256;                      // token rows per workgroup

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// sum over the 16 lanes of a DPP row; every lane of the row gets the total
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return v;
}

// max / sum over the lanes l, l^16, l^32, l^48 (the four rows of a wave)
__device__ __forceinline__ float rows_max(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Butterfly reduction of G per-lane partial sums over the 16 lanes of a DPP
// row: at each of four levels a lane adds its partner's values for the half
// of its heads it keeps (partners c^8 by row_ror:8, c^7 by row_half_mirror,
// c^2 and c^1 by quad_perm; these span all 16 lanes).  Afterwards lane c
// holds the full sum of head c >> (4 - log2 G), on 16 / G lanes each.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float keep, float send) {
  return keep + __int_as_float(
                    __builtin_amdgcn_update_dpp(0, __float_as_int(send), CTRL, 0xF, 0xF, false));
}
template <int G>
__device__ __forceinline__ float head_reduce(const float (&d)[G], int c) {
  float v[G];
#pragma unroll
  for (int h = 0; h < G; ++h) v[h] = d[h];
  int n = G;
#pragma unroll
  for (int lvl = 0; lvl < 4; ++lvl) {
    const bool up = (c >> (3 - lvl)) & 1;
    const int half = n > 1 ? n / 2 : 1;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float keep = n > 1 ? (up ? v[half + i] : v[i]) : v[i];
      const float send = n > 1 ? (up ? v[i] : v[half + i]) : v[i];
      if (lvl == 0) v[i] = dpp_add<0x128>(keep, send);       // row_ror:8
      else if (lvl == 1) v[i] = dpp_add<0x141>(keep, send);  // row_half_mirror
      else if (lvl == 2) v[i] = dpp_add<0x4E>(keep, send);   // quad_perm [2,3,0,1]
      else v[i] = dpp_add<0xB1>(keep, send);                 // quad_perm [1,0,3,2]
    }
    n = half;
  }
  return v[0];
}
// Value of lane c - k * 16 / G (mod 16, by DPP row rotation): with head h on
// lanes h * 16 / G .., slot k of a lane sees head (own head - k) mod G.
template <int G, int K>
__device__ __forceinline__ float rot(float v) {
  if constexpr (K == 0) {
    return v;
  } else {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + K * (16 / G),
                                                      0xF, 0xF, false));
  }
}
template <int G, int K>
__device__ __forceinline__ int rot_i(int v) {
  if constexpr (K == 0) {
    return v;
  } else {
    return __builtin_amdgcn_update_dpp(0, v, 0x120 + K * (16 / G), 0xF, 0xF, false);
  }
}
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void*)p;
}
__device__ __forceinline__ void ds_b128(u32x4& d, uint32_t a) {
  asm volatile("ds_read_b128 %0, %1" : "=v"(d) : "v"(a));
}
__device__ __forceinline__ void ds_b64(int2& d, uint32_t a) {
  asm volatile("ds_read_b64 %0, %1" : "=v"(d) : "v"(a));
}
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int G>
__global__ __launch_bounds__(kAttnThreads) void attn_split_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t sTile[kBufs * kTileBytes];
  __shared__ int2 sRow[kSplitRows];   // per entry of the split: (slot, host id or -1)
  __shared__ int32_t sHost[kSplitRows];  // entries to fetch (gather-first)
  __shared__ int32_t sNHost;
  __shared__ float sMw[kWaves][G], sLw[kWaves][G];

  const int nsplit = p.nsplit;
  const int u = blockIdx.x / nsplit;
  const int sp = blockIdx.x - u * nsplit;
  const int j = p.token;
  const int uj = u * p.T + j;
  const int b = u / p.Hkv, g = u - b * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rg = lane >> 4, c = lane & 15;
  const int tpe = p.tpe;
  const int n_rows = p.k * tpe;
  const int r0 = sp * p.split_rows, r1 = min(r0 + p.split_rows, n_rows);
  float* orow = p.out + (((size_t)b * p.T + j) * p.Hq + g * G) * kD;
  if (p.unit_status[u] != 0) {
    if (nsplit == 1)
      for (int idx = tid; idx < G * kD; idx += kAttnThreads) orow[idx] = 0.f;
    return;
  }

  const int e0 = r0 / tpe, e1 = (r1 - 1) / tpe + 1;
  if (tid == 0) sNHost = 0;
  __syncthreads();
  for (int i0 = 0; i0 < e1 - e0; i0 += kAttnThreads) {
    const int i = i0 + tid;
    const size_t at = (size_t)uj * p.k + e0 + i;
    const bool in = i < e1 - e0;
    const bool fetch = in && p.fetch && p.fetch[at];
    if (in) sRow[i] = make_int2(p.sel_slot[at], fetch ? p.sel[at] : -1);
    if (p.gather_first) {
      // list the entries this split fetches (their order does not matter)
      const uint64_t m = __builtin_amdgcn_ballot_w64(fetch);
      int base = 0;
      if (lane == 0 && m) base = atomicAdd(&sNHost, __popcll(m));
      base = __shfl(base, 0, 64);
      if (fetch)
        sHost[base + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                               __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] = i;
    }
  }
  uint32_t qf[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 qq = *reinterpret_cast<const uint4*>(
        p.q + (((size_t)b * p.T + j) * p.Hq + g * G + h) * kD + c * 8);
    qf[h][0] = qq.x; qf[h][1] = qq.y; qf[h][2] = qq.z; qf[h][3] = qq.w;
  }
  __syncthreads();
  // the queries are in registers before any copy is issued
#pragma unroll
  for (int h = 0; h < G; ++h)
    asm volatile("" : "+v"(qf[h][0]), "+v"(qf[h][1]), "+v"(qf[h][2]), "+v"(qf[h][3]));

  uint16_t* ubase = p.buf_kv + (size_t)u * p.S * p.row_elems;
  const uint16_t* hbase = p.host_kv + (size_t)u * p.N * p.row_elems;
  const int v_off = tpe * kD;  // elements from an entry's K rows to its V rows
  const uint32_t row_lds = lds_addr(sRow);
  const uint32_t tile_lds = lds_addr(sTile);

  // Gather-first: the split's missed entries go from pinned host memory into
  // their slots before any tile, all of the workgroup's host reads in flight
  // together (8 16-byte pieces per lane per round), and the tiles then read
  // them from HBM.  Chosen when the grid runs in several rounds of resident
  // workgroups: the host latency is then paid once per workgroup.
  if (p.gather_first) {
    const int pe = p.row_elems >> 3;  // 16-byte pieces per entry
    const int total = sNHost * pe;
    for (int q0 = 0; q0 < total; q0 += 8 * kAttnThreads) {
      u32x4 v[8];
#pragma unroll
      for (int bq = 0; bq < 8; ++bq) {
        const int q = q0 + bq * kAttnThreads + tid;
        if (q < total) {
          const int k = q / pe, col = q - k * pe;
          v[bq] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
              hbase + (size_t)(uint32_t)sRow[sHost[k]].y * p.row_elems + col * 8));
        }
      }
#pragma unroll
      for (int bq = 0; bq < 8; ++bq) {
        const int q = q0 + bq * kAttnThreads + tid;
        if (q < total) {
          const int k = q / pe, col = q - k * pe;
          *reinterpret_cast<u32x4*>(ubase + (size_t)(uint32_t)sRow[sHost[k]].x * p.row_elems +
                                    col * 8) = v[bq];
        }
      }
    }
    __syncthreads();  // every read of sRow above is done
    for (int k = tid; k < sNHost; k += kAttnThreads) sRow[sHost[k]].y = -1;
    // the stores are in L2 before any wave copies those rows into LDS
    vm_wait<0>();
    __syncthreads();
  }

  // This lane's copies of a tile: copy x is row 8w + 2x + lane/32 of the
  // tile, half (K or V) (lane/16)%2, 16-byte column lane%16; instruction
  // w*kCopies + x fills bytes [1024 (w*kCopies + x), +1024) of the tile.
  // Entry of a row: r itself for token entries, else r / tpe by an exact
  // multiply-high with ceil(2^32 / tpe) (exact while r * tpe < 2^32).
  const uint32_t tpe_magic = tpe == 1 ? 0u : (uint32_t)((0x100000000ull + tpe - 1) / tpe);
  auto entry_of = [&](int r) -> int {
    return tpe == 1 ? r : (int)__umulhi((uint32_t)r, tpe_magic);
  };
  const int row_base = 8 * w + (lane >> 5);
  const int wu = __builtin_amdgcn_readfirstlane(w);  // the wave index, in a scalar register
  const int copy_off = ((lane >> 4) & 1) * v_off + (lane & 15) * 8;  // elements
  // Copies tile t into buffer `buf`; rows past the split repeat its last row
  // (their scores are masked) so every wave issues exactly kCopies copies.
  // Returns the copies whose row came from host memory (bit x).
  auto stage = [&](int t, int buf) -> uint32_t {
    int2 ri[kCopies];
    int ent[kCopies];
    const int rt = r0 + t * kTileRows + row_base;
#pragma unroll
    for (int x = 0; x < kCopies; ++x) {
      const int r = min(rt + 2 * x, r1 - 1);
      ent[x] = entry_of(r);
      ds_b64(ri[x], row_lds + 8 * (ent[x] - e0));
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int x = 0; x < kCopies; ++x) asm volatile("" : "+v"(ri[x]));
    uint32_t fetched = 0;
    uint8_t* tile = sTile + buf * kTileBytes;
#pragma unroll
    for (int x = 0; x < kCopies; ++x) {
      const int r = min(rt + 2 * x, r1 - 1);
      const uint32_t off = (uint32_t)((r - ent[x] * tpe) * kD + copy_off);
      const bool host = ri[x].y >= 0;
      const uint16_t* base = host ? hbase : ubase;
      const uint32_t idx = (uint32_t)(host ? ri[x].y : ri[x].x);
      // one 32 x 32 -> 64-bit multiply per copy
      const uint16_t* src = base + (uint64_t)idx * (uint32_t)p.row_elems + off;
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(tile + (wu * kCopies + x) * 1024), 16, 0,
                                       0);
      if (host && rt + 2 * x < r1) fetched |= 1u << x;
    }
    return fetched;
  };
  // Stores this lane's host-fetched pieces of tile t from LDS into their slots.
  auto write_back = [&](int t, int buf, uint32_t fetched) {
    if (!__builtin_amdgcn_ballot_w64(fetched != 0)) return;
    const int rt = r0 + t * kTileRows + row_base;
    int2 ri[kCopies];
    u32x4 d[kCopies];
#pragma unroll
    for (int x = 0; x < kCopies; ++x) {
      const int r = min(rt + 2 * x, r1 - 1);
      ds_b64(ri[x], row_lds + 8 * (entry_of(r) - e0));
      ds_b128(d[x], tile_lds + buf * kTileBytes + (w * kCopies + x) * 1024 + lane * 16);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int x = 0; x < kCopies; ++x) asm volatile("" : "+v"(ri[x]), "+v"(d[x]));
#pragma unroll
    for (int x = 0; x < kCopies; ++x) {
      if (fetched & (1u << x)) {
        const int r = rt + 2 * x;
        const int e = entry_of(r);
        const uint32_t off = (uint32_t)((r - e * tpe) * kD + copy_off);
        *reinterpret_cast<u32x4*>(ubase + (size_t)(uint32_t)ri[x].x * p.row_elems + off) = d[x];
      }
    }
  };

  // o[k]: dims c*8 .. c*8+7 of head (hl - k) mod G, hl = this lane's head;
  // m_run, l_run: the online softmax of head hl over this lane's rows
  const int hl = c / (16 / G);
  float o[G][8];
  float m_run = -INFINITY, l_run = 0.f;
#pragma unroll
  for (int k = 0; k < G; ++k)
#pragma unroll
    for (int x = 0; x < 8; ++x) o[k][x] = 0.f;

  const int ntiles = (r1 - r0 + kTileRows - 1) / kTileRows;
  // fmask[i]: this lane's host-fetched copies of tile t + i
  uint32_t fmask[kAhead];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) fmask[i] = i < ntiles ? stage(i, i) : 0u;
  // this lane's two rows of a tile: 8w + rg and 8w + 4 + rg
  const uint32_t lane_off = (8 * w + rg) * kRowBytes + c * 16;

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t % kBufs;
    // tile t has landed once only the copies of the later tiles in flight
    // (kCopies each) may still be outstanding
    const int later = min(kAhead - 1, ntiles - 1 - t);
    if (later <= 0) vm_wait<0>();
    else if (later == 1) vm_wait<kCopies>();
    else vm_wait<2 * kCopies>();
    asm volatile("s_barrier" ::: "memory");  // tile t in LDS; tile t-1's buffer free
    const uint32_t f_now = fmask[0];
#pragma unroll
    for (int i = 0; i + 1 < kAhead; ++i) fmask[i] = fmask[i + 1];
    fmask[kAhead - 1] = t + kAhead < ntiles ? stage(t + kAhead, (t + kAhead) % kBufs) : 0u;
    // slot stores of tile t's host rows, issued after the copies of tile
    // t + kAhead: the next tile's wait (its copies are older) does not wait
    // for them
    write_back(t, buf, f_now);

    const uint32_t a = tile_lds + buf * kTileBytes + lane_off;
    u32x4 k0, k1, v0, v1;
    ds_b128(k0, a);
    ds_b128(k1, a + 4 * kRowBytes);
    ds_b128(v0, a + 2 * kD);
    ds_b128(v1, a + 4 * kRowBytes + 2 * kD);
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(k0), "+v"(k1), "+v"(v0), "+v"(v1));

    const int ra = r0 + t * kTileRows + 8 * w + rg, rb = ra + 4;
    const float va[8] = {bf_lo(v0.x), bf_hi(v0.x), bf_lo(v0.y), bf_hi(v0.y),
                         bf_lo(v0.z), bf_hi(v0.z), bf_lo(v0.w), bf_hi(v0.w)};
    const float vb[8] = {bf_lo(v1.x), bf_hi(v1.x), bf_lo(v1.y), bf_hi(v1.y),
                         bf_lo(v1.z), bf_hi(v1.z), bf_lo(v1.w), bf_hi(v1.w)};
    float da[G], db[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float x0 = dot2(qf[h][0], k0.x, 0.f);
      x0 = dot2(qf[h][1], k0.y, x0);
      x0 = dot2(qf[h][2], k0.z, x0);
      da[h] = dot2(qf[h][3], k0.w, x0);
      float x1 = dot2(qf[h][0], k1.x, 0.f);
      x1 = dot2(qf[h][1], k1.y, x1);
      x1 = dot2(qf[h][2], k1.z, x1);
      db[h] = dot2(qf[h][3], k1.w, x1);
    }
    // scores of head hl for rows a and b; rows past the split hold a copy
    // of its last row and are masked here
    float sa = head_reduce<G>(da, c) * p.scale_log2e;
    float sb = head_reduce<G>(db, c) * p.scale_log2e;
    sa = ra < r1 ? sa : -INFINITY;
    sb = rb < r1 ? sb : -INFINITY;
    const float cm = rows_max(fmaxf(sa, sb));
    const bool move = cm > m_run + 8.f;
    if (__builtin_amdgcn_ballot_w64(move)) {
      const float corr = move ? __builtin_amdgcn_exp2f(m_run - cm) : 1.f;  // 0 on a first move
      m_run = move ? cm : m_run;
      l_run *= corr;
      static_for<0, G>([&](auto k_) {
        constexpr int k = decltype(k_)::value;
        const float ck = rot<G, k>(corr);
#pragma unroll
        for (int x = 0; x < 8; ++x) o[k][x] *= ck;
      });
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;  // no valid row yet
    const float pa = __builtin_amdgcn_exp2f(sa - m_use);
    const float pb = __builtin_amdgcn_exp2f(sb - m_use);
    l_run += pa + pb;
    static_for<0, G>([&](auto k_) {
      constexpr int k = decltype(k_)::value;
      const float pak = rot<G, k>(pa), pbk = rot<G, k>(pb);
#pragma unroll
      for (int x = 0; x < 8; ++x) o[k][x] = fmaf(pbk, vb[x], fmaf(pak, va[x], o[k][x]));
    });
  }

  // merge the four row groups of the wave, then the four waves (in order)
  float* sO = reinterpret_cast<float*>(sTile + (ntiles % kBufs) * kTileBytes);  // [4][G][kD]
  const float l = rows_sum(l_run);
  static_for<0, G>([&](auto k_) {
    constexpr int k = decltype(k_)::value;
    const int hk = rot_i<G, k>(hl);
#pragma unroll
    for (int x = 0; x < 8; ++x) o[k][x] = rows_sum(o[k][x]);
    if (rg == 0) {
      *reinterpret_cast<float4*>(sO + (w * G + hk) * kD + c * 8) =
          make_float4(o[k][0], o[k][1], o[k][2], o[k][3]);
      *reinterpret_cast<float4*>(sO + (w * G + hk) * kD + c * 8 + 4) =
          make_float4(o[k][4], o[k][5], o[k][6], o[k][7]);
    }
  });
  if (rg == 0 && (c & (16 / G - 1)) == 0) {
    sMw[w][hl] = m_run;
    sLw[w][hl] = l;
  }
  __syncthreads();
  const size_t part_stride = partial_stride(G, kD);
  float* part = p.partials + ((size_t)uj * nsplit + sp) * part_stride;
  for (int idx = tid; idx < G * kD; idx += kAttnThreads) {
    const int h = idx / kD, d = idx - h * kD;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, sMw[v][h]);
    float O = 0.f, L = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const float f = sMw[v][h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sMw[v][h] - M);
      O = fmaf(f, sO[(v * G + h) * kD + d], O);
      L = fmaf(f, sLw[v][h], L);
    }
    if (nsplit == 1) {
      orow[idx] = O / L;
    } else {
      part[idx] = O;
      if (d == 0) {
        part[G * kD + h] = M;
        part[G * kD + G + h] = L;
      }
    }
  }
}

}  // namespace

template <int G>
static hipError_t launch_g(const AttnParams& p0, hipStream_t s) {
  // one launch per query token: a row that several tokens select is fetched
  // by the first of them, and later tokens read it from the buffer
  const dim3 grid((unsigned)(p0.units * p0.nsplit));
  static int resident = 0;  // workgroups the device holds at once
  if (resident == 0) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_split_kernel<G>, kAttnThreads,
                                                     0) != hipSuccess)
      return hipErrorUnknown;
    resident = cus * per_cu;
  }
  AttnParams p = p0;
  if ((int64_t)grid.x > resident) p.gather_first = 1;
  for (int j = 0; j < p0.T; ++j) {
    p.token = j;
    hipLaunchKernelGGL(attn_split_kernel<G>, grid, dim3(kAttnThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.nsplit == 1) return hipSuccess;
  return launch_attn_combine(p0, G, kD, s);
}

hipError_t launch_attn_split(const AttnParams& p, int G, hipStream_t s) {
  if (p.split_rows != kSplitRows) return hipErrorInvalidValue;
  switch (G) {
    case 1: return launch_g<1>(p, s);
    case 2: return launch_g<2>(p, s);
    case 4: return launch_g<4>(p, s);
    case 8: return launch_g<8>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace avsg
