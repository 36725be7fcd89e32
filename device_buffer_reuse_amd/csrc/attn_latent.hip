// K3m: split-k decode attention for the latent layout (one shared 576-wide
// latent row per token, 64 or 128 query heads), on MFMA.
//
// What it computes: for each request and query head h, softmax(scale * q_h
// K^T) V over exactly the selected tokens, where a selected token's row is
// the key (576 values) and its first 512 values are the value.  With many
// heads sharing each row, QK^T [H x 576] x [576 x n] and PV [H x n] x
// [n x 512] are real contractions, so they run on v_mfma_f32_16x16x32_bf16.
//
// gfx950 mapping:
//  * A workgroup of Hq/16 waves owns `split_rows` selected tokens of one
//    request; each wave owns 16 heads (their queries stay in 72 registers,
//    their 16 x 512 accumulators in 128).
//  * Rows are staged through three LDS tiles of 32 rows by direct
//    global-to-LDS loads, 16 bytes per lane, with no staging registers.
//    Rows are padded to 1184 bytes and 16-byte piece c of tile row r sits
//    at position c ^ swz(r), swz(r) = bit 2 of r xor bit 3 of r: with the 64
//    four-byte LDS banks of gfx950 (and with 32) both operand reads are then
//    free of bank conflicts (the K read, 16 rows x 16 bytes per 16 lanes,
//    and the transposing V read, 8 rows x 32 bytes per 32 lanes).  swz
//    depends on row bits 0..3 only, so rows r and r + 16 share it and the
//    second half of a tile is reached by a constant offset.  Two chunks are in flight while one is multiplied; each wave
//    issues the same number of copies per chunk, so a vmcnt wait with a
//    constant count tells it that its copies of the chunk it needs have
//    landed, and one barrier per chunk makes everybody's copies visible.
//  * Missed rows (fetch flag set by the matching kernel) are copied from
//    pinned host memory into the tile; the wave that copied a piece then
//    stores it from LDS into its slot, so a row crosses the host link once.
//  * All LDS reads in the loop are inline assembly with waits tied to their
//    results: the compiler would otherwise order every LDS read after all
//    outstanding global-to-LDS copies.  K operands and V^T operands are read
//    one step ahead of the MFMAs that use them.
//  * Scores are computed transposed, S^T = K Q^T (M = 16 tokens, N = 16
//    heads, K = 576).  In that result layout each lane owns one head's
//    column, so the online softmax reduces over 4 lanes with the gfx950 lane
//    swaps (v_permlane16_swap, v_permlane32_swap), and the probabilities are
//    already the B operand of O^T = V^T P^T.  V^T operands come from
//    ds_read_b64_tr_b16, the transposing LDS read (lane i of each 16-lane
//    group receives element i%4 of the 4 halfwords that lane 4r + i/4
//    addressed, r = 0..3), so V is never transposed in memory.
//  * P is split into bf16 hi + lo parts (two MFMAs on the same V fragment):
//    rounding P to bf16 alone would leave about 1e-3 relative error.
//  * The reference maximum of the online softmax moves only when a chunk
//    exceeds it by 2^8, so the accumulators are rescaled rarely; the result
//    does not depend on the reference chosen.
//  * Split partials are merged by the combine kernel: each holds the split's
//    output normalized by its own sum, as fp16 (half the bytes of fp32; the
//    normalized values are convex combinations of value rows, bounded by
//    them, and fp16 rounding adds about 1.5e-4 relative L1 to the merged
//    output, against the 1e-3 tolerance), with the split's maximum and sum
//    in fp32.
#include <type_traits>
#include <utility>

#include "avsg_internal.h"

namespace avsg {
namespace {

constexpr int kDqk = 576, kDv = 512;
constexpr int kChunk = 32;                       // tokens per LDS tile
constexpr int kRow = kDqk + 16;                  // bf16 per padded LDS row (1184 B)
constexpr int kRowBytes = 2 * kRow;
constexpr int kRowPieces = kRow / 8;             // 74 16-byte pieces per padded row
constexpr int kPiecesPerRow = kDqk / 8;          // 72 of them carry data
constexpr int kTilePieces = kChunk * kRowPieces; // 2368
constexpr int kTileInstr = (kTilePieces + 63) / 64;  // 37 wave-wide copies per tile
constexpr int kTileElems = kChunk * kRow;
constexpr int kKSteps = kDqk / 32;               // 18 MFMA k-steps for QK^T
constexpr int kMTiles = kDv / 16;                // 32 output tiles per wave
constexpr int kBufs = 3;                         // LDS tiles
constexpr int kAhead = kBufs - 1;                // chunks in flight beyond the one in use
static_assert(kAhead >= 1 && kAhead <= 3, "chunk pipeline depth");
constexpr int kMaxSplit = 512;

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

// position offset (xor) of the pieces of tile row r: bit 2 of r xor bit 3
__device__ __forceinline__ int swz(int r) { return ((r >> 2) ^ (r >> 3)) & 1; }

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
// LDS wait that the compiler sees as producing the tied registers
template <int N, class A, class B>
__device__ __forceinline__ void lgkm_wait(A& a, B& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N));
}
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

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

template <int NW>
__global__ __launch_bounds__(NW * 64) void attn_latent_kernel(AttnParams p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t sTile[];  // [kBufs][kChunk][kRow]
  __shared__ int2 sRow[kMaxSplit];  // (slot, id to fetch from host or -1)
  constexpr int kThreads = NW * 64;
  constexpr int G = NW * 16;  // query heads
  constexpr int kInstr = (kTileInstr + NW - 1) / NW;     // copies per chunk, first waves
  constexpr int kFull = kTileInstr - (kInstr - 1) * NW;  // waves issuing kInstr copies

  // the context's step counter advances once per step, here: the match
  // kernel that read it has finished (a non-returning atomic: no wait)
  if (p.step && p.token == 0 && blockIdx.x == 0 && threadIdx.x == 0)
    __hip_atomic_fetch_add(p.step, (int64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int nsplit = p.nsplit;
  // workgroups are dealt to the 8 XCDs in turn; when the grid divides by 8,
  // XCD x takes the x-th eighth of the (request, split) range, so a
  // request's splits, and later its combine, share one L2
  const int nb = (int)gridDim.x;
  const int bid = (nb & 7) == 0 ? (int)(blockIdx.x & 7) * (nb >> 3) + (int)(blockIdx.x >> 3)
                                : (int)blockIdx.x;
  const int u = bid / nsplit;
  const int sp = bid - u * nsplit;
  const int j = p.token;
  const int uj = u * p.T + j;
  const int b = u;  // one latent head per request
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  // a shortened list (length array): its first sel_len[u][j] entries (clamped
  // into [1, k]; a unit with an invalid length has failed and is zeroed)
  const int len = p.sel_len ? min(max(p.sel_len[uj], 1), p.k) : p.k;
  const int e0 = sp * p.split_rows, e1 = min(e0 + p.split_rows, len);
  if (e0 >= e1) return;  // a split past the list's end (merged as empty)
  const int ne = e1 - e0;
  // (recomputed where it is written: kept live across the chunk loop it
  // would take a register the loop needs)
  auto out_rows = [&]() { return p.out + ((size_t)b * p.T + j) * p.Hq * kDv; };
  if (p.unit_status[u] != 0) {
    if (nsplit == 1)
      for (int idx = tid; idx < G * kDv; idx += kThreads) out_rows()[idx] = 0.f;
    return;
  }
  for (int i = tid; i < ne; i += kThreads) {
    const size_t at = (size_t)uj * p.k + e0 + i;
    // host row of a fetched entry: its id (flat host KV) or its pool row
    sRow[i] = make_int2(p.sel_slot[at],
                        (p.fetch && p.fetch[at]) ? (p.host_row ? p.host_row : p.sel)[at] : -1);
  }
  // this lane's Q operand: head w*16 + li, dims 32*ks + 8*g .. +8
  bf16x8 qf[kKSteps];
  {
    const uint16_t* qrow = p.q + (((size_t)b * p.T + j) * p.Hq + w * 16 + li) * kDqk + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
  }
  __syncthreads();
  // the queries are in registers before any copy is issued
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) asm volatile("" : "+v"(qf[ks]));

  // this lane's piece of copy x: row << 8 | column, -1 for padding.  The lane
  // index passes through an empty asm so that the pieces are recomputed per
  // chunk instead of being held (or spilled) across the loop.
  auto piece = [&](int x) -> int {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int n = w + x * NW;
    const int P = n * 64 + ln;
    const int r = P / kRowPieces, col = P - r * kRowPieces;
    return (n < kTileInstr && P < kTilePieces && col < kPiecesPerRow) ? (r << 8 | col) : -1;
  };
  uint16_t* ubase = p.buf_kv + (size_t)u * p.S * kDqk;
  const uint16_t* hbase = p.host_kv + (p.host_row ? 0 : (size_t)u * p.N * kDqk);
  const uint32_t row_lds = lds_addr(sRow);
  const uint32_t tile_lds = lds_addr(sTile);

  // Copies chunk c into tile `buf`.  Rows past the split repeat the split's
  // last row (their scores are masked), so every wave issues exactly its
  // kInstr or kInstr-1 copies.  Returns the copies whose row came from host
  // memory (bit x), which the wave later stores into the rows' slots.
  auto stage = [&](int c, int buf) -> uint32_t {
    int2 ri[kInstr];
    int rc[kInstr];
#pragma unroll
    for (int x = 0; x < kInstr; ++x) {
      rc[x] = piece(x);
      const int e = min(c * kChunk + (rc[x] < 0 ? 0 : rc[x] >> 8), ne - 1);
      ds_b64(ri[x], row_lds + 8 * e);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int x = 0; x < kInstr; ++x) asm volatile("" : "+v"(ri[x]));
    uint32_t fetched = 0;
    uint16_t* tile = sTile + buf * kTileElems;
#pragma unroll
    for (int x = 0; x < kInstr; ++x) {
      const int n = w + x * NW;
      if (n < kTileInstr) {  // wave-uniform
        const int r = rc[x] >> 8, col = (rc[x] & 255) ^ swz(rc[x] >> 8);  // the row's piece
        const bool host = ri[x].y >= 0;
        const uint16_t* src = host ? hbase + (size_t)ri[x].y * kDqk + col * 8
                                   : ubase + (size_t)ri[x].x * kDqk + col * 8;
        if (rc[x] >= 0) {
          __builtin_amdgcn_global_load_lds(src, (lds_void*)(tile + n * 512), 16, 0, 0);
          if (host && c * kChunk + r < ne) fetched |= 1u << x;
        }
      }
    }
    return fetched;
  };
  // Stores this wave's host-fetched pieces of chunk c from LDS into their slots.
  auto write_back = [&](int c, int buf, uint32_t fetched) {
    if (!__builtin_amdgcn_ballot_w64(fetched != 0)) return;
    int2 ri[kInstr];
    u32x4 d[kInstr];
    int rc[kInstr];
#pragma unroll
    for (int x = 0; x < kInstr; ++x) {
      rc[x] = piece(x);
      const int n = w + x * NW;
      const int e = min(c * kChunk + (rc[x] < 0 ? 0 : rc[x] >> 8), ne - 1);
      ds_b64(ri[x], row_lds + 8 * e);
      const int nn = n < kTileInstr ? n : 0;
      ds_b128<0>(d[x], tile_lds + buf * kTileElems * 2 + nn * 1024 + lane * 16);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int x = 0; x < kInstr; ++x) asm volatile("" : "+v"(ri[x]), "+v"(d[x]));
#pragma unroll
    for (int x = 0; x < kInstr; ++x) {
      if (fetched & (1u << x)) {
        const int col = (rc[x] & 255) ^ swz(rc[x] >> 8);
        *reinterpret_cast<u32x4*>(ubase + (size_t)ri[x].x * kDqk + col * 8) = d[x];
      }
    }
  };

  f32x4 acc[kMTiles];
#pragma unroll
  for (int t = 0; t < kMTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int nchunks = (ne + kChunk - 1) / kChunk;
  // fmask[i]: this wave's host-fetched copies of chunk c + i
  uint32_t fmask[kAhead];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) fmask[i] = i < nchunks ? stage(i, i) : 0u;
  // per-lane operand addresses within a tile
  // K: row li, piece 4 ks + g.  V^T: row 4g + li/4, bytes 8 (li & 3) of the
  // group's first 32 bytes (pieces 0, 1) and of its last 32 (pieces 2, 3)
  const uint32_t k_off = li * kRowBytes + 16 * (g ^ swz(li));
  const int vr_row = 4 * g + (li >> 2);
  const uint32_t v_off0 = vr_row * kRowBytes + 16 * (((li & 3) >> 1) ^ swz(vr_row)) + 8 * (li & 1);
  const uint32_t v_off1 = vr_row * kRowBytes + 16 * ((((li & 3) >> 1) | 2) ^ swz(vr_row)) + 8 * (li & 1);

  for (int c = 0; c < nchunks; ++c) {
    const int buf = c % kBufs;
    // chunk c has landed once only this wave's copies of the later chunks in
    // flight (kInstr or kInstr - 1 each) may still be outstanding
    const int later = min(kAhead - 1, nchunks - 1 - c);
    if (later <= 0) {
      vm_wait<0>();
    } else if (later == 1) {
      if (w < kFull) vm_wait<kInstr>();
      else vm_wait<kInstr - 1>();
    } else {
      if (w < kFull) vm_wait<2 * kInstr>();
      else vm_wait<2 * (kInstr - 1)>();
    }
    block_barrier();  // chunk c is in LDS; nobody reads chunk c-1's tile any more
    const uint32_t f_now = fmask[0];
#pragma unroll
    for (int i = 0; i + 1 < kAhead; ++i) fmask[i] = fmask[i + 1];
    fmask[kAhead - 1] = c + kAhead < nchunks ? stage(c + kAhead, (c + kAhead) % kBufs) : 0u;
    // slot stores of chunk c's host rows, issued after the copies of chunk
    // c + kAhead: the next chunk's wait (its copies are older) does not wait
    // for them
    write_back(c, buf, f_now);

    // S^T = K Q^T for tokens 0..15 and 16..31 of the chunk, this wave's heads
    const uint32_t ka = tile_lds + buf * kTileElems * 2 + k_off;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
    u32x4 kf0[2], kf1[2];
    ds_b128<0>(kf0[0], ka);
    ds_b128<16 * kRowBytes>(kf1[0], ka);
    ds_b128<64>(kf0[1], ka);
    ds_b128<64 + 16 * kRowBytes>(kf1[1], ka);
    static_for<0, kKSteps>([&](auto ks_) {
      constexpr int ks = decltype(ks_)::value, st = ks & 1;
      if constexpr (ks + 1 < kKSteps) lgkm_wait<2>(kf0[st], kf1[st]);
      else lgkm_wait<0>(kf0[st], kf1[st]);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf0[st]), qf[ks], s0,
                                                   0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf1[st]), qf[ks], s1,
                                                   0, 0, 0);
      if constexpr (ks + 2 < kKSteps) {
        ds_b128<64 * (ks + 2)>(kf0[st], ka);
        ds_b128<64 * (ks + 2) + 16 * kRowBytes>(kf1[st], ka);
      }
    });

    // lane owns head li: tokens 4g+i (s0) and 16+4g+i (s1) of the chunk
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t0 = c * kChunk + 4 * g + i, t1 = t0 + 16;
      sv[i] = t0 < ne ? s0[i] * p.scale_log2e : -INFINITY;
      sv[4 + i] = t1 < ne ? s1[i] * p.scale_log2e : -INFINITY;
    }
    float cm = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) cm = fmaxf(cm, sv[i]);
    cm = col_max(cm);
    const bool move = cm > m_run + 8.f;
    const float m_new = move ? cm : m_run;
    const float corr = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first chunk
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
      for (int t = 0; t < kMTiles; ++t) acc[t] *= corr;
    }

    const uint32_t va0 = tile_lds + buf * kTileElems * 2 + v_off0;
    const uint32_t va1 = tile_lds + buf * kTileElems * 2 + v_off1;
    u32x2 vr[2][4];
    ds_tr<0>(vr[0][0], va0);
    ds_tr<16 * kRowBytes>(vr[0][1], va0);
    ds_tr<0>(vr[0][2], va1);
    ds_tr<16 * kRowBytes>(vr[0][3], va1);
    // O^T += V^T P^T, output tiles in pairs.  k slot 8g+r is token 4g+r for
    // r < 4 and 16+4g+(r-4) otherwise, matching the probabilities above.
    static_for<0, kMTiles / 2>([&](auto pr_) {
      constexpr int pr = decltype(pr_)::value, st = pr & 1;
      if constexpr (pr + 1 < kMTiles / 2) {
        constexpr int o = 64 * (pr + 1);
        ds_tr<o>(vr[st ^ 1][0], va0);
        ds_tr<o + 16 * kRowBytes>(vr[st ^ 1][1], va0);
        ds_tr<o>(vr[st ^ 1][2], va1);
        ds_tr<o + 16 * kRowBytes>(vr[st ^ 1][3], va1);
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
  }

  // lane holds O[h = w*16 + li][d = 16t + 4g + i]
  // (from a fresh thread index: a value kept from before the chunk loop
  // would occupy a register through it)
  int tid_end = (int)threadIdx.x;
  asm volatile("" : "+v"(tid_end));
  const int h = (tid_end >> 6) * 16 + (tid_end & 15);
  if (nsplit == 1) {
    const float inv = 1.f / l_run;
#pragma unroll
    for (int t = 0; t < kMTiles; ++t)
      *reinterpret_cast<f32x4*>(out_rows() + (size_t)h * kDv + 16 * t + 4 * g) = acc[t] * inv;
    return;
  }
  uint8_t* part = reinterpret_cast<uint8_t*>(p.partials) +
                  ((size_t)uj * nsplit + sp) * latent_partial_bytes(G, kDv);
  _Float16* po = reinterpret_cast<_Float16*>(part);
  float* pm = reinterpret_cast<float*>(part + (size_t)G * kDv * 2);
  const float inv = 1.f / l_run;
#pragma unroll
  for (int t = 0; t < kMTiles; ++t) {
    const f32x4 v = acc[t] * inv;
    typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
    const f16x4 hv = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    *reinterpret_cast<f16x4*>(po + (size_t)h * kDv + 16 * t + 4 * g) = hv;
  }
  if (g == 0) {
    pm[h] = m_run;
    pm[G + h] = l_run;
  }
}

}  // namespace

size_t attn_latent_lds() { return sizeof(uint16_t) * kBufs * kTileElems; }

hipError_t launch_attn_latent(const AttnParams& p0, int dqk, int dv, hipStream_t s) {
  if (dqk != kDqk || dv != kDv || p0.split_rows % kChunk != 0 || p0.split_rows > kMaxSplit)
    return hipErrorInvalidValue;
  const size_t lds = attn_latent_lds();
  const dim3 grid((unsigned)(p0.units * p0.nsplit));
  AttnParams p = p0;
  for (int j = 0; j < p0.T; ++j) {
    p.token = j;
    if (p.Hq == 128) {
      hipLaunchKernelGGL(attn_latent_kernel<8>, grid, dim3(512), lds, s, p);
    } else if (p.Hq == 64) {
      hipLaunchKernelGGL(attn_latent_kernel<4>, grid, dim3(256), lds, s, p);
    } else {
      return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t attn_latent_set_lds() {
  const int lds = (int)attn_latent_lds();
  hipError_t e = hipFuncSetAttribute((const void*)attn_latent_kernel<8>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute((const void*)attn_latent_kernel<4>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, lds);
}

}  // namespace avsg
