// K3m: split-k decode attention for the latent layout (one shared 576-wide
// latent row per token, 128 query heads), on MFMA.
//
// What it computes: for each request and query head h, softmax(scale * q_h
// K^T) V over exactly the selected tokens, where a selected token's row is
// the key (576 values) and its first 512 values are the value.  With 128
// heads sharing each row, QK^T [128 x 576] x [576 x n] and PV [128 x n] x
// [n x 512] are real contractions, so they run on v_mfma_f32_16x16x32_bf16.
//
// gfx950 mapping:
//  * A workgroup of Hq/16 waves owns `split_rows` selected tokens of one
//    request; each wave owns 16 heads.  The tokens' rows are staged through
//    LDS in chunks of 32 (double buffered, rows padded to 1168 bytes so the
//    16 rows an MFMA operand reads fall in distinct banks); the loads of the
//    next chunk are in flight while the current one is multiplied.
//  * Scores are computed transposed, S^T = K Q^T (M = 16 tokens, N = 16
//    heads, K = 576): the K operand is a plain 16-byte LDS read of a row and
//    the Q operand stays in registers for the whole split.  In the result
//    layout each lane owns one head's column, so the online softmax needs only
//    two cross-lane steps, and the probabilities are already laid out as the B
//    operand of O^T = V^T P^T.
//  * V^T operands come from ds_read_b64_tr_b16, the transposing LDS read, so V
//    is never transposed in memory.
//  * P is split into bf16 hi + lo parts (two MFMAs on the same V fragment):
//    rounding P to bf16 alone would leave about 1e-3 relative error.
//  * Missed rows are read from pinned host memory while staging and stored
//    into their slot (fused transfer), as in the split-layout kernel.
//  * Split partials (max, sum, o) are merged by the combine kernel.
#include "avsg_internal.h"

namespace avsg {
namespace {

constexpr int kDqk = 576, kDv = 512;
constexpr int kChunk = 32;                  // tokens per LDS tile
constexpr int kRow = kDqk + 8;              // bf16 per padded LDS row (1168 B)
constexpr int kKSteps = kDqk / 32;          // 18 MFMA k-steps for QK^T
constexpr int kMTiles = kDv / 16;           // 32 output tiles per wave
constexpr int kPiecesPerRow = kDqk / 8;     // 72 16-byte pieces
constexpr int kPieces = kChunk * kPiecesPerRow;
constexpr int kMaxSplit = 512;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ bf16x8 lds_row8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// V^T fragment of 8 tokens (k slots) x 16 dims (m) for the A operand
__device__ __forceinline__ bf16x8 lds_vt(const uint16_t* p0, const uint16_t* p1) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
  const s16x4 v[2] = {a, b};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float xor_max(float v, int m) { return fmaxf(v, __shfl_xor(v, m, 64)); }

template <int NW>
__global__ __launch_bounds__(NW * 64) void attn_latent_kernel(AttnParams p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t sKV[];  // [2][kChunk][kRow]
  __shared__ int32_t sSlot[kMaxSplit];
  __shared__ int32_t sSrc[kMaxSplit];
  constexpr int kThreads = NW * 64;
  constexpr int G = NW * 16;  // query heads

  const int nsplit = p.nsplit;
  const int u = blockIdx.x / nsplit;
  const int sp = blockIdx.x - u * nsplit;
  const int j = p.token;
  const int uj = u * p.T + j;
  const int b = u;  // one latent head per request
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int e0 = sp * p.split_rows, e1 = min(e0 + p.split_rows, p.k);
  const int ne = e1 - e0;
  float* orow = p.out + ((size_t)b * p.T + j) * p.Hq * kDv;
  if (p.unit_status[u] != 0) {
    if (nsplit == 1)
      for (int idx = tid; idx < G * kDv; idx += kThreads) orow[idx] = 0.f;
    return;
  }
  for (int i = tid; i < ne; i += kThreads) {
    const size_t at = (size_t)uj * p.k + e0 + i;
    sSlot[i] = p.sel_slot[at];
    sSrc[i] = (p.fetch && p.fetch[at]) ? p.sel[at] : -1;
  }

  // this lane's Q operand: head w*16 + li, dims 32*ks + 8*g .. +8
  bf16x8 qf[kKSteps];
  {
    const uint16_t* qrow = p.q + (((size_t)b * p.T + j) * p.Hq + w * 16 + li) * kDqk + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
  }
  __syncthreads();

  uint16_t* ubase = p.buf_kv + (size_t)u * p.S * kDqk;
  const uint16_t* hbase = p.host_kv + (size_t)u * p.N * kDqk;
  constexpr int kPer = (kPieces + kThreads - 1) / kThreads;
  u32x4 pre[kPer];
  uint32_t fetched = 0;  // bit x: piece x came from host memory

  // stage chunk c's rows into registers (rows past the split are zero)
  auto load_chunk = [&](int c) {
    fetched = 0;
#pragma unroll
    for (int x = 0; x < kPer; ++x) {
      const int pc = tid + x * kThreads;
      pre[x] = u32x4{0u, 0u, 0u, 0u};
      if (pc < kPieces) {
        const int r = pc / kPiecesPerRow, col = pc - r * kPiecesPerRow;
        const int e = c * kChunk + r;
        if (e < ne) {
          const int src = sSrc[e];
          if (src >= 0) {
            pre[x] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(hbase + (size_t)src * kDqk + col * 8));
            fetched |= 1u << x;
          } else {
            pre[x] = *reinterpret_cast<const u32x4*>(ubase + (size_t)sSlot[e] * kDqk + col * 8);
          }
        }
      }
    }
  };
  auto store_chunk = [&](int c, int buf) {
#pragma unroll
    for (int x = 0; x < kPer; ++x) {
      const int pc = tid + x * kThreads;
      if (pc < kPieces) {
        const int r = pc / kPiecesPerRow, col = pc - r * kPiecesPerRow;
        *reinterpret_cast<u32x4*>(sKV + (buf * kChunk + r) * kRow + col * 8) = pre[x];
        if (fetched & (1u << x))
          *reinterpret_cast<u32x4*>(ubase + (size_t)sSlot[c * kChunk + r] * kDqk + col * 8) = pre[x];
      }
    }
  };

  f32x4 acc[kMTiles];
#pragma unroll
  for (int t = 0; t < kMTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int nchunks = (ne + kChunk - 1) / kChunk;
  load_chunk(0);
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    store_chunk(c, buf);
    __syncthreads();
    if (c + 1 < nchunks) load_chunk(c + 1);
    const uint16_t* tile = sKV + buf * kChunk * kRow;

    // S^T = K Q^T for tokens 0..15 and 16..31 of the chunk, this wave's heads
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      const bf16x8 k0 = lds_row8(tile + li * kRow + 32 * ks + 8 * g);
      const bf16x8 k1 = lds_row8(tile + (16 + li) * kRow + 32 * ks + 8 * g);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[ks], s1, 0, 0, 0);
    }
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
    cm = xor_max(xor_max(cm, 16), 32);
    // lazy rescaling: the reference maximum only moves when the chunk's
    // maximum exceeds it by more than 8 (log2 units), so the weights stay
    // below 2^8 and the accumulators are rescaled rarely; the result does not
    // depend on which reference is used
    const bool move = cm > m_run + 8.f;
    const float m_new = move ? cm : m_run;
    const float corr = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first chunk
    float ps = 0.f;
    bf16x8 phi, plo;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float pv = __builtin_amdgcn_exp2f(sv[i] - m_new);
      ps += pv;
      const __bf16 h = (__bf16)pv;
      phi[i] = h;
      plo[i] = (__bf16)(pv - (float)h);
    }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l_run = l_run * corr + ps;
    m_run = m_new;
    if (__ballot(move)) {
#pragma unroll
      for (int t = 0; t < kMTiles; ++t) acc[t] *= corr;
    }

    // O^T += V^T P^T: V^T fragments by transposing LDS reads.  k slot 8g+r
    // is token 4g+r for r < 4 and 16+4g+(r-4) otherwise, matching the
    // layout of the probabilities above.
    const uint16_t* v0 = tile + (4 * g + (li >> 2)) * kRow + 4 * (li & 3);
    const uint16_t* v1 = v0 + 16 * kRow;
#pragma unroll
    for (int t = 0; t < kMTiles; ++t) {
      const bf16x8 vt = lds_vt(v0 + 16 * t, v1 + 16 * t);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, phi, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, plo, acc[t], 0, 0, 0);
    }
  }

  // lane holds O[h = w*16 + li][d = 16t + 4g + i]
  const int h = w * 16 + li;
  if (nsplit == 1) {
    const float inv = 1.f / l_run;
#pragma unroll
    for (int t = 0; t < kMTiles; ++t)
      *reinterpret_cast<f32x4*>(orow + (size_t)h * kDv + 16 * t + 4 * g) = acc[t] * inv;
    return;
  }
  const size_t part_stride = (size_t)G * (kDv + 2);
  float* part = p.partials + ((size_t)uj * nsplit + sp) * part_stride;
#pragma unroll
  for (int t = 0; t < kMTiles; ++t)
    *reinterpret_cast<f32x4*>(part + (size_t)h * kDv + 16 * t + 4 * g) = acc[t];
  if (g == 0) {
    part[G * kDv + h] = m_run;
    part[G * kDv + G + h] = l_run;
  }
}

}  // namespace

size_t attn_latent_lds() { return sizeof(uint16_t) * 2 * kChunk * kRow; }

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
  if (p.nsplit == 1) return hipSuccess;
  return launch_attn_combine(p0, p0.Hq, kDv, s);
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
