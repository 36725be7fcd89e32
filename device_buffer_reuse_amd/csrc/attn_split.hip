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
//  * A workgroup (4 waves) owns 128 token rows of one (unit, token).  16 lanes
//    cover one 256-byte K or V half-row of a token (16 bytes each), so a wave
//    reads 4 half-rows (1 KiB) per load instruction; each lane issues the K
//    and V loads of its 8 rows before any use, so a workgroup has its whole
//    64 KiB in flight at once and every selected byte is read exactly once.
//  * q.k uses v_dot2_f32_bf16 on bf16 pairs (products exact, fp32 sums); the
//    16 partial sums of a row are added by four DPP steps inside the row.
//  * Scores go to LDS; one wave per head takes the split's maximum and the
//    exp2 weights; p * v accumulates in fp32 from the V halves in registers.
//  * Split partials (max, sum, o) go to the workspace and the combine kernel
//    merges them in split order, so the result does not depend on workgroup
//    timing.  (Merging inside the last workgroup of each (unit,
//    token) needs an agent-scope release in every workgroup, which writes
//    back the XCD's L2 each time and cost more than the extra launch.)
#include "avsg_internal.h"

namespace avsg {
namespace {

constexpr int kD = 128;           // head dim of the split layout
constexpr int kUnr = 8;           // rows in flight per lane group
constexpr int kSplitRows = 16 * kUnr;  // token rows per workgroup

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

template <int G>
__global__ __launch_bounds__(kAttnThreads) void attn_split_kernel(AttnParams p) {
  __shared__ float sScore[G][kSplitRows];
  __shared__ int32_t sSlot[kSplitRows];
  __shared__ int32_t sSrc[kSplitRows];  // host row of a fetched entry, else -1
  __shared__ float sO[4][G][kD];
  __shared__ float sM[G], sL[G];

  const int nsplit = p.nsplit;
  const int u = blockIdx.x / nsplit;
  const int sp = blockIdx.x - u * nsplit;
  const int j = p.token;
  const int uj = u * p.T + j;
  const int b = u / p.Hkv, g = u - b * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rg = lane >> 4, c = lane & 15;
  const int tpe = p.tpe;
  const bool bad = p.unit_status[u] != 0;
  const int n_rows = p.k * tpe;
  const int r0 = sp * kSplitRows, r1 = min(r0 + kSplitRows, n_rows);
  const int nr = r1 - r0;
  float* orow = p.out + (((size_t)b * p.T + j) * p.Hq + g * G) * kD;
  if (bad) {
    if (nsplit == 1)
      for (int idx = tid; idx < G * kD; idx += kAttnThreads) orow[idx] = 0.f;
    return;
  }

  const int e0 = r0 / tpe, e1 = (r1 - 1) / tpe + 1;
  for (int i = tid; i < e1 - e0; i += kAttnThreads) {
    const size_t at = (size_t)uj * p.k + e0 + i;
    sSlot[i] = p.sel_slot[at];
    sSrc[i] = (p.fetch && p.fetch[at]) ? p.sel[at] : -1;
  }

  uint32_t qf[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 qq = *reinterpret_cast<const uint4*>(
        p.q + (((size_t)b * p.T + j) * p.Hq + g * G + h) * kD + c * 8);
    qf[h][0] = qq.x; qf[h][1] = qq.y; qf[h][2] = qq.z; qf[h][3] = qq.w;
  }
  __syncthreads();

  uint16_t* ubase = p.buf_kv + (size_t)u * p.S * p.row_elems;
  const uint16_t* hbase = p.host_kv + (size_t)u * p.N * p.row_elems;
  const int v_off = tpe * kD;
  float o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int x = 0; x < 8; ++x) o[h][x] = 0.f;

  // K and V halves of this lane group's rows, all in flight together: rows
  // that missed come from pinned host memory (and are stored into their slot
  // below), the others from the buffer in HBM
  uint4 kr[kUnr], vr[kUnr];
  uint16_t* dst[kUnr];
#pragma unroll
  for (int e = 0; e < kUnr; ++e) {
    const int rr = e * 16 + w * 4 + rg;
    dst[e] = nullptr;
    if (rr < nr) {
      const int row = r0 + rr;
      const int ent = row / tpe, sub = row - ent * tpe;
      const int off = sub * kD + c * 8;
      uint16_t* slot_row = ubase + (size_t)sSlot[ent - e0] * p.row_elems + off;
      const int src = sSrc[ent - e0];
      if (src >= 0) {
        const u32x4* h = reinterpret_cast<const u32x4*>(hbase + (size_t)src * p.row_elems + off);
        const u32x4 a = __builtin_nontemporal_load(h);
        const u32x4 bb = __builtin_nontemporal_load(h + v_off / 8);
        kr[e] = make_uint4(a.x, a.y, a.z, a.w);
        vr[e] = make_uint4(bb.x, bb.y, bb.z, bb.w);
        dst[e] = slot_row;
      } else {
        kr[e] = *reinterpret_cast<const uint4*>(slot_row);
        vr[e] = *reinterpret_cast<const uint4*>(slot_row + v_off);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < kUnr; ++e) {
    const int rr = e * 16 + w * 4 + rg;
    if (rr < nr) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc = dot2(qf[h][0], kr[e].x, 0.f);
        acc = dot2(qf[h][1], kr[e].y, acc);
        acc = dot2(qf[h][2], kr[e].z, acc);
        acc = dot2(qf[h][3], kr[e].w, acc);
        acc = row_sum16(acc);
        if (c == h) sScore[h][rr] = acc * p.scale_log2e;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < kUnr; ++e)
    if (dst[e]) {
      *reinterpret_cast<uint4*>(dst[e]) = kr[e];
      *reinterpret_cast<uint4*>(dst[e] + v_off) = vr[e];
    }
  __syncthreads();
  // split maximum and exp2 weights, one wave per head
  for (int h = w; h < G; h += 4) {
    float mx = -INFINITY;
    for (int i = lane; i < nr; i += 64) mx = fmaxf(mx, sScore[h][i]);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int i = lane; i < nr; i += 64) {
      const float e = __builtin_amdgcn_exp2f(sScore[h][i] - mx);
      sScore[h][i] = e;
      sum += e;
    }
    sum = wave_sum(sum);
    if (lane == 0) { sM[h] = mx; sL[h] = sum; }
  }
  __syncthreads();
  // o += p v
#pragma unroll
  for (int e = 0; e < kUnr; ++e) {
    const int rr = e * 16 + w * 4 + rg;
    if (rr < nr) {
      float vf[8] = {bf_lo(vr[e].x), bf_hi(vr[e].x), bf_lo(vr[e].y), bf_hi(vr[e].y),
                     bf_lo(vr[e].z), bf_hi(vr[e].z), bf_lo(vr[e].w), bf_hi(vr[e].w)};
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pw = sScore[h][rr];
#pragma unroll
        for (int x = 0; x < 8; ++x) o[h][x] = fmaf(pw, vf[x], o[h][x]);
      }
    }
  }
  // reduce over the 4 row groups of the wave, then over the 4 waves
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      o[h][x] += __shfl_xor(o[h][x], 16, 64);
      o[h][x] += __shfl_xor(o[h][x], 32, 64);
    }
  if (rg == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int x = 0; x < 8; ++x) sO[w][h][c * 8 + x] = o[h][x];
  }
  __syncthreads();
  if (nsplit == 1) {
    for (int idx = tid; idx < G * kD; idx += kAttnThreads) {
      const int h = idx / kD, d = idx - h * kD;
      orow[idx] = ((sO[0][h][d] + sO[1][h][d]) + (sO[2][h][d] + sO[3][h][d])) / sL[h];
    }
    return;
  }
  const size_t part_stride = (size_t)G * (kD + 2);
  float* part = p.partials + ((size_t)uj * nsplit + sp) * part_stride;
  for (int idx = tid; idx < G * kD; idx += kAttnThreads) {
    const int h = idx / kD, d = idx - h * kD;
    part[idx] = (sO[0][h][d] + sO[1][h][d]) + (sO[2][h][d] + sO[3][h][d]);
  }
  if (tid < G) {
    part[G * kD + tid] = sM[tid];
    part[G * kD + G + tid] = sL[tid];
  }
}

}  // namespace

template <int G>
static hipError_t launch_g(const AttnParams& p0, hipStream_t s) {
  // one launch per query token: a row that several tokens select is fetched
  // by the first of them, and later tokens read it from the buffer
  const dim3 grid((unsigned)(p0.units * p0.nsplit));
  AttnParams p = p0;
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
