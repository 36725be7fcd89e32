// K3 + K4: split-k decode attention over the buffer slots of the selected
// entries (K/V split layout, grouped-query heads), with the split merge fused
// into the last workgroup of each (unit, token).
//
// What it computes: for each unit, query token and query head of the unit,
// softmax(scale * q K^T) V over exactly the selected entries (all tokens of a
// selected page), reading every row from the slot that match_reserve assigned.
// The AVSG abstract (arxivdaily 2609.37538) requires the selections to stay
// exact, so this equals attention over the same rows read from host memory.
//
// gfx950 mapping (HBM-bound, VALU):
//  * A workgroup (4 waves) owns `split_rows` token rows of one (unit, token).
//    16 lanes cover one 256-byte K or V row of a token (16 bytes each), so a
//    wave reads 4 rows (1 KiB) per load instruction and a workgroup 16; the
//    8 iterations of a 128-row split are issued before any use.
//  * q.k uses v_dot2_f32_bf16 on bf16 pairs (products exact, fp32 sums); the
//    16 partial sums of a row are added by four DPP steps inside the row.
//  * Scores go to LDS; one wave per head takes the split's maximum and the
//    exp2 weights; the V pass reads the other half of each row (each byte of
//    a selected row is read once) and accumulates p * v in fp32.
//  * Split partials (max, sum, o) go to the workspace; the last workgroup of a
//    (unit, token), found with an agent-scope counter, merges them in split
//    order, so the result does not depend on workgroup timing.
#include "avsg_internal.h"

namespace avsg {
namespace {

constexpr int kD = 128;           // head dim of the split layout
constexpr int kMaxSplitRows = 256;
constexpr int kUnr = 8;           // row batches in flight per lane

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

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
  __shared__ float sScore[G][kMaxSplitRows];
  __shared__ int32_t sSlot[kMaxSplitRows];
  __shared__ float sO[4][G][kD];
  __shared__ float sM[G], sL[G];
  __shared__ int sLast;

  const int nsplit = p.nsplit;
  const int uj = blockIdx.x / nsplit;
  const int sp = blockIdx.x - uj * nsplit;
  const int u = uj / p.T, j = uj - u * p.T;
  const int b = u / p.Hkv, g = u - b * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rg = lane >> 4, c = lane & 15;
  const int tpe = p.tpe;
  const bool bad = p.unit_status[u] != 0;
  const int n_rows = p.k * tpe;
  const int r0 = sp * p.split_rows, r1 = min(r0 + p.split_rows, n_rows);
  const int nr = r1 - r0;
  const size_t part_stride = (size_t)G * (kD + 2);
  float* part = p.partials + ((size_t)uj * nsplit + sp) * part_stride;

  if (!bad) {
    const int e0 = r0 / tpe, e1 = (r1 - 1) / tpe + 1;
    for (int i = tid; i < e1 - e0; i += kAttnThreads) sSlot[i] = p.sel_slot[(size_t)uj * p.k + e0 + i];

    uint32_t qf[G][4];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint4 qq = *reinterpret_cast<const uint4*>(
          p.q + (((size_t)b * p.T + j) * p.Hq + g * G + h) * kD + c * 8);
      qf[h][0] = qq.x; qf[h][1] = qq.y; qf[h][2] = qq.z; qf[h][3] = qq.w;
    }
    __syncthreads();

    const uint16_t* ubase = p.buf_kv + (size_t)u * p.S * p.row_elems;
    const int v_off = tpe * kD;

    // pass 1: scores
    for (int rb = 0; rb < nr; rb += 16 * kUnr) {
      uint4 kr[kUnr];
#pragma unroll
      for (int e = 0; e < kUnr; ++e) {
        const int rr = rb + e * 16 + w * 4 + rg;
        if (rr < nr) {
          const int row = r0 + rr;
          const int ent = row / tpe, sub = row - ent * tpe;
          const int slot = sSlot[ent - e0];
          kr[e] = *reinterpret_cast<const uint4*>(ubase + (size_t)slot * p.row_elems + sub * kD + c * 8);
        }
      }
#pragma unroll
      for (int e = 0; e < kUnr; ++e) {
        const int rr = rb + e * 16 + w * 4 + rg;
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

    // pass 2: o = sum p v
    float o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int x = 0; x < 8; ++x) o[h][x] = 0.f;
    for (int rb = 0; rb < nr; rb += 16 * kUnr) {
      uint4 vr[kUnr];
#pragma unroll
      for (int e = 0; e < kUnr; ++e) {
        const int rr = rb + e * 16 + w * 4 + rg;
        if (rr < nr) {
          const int row = r0 + rr;
          const int ent = row / tpe, sub = row - ent * tpe;
          const int slot = sSlot[ent - e0];
          vr[e] = *reinterpret_cast<const uint4*>(ubase + (size_t)slot * p.row_elems + v_off + sub * kD + c * 8);
        }
      }
#pragma unroll
      for (int e = 0; e < kUnr; ++e) {
        const int rr = rb + e * 16 + w * 4 + rg;
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
    for (int idx = tid; idx < G * kD; idx += kAttnThreads) {
      const int h = idx / kD, d = idx - h * kD;
      part[h * kD + d] = (sO[0][h][d] + sO[1][h][d]) + (sO[2][h][d] + sO[3][h][d]);
    }
    if (tid < G) {
      part[G * kD + tid] = sM[tid];
      part[G * kD + G + tid] = sL[tid];
    }
  }

  // merge of the splits by the last workgroup of this (unit, token)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(&p.counters[uj], 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    sLast = (prev == (unsigned)(nsplit - 1));
  }
  __syncthreads();
  if (!sLast) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  const float* pbase = p.partials + (size_t)uj * nsplit * part_stride;
  float* orow = p.out + (((size_t)b * p.T + j) * p.Hq + g * G) * kD;
  for (int idx = tid; idx < G * kD; idx += kAttnThreads) {
    const int h = idx / kD, d = idx - h * kD;
    if (bad) { orow[idx] = 0.f; continue; }
    float mx = -INFINITY;
    for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, pbase[s * part_stride + G * kD + h]);
    float acc = 0.f, lsum = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float* ps = pbase + s * part_stride;
      const float wgt = __builtin_amdgcn_exp2f(ps[G * kD + h] - mx);
      lsum = fmaf(ps[G * kD + G + h], wgt, lsum);
      acc = fmaf(ps[h * kD + d], wgt, acc);
    }
    orow[idx] = acc / lsum;
  }
  if (tid == 0) p.counters[uj] = 0u;
}

}  // namespace

hipError_t launch_attn_split(const AttnParams& p, int G, hipStream_t s) {
  const dim3 grid((unsigned)(p.units * p.T * p.nsplit));
  switch (G) {
    case 1: hipLaunchKernelGGL(attn_split_kernel<1>, grid, dim3(kAttnThreads), 0, s, p); break;
    case 2: hipLaunchKernelGGL(attn_split_kernel<2>, grid, dim3(kAttnThreads), 0, s, p); break;
    case 4: hipLaunchKernelGGL(attn_split_kernel<4>, grid, dim3(kAttnThreads), 0, s, p); break;
    case 8: hipLaunchKernelGGL(attn_split_kernel<8>, grid, dim3(kAttnThreads), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace avsg
