// K4: merge of the split-k attention partials of each (unit, token, head), in
// split order: out = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M), with
// M = max_s m_s (scores are kept in log2 units).  One workgroup per head row;
// the split weights are formed once in LDS, then every output element reads
// its nsplit partials with independent loads.
#include "avsg_internal.h"

namespace avsg {
namespace {

constexpr int kCombineThreads = 128;

__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(AttnParams p, int G, int D) {
  extern __shared__ float sW[];  // [nsplit] weights
  __shared__ float sInvL;
  const int uj = blockIdx.x / G, h = blockIdx.x - (blockIdx.x / G) * G;
  const int u = uj / p.T, j = uj - u * p.T;
  const int b = u / p.Hkv, g = u - b * p.Hkv;
  const int nsplit = p.nsplit, tid = threadIdx.x;
  float* orow = p.out + ((((size_t)b * p.T + j) * p.Hq) + (size_t)g * G + h) * D;
  if (p.unit_status[u] != 0) {
    for (int d = tid; d < D; d += kCombineThreads) orow[d] = 0.f;
    return;
  }
  const size_t ps = (size_t)G * (D + 2);
  const float* pbase = p.partials + (size_t)uj * nsplit * ps;
  for (int s = tid; s < nsplit; s += kCombineThreads) sW[s] = pbase[s * ps + (size_t)G * D + h];
  __syncthreads();
  if (tid == 0) {
    float mx = -INFINITY;
    for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, sW[s]);
    float lsum = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float wgt = __builtin_amdgcn_exp2f(sW[s] - mx);
      lsum = fmaf(pbase[s * ps + (size_t)G * D + G + h], wgt, lsum);
      sW[s] = wgt;
    }
    sInvL = 1.f / lsum;
  }
  __syncthreads();
  const float inv = sInvL;
  for (int d = tid; d < D; d += kCombineThreads) {
    float acc = 0.f;
#pragma unroll 8
    for (int s = 0; s < nsplit; ++s) acc = fmaf(pbase[s * ps + (size_t)h * D + d], sW[s], acc);
    orow[d] = acc * inv;
  }
}

}  // namespace

hipError_t launch_attn_combine(const AttnParams& p, int G, int D, hipStream_t s) {
  const size_t lds = sizeof(float) * (size_t)p.nsplit;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(p.units * p.T * G)),
                     dim3(kCombineThreads), lds, s, p, G, D);
  return hipGetLastError();
}

}  // namespace avsg
