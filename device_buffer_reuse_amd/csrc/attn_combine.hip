// K4: merge of the split-k attention partials of each (unit, token, head), in
// split order: out = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M), with
// M = max_s m_s (scores are kept in log2 units).
//
// One thread per 4 consecutive output values.  With at most 16 splits (every
// configured workload) a thread issues the loads of all the splits' maxima,
// sums and 16-byte partial vectors together, so the merge costs one memory
// round trip; more splits take a loop over the splits.
#include "avsg_internal.h"

namespace avsg {
namespace {

constexpr int kCombineThreads = 256;
constexpr int kMaxFastSplits = 16;

template <int NS>  // NS > 0: exactly NS splits, all loads in flight at once
__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(AttnParams p, int G, int D) {
  const int dv4 = D >> 2;
  // the same XCD-aware order as the attention launches: XCD x merges the
  // x-th eighth of the outputs, whose partials its own L2 wrote
  const int nb = (int)gridDim.x;
  const int bid = (nb & 7) == 0 ? (int)(blockIdx.x & 7) * (nb >> 3) + (int)(blockIdx.x >> 3)
                                : (int)blockIdx.x;
  const int64_t idx = (int64_t)bid * kCombineThreads + threadIdx.x;
  const int64_t total = (int64_t)p.units * p.T * G * dv4;
  if (idx >= total) return;
  const int d4 = (int)(idx % dv4);
  const int64_t rest = idx / dv4;
  const int h = (int)(rest % G);
  const int uj = (int)(rest / G);
  const int u = uj / p.T, j = uj - u * p.T;
  const int b = u / p.Hkv, g = u - b * p.Hkv;
  float4* orow = reinterpret_cast<float4*>(
      p.out + ((((size_t)b * p.T + j) * p.Hq) + (size_t)g * G + h) * D) + d4;
  const int nsplit = NS > 0 ? NS : p.nsplit;
  const size_t ps = partial_stride(G, D);  // floats per split partial, multiple of 4
  const float* pbase = p.partials + (size_t)uj * nsplit * ps;
  const float* mrow = pbase + (size_t)G * D + h;
  const float* lrow = mrow + G;
  const float4* orow_s = reinterpret_cast<const float4*>(pbase + (size_t)h * D) + d4;
  if constexpr (NS > 0) {
    // every split's partial is loaded together with the unit's status and
    // list length (one memory round trip); splits past a shortened list
    // hold stale values and are dropped by selection, never by a weight
    const int status = p.unit_status[u];
    const int len_in = p.sel_len ? p.sel_len[uj] : p.k;
    float m[NS], l[NS];
    float4 o[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      m[s] = mrow[s * ps];
      l[s] = lrow[s * ps];
      o[s] = orow_s[s * (ps / 4)];
    }
    if (status != 0) {
      *orow = make_float4(0.f, 0.f, 0.f, 0.f);
      return;
    }
    // splits holding rows: all of them, or those covering a shortened list
    const int len = min(max(len_in, 1), p.k);
    const int nused = min(nsplit, (len * p.tpe + p.split_rows - 1) / p.split_rows);
    float mx = -INFINITY;
#pragma unroll
    for (int s = 0; s < NS; ++s) mx = s < nused ? fmaxf(mx, m[s]) : mx;
    float lsum = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s < nused) {
        const float wgt = __builtin_amdgcn_exp2f(m[s] - mx);
        lsum = fmaf(l[s], wgt, lsum);
        acc.x = fmaf(o[s].x, wgt, acc.x);
        acc.y = fmaf(o[s].y, wgt, acc.y);
        acc.z = fmaf(o[s].z, wgt, acc.z);
        acc.w = fmaf(o[s].w, wgt, acc.w);
      }
    }
    const float inv = 1.f / lsum;
    *orow = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  } else {
    if (p.unit_status[u] != 0) {
      *orow = make_float4(0.f, 0.f, 0.f, 0.f);
      return;
    }
    const int len = p.sel_len ? min(max(p.sel_len[uj], 1), p.k) : p.k;
    const int nused = min(nsplit, (len * p.tpe + p.split_rows - 1) / p.split_rows);
    float mx = -INFINITY;
    for (int s = 0; s < nused; ++s) mx = fmaxf(mx, mrow[s * ps]);
    float lsum = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < nused; ++s) {
      const float wgt = __builtin_amdgcn_exp2f(mrow[s * ps] - mx);
      lsum = fmaf(lrow[s * ps], wgt, lsum);
      const float4 o = orow_s[s * (ps / 4)];
      acc.x = fmaf(o.x, wgt, acc.x);
      acc.y = fmaf(o.y, wgt, acc.y);
      acc.z = fmaf(o.z, wgt, acc.z);
      acc.w = fmaf(o.w, wgt, acc.w);
    }
    const float inv = 1.f / lsum;
    *orow = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
}

// The latent layout's partials: each split's output normalized by its own
// sum, as fp16, then its maxima and sums as fp32 (latent_partial_bytes):
// out = sum_s l_s 2^(m_s - M) on_s / sum_s l_s 2^(m_s - M).  One thread per 4
// consecutive outputs; with NS > 0 splits all loads are issued together, NS
// = 0 loops over the context's split count.
template <int NS>
__global__ __launch_bounds__(kCombineThreads) void attn_combine_latent_kernel(AttnParams p, int G,
                                                                              int D) {
  typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
  const int dv4 = D >> 2;
  const int nb = (int)gridDim.x;
  const int bid = (nb & 7) == 0 ? (int)(blockIdx.x & 7) * (nb >> 3) + (int)(blockIdx.x >> 3)
                                : (int)blockIdx.x;
  const int64_t idx = (int64_t)bid * kCombineThreads + threadIdx.x;
  const int64_t total = (int64_t)p.units * p.T * G * dv4;
  if (idx >= total) return;
  const int d4 = (int)(idx % dv4);
  const int64_t rest = idx / dv4;
  const int h = (int)(rest % G);
  const int uj = (int)(rest / G);
  const int u = uj / p.T, j = uj - u * p.T;
  float4* orow = reinterpret_cast<float4*>(p.out + (((size_t)u * p.T + j) * p.Hq + h) * D) + d4;
  const int nsplit = NS > 0 ? NS : p.nsplit;
  const size_t pb = latent_partial_bytes(G, D);
  const uint8_t* base = reinterpret_cast<const uint8_t*>(p.partials) + (size_t)uj * nsplit * pb;
  auto load = [&](int s, float& m, float& l, f16x4& o) {
    const uint8_t* ps = base + (size_t)s * pb;
    const float* pm = reinterpret_cast<const float*>(ps + (size_t)G * D * 2);
    m = pm[h];
    l = pm[G + h];
    o = *(reinterpret_cast<const f16x4*>(ps + ((size_t)h * D) * 2) + d4);
  };
  float lsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto add = [&](float wgt, const f16x4& o) {
    lsum += wgt;
    acc.x = fmaf((float)o[0], wgt, acc.x);
    acc.y = fmaf((float)o[1], wgt, acc.y);
    acc.z = fmaf((float)o[2], wgt, acc.z);
    acc.w = fmaf((float)o[3], wgt, acc.w);
  };
  if constexpr (NS > 0) {
    // all splits' partials, the unit's status and its list length in one
    // memory round trip; splits past a shortened list are dropped by
    // selection
    const int status = p.unit_status[u];
    const int len_in = p.sel_len ? p.sel_len[uj] : p.k;
    float m[NS], l[NS];
    f16x4 o[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) load(s, m[s], l[s], o[s]);
    if (status != 0) {
      *orow = make_float4(0.f, 0.f, 0.f, 0.f);
      return;
    }
    const int len = min(max(len_in, 1), p.k);
    const int nused = min(nsplit, (len + p.split_rows - 1) / p.split_rows);
    float mx = -INFINITY;
#pragma unroll
    for (int s = 0; s < NS; ++s) mx = s < nused ? fmaxf(mx, m[s]) : mx;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      if (s < nused) add(l[s] * __builtin_amdgcn_exp2f(m[s] - mx), o[s]);
  } else {
    if (p.unit_status[u] != 0) {
      *orow = make_float4(0.f, 0.f, 0.f, 0.f);
      return;
    }
    const int len = p.sel_len ? min(max(p.sel_len[uj], 1), p.k) : p.k;
    const int nused = min(nsplit, (len + p.split_rows - 1) / p.split_rows);
    float mx = -INFINITY;
    for (int s = 0; s < nused; ++s) {
      float m, l;
      f16x4 o;
      load(s, m, l, o);
      mx = fmaxf(mx, m);
    }
    for (int s = 0; s < nused; ++s) {
      float m, l;
      f16x4 o;
      load(s, m, l, o);
      add(l * __builtin_amdgcn_exp2f(m - mx), o);
    }
  }
  const float inv = 1.f / lsum;
  *orow = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

template <int NS>
hipError_t launch_ns(const AttnParams& p, int G, int D, bool latent, hipStream_t s) {
  const int64_t total = (int64_t)p.units * p.T * G * (D / 4);
  const dim3 grid((unsigned)((total + kCombineThreads - 1) / kCombineThreads));
  if (latent) {
    hipLaunchKernelGGL(attn_combine_latent_kernel<NS>, grid, dim3(kCombineThreads), 0, s, p, G, D);
  } else {
    hipLaunchKernelGGL(attn_combine_kernel<NS>, grid, dim3(kCombineThreads), 0, s, p, G, D);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_combine(const AttnParams& p, int G, int D, bool latent, hipStream_t s) {
  if (D % 4 != 0) return hipErrorInvalidValue;
  switch (p.nsplit) {
    case 2: return launch_ns<2>(p, G, D, latent, s);
    case 3: return launch_ns<3>(p, G, D, latent, s);
    case 4: return launch_ns<4>(p, G, D, latent, s);
    case 8: return launch_ns<8>(p, G, D, latent, s);
    case 16: return launch_ns<kMaxFastSplits>(p, G, D, latent, s);
    default: return launch_ns<0>(p, G, D, latent, s);
  }
}

}  // namespace avsg
