// K2: miss-only transfer of KV rows from pinned host memory into the reserved
// buffer slots, split evenly over all compute units.
//
// Method (AVSG abstract, arxivdaily 2609.37538): only the entries that missed
// are transferred, and the transfers are partitioned evenly across the
// accelerator's cores instead of being assigned per request, which would
// leave cores idle when requests miss unevenly.  Head-wise rows (Spin summary,
// gist.science 2604.26837, section 2B) mean only the selected head's bytes
// cross PCIe.
//
// gfx950 mapping: every workgroup reads the per-unit miss counts written by
// match_reserve (no host round trip), forms their prefix sum in LDS, and
// takes an equal share of the global list of 16-byte pieces of missed rows
// (or, in the request-level mode kept for comparison, one unit's rows).
// Each lane issues several 16-byte loads from host memory before storing
// them, so thousands of PCIe reads are in flight across the chip; a wave
// reads 1 KiB of consecutive row bytes per instruction.
#include "avsg_internal.h"

namespace avsg {
namespace {

constexpr int kUnroll = 8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kGatherThreads) void gather_kernel(GatherParams p) {
  extern __shared__ int32_t sPre[];  // [units + 1] exclusive prefix of miss counts
  const int tid = threadIdx.x;
  const int units = p.units;

  // prefix sum of miss counts, each thread owning a contiguous run of units
  __shared__ int32_t sPart[kGatherThreads];
  const int per = (units + kGatherThreads - 1) / kGatherThreads;
  const int a0 = min(tid * per, units), a1 = min(a0 + per, units);
  int sum = 0;
  for (int i = a0; i < a1; ++i) sum += p.miss_count[i];
  sPart[tid] = sum;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < kGatherThreads; ++i) {
      int v = sPart[i];
      sPart[i] = run;
      run += v;
    }
    sPre[units] = run;
  }
  __syncthreads();
  {
    int run = sPart[tid];
    for (int i = a0; i < a1; ++i) {
      sPre[i] = run;
      run += p.miss_count[i];
    }
  }
  __syncthreads();

  const uint32_t rows = (uint32_t)sPre[units];
  const uint32_t row16 = (uint32_t)p.row16;
  const uint64_t pieces = (uint64_t)rows * row16;
  uint32_t c0, c1;
  if (p.per_unit) {
    // request-level assignment: workgroup u copies exactly unit u's rows
    c0 = (uint32_t)sPre[blockIdx.x] * row16;
    c1 = (uint32_t)sPre[blockIdx.x + 1] * row16;
  } else {
    // equal shares of the global list of row pieces
    c0 = (uint32_t)(pieces * blockIdx.x / gridDim.x);
    c1 = (uint32_t)(pieces * (blockIdx.x + 1) / gridDim.x);
  }

  int cur_unit = 0;
  for (uint32_t c = c0 + tid; c < c1; c += kGatherThreads * kUnroll) {
    uint4 v[kUnroll];
    uint4* dst[kUnroll];
#pragma unroll
    for (int e = 0; e < kUnroll; ++e) {
      const uint32_t cc = c + (uint32_t)e * kGatherThreads;
      dst[e] = nullptr;
      if (cc < c1) {
        const uint32_t row = cc / row16;
        const uint32_t col = cc - row * row16;
        // unit owning this row: last unit whose prefix is <= row
        if (!((uint32_t)sPre[cur_unit] <= row && row < (uint32_t)sPre[cur_unit + 1])) {
          int lo = 0, hi = units - 1;
          while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if ((uint32_t)sPre[mid] <= row) lo = mid; else hi = mid - 1;
          }
          cur_unit = lo;
        }
        const int2 ms = p.misses[(size_t)cur_unit * p.ucap + (row - (uint32_t)sPre[cur_unit])];
        // ms.y: the row's id in its unit, or its pool row (host directory)
        const u32x4* src = reinterpret_cast<const u32x4*>(p.host_kv) +
                           ((p.pooled ? 0 : (size_t)cur_unit * p.N) + (uint32_t)ms.y) * row16 + col;
        const u32x4 x = __builtin_nontemporal_load(src);
        v[e] = make_uint4(x.x, x.y, x.z, x.w);
        dst[e] = p.buf_kv + ((size_t)cur_unit * p.S + ms.x) * row16 + col;
      }
    }
#pragma unroll
    for (int e = 0; e < kUnroll; ++e)
      if (dst[e]) *dst[e] = v[e];
  }
}

}  // namespace

hipError_t launch_gather(const GatherParams& p, int grid, hipStream_t s) {
  const size_t lds = sizeof(int32_t) * (size_t)(p.units + 1);
  hipLaunchKernelGGL(gather_kernel, dim3(grid), dim3(kGatherThreads), lds, s, p);
  return hipGetLastError();
}

}  // namespace avsg
