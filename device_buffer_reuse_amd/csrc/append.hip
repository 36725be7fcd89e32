// Offload of a newly decoded token.  The Spin summary (gist.science
// 2604.26837, section 2A) lists Offload, placing KV data into memory, among
// the system-managed operations over a page-based KV substrate, and keeps the
// physical pages per attention head (section 2B).  Here the token's K and V
// (or its latent vector) are written into its row of the head-wise host
// store, and into the slot holding that entry if the entry is resident, so
// the device buffer keeps exact copies of host rows and later hits stay
// exact.  Slots, lifetimes and stamps are not touched.
//
// One workgroup per unit: the slot table is scanned for the entry (S int32
// reads, coalesced), then one lane per 16-byte piece of the token copies it
// to host memory and to each slot found.  With a two-level host directory
// (Spin summary, section 2C) the host row is the entry's pool row.
#include "avsg_internal.h"

namespace avsg {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kAppendThreads = 256;
constexpr int kMaxHolders = 32;  // slots recorded per entry (1 in a valid state)

__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendParams p) {
  __shared__ int32_t sHolder[kMaxHolders];
  __shared__ int32_t sCount;
  __shared__ int64_t sHostRow;
  const int u = blockIdx.x;
  const int b = u / p.Hkv;
  const int tid = threadIdx.x;
  const int64_t pos = p.pos[b];
  if (pos < 0 || pos >= (int64_t)p.N * p.tpe) {
    if (tid == 0 && u == b * p.Hkv) atomicOr(p.err_word, 1u << (AVSG_ERR_RANGE - 16));
    return;
  }
  const int e = (int)(pos / p.tpe);
  const int r = (int)(pos - (int64_t)e * p.tpe);
  if (tid == 0) {
    sCount = 0;
    // the entry's host row: u * N + e, or its pool row through the two-level
    // directory (-1: not mapped, a range error of the unit)
    int64_t hrow = (int64_t)u * p.N + e;
    if (p.dir.top) {
      const int32_t seg = p.dir.top[(size_t)u * p.dir.n_seg + (e >> p.dir.seg_log2)];
      int32_t row = -1;
      if (seg >= 0 && seg < p.dir.n_segments)
        row = p.dir.segments[((size_t)seg << p.dir.seg_log2) + (e & ((1 << p.dir.seg_log2) - 1))];
      hrow = (row >= 0 && (int64_t)row < p.dir.pool_rows) ? row : -1;
    }
    sHostRow = hrow;
  }
  __syncthreads();
  const int64_t hrow = sHostRow;
  if (hrow < 0) {
    if (tid == 0) atomicOr(p.err_word, 1u << (AVSG_ERR_RANGE - 16));
    return;
  }
  const int32_t* st = p.slot_table + (size_t)u * p.S;
  for (int s = tid; s < p.S; s += kAppendThreads) {
    if (st[s] == e) {
      const int at = atomicAdd(&sCount, 1);
      if (at < kMaxHolders) sHolder[at] = s;
    }
  }
  __syncthreads();
  const int holders = sCount;
  if (holders > kMaxHolders) {
    // more slots than a valid state allows hold the entry: nothing is written
    if (tid == 0) atomicOr(p.err_word, 1u << (AVSG_ERR_STATE - 16));
    return;
  }
  // piece i of the token: key pieces first, then value pieces (split layout)
  const int kp = p.dqk >> 3, vp = p.latent ? 0 : p.dv >> 3;
  if (tid >= kp + vp) return;
  const int64_t off = tid < kp ? (int64_t)(p.latent ? 0 : r * p.dqk) + 8 * tid
                               : (int64_t)p.tpe * p.dqk + (int64_t)r * p.dv + 8 * (tid - kp);
  const u32x4 v = *reinterpret_cast<const u32x4*>(p.new_kv + (size_t)u * p.tok_elems + 8 * tid);
  *reinterpret_cast<u32x4*>(p.host_kv + (size_t)hrow * p.row_elems + off) = v;
  for (int h = 0; h < holders; ++h)
    *reinterpret_cast<u32x4*>(p.buf_kv + ((size_t)u * p.S + sHolder[h]) * p.row_elems + off) = v;
}

}  // namespace

hipError_t launch_append(const AppendParams& p, int units, hipStream_t s) {
  if (p.dqk % 8 != 0 || p.dv % 8 != 0 || (p.dqk >> 3) + (p.latent ? 0 : p.dv >> 3) > kAppendThreads)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)units), dim3(kAppendThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace avsg
