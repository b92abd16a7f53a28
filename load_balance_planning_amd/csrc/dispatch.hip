// Dispatch layout and bf16 row gather on gfx950.
//
// [TopoEP] section 5: the plan stays on the device and the receive counts are
// derived there.  The layout is a stable counting sort of the slots by
// instance: instance offsets are the exclusive prefix of the instance loads,
// and the plan already gives each slot its position inside its instance
// (slot_rank), so slot_pos = inst_offset[slot_inst] + slot_rank with no sort.
//
// The copy is source-ordered: each hidden row is read from HBM once and
// written to its k dispatch rows, so HBM traffic is T*H*2 bytes read plus
// T*k*H*2 bytes written -- a destination-ordered gather would read each row
// k times (and measured slower on MI355X).  Plain stores: on MI355X they beat
// non-temporal ones for this write pattern.
#include "internal.h"

namespace moe {
namespace {

constexpr int kOffThreads = 1024;

__global__ __launch_bounds__(kOffThreads) void offsets_kernel(Dims d, const int32_t* __restrict__ n_inst_p,
                                                              const int32_t* __restrict__ inst_rank,
                                                              const int32_t* __restrict__ inst_load,
                                                              int32_t* __restrict__ inst_offset,
                                                              int32_t* __restrict__ rank_offset,
                                                              int32_t* __restrict__ status) {
  extern __shared__ int32_t sa[];  // [cap]
  __shared__ int32_t wave_tot[kOffThreads / 64 + 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int n = n_inst_p[0];
  if (n < 0 || n > d.cap) {
    if (tid == 0) atomicOr(status, MOE_STATUS_PLAN_CHECK);
    n = 0;
  }
  for (int i = tid; i < n; i += kOffThreads) sa[i] = inst_load[i];
  __syncthreads();
  const int per = (n + kOffThreads - 1) / kOffThreads;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int sum = 0;
  for (int q = lo; q < hi; ++q) sum += sa[q];
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < kOffThreads / 64; ++w) {
      const int v = wave_tot[w];
      wave_tot[w] = run;
      run += v;
    }
    wave_tot[kOffThreads / 64] = run;
  }
  __syncthreads();
  int run = wave_tot[wave] + incl - sum;
  for (int q = lo; q < hi; ++q) {
    const int v = sa[q];
    sa[q] = run;
    run += v;
  }
  __syncthreads();
  const int total = wave_tot[kOffThreads / 64];
  for (int i = tid; i <= d.cap; i += kOffThreads) inst_offset[i] = i < n ? sa[i] : (i == n ? total : -1);
  // Instances are rank-major, so a rank starts at its first instance.
  for (int i = tid; i < n; i += kOffThreads) {
    const int r = inst_rank[i];
    if ((unsigned)r < (unsigned)d.R && (i == 0 || inst_rank[i - 1] != r)) rank_offset[r] = sa[i];
  }
  if (tid == 0) rank_offset[d.R] = total;
}

// One workgroup per token: threads j < k place slot t*k+j, then the whole
// workgroup streams the row into its k destinations (16-byte vectors).
template <int VPT>
__global__ __launch_bounds__(256) void gather_vec_kernel(Dims d, const int32_t* __restrict__ slot_inst,
                                                         const int32_t* __restrict__ slot_rank,
                                                         const int32_t* __restrict__ inst_offset,
                                                         const uint4* __restrict__ hidden, int32_t* __restrict__ perm,
                                                         int32_t* __restrict__ slot_pos, uint4* __restrict__ dispatch,
                                                         int32_t* __restrict__ status) {
  __shared__ int32_t pos_s[kMaxK];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t N = (int64_t)d.T * d.k;
  const int vpr = d.H / 8;
  if (tid < d.k) {
    const int64_t sigma = t * d.k + tid;
    const int i = slot_inst[sigma];
    int64_t p = -1;
    if ((unsigned)i < (unsigned)d.cap) p = (int64_t)inst_offset[i] + slot_rank[sigma];
    if (p < 0 || p >= N) {
      atomicOr(status, MOE_STATUS_PLAN_CHECK);
      p = -1;
    } else {
      perm[p] = (int32_t)sigma;
    }
    slot_pos[sigma] = (int32_t)p;
    pos_s[tid] = (int32_t)p;
  }
  __syncthreads();
  const uint4* src = hidden + t * vpr;
  for (int base = 0; base < vpr; base += 256 * VPT) {
    uint4 v[VPT];
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int c = base + tid + u * 256;
      if (c < vpr) v[u] = src[c];
    }
    for (int j = 0; j < d.k; ++j) {
      const int p = pos_s[j];
      if (p < 0) continue;
      uint4* dst = dispatch + (int64_t)p * vpr;
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        const int c = base + tid + u * 256;
        if (c < vpr) dst[c] = v[u];
      }
    }
  }
}

// Any H: element-wise copy of bf16 bit patterns.
__global__ __launch_bounds__(256) void gather_u16_kernel(Dims d, const int32_t* __restrict__ slot_inst,
                                                         const int32_t* __restrict__ slot_rank,
                                                         const int32_t* __restrict__ inst_offset,
                                                         const uint16_t* __restrict__ hidden,
                                                         int32_t* __restrict__ perm, int32_t* __restrict__ slot_pos,
                                                         uint16_t* __restrict__ dispatch, int32_t* __restrict__ status) {
  __shared__ int32_t pos_s[kMaxK];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t N = (int64_t)d.T * d.k;
  if (tid < d.k) {
    const int64_t sigma = t * d.k + tid;
    const int i = slot_inst[sigma];
    int64_t p = -1;
    if ((unsigned)i < (unsigned)d.cap) p = (int64_t)inst_offset[i] + slot_rank[sigma];
    if (p < 0 || p >= N) {
      atomicOr(status, MOE_STATUS_PLAN_CHECK);
      p = -1;
    } else {
      perm[p] = (int32_t)sigma;
    }
    slot_pos[sigma] = (int32_t)p;
    pos_s[tid] = (int32_t)p;
  }
  __syncthreads();
  const uint16_t* src = hidden + t * d.H;
  for (int c = tid; c < d.H; c += 256) {
    const uint16_t v = src[c];
    for (int j = 0; j < d.k; ++j) {
      const int p = pos_s[j];
      if (p >= 0) dispatch[(int64_t)p * d.H + c] = v;
    }
  }
}

}  // namespace

hipError_t launch_offsets(const Dims& d, const int32_t* n_inst, const int32_t* inst_rank, const int32_t* inst_load,
                          int32_t* inst_offset, int32_t* rank_offset, int32_t* status, hipStream_t st) {
  const size_t lds = sizeof(int32_t) * (size_t)d.cap;
  hipLaunchKernelGGL(offsets_kernel, dim3(1), dim3(kOffThreads), lds, st, d, n_inst, inst_rank, inst_load,
                     inst_offset, rank_offset, status);
  return hipGetLastError();
}

hipError_t launch_gather(const Dims& d, const int32_t* slot_inst, const int32_t* slot_rank,
                         const int32_t* inst_offset, const uint16_t* hidden, int32_t* perm, int32_t* slot_pos,
                         uint16_t* dispatch, int32_t* status, hipStream_t st) {
  if (d.T == 0) return hipSuccess;
  const bool vec = (d.H % 8) == 0 && ((uintptr_t)hidden % 16) == 0 && ((uintptr_t)dispatch % 16) == 0;
  if (vec) {
    hipLaunchKernelGGL((gather_vec_kernel<4>), dim3(d.T), dim3(256), 0, st, d, slot_inst, slot_rank, inst_offset,
                       reinterpret_cast<const uint4*>(hidden), perm, slot_pos, reinterpret_cast<uint4*>(dispatch),
                       status);
  } else {
    hipLaunchKernelGGL(gather_u16_kernel, dim3(d.T), dim3(256), 0, st, d, slot_inst, slot_rank, inst_offset, hidden,
                       perm, slot_pos, dispatch, status);
  }
  return hipGetLastError();
}

}  // namespace moe
