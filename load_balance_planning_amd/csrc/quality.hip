// Plan-quality counters on gfx950.
//
// [TopoEP] section 6.2 Fig. 10 and section 6.4 Fig. 13(b) judge a plan by its
// rank-load imbalance (the largest rank load over the mean); section 6.6
// Fig. 16 by the share of assignments executed on another node than their
// source and the share executed by replicas.  From the plan's quotas
// q[s][i], instance ranks and experts and the rank loads, one workgroup sums
// (int64): all assignments, those on the source's rank, on its node, on
// another node, on a replica (an instance not on its expert's main rank
// e / (E/R)); and takes the largest and smallest rank load and the replica
// count.  The quota matrix is R x (E+B) int32 -- tens of KiB -- read once,
// coalesced along instances, one source row per wave at a time.
#include "internal.h"

namespace moe {
namespace {

constexpr int kQualThreads = 1024;

__device__ __forceinline__ int64_t wave_sum64(int64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__global__ __launch_bounds__(kQualThreads) void quality_kernel(Dims d, const int32_t* __restrict__ n_inst_p,
                                                               const int32_t* __restrict__ inst_expert,
                                                               const int32_t* __restrict__ inst_rank,
                                                               const int32_t* __restrict__ rank_load,
                                                               const int32_t* __restrict__ quota,
                                                               int64_t* __restrict__ out, int32_t* __restrict__ status) {
  extern __shared__ int32_t smem_q[];
  int32_t* rank_s = smem_q;              // [cap] rank of each instance
  int32_t* repl_s = smem_q + d.cap;      // [cap] 1 when the instance is a replica
  int32_t* node_s = smem_q + 2 * d.cap;  // [cap] node of each instance's rank
  __shared__ int64_t part[4][kQualThreads / 64];
  __shared__ int32_t lo_s[kQualThreads / 64], hi_s[kQualThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int n = *n_inst_p;
  if (n < d.E || n > d.cap) {
    if (tid == 0) atomicOr(status, MOE_STATUS_PLAN_CHECK);
    n = n < d.E ? d.E : d.cap;
  }
  bool bad = false;
  for (int i = tid; i < n; i += kQualThreads) {
    const int r = inst_rank[i], e = inst_expert[i];
    const bool ok = (unsigned)r < (unsigned)d.R && (unsigned)e < (unsigned)d.E;
    bad |= !ok;
    rank_s[i] = ok ? r : -1;
    repl_s[i] = ok && r != e / d.Er;
    node_s[i] = ok ? r / d.G : -1;
  }
  if (bad) atomicOr(status, MOE_STATUS_PLAN_CHECK);
  __syncthreads();
  int64_t tot = 0, same_rank = 0, same_node = 0, repl = 0;
  // one source row per wave at a time, lanes along the instances
  for (int s = wave; s < d.R; s += kQualThreads / 64) {
    const int32_t* row = quota + (int64_t)s * d.cap;
    const int sn = s / d.G;
#pragma unroll 4
    for (int i = lane; i < n; i += 64) {
      const int64_t q = row[i];
      const int r = rank_s[i];
      tot += q;
      same_rank += r == s ? q : 0;
      same_node += node_s[i] == sn ? q : 0;
      repl += repl_s[i] ? q : 0;
    }
  }
  int lo = INT32_MAX, hi = INT32_MIN;
  for (int r = tid; r < d.R; r += kQualThreads) {
    lo = min(lo, rank_load[r]);
    hi = max(hi, rank_load[r]);
  }
  tot = wave_sum64(tot);
  same_rank = wave_sum64(same_rank);
  same_node = wave_sum64(same_node);
  repl = wave_sum64(repl);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    lo = min(lo, __shfl_xor(lo, off));
    hi = max(hi, __shfl_xor(hi, off));
  }
  if (lane == 0) {
    part[0][wave] = tot;
    part[1][wave] = same_rank;
    part[2][wave] = same_node;
    part[3][wave] = repl;
    lo_s[wave] = lo;
    hi_s[wave] = hi;
  }
  __syncthreads();
  if (tid == 0) {
    int64_t v[4] = {0, 0, 0, 0};
    int mn = INT32_MAX, mx = INT32_MIN;
    for (int w = 0; w < kQualThreads / 64; ++w) {
      for (int j = 0; j < 4; ++j) v[j] += part[j][w];
      mn = min(mn, lo_s[w]);
      mx = max(mx, hi_s[w]);
    }
    out[0] = v[0];
    out[1] = v[1];
    out[2] = v[2];
    out[3] = v[0] - v[2];
    out[4] = v[3];
    out[5] = mx;
    out[6] = mn;
    out[7] = n - d.E;
  }
}

}  // namespace

hipError_t launch_quality(const Dims& d, const moe_plan_out& plan, int64_t* out, int32_t* status, hipStream_t st) {
  const size_t lds = sizeof(int32_t) * 3 * (size_t)d.cap;
  hipLaunchKernelGGL(quality_kernel, dim3(1), dim3(kQualThreads), lds, st, d, plan.n_inst, plan.inst_expert,
                     plan.inst_rank, plan.rank_load, plan.quota, out, status);
  return hipGetLastError();
}

}  // namespace moe
