// Replica slots and their parameter / gradient transfers on gfx950.
//
// [TopoEP] section 3.2 (Replica Buffer Management) and Fig. 6: each rank keeps
// N_slot replica slots, reused across layers and microbatches; the plan maps
// every occupied slot to an expert and so to the expert's main rank, which
// supplies the BF16 parameters in the forward pass and receives the
// gradients in the backward pass (the optimizer state never moves).  The
// replicas of a rank fill its slots in instance order (ascending expert):
// instances are rank-major with a rank's E/R main experts first, so the slot
// of replica instance i on rank r is i - first(r) - E/R.
//
// The transfers are row copies of P bf16 elements per expert: the pull
//   replica_params[r][j] = main_params[e]                    ([R][N_slot][P] <- [E][P])
// and the return
//   grad_accum[main(e)][r][e - main(e)*E/R] = replica_grads[r][j]   ([R][R][E/R][P])
// One workgroup column per slot (grid.x), chunks of 8192 elements along the
// row (grid.y, strided), 16-byte vectors when the rows allow; HBM traffic is
// one read and one write of every occupied slot's row.  The vector stores
// carry the nontemporal hint (nothing here reads the copied rows back): on
// MI355X that lifts the copy from 4.7 to 5.3 TB/s, with 512 threads of two
// vectors each (256 x 4 reaches 5.2).
#include "internal.h"

namespace moe {
namespace {

constexpr int kMapThreads = 1024;
constexpr int kCopyThreads = 512;
constexpr int kCopyVpt = 2;                                  // 16-byte vectors per thread
constexpr int64_t kChunk = (int64_t)kCopyThreads * kCopyVpt * 8;  // bf16 elements per chunk

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void store_stream(uint4* p, const uint4& v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}

__global__ __launch_bounds__(kMapThreads) void slot_map_kernel(Dims d, const int32_t* __restrict__ n_inst_p,
                                                               const int32_t* __restrict__ inst_expert,
                                                               const int32_t* __restrict__ inst_rank,
                                                               int32_t* __restrict__ slot_expert,
                                                               int32_t* __restrict__ slot_main,
                                                               int32_t* __restrict__ inst_slot,
                                                               int32_t* __restrict__ status) {
  __shared__ int32_t first[kMaxR];
  const int tid = threadIdx.x;
  int n = *n_inst_p;
  bool bad = n < d.E || n > d.cap;
  n = n < d.E ? d.E : n > d.cap ? d.cap : n;
  const int64_t nslots = (int64_t)d.R * d.n_slot;
  for (int64_t q = tid; q < nslots; q += kMapThreads) slot_expert[q] = slot_main[q] = -1;
  for (int i = tid; i < d.cap; i += kMapThreads) inst_slot[i] = -1;
  for (int r = tid; r < d.R; r += kMapThreads) first[r] = -1;
  __syncthreads();
  for (int i = tid; i < n; i += kMapThreads) {
    const int r = inst_rank[i];
    if ((unsigned)r >= (unsigned)d.R) continue;
    if (i == 0 || inst_rank[i - 1] != r) first[r] = i;
  }
  __syncthreads();
  for (int i = tid; i < n; i += kMapThreads) {
    const int r = inst_rank[i], e = inst_expert[i];
    if ((unsigned)r >= (unsigned)d.R || (unsigned)e >= (unsigned)d.E || first[r] < 0) {
      bad = true;
      continue;
    }
    const int m = e / d.Er, pos = i - first[r];
    if (m == r) {
      bad |= pos >= d.Er;  // main instances come first on their rank
      continue;
    }
    const int j = pos - d.Er;
    if (j < 0 || j >= d.n_slot) {
      bad = true;
      continue;
    }
    slot_expert[(int64_t)r * d.n_slot + j] = e;
    slot_main[(int64_t)r * d.n_slot + j] = m;
    inst_slot[i] = j;
  }
  if (bad) atomicOr(status, MOE_STATUS_PLAN_CHECK);
}

// Copies row src_row(slot) to dst_row(slot) for every occupied slot.  PUSH
// selects the gradient return's addressing, else the parameter pull's.
template <bool PUSH, bool VEC>
__global__ __launch_bounds__(kCopyThreads) void slot_copy_kernel(Dims d, const int32_t* __restrict__ slot_expert,
                                                                 const uint16_t* __restrict__ src,
                                                                 uint16_t* __restrict__ dst, int64_t P,
                                                                 int32_t* __restrict__ status) {
  const int64_t q = blockIdx.x;  // slot r * N_slot + j
  const int e = slot_expert[q];
  if (e < 0) return;
  if (e >= d.E) {
    if (threadIdx.x == 0) atomicOr(status, MOE_STATUS_PLAN_CHECK);
    return;
  }
  const int64_t r = q / d.n_slot, m = e / d.Er;
  const uint16_t* s;
  uint16_t* t;
  if (PUSH) {
    s = src + q * P;
    t = dst + ((m * d.R + r) * d.Er + (e - m * d.Er)) * P;
  } else {
    s = src + (int64_t)e * P;
    t = dst + q * P;
  }
  for (int64_t c0 = (int64_t)blockIdx.y * kChunk; c0 < P; c0 += (int64_t)gridDim.y * kChunk) {
    if (VEC) {
      const uint4* sv = reinterpret_cast<const uint4*>(s + c0);
      uint4* tv = reinterpret_cast<uint4*>(t + c0);
      const int64_t nv = min((int64_t)kCopyThreads * kCopyVpt, (P - c0) / 8);
      uint4 v[kCopyVpt];
#pragma unroll
      for (int u = 0; u < kCopyVpt; ++u) {
        const int64_t i = threadIdx.x + (int64_t)u * kCopyThreads;
        if (i < nv) v[u] = sv[i];
      }
#pragma unroll
      for (int u = 0; u < kCopyVpt; ++u) {
        const int64_t i = threadIdx.x + (int64_t)u * kCopyThreads;
        if (i < nv) store_stream(tv + i, v[u]);
      }
    } else {
      const int64_t n = min(kChunk, P - c0);
      for (int64_t i = threadIdx.x; i < n; i += kCopyThreads) t[c0 + i] = s[c0 + i];
    }
  }
}

template <bool PUSH>
hipError_t launch_copy(const Dims& d, const int32_t* slot_expert, const uint16_t* src, uint16_t* dst, int64_t P,
                       int32_t* status, hipStream_t st) {
  const int64_t rows = (int64_t)d.R * d.n_slot;
  if (rows == 0 || P == 0) return hipSuccess;
  const int64_t chunks = (P + kChunk - 1) / kChunk;
  const dim3 grid((unsigned)rows, (unsigned)(chunks < 65535 ? chunks : 65535));
  const bool vec = P % 8 == 0 && (uintptr_t)src % 16 == 0 && (uintptr_t)dst % 16 == 0;
  if (vec)
    hipLaunchKernelGGL((slot_copy_kernel<PUSH, true>), grid, dim3(kCopyThreads), 0, st, d, slot_expert, src, dst, P,
                       status);
  else
    hipLaunchKernelGGL((slot_copy_kernel<PUSH, false>), grid, dim3(kCopyThreads), 0, st, d, slot_expert, src, dst, P,
                       status);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_slot_map(const Dims& d, const moe_plan_out& plan, const moe_slot_out& out, int32_t* status,
                           hipStream_t st) {
  hipLaunchKernelGGL(slot_map_kernel, dim3(1), dim3(kMapThreads), 0, st, d, plan.n_inst, plan.inst_expert,
                     plan.inst_rank, out.slot_expert, out.slot_main, out.inst_slot, status);
  return hipGetLastError();
}

hipError_t launch_replica_pull(const Dims& d, const int32_t* slot_expert, const uint16_t* main_params, int64_t P,
                               uint16_t* replica_params, int32_t* status, hipStream_t st) {
  return launch_copy<false>(d, slot_expert, main_params, replica_params, P, status, st);
}

hipError_t launch_replica_push(const Dims& d, const int32_t* slot_expert, const uint16_t* replica_grads, int64_t P,
                               uint16_t* grad_accum, int32_t* status, hipStream_t st) {
  return launch_copy<true>(d, slot_expert, replica_grads, grad_accum, P, status, st);
}

}  // namespace moe
