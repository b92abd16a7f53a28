// Dispatch layout and bf16 row gather on gfx950.
//
// [TopoEP] section 5: the plan stays on the device and the receive counts are
// derived there.  The layout is a stable counting sort of the slots by
// instance: the plan gives the instance offsets (exclusive prefix of the
// instance loads) and each slot's position inside its instance (slot_rank),
// so slot_pos = inst_offset[slot_inst] + slot_rank with no sort, and the
// whole dispatch is one kernel.
//
// The copy is source-ordered: each hidden row is read from HBM once and
// written to its k dispatch rows, so HBM traffic is T*H*2 bytes read plus
// T*k*H*2 bytes written -- a destination-ordered gather would read each row
// k times (and measured slower on MI355X).  Plain stores: on MI355X they beat
// non-temporal ones for this write pattern.
#include "internal.h"
#include "slot_assign.h"

namespace moe {
namespace {

// Inputs of the slot assignment when the gather does it (single-call step).
struct AssignIn {
  const int32_t* topk;
  const uint64_t* tile_mask;
  const int32_t* tile_base;
  const int32_t* quota;
  int32_t* slot_inst;  // written
  int32_t* slot_rank;  // written
  int32_t* clear;      // zeroed, [0, clear_n) (nullable): a buffer no earlier kernel still reads
  int64_t clear_n;
};

// One workgroup per token.  Threads j < k place slot t*k+j -- reading its
// instance and rank, or with ASSIGN computing them from the plan
// (slot_assign.h) and writing them; the workgroup loads its hidden row (the
// first 256*VPT vectors) and writes it to its k destinations (16-byte
// vectors, plain stores).
template <int VPT, bool ASSIGN>
__global__ __launch_bounds__(256) void gather_vec_kernel(Dims d, const int32_t* __restrict__ slot_inst,
                                                         const int32_t* __restrict__ slot_rank,
                                                         const int32_t* __restrict__ inst_offset,
                                                         const uint4* __restrict__ hidden, int32_t* __restrict__ perm,
                                                         int32_t* __restrict__ slot_pos, uint4* __restrict__ dispatch,
                                                         AssignIn as, Workspace ws) {
  __shared__ int32_t pos_s[kMaxK];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t N = (int64_t)d.T * d.k;
  const int vpr = d.H / 8;
  const uint4* src = hidden + t * vpr;
  // Measured on MI355X: with the long chain of the assignment, issuing the
  // row loads first and overlapping them pays; with the two loads of a plain
  // placement, loading after the positions is faster.
  constexpr bool kLoadFirst = ASSIGN;
  uint4 v[VPT];
  if (kLoadFirst) {
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int c = tid + u * 256;
      if (c < vpr) v[u] = src[c];
    }
  }
  if (ASSIGN)
    for (int64_t q = t * 256 + tid; q < as.clear_n; q += (int64_t)gridDim.x * 256) as.clear[q] = 0;
  if (tid < d.k) {
    const int64_t sigma = t * d.k + tid;
    int i, r;
    if (ASSIGN) {
      assign_slot(d, sigma, as.topk, as.tile_mask, as.tile_base, as.quota, ws, i, r);
      as.slot_inst[sigma] = i;
      as.slot_rank[sigma] = r;
    } else {
      i = slot_inst[sigma];
      r = slot_rank[sigma];
    }
    int64_t p = -1;
    if ((unsigned)i < (unsigned)d.cap) p = (int64_t)inst_offset[i] + r;
    if (p < 0 || p >= N) {
      atomicOr(ws.status, MOE_STATUS_PLAN_CHECK);
      p = -1;
    } else {
      perm[p] = (int32_t)sigma;
    }
    slot_pos[sigma] = (int32_t)p;
    pos_s[tid] = (int32_t)p;
  }
  if (!kLoadFirst) {
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int c = tid + u * 256;
      if (c < vpr) v[u] = src[c];
    }
  }
  __syncthreads();
  for (int base = 0; base < vpr; base += 256 * VPT) {
    if (base > 0) {
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        const int c = base + tid + u * 256;
        if (c < vpr) v[u] = src[c];
      }
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

// A row of at most 256 vectors is one store round of the workgroup: the
// VPT = 1 instantiation then carries no dead loads, stores or registers
// (measured on MI355X: Qwen3-shaped step 160 -> 154 us, Mixtral-shaped 45 -> 32 us).
bool one_round(const Dims& d) { return d.H / 8 <= 256; }

}  // namespace

hipError_t launch_gather(const Dims& d, const int32_t* slot_inst, const int32_t* slot_rank,
                         const int32_t* inst_offset, const uint16_t* hidden, int32_t* perm, int32_t* slot_pos,
                         uint16_t* dispatch, const Workspace& ws, hipStream_t st) {
  if (d.T == 0) return hipSuccess;
  const bool vec = (d.H % 8) == 0 && ((uintptr_t)hidden % 16) == 0 && ((uintptr_t)dispatch % 16) == 0;
  if (vec) {
    if (one_round(d))
      hipLaunchKernelGGL((gather_vec_kernel<1, false>), dim3(d.T), dim3(256), 0, st, d, slot_inst, slot_rank,
                         inst_offset, reinterpret_cast<const uint4*>(hidden), perm, slot_pos,
                         reinterpret_cast<uint4*>(dispatch), AssignIn{}, ws);
    else
      hipLaunchKernelGGL((gather_vec_kernel<4, false>), dim3(d.T), dim3(256), 0, st, d, slot_inst, slot_rank,
                         inst_offset, reinterpret_cast<const uint4*>(hidden), perm, slot_pos,
                         reinterpret_cast<uint4*>(dispatch), AssignIn{}, ws);
  } else {
    hipLaunchKernelGGL(gather_u16_kernel, dim3(d.T), dim3(256), 0, st, d, slot_inst, slot_rank, inst_offset, hidden,
                       perm, slot_pos, dispatch, ws.status);
  }
  return hipGetLastError();
}

bool gather_can_assign(const Dims& d, const uint16_t* hidden, const uint16_t* dispatch) {
  return (d.H % 8) == 0 && ((uintptr_t)hidden % 16) == 0 && ((uintptr_t)dispatch % 16) == 0;
}

hipError_t launch_assign_gather(const Dims& d, const int32_t* topk_idx, const uint64_t* tile_mask,
                                const int32_t* tile_base, const moe_plan_out& plan, const uint16_t* hidden,
                                int32_t* perm, int32_t* slot_pos, uint16_t* dispatch, const Workspace& ws,
                                int32_t* clear, int64_t clear_n, hipStream_t st) {
  if (d.T == 0) return hipSuccess;
  const AssignIn as{topk_idx, tile_mask, tile_base, plan.quota, plan.slot_inst, plan.slot_rank, clear,
                    clear ? clear_n : 0};
  if (one_round(d))
    hipLaunchKernelGGL((gather_vec_kernel<1, true>), dim3(d.T), dim3(256), 0, st, d, nullptr, nullptr,
                       plan.inst_offset, reinterpret_cast<const uint4*>(hidden), perm, slot_pos,
                       reinterpret_cast<uint4*>(dispatch), as, ws);
  else
    hipLaunchKernelGGL((gather_vec_kernel<4, true>), dim3(d.T), dim3(256), 0, st, d, nullptr, nullptr,
                       plan.inst_offset, reinterpret_cast<const uint4*>(hidden), perm, slot_pos,
                       reinterpret_cast<uint4*>(dispatch), as, ws);
  return hipGetLastError();
}

}  // namespace moe
