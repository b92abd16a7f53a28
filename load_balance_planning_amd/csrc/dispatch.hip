// Dispatch layout and bf16 row gather on gfx950.
//
// [TopoEP] section 5: the plan stays on the device and the receive counts are
// derived there.  The layout is a stable counting sort of the slots by
// instance: the instance offsets are the exclusive prefix of the instance
// loads (one small workgroup computes them), and the plan gives each slot's
// position inside its instance (slot_rank), so slot_pos =
// inst_offset[slot_inst] + slot_rank with no sort, and the row copy is one
// kernel.  (Scanning the loads inside every gather workgroup instead made the
// compiler keep the row in scratch memory while the scan ran: the DeepSeek-V3
// dispatch slowed from 0.83 to 1.34 ms on MI355X.)
//
// The copy is source-ordered: each hidden row is read from HBM once and
// written to its k dispatch rows, so HBM traffic is T*H*2 bytes read plus
// T*k*H*2 bytes written -- a destination-ordered gather would read each row
// k times (and measured slower on MI355X).  Plain stores: on MI355X they beat
// non-temporal ones for this write pattern.
#include "internal.h"
#include "row_stage.h"
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

// The plan's instance loads, for a dispatch that derives its own offsets.
struct OffsetsIn {
  const int32_t* n_inst;
  const int32_t* inst_load;
  const int32_t* inst_rank;
  int32_t* inst_offset;  // written by workgroup 0
  int32_t* rank_offset;  // written by workgroup 0
};

// Exclusive prefix of the instance loads and each rank's first row (instances
// are rank-major): one workgroup of 256 threads.  inst_offset gets -1 after
// entry n_inst; a rank without instances -- impossible in a plan of this
// library -- takes the next rank's offset.  An n_inst outside [0, cap] sets
// MOE_STATUS_PLAN_CHECK and is taken as 0.
__global__ __launch_bounds__(256) void offsets_kernel(Dims d, OffsetsIn in, int32_t* __restrict__ status) {
  extern __shared__ int32_t pre[];
  __shared__ int wsum[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int n = in.n_inst[0];
  if (n < 0 || n > d.cap) {
    if (tid == 0) atomicOr(status, MOE_STATUS_PLAN_CHECK);
    n = 0;
  }
  const int per = (n + 255) / 256;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int sum = 0;
  for (int q = lo; q < hi; ++q) sum += in.inst_load[q];
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  for (int r = tid; r < d.R; r += 256) in.rank_offset[r] = -1;
  __syncthreads();
  int run = incl - sum;
  for (int w = 0; w < wave; ++w) run += wsum[w];
  for (int q = lo; q < hi; ++q) {
    pre[q] = run;
    run += in.inst_load[q];
  }
  if (tid == 0) pre[n] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();
  for (int i = tid; i <= d.cap; i += 256) in.inst_offset[i] = i <= n ? pre[i] : -1;
  for (int q = tid; q < n; q += 256) {
    const int r = in.inst_rank[q];
    if ((unsigned)r < (unsigned)d.R && (q == 0 || in.inst_rank[q - 1] != r)) in.rank_offset[r] = pre[q];
  }
  __syncthreads();
  if (tid == 0) {
    int next = pre[n];
    for (int r = d.R - 1; r >= 0; --r) {
      if (in.rank_offset[r] < 0) in.rank_offset[r] = next;
      next = in.rank_offset[r];
    }
    in.rank_offset[d.R] = pre[n];
  }
}

// split * csplit adjacent workgroups per token: workgroup (part, half) takes
// the token's slots j in [part*k/split, (part+1)*k/split) and the half-th of
// csplit equal column ranges of the row.  Its first threads place those slots
// -- reading instance and rank, or with ASSIGN computing them from the plan
// (slot_assign.h) and writing them; the workgroup loads its range of the
// hidden row (256*VPT vectors at a time, staged through LDS: row_stage.h) and
// writes it to those destinations (16-byte vectors, plain stores).  Every
// column part writes the same perm / slot_pos entries with the same values.
template <int VPT, bool ASSIGN>
__global__ __launch_bounds__(256) void gather_vec_kernel(Dims d, const int32_t* __restrict__ slot_inst,
                                                         const int32_t* __restrict__ slot_rank,
                                                         const int32_t* __restrict__ inst_offset,
                                                         const uint4* __restrict__ hidden, int32_t* __restrict__ perm,
                                                         int32_t* __restrict__ slot_pos, uint4* __restrict__ dispatch,
                                                         AssignIn as, Workspace ws, int split, int csplit) {
  __shared__ int32_t pos_s[kMaxK];
  static_assert(sizeof(uint4) * VPT * 256 + sizeof(pos_s) <= kGatherWgLds, "the row copy's LDS");
  const int64_t t = blockIdx.x / (split * csplit);
  const int rem = (int)(blockIdx.x - t * (split * csplit)), part = rem / csplit, half = rem - part * csplit;
  const int j0 = part * d.k / split, kp = (part + 1) * d.k / split - j0;
  const int tid = threadIdx.x;
  const int64_t N = (int64_t)d.T * d.k;
  const int vpr = d.H / 8;
  const uint4* src = hidden + t * vpr;
  const int chunk = (vpr + csplit - 1) / csplit, cbeg = half * chunk, cend = min(vpr, cbeg + chunk);
  // Measured on MI355X: with the long chain of the assignment, issuing the
  // row loads first and overlapping them pays; with the two loads of a plain
  // placement, loading after the positions is faster.
  constexpr bool kLoadFirst = ASSIGN;
  __shared__ uint4 stage_s[VPT * 256];
  RowStage<VPT> v{stage_s};
  if (kLoadFirst) v.load(src, cbeg + tid, cend);
  if (ASSIGN)
    for (int64_t q = (int64_t)blockIdx.x * 256 + tid; q < as.clear_n; q += (int64_t)gridDim.x * 256) as.clear[q] = 0;
  if (tid < kp) {
    const int64_t sigma = t * d.k + j0 + tid;
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
  if (!kLoadFirst) v.load(src, cbeg + tid, cend);
  __syncthreads();
  for (int base = cbeg; base < cend; base += 256 * VPT) {
    if (base > cbeg) v.load(src, base + tid, cend);
    for (int j = 0; j < kp; ++j) {
      const int p = pos_s[j];
      if (p >= 0) v.store(dispatch + (int64_t)p * vpr, base + tid, cend);
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

// Parts per token of the row copy, measured on MI355X: the copy runs fastest
// when each workgroup writes about 56 KiB (3584 16-byte vectors), so a token
// writing k rows of vpr vectors takes floor(k * vpr / 3584) parts (at least
// one, at most four), split by columns first (each hidden row is then read
// once) and by destinations after.  DeepSeek-V3-shaped (k 8, 896 vectors):
// one part 780-797 us, two column parts 771-776, two destination parts
// 771-775 (reading each row twice), four parts 837; Kimi-K2-shaped (k 16):
// one part 783-790 us, two destination parts 735-740, two column parts 771,
// two of each 721; Qwen3-shaped (k 8, 256 vectors): one part 118 us, two
// 127-137.  Narrower column parts write shorter pieces of each row and run
// slower: four column parts (3.5 KiB pieces) 793 us on the DeepSeek-V3 shape
// and 747 us on the Kimi-K2 one, eight 1 000 and 791 us, four by two
// destination parts 954 and 784 us (against 777 and 727 us, same box).
constexpr int kCopyVectorsPerPart = 3584;
struct CopyParts {
  int split;   // destination parts
  int csplit;  // column parts
};
CopyParts copy_parts(const Dims& d) {
  const int vpr = d.H / 8;
  const int64_t n = std::min<int64_t>(4, std::max<int64_t>(1, (int64_t)d.k * vpr / kCopyVectorsPerPart));
  const int cs = n >= 2 && vpr >= 512 ? 2 : 1;
  return CopyParts{std::min(d.k, (int)n / cs), cs};
}

}  // namespace

hipError_t launch_gather(const Dims& d, const moe_plan_out& plan, const uint16_t* hidden, int32_t* perm,
                         int32_t* slot_pos, int32_t* inst_offset, int32_t* rank_offset, uint16_t* dispatch,
                         const Workspace& ws, const KernelEvents& ev, hipStream_t st) {
  const OffsetsIn oi{plan.n_inst, plan.inst_load, plan.inst_rank, inst_offset, rank_offset};
  hipLaunchKernelGGL(offsets_kernel, dim3(1), dim3(256), sizeof(int32_t) * (size_t)(d.cap + 1), st, d, oi, ws.status);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_gather_rows(d, plan, hidden, perm, slot_pos, inst_offset, dispatch, ws, ev, st);
}

hipError_t launch_gather_rows(const Dims& d, const moe_plan_out& plan, const uint16_t* hidden, int32_t* perm,
                              int32_t* slot_pos, const int32_t* inst_offset, uint16_t* dispatch, const Workspace& ws,
                              const KernelEvents& ev, hipStream_t st) {
  if (d.T == 0) return hipSuccess;
  hipError_t e;
  if ((e = gather_hooks_before(ev, st)) != hipSuccess) return e;
  if (gather_can_assign(d, hidden, dispatch)) {
    const CopyParts cp = copy_parts(d);
    const dim3 grid((unsigned)(d.T * cp.split * cp.csplit));
    if (one_round(d))
      hipLaunchKernelGGL((gather_vec_kernel<1, false>), grid, dim3(256), 0, st, d, plan.slot_inst, plan.slot_rank,
                         inst_offset, reinterpret_cast<const uint4*>(hidden), perm, slot_pos,
                         reinterpret_cast<uint4*>(dispatch), AssignIn{}, ws, cp.split, cp.csplit);
    else
      hipLaunchKernelGGL((gather_vec_kernel<4, false>), grid, dim3(256), 0, st, d, plan.slot_inst, plan.slot_rank,
                         inst_offset, reinterpret_cast<const uint4*>(hidden), perm, slot_pos,
                         reinterpret_cast<uint4*>(dispatch), AssignIn{}, ws, cp.split, cp.csplit);
  } else {
    hipLaunchKernelGGL(gather_u16_kernel, dim3(d.T), dim3(256), 0, st, d, plan.slot_inst, plan.slot_rank,
                       inst_offset, hidden, perm, slot_pos, dispatch, ws.status);
  }
  e = hipGetLastError();
  if (e == hipSuccess) e = gather_hooks_after(ev, st);
  return e;
}

hipError_t gather_hooks_before(const KernelEvents& ev, hipStream_t st) {
  hipError_t e = hipSuccess;
  if (ev.wait) e = hipStreamWaitEvent(st, ev.wait, 0);
  if (e == hipSuccess && ev.begin) e = hipEventRecord(ev.begin, st);
  return e;
}

hipError_t gather_hooks_after(const KernelEvents& ev, hipStream_t st) {
  hipError_t e = hipSuccess;
  if (ev.end) e = hipEventRecord(ev.end, st);
  if (e == hipSuccess && ev.done) e = hipEventRecord(ev.done, st);
  return e;
}

bool gather_can_assign(const Dims& d, const uint16_t* hidden, const uint16_t* dispatch) {
  return (d.H % 8) == 0 && ((uintptr_t)hidden % 16) == 0 && ((uintptr_t)dispatch % 16) == 0;
}

bool copy_in_one_part(const Dims& d) {
  const CopyParts cp = copy_parts(d);
  return cp.split * cp.csplit == 1;
}

hipError_t launch_assign_gather(const Dims& d, const int32_t* topk_idx, const uint64_t* tile_mask,
                                const int32_t* tile_base, const moe_plan_out& plan, const int32_t* inst_offset,
                                const uint16_t* hidden, int32_t* perm, int32_t* slot_pos, uint16_t* dispatch,
                                const Workspace& ws, int32_t* clear, int64_t clear_n, const KernelEvents& ev,
                                hipStream_t st) {
  if (d.T == 0) return hipSuccess;
  hipError_t e;
  if ((e = gather_hooks_before(ev, st)) != hipSuccess) return e;
  const AssignIn as{topk_idx, tile_mask, tile_base, plan.quota, plan.slot_inst, plan.slot_rank, clear,
                    clear ? clear_n : 0};
  if (one_round(d))
    hipLaunchKernelGGL((gather_vec_kernel<1, true>), dim3(d.T), dim3(256), 0, st, d, nullptr, nullptr, inst_offset,
                       reinterpret_cast<const uint4*>(hidden), perm, slot_pos, reinterpret_cast<uint4*>(dispatch), as,
                       ws, 1, 1);
  else
    hipLaunchKernelGGL((gather_vec_kernel<4, true>), dim3(d.T), dim3(256), 0, st, d, nullptr, nullptr, inst_offset,
                       reinterpret_cast<const uint4*>(hidden), perm, slot_pos, reinterpret_cast<uint4*>(dispatch), as,
                       ws, 1, 1);
  e = hipGetLastError();
  if (e == hipSuccess) e = gather_hooks_after(ev, st);
  return e;
}

}  // namespace moe
