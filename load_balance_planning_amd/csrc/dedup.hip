// Deduplicated dispatch on gfx950.
//
// [Coupling] "Moving Correlated Experts Together", Fig. 3: a token whose
// selected experts share a destination rank travels there once, with the list
// of its slots that rank serves.  Slot q = t*k+j goes to rank key_rank[key[q]]
// (expert ids with a placement table, or instance ids with the planner's
// instance ranks; without a table the contiguous placement key / (E/R)).
// Rows are ordered by destination rank, then token.
//
// Three launches, the rank-keyed twin of the routing histogram:
//   masks   one workgroup per 64-token tile of one source: bit i of
//           mask[x][r] is set when token i of tile x has a slot on rank r
//           (plus per-tile slot counts); each token's distinct-rank count;
//   scan    tile_scan_block with ranks as the columns: rows per (source, rank),
//           rows per rank, and every tile's exclusive row prefix per rank;
//   gather  one workgroup per token: the row of (rank r, token t) is
//           offset[r] + base[x][r] + popcount(mask[x][r] below t); the first
//           slot of each rank writes the row's token and slot mask, every slot
//           its row, and the hidden row is read once and written to the
//           token's distinct ranks.  HBM traffic T*H*2 read plus
//           n_rows*H*2 written, n_rows = sum of the distinct-rank counts.
#include "internal.h"
#include "row_stage.h"
#include "tile_scan.h"

namespace moe {
namespace {

struct KeyMap {
  const int32_t* key;   // [T*k] slot keys
  const int32_t* rank;  // [n] key -> rank, or null: key / Er
  int32_t n;
};

__device__ __forceinline__ int slot_dest(const Dims& d, const KeyMap& km, int64_t q) {
  const int32_t key = km.key[q];
  int r;
  if (km.rank) r = (unsigned)key < (unsigned)km.n ? km.rank[key] : -1;
  else r = (unsigned)key < (unsigned)d.E ? key / d.Er : -1;
  return (unsigned)r < (unsigned)d.R ? r : -1;
}

constexpr int kMaskThreads = 256;

__global__ __launch_bounds__(kMaskThreads) void dedup_mask_kernel(Dims d, KeyMap km, uint64_t* __restrict__ mask,
                                                                  int32_t* __restrict__ cnt,
                                                                  int32_t* __restrict__ tok_ranks,
                                                                  int32_t* __restrict__ status) {
  __shared__ uint64_t rmask[kMaxR];
  __shared__ int32_t rcnt[kMaxR];
  __shared__ int32_t part[kMaskThreads / 64][64];
  const int x = blockIdx.x, tid = threadIdx.x;
  const int s = x / d.C, c = x - s * d.C;
  const int64_t t0 = (int64_t)s * d.Tr + (int64_t)c * kTile;
  const int nt = min(kTile, d.Tr - c * kTile);
  for (int r = tid; r < d.R; r += kMaskThreads) {
    rmask[r] = 0;
    rcnt[r] = 0;
  }
  __syncthreads();
  bool bad = false;
  for (int q = tid; q < nt * d.k; q += kMaskThreads) {
    const int i = q / d.k;
    const int r = slot_dest(d, km, t0 * d.k + q);
    if (r < 0) {
      bad = true;
      continue;
    }
    atomicOr(&rmask[r], 1ull << i);
    atomicAdd(&rcnt[r], 1);
  }
  if (bad) atomicOr(status, MOE_STATUS_BAD_KEY);
  __syncthreads();
  {
    const int i = tid & 63, g = tid >> 6;
    int n = 0;
    for (int r = g; r < d.R; r += kMaskThreads / 64) n += (int)(rmask[r] >> i & 1ull);
    part[g][i] = n;
  }
  __syncthreads();
  if (tid < nt) {
    int n = 0;
#pragma unroll
    for (int g = 0; g < kMaskThreads / 64; ++g) n += part[g][tid];
    tok_ranks[t0 + tid] = n;
  }
  for (int r = tid; r < d.R; r += kMaskThreads) {
    mask[(int64_t)x * d.R + r] = rmask[r];
    cnt[(int64_t)x * d.R + r] = rcnt[r];
  }
}

__global__ __launch_bounds__(1024) void dedup_scan_kernel(Dims d, const uint64_t* __restrict__ mask,
                                                          const int32_t* __restrict__ cnt, int32_t* __restrict__ base,
                                                          int32_t* __restrict__ rank_rows,
                                                          int32_t* __restrict__ rank_count,
                                                          int32_t* __restrict__ rank_slots) {
  extern __shared__ int32_t smem_dscan[];
  Dims dr = d;
  dr.E = d.R;  // ranks are the columns
  tile_scan_block<1024>(dr, mask, base, rank_rows, rank_count, nullptr, nullptr, blockIdx.x, smem_dscan);
  if (rank_slots) {
    for (int q = threadIdx.x; q < d.R * kScanEB; q += 1024) {
      const int src = q / kScanEB, r = blockIdx.x * kScanEB + (q - src * kScanEB);
      if (r >= d.R) continue;
      int sum = 0;
      for (int c = 0; c < d.C; ++c) sum += cnt[((int64_t)src * d.C + c) * d.R + r];
      rank_slots[(int64_t)src * d.R + r] = sum;
    }
  }
}

struct GatherOut {
  int32_t* row_token;
  int32_t* row_slots;
  int32_t* slot_row;
  int32_t* rank_row_offset;
  int32_t* n_rows;
  int32_t* status;
};

// One workgroup per token (the grid has at least one workgroup, which also
// writes the rank offsets when T = 0).
template <bool VEC, int VPT>
__global__ __launch_bounds__(256) void dedup_gather_kernel(Dims d, KeyMap km, const uint64_t* __restrict__ mask,
                                                           const int32_t* __restrict__ base,
                                                           const int32_t* __restrict__ rank_count,
                                                           const uint16_t* __restrict__ hidden,
                                                           uint16_t* __restrict__ out, GatherOut go) {
  __shared__ int32_t off_s[kMaxR + 1];
  __shared__ int32_t wtot[4];
  __shared__ int32_t row_s[kMaxK];
  __shared__ int32_t nd_s;
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool live = t < d.T;
  const int64_t N = (int64_t)d.T * d.k;
  const int vpr = VEC ? d.H / 8 : d.H;
  __shared__ uint4 stage_s[VPT * 256];
  RowStage<VPT> v{stage_s};
  if (VEC && live) v.load(reinterpret_cast<const uint4*>(hidden) + t * vpr, tid, vpr);
  // Exclusive prefix of the per-rank row counts (R <= 256: one per thread).
  int cntv = tid < d.R ? rank_count[tid] : 0;
  int inc = cntv;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  if (lane == 63) wtot[wave] = inc;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wtot[w];
  if (tid < d.R) off_s[tid] = before + inc - cntv;
  if (tid == 0) off_s[d.R] = wtot[0] + wtot[1] + wtot[2] + wtot[3];
  __syncthreads();
  const int n_rows = off_s[d.R];
  if (t == 0)
    for (int r = tid; r <= d.R; r += 256) go.rank_row_offset[r] = off_s[r];
  if (t == 0 && tid == 0) *go.n_rows = n_rows;
  if (!live) return;

  if (wave == 0) {
    const int s = (int)(t / d.Tr), ti = (int)(t - (int64_t)s * d.Tr);
    const int64_t x = (int64_t)s * d.C + ti / kTile;
    const int i = ti % kTile;
    const bool on = lane < d.k;
    const int r = on ? slot_dest(d, km, t * d.k + lane) : -2;
    uint32_t same = 0;  // slots of this token with the same destination
    for (int jj = 0; jj < d.k; ++jj) same |= (uint32_t)(__shfl(r, jj) == r) << jj;
    const bool lead = on && r >= 0 && (__ffs(same) - 1) == lane;
    int p = -1;
    if (lead) {
      const uint64_t m = mask[x * d.R + r];
      const int64_t pp = (int64_t)off_s[r] + base[x * d.R + r] + __popcll(m & ((1ull << i) - 1));
      if (pp >= 0 && pp < N && (m >> i & 1ull)) {
        p = (int)pp;
        go.row_token[p] = (int32_t)t;
        go.row_slots[p] = (int32_t)same;
      } else {
        atomicOr(go.status, MOE_STATUS_PLAN_CHECK);
      }
    }
    const int pr = __shfl(p, on && r >= 0 ? __ffs(same) - 1 : lane);
    if (on) {
      go.slot_row[t * d.k + lane] = r >= 0 ? pr : -1;
      if (r < 0) atomicOr(go.status, MOE_STATUS_BAD_KEY);
    }
    const uint64_t leaders = __ballot(lead && p >= 0);
    if (lead && p >= 0) row_s[__popcll(leaders & ((1ull << lane) - 1))] = p;
    if (lane == 0) nd_s = __popcll(leaders);
  }
  __syncthreads();
  const int nd = nd_s;
  if (VEC) {
    const uint4* src = reinterpret_cast<const uint4*>(hidden) + t * vpr;
    for (int b0 = 0; b0 < vpr; b0 += 256 * VPT) {
      if (b0 > 0) v.load(src, b0 + tid, vpr);
      for (int j = 0; j < nd; ++j) v.store(reinterpret_cast<uint4*>(out) + (int64_t)row_s[j] * vpr, b0 + tid, vpr);
    }
  } else {
    const uint16_t* src = hidden + t * d.H;
    for (int c = tid; c < d.H; c += 256) {
      const uint16_t h = src[c];
      for (int j = 0; j < nd; ++j) out[(int64_t)row_s[j] * d.H + c] = h;
    }
  }
  // Rows past n_rows: -1.
  for (int64_t q = n_rows + t; q < N; q += d.T) {
    go.row_token[q] = -1;
    go.row_slots[q] = -1;
  }
}

hipError_t launch_counts(const Dims& d, const KeyMap& km, const moe_dedup_out& out, const Workspace& ws,
                         hipStream_t st) {
  if (d.NT > 0)
    hipLaunchKernelGGL(dedup_mask_kernel, dim3(d.NT), dim3(kMaskThreads), 0, st, d, km, ws.dd_mask, ws.dd_cnt,
                       out.tok_ranks, ws.status);
  const size_t lds = dedup_scan_lds_bytes(d);
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(dedup_scan_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(dedup_scan_kernel, dim3((d.R + kScanEB - 1) / kScanEB), dim3(1024), lds, st, d, ws.dd_mask,
                     ws.dd_cnt, ws.dd_base, out.rank_rows, ws.dd_count, out.rank_slots);
  return hipGetLastError();
}

}  // namespace

size_t dedup_scan_lds_bytes(const Dims& d) {
  Dims dr = d;
  dr.E = d.R;
  return tile_scan_lds_bytes(dr, 1024);
}

hipError_t launch_dedup(const Dims& d, const int32_t* slot_key, const int32_t* key_rank, int32_t n_keys,
                        const uint16_t* hidden, const moe_dedup_out& out, const Workspace& ws, hipStream_t st) {
  const KeyMap km{slot_key, key_rank, n_keys};
  hipError_t e = launch_counts(d, km, out, ws, st);
  if (e != hipSuccess || !hidden) return e;
  const GatherOut go{out.row_token, out.row_slots, out.slot_row, out.rank_row_offset, out.n_rows, ws.status};
  const bool vec = (d.H % 8) == 0 && ((uintptr_t)hidden % 16) == 0 && ((uintptr_t)out.ddispatch % 16) == 0;
  const dim3 grid(d.T > 0 ? d.T : 1);
  // a row of at most 256 vectors takes one store round: no dead registers
  if (vec && d.H / 8 <= 256)
    hipLaunchKernelGGL((dedup_gather_kernel<true, 1>), grid, dim3(256), 0, st, d, km, ws.dd_mask, ws.dd_base,
                       ws.dd_count, hidden, out.ddispatch, go);
  else if (vec)
    hipLaunchKernelGGL((dedup_gather_kernel<true, 4>), grid, dim3(256), 0, st, d, km, ws.dd_mask, ws.dd_base,
                       ws.dd_count, hidden, out.ddispatch, go);
  else
    hipLaunchKernelGGL((dedup_gather_kernel<false, 4>), grid, dim3(256), 0, st, d, km, ws.dd_mask, ws.dd_base,
                       ws.dd_count, hidden, out.ddispatch, go);
  return hipGetLastError();
}

}  // namespace moe
