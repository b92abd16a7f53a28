// Per-tile histogram scan shared by the route kernels and the plan launch.
//
// For a block of kScanEB experts and every source rank: the routing matrix
// row sums omega[s][e] = sum of popcount(tile_mask[x][e]) over the tiles x of
// source s ([TopoEP] Eq. 3), the expert counts, and tile_base[x][e], the
// exclusive prefix of those popcounts over all tiles in token order; or,
// instead of writing the routing matrix, a comparison with a given one.  Thread
// (row, e) of the workgroup: NTHR / kScanEB rows; when there are fewer
// sources than rows each source's tiles are split over several rows.
// Prefixes go over the rows of a source (chunks of tiles), then over sources.
#pragma once

#include "internal.h"

namespace moe {

constexpr int kScanEB = 16;

// LDS (bytes) of one scan workgroup of nthr threads.
inline size_t tile_scan_lds_bytes(const Dims& d, int nthr) {
  const int rows = nthr / kScanEB;
  const int rps = d.R < rows ? rows / d.R : 1;
  return sizeof(int32_t) * ((size_t)d.R * rps * kScanEB + (size_t)d.R * kScanEB);
}

// Expert block blk (experts blk*kScanEB ...).  tile_base, omega, count and
// check may be null; a routing-matrix entry that differs from check sets
// MOE_STATUS_BAD_OMEGA in *status.
template <int NTHR>
__device__ __forceinline__ void tile_scan_block(const Dims& d, const uint64_t* __restrict__ tile_mask,
                                                int32_t* __restrict__ tile_base, int32_t* __restrict__ omega,
                                                int32_t* __restrict__ count, const int32_t* __restrict__ check,
                                                int32_t* __restrict__ status, int blk, int32_t* smem) {
  constexpr int kRows = NTHR / kScanEB;
  const int el = threadIdx.x % kScanEB, row = threadIdx.x / kScanEB;
  const int e = blk * kScanEB + el;
  const bool ok = e < d.E;
  const int R = d.R, C = d.C;
  const int rps = R < kRows ? kRows / R : 1;  // rows per source
  const int cc = (C + rps - 1) / rps;         // tiles per row
  int32_t* part = smem;                       // [R][rps][EB] chunk sums -> chunk prefixes
  int32_t* tot = smem + R * rps * kScanEB;    // [R][EB] source sums -> source prefixes
  // rows handle the (source, chunk) pairs r = row, row + kRows, ... of R * rps
  for (int r = row; r < R * rps; r += kRows) {
    const int src = r / rps, ch = r - src * rps;
    const int c0 = ch * cc, c1 = min(C, c0 + cc);
    int sum = 0;
    if (ok) {
      const uint64_t* m = tile_mask + ((int64_t)src * C) * d.E + e;
#pragma unroll 4
      for (int c2 = c0; c2 < c1; ++c2) sum += __popcll(m[(int64_t)c2 * d.E]);
    }
    part[r * kScanEB + el] = sum;
  }
  __syncthreads();
  for (int q = threadIdx.x; q < R * kScanEB; q += NTHR) {
    const int src = q / kScanEB, l = q - src * kScanEB;
    int run = 0;
    for (int ch = 0; ch < rps; ++ch) {
      const int v = part[(src * rps + ch) * kScanEB + l];
      part[(src * rps + ch) * kScanEB + l] = run;
      run += v;
    }
    tot[src * kScanEB + l] = run;
    if (blk * kScanEB + l < d.E) {
      const int64_t at = (int64_t)src * d.E + blk * kScanEB + l;
      if (omega) omega[at] = run;
      if (check && check[at] != run) atomicOr(status, MOE_STATUS_BAD_OMEGA);
    }
  }
  __syncthreads();
  if (threadIdx.x < kScanEB) {
    int run = 0;
    for (int src = 0; src < R; ++src) {
      const int v = tot[src * kScanEB + el];
      tot[src * kScanEB + el] = run;
      run += v;
    }
    if (ok && count) count[e] = run;
  }
  __syncthreads();
  if (!tile_base) return;
  for (int r = row; r < R * rps; r += kRows) {
    const int src = r / rps, ch = r - src * rps;
    const int c0 = ch * cc, c1 = min(C, c0 + cc);
    if (!ok) continue;
    int run = tot[src * kScanEB + el] + part[r * kScanEB + el];
    const int64_t base = ((int64_t)src * C) * d.E + e;
#pragma unroll 4
    for (int c2 = c0; c2 < c1; ++c2) {
      const int64_t idx = base + (int64_t)c2 * d.E;
      tile_base[idx] = run;
      run += __popcll(tile_mask[idx]);
    }
  }
}

}  // namespace moe
