// Pair counts (co-selection, layer-to-layer transitions) as a binary product
// over tiles, shared by the route kernels and the plan launch.
//
//   out[a][b] = sum_x popcount(A[x][a] & B[x][b])      ([Coupling])
//
// Output blocks of 64 a x kPairB b.  Lane l of a wave holds A[x][a0 + l]; the
// kPairB masks B[x][b0 ..] are wave-uniform: the workgroup stages them in LDS
// for a chunk of tiles at a time (one vector load per mask, all in flight)
// and every wave reads them back as LDS broadcasts, so one b costs two AND
// and two popcount-accumulate VALU operations for 64 experts a and 64
// tokens.  (Fetched with scalar loads, one per mask and tile, they made the
// pair workgroups the longest part of the solver launch: measured on MI355X,
// DeepSeek-V3-shaped launch 31.5 -> 24.9 us, Kimi-K2-shaped 98.8 -> 59.6 us.)
// The tiles of a block are split over `splits`
// workgroups (and over the waves of each) so that a launch fills the chip;
// the waves meet in LDS and each workgroup stores its partial block, which
// pair_reduce_one adds up in split order (with one split the block is
// written directly).  The co-selection matrix is symmetric: blocks strictly
// below the diagonal are skipped and each off-diagonal count is written to
// (a, b) and (b, a).  Slice z: 0 co-selection (A = B = this layer, zero
// diagonal), 1 transitions (A = previous layer, B = this layer).
#pragma once

#include "internal.h"

namespace moe {

constexpr int kPairB = 16;
constexpr int kPairBlock = 64 * kPairB;

__host__ __device__ inline int pair_blocks(const Dims& d) { return ((d.E + 63) / 64) * ((d.E + kPairB - 1) / kPairB); }

// Tile splits for workgroups of nthr threads: about 256K threads in all, at
// least 8 tiles per workgroup.
inline int pair_splits(const Dims& d, int nthr) {
  int s = (1024 * 256 / nthr) / pair_blocks(d);
  if (s > d.NT / 8) s = d.NT / 8;
  return s < 1 ? 1 : s;
}

__device__ __forceinline__ bool pair_block_skipped(const Dims& d, int z, int blk) {
  const int nb = (d.E + kPairB - 1) / kPairB;
  return z == 0 && (blk % nb) * kPairB + kPairB - 1 < (blk / nb) * 64;
}

// Write one finished 64 x kPairB block (co-selection: upper part mirrored).
__device__ __forceinline__ void pair_store(const Dims& d, int32_t* __restrict__ out, bool is_trans, int a0, int b0,
                                           int q, int v) {
  const int al = q / kPairB, bl = q - al * kPairB;
  const int aa = a0 + al, bb = b0 + bl;
  if (aa >= d.E || bb >= d.E) return;
  if (is_trans) {
    out[(int64_t)aa * d.E + bb] = v;
  } else if (aa == bb) {
    out[(int64_t)aa * d.E + bb] = 0;
  } else if (aa < bb) {
    out[(int64_t)aa * d.E + bb] = v;
    out[(int64_t)bb * d.E + aa] = v;
  }
}

// Tiles per LDS chunk of B masks, for workgroups of nthr threads (four per wave).
__host__ __device__ constexpr int pair_chunk(int nthr) { return 4 * (nthr / 64); }
// LDS bytes of pair_partial_block for workgroups of nthr threads.
__host__ __device__ constexpr size_t pair_lds_bytes(int nthr) {
  return sizeof(int32_t) * kPairBlock + sizeof(uint64_t) * kPairB * pair_chunk(nthr);
}

// Split `split` of block blk of slice z, by a workgroup of NTHR threads;
// acc_s: pair_lds_bytes(NTHR) bytes of LDS (the block's sums, then a chunk
// of B masks).
template <int NTHR, int KCHUNK = pair_chunk(NTHR)>
__device__ __forceinline__ void pair_partial_block(const Dims& d, const PairArgs& pa, int z, int blk, int split,
                                                   int32_t* acc_s) {
  if (pair_block_skipped(d, z, blk)) return;  // strictly below the diagonal: written as mirrors
  const bool is_trans = z == 1;
  const uint64_t* A = is_trans ? pa.prev : pa.cur;
  const int nb = (d.E + kPairB - 1) / kPairB;
  const int a0 = (blk / nb) * 64, b0 = (blk % nb) * kPairB;
  const int splits = pa.splits;
  const int x0 = (int)((int64_t)d.NT * split / splits), x1 = (int)((int64_t)d.NT * (split + 1) / splits);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int q = threadIdx.x; q < kPairBlock; q += NTHR) acc_s[q] = 0;
  __syncthreads();
  const int a = a0 + lane;
  const bool a_ok = a < d.E;
  uint32_t acc[kPairB];
#pragma unroll
  for (int bb = 0; bb < kPairB; ++bb) acc[bb] = 0;
  constexpr int kWaves = NTHR / 64;
  constexpr int kPer = KCHUNK / kWaves;  // tiles of a chunk per wave
  uint64_t* bst = reinterpret_cast<uint64_t*>(acc_s + kPairBlock);
  for (int c0 = x0; c0 < x1; c0 += KCHUNK) {
    const int cn = min(KCHUNK, x1 - c0);
    __syncthreads();
    for (int q = threadIdx.x; q < cn * kPairB; q += NTHR) {
      const int u = q / kPairB, bb = q - u * kPairB;
      bst[q] = b0 + bb < d.E ? pa.cur[(int64_t)(c0 + u) * d.E + b0 + bb] : 0ull;
    }
    __syncthreads();
    uint64_t am[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int u = wave + j * kWaves;
      am[j] = (a_ok && u < cn) ? A[(int64_t)(c0 + u) * d.E + a] : 0ull;
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int u = wave + j * kWaves;
      if (u >= cn) break;
      const uint64_t* brow = bst + u * kPairB;
      const uint32_t alo = (uint32_t)am[j], ahi = (uint32_t)(am[j] >> 32);
#pragma unroll
      for (int bb = 0; bb < kPairB; ++bb) {
        const uint64_t bv = brow[bb];
        acc[bb] += __popc(alo & (uint32_t)bv) + __popc(ahi & (uint32_t)(bv >> 32));
      }
    }
  }
#pragma unroll
  for (int bb = 0; bb < kPairB; ++bb)
    if (acc[bb] != 0) atomicAdd(&acc_s[lane * kPairB + bb], (int)acc[bb]);
  __syncthreads();
  if (splits > 1) {
    int32_t* mine = pa.part + ((int64_t)(z * pair_blocks(d) + blk) * splits + split) * kPairBlock;
    for (int q = threadIdx.x; q < kPairBlock; q += NTHR) mine[q] = acc_s[q];
    return;
  }
  int32_t* out = is_trans ? pa.trans : pa.cooc;
  for (int q = threadIdx.x; q < kPairBlock; q += NTHR) pair_store(d, out, is_trans, a0, b0, q, acc_s[q]);
}

// Element q of block blk of slice z: the sum of its split partials, in split order.
__device__ __forceinline__ void pair_reduce_one(const Dims& d, const PairArgs& pa, int z, int blk, int q) {
  if (q >= kPairBlock || pair_block_skipped(d, z, blk)) return;
  const bool is_trans = z == 1;
  const int nb = (d.E + kPairB - 1) / kPairB;
  const int a0 = (blk / nb) * 64, b0 = (blk % nb) * kPairB;
  const int32_t* all = pa.part + (int64_t)(z * pair_blocks(d) + blk) * pa.splits * kPairBlock + q;
  int sum = 0;
  for (int sp = 0; sp < pa.splits; ++sp) sum += all[(int64_t)sp * kPairBlock];
  pair_store(d, is_trans ? pa.trans : pa.cooc, is_trans, a0, b0, q, sum);
}

}  // namespace moe
