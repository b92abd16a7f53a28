// Top-k gating and load histograms on gfx950.
//
// [TopoEP] section 2.1: each rank's router picks the top-k experts of its
// local tokens; Eq. 3: the routing matrix omega[s][e] counts the assignments
// of source rank s to expert e.  [Coupling]: co-selection counts within a
// layer and transition counts between consecutive layers.
//
// Data layout.  Tokens are cut into tiles of up to 64 consecutive tokens of
// one source rank.  For every tile x and expert e a 64-bit presence mask
// records which tokens of the tile selected e.  Every histogram of the path
// comes from these masks:
//   omega[s][e]      = sum over the tiles of s of popcount(mask[x][e])
//   tile_base[x][e]  = exclusive prefix of those popcounts over tiles
//   stable rank of token t among the tokens of its source that chose e
//                    = tile_base[x][e] - tile_base[first tile of s][e]
//                      + popcount(mask[x][e] & bits below t)
//   cooc[a][b]       = sum over tiles of popcount(mask[x][a] & mask[x][b])
//   trans[a][b]      = sum over tiles of popcount(prev[x][a] & mask[x][b])
// so the route step writes NT*E*8 bytes of masks instead of sorting slots.
#include "internal.h"

namespace moe {
namespace {

// Total order of IEEE floats as unsigned integers, with -0.0 mapped onto +0.0.
__device__ __forceinline__ uint32_t float_order_key(uint32_t u) {
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
  lo = __shfl_xor(lo, m);
  hi = __shfl_xor(hi, m);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// One workgroup per tile.  A group of P lanes handles one token: lane l holds
// logits l, l+P, l+2P, ... as 64-bit keys (order key << 32 | ~e), so the
// largest key is the largest logit with ties going to the lower expert.
// k rounds of a group max (butterfly over P lanes) pick the experts in order.
template <int P, int VPL>
__global__ __launch_bounds__(1024) void route_topk_kernel(Dims d, const float* __restrict__ logits,
                                                          const int32_t* __restrict__ prev_topk,
                                                          int32_t* __restrict__ topk_idx,
                                                          float* __restrict__ topk_val,
                                                          uint64_t* __restrict__ tile_mask,
                                                          uint64_t* __restrict__ prev_mask,
                                                          int32_t* __restrict__ status) {
  extern __shared__ unsigned long long smem_masks[];
  unsigned long long* smask = smem_masks;
  unsigned long long* pmask = smem_masks + d.E;
  const int x = blockIdx.x;
  const int s = x / d.C, c = x - s * d.C;
  const int64_t t0 = (int64_t)s * d.Tr + (int64_t)c * kTile;
  const int nt = min(kTile, d.Tr - c * kTile);
  const int tid = threadIdx.x, nthr = blockDim.x;
  const bool want_prev = prev_topk != nullptr;
  for (int e = tid; e < d.E; e += nthr) {
    smask[e] = 0ull;
    if (want_prev) pmask[e] = 0ull;
  }
  __syncthreads();

  const int lane = tid % P;
  const int ngrp = nthr / P;
  bool bad = false;
  for (int i = tid / P; i < nt; i += ngrp) {
    const int64_t t = t0 + i;
    const float* row = logits + t * d.E;
    uint64_t key[VPL];
    float val[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = lane + v * P;
      if (e < d.E) {
        const float f = row[e];
        const uint32_t u = __float_as_uint(f);
        bad |= (u & 0x7fffffffu) > 0x7f800000u;
        key[v] = ((uint64_t)float_order_key(u) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
        val[v] = f;
      } else {
        key[v] = 0ull;  // below every real key (the smallest real order key is that of -inf)
        val[v] = 0.f;
      }
    }
    for (int j = 0; j < d.k; ++j) {
      uint64_t best = 0ull;
#pragma unroll
      for (int v = 0; v < VPL; ++v) best = key[v] > best ? key[v] : best;
#pragma unroll
      for (int m = P / 2; m >= 1; m >>= 1) {
        const uint64_t o = shfl_xor_u64(best, m);
        best = o > best ? o : best;
      }
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        if (key[v] == best) {  // keys are distinct: exactly one (lane, v) matches
          const int e = lane + v * P;
          topk_idx[t * d.k + j] = e;
          if (topk_val) topk_val[t * d.k + j] = val[v];
          atomicOr(&smask[e], 1ull << i);
          key[v] = 0ull;
        }
      }
    }
  }
  if (want_prev) {
    for (int q = tid; q < nt * d.k; q += nthr) {
      const int i = q / d.k;
      const int e = prev_topk[(t0 + i) * d.k + (q - i * d.k)];
      if ((unsigned)e < (unsigned)d.E) {
        const unsigned long long old = atomicOr(&pmask[e], 1ull << i);
        if (old & (1ull << i)) atomicOr(status, MOE_STATUS_BAD_TOPK);
      } else {
        atomicOr(status, MOE_STATUS_BAD_TOPK);
      }
    }
  }
  if (bad) atomicOr(status, MOE_STATUS_NAN_LOGIT);
  __syncthreads();
  for (int e = tid; e < d.E; e += nthr) {
    tile_mask[(int64_t)x * d.E + e] = smask[e];
    if (want_prev) prev_mask[(int64_t)x * d.E + e] = pmask[e];
  }
}

// Presence masks from a given top-k (and optionally the previous layer's).
__global__ __launch_bounds__(256) void build_masks_kernel(Dims d, const int32_t* __restrict__ topk,
                                                          const int32_t* __restrict__ prev_topk,
                                                          uint64_t* __restrict__ tile_mask,
                                                          uint64_t* __restrict__ prev_mask,
                                                          int32_t* __restrict__ status) {
  extern __shared__ unsigned long long smem_masks[];
  unsigned long long* smask = smem_masks;
  unsigned long long* pmask = smem_masks + d.E;
  const int x = blockIdx.x;
  const int s = x / d.C, c = x - s * d.C;
  const int64_t t0 = (int64_t)s * d.Tr + (int64_t)c * kTile;
  const int nt = min(kTile, d.Tr - c * kTile);
  const int tid = threadIdx.x, nthr = blockDim.x;
  const bool want_prev = prev_topk != nullptr;
  for (int e = tid; e < d.E; e += nthr) {
    smask[e] = 0ull;
    if (want_prev) pmask[e] = 0ull;
  }
  __syncthreads();
  bool bad = false;
  for (int q = tid; q < nt * d.k; q += nthr) {
    const int i = q / d.k;
    const int64_t off = (t0 + i) * d.k + (q - i * d.k);
    const int e = topk[off];
    if ((unsigned)e < (unsigned)d.E) {
      bad |= (atomicOr(&smask[e], 1ull << i) & (1ull << i)) != 0ull;
    } else {
      bad = true;
    }
    if (want_prev) {
      const int ep = prev_topk[off];
      if ((unsigned)ep < (unsigned)d.E) {
        bad |= (atomicOr(&pmask[ep], 1ull << i) & (1ull << i)) != 0ull;
      } else {
        bad = true;
      }
    }
  }
  if (bad) atomicOr(status, MOE_STATUS_BAD_TOPK);
  __syncthreads();
  for (int e = tid; e < d.E; e += nthr) {
    tile_mask[(int64_t)x * d.E + e] = smask[e];
    if (want_prev) prev_mask[(int64_t)x * d.E + e] = pmask[e];
  }
}

// omega, expert counts and the exclusive tile prefix.  One workgroup per 64
// experts (a lane per expert, coalesced 512-byte mask rows); its 16 wave rows
// split the source ranks.
__global__ __launch_bounds__(1024) void scan_kernel(Dims d, const uint64_t* __restrict__ tile_mask,
                                                    int32_t* __restrict__ tile_base, int32_t* __restrict__ omega,
                                                    int32_t* __restrict__ count) {
  extern __shared__ int32_t smem_scan[];  // [R][64]
  const int el = threadIdx.x & 63, row = threadIdx.x >> 6, nrow = blockDim.x >> 6;
  const int e = blockIdx.x * 64 + el;
  const bool ok = e < d.E;
  for (int s = row; s < d.R; s += nrow) {
    int sum = 0;
    if (ok)
      for (int c = 0; c < d.C; ++c) sum += __popcll(tile_mask[((int64_t)s * d.C + c) * d.E + e]);
    smem_scan[s * 64 + el] = sum;
    if (ok) omega[(int64_t)s * d.E + e] = sum;
  }
  __syncthreads();
  if (row == 0) {
    int run = 0;
    for (int s = 0; s < d.R; ++s) {
      const int v = smem_scan[s * 64 + el];
      smem_scan[s * 64 + el] = run;
      run += v;
    }
    if (ok) count[e] = run;
  }
  __syncthreads();
  for (int s = row; s < d.R; s += nrow) {
    int run = smem_scan[s * 64 + el];
    if (ok)
      for (int c = 0; c < d.C; ++c) {
        const int64_t idx = ((int64_t)s * d.C + c) * d.E + e;
        tile_base[idx] = run;
        run += __popcll(tile_mask[idx]);
      }
  }
}

// Pair counts as a binary product over tiles: out[a][b] = sum_x popcount(A[x][a] & B[x][b]).
// blockIdx.z = 0: co-selection (A = B = this layer, zero diagonal);
// blockIdx.z = 1: transitions (A = previous layer, B = this layer).
constexpr int kPairBS = 16;
constexpr int kPairChunk = 64;

__global__ __launch_bounds__(256) void pair_kernel(Dims d, const uint64_t* __restrict__ cur,
                                                   const uint64_t* __restrict__ prev, int32_t* __restrict__ cooc,
                                                   int32_t* __restrict__ trans, int zbase) {
  __shared__ uint64_t As[kPairChunk][kPairBS];
  __shared__ uint64_t Bs[kPairChunk][kPairBS];
  const bool is_trans = (int)blockIdx.z + zbase == 1;
  const uint64_t* A = is_trans ? prev : cur;
  int32_t* out = is_trans ? trans : cooc;
  const int a0 = blockIdx.y * kPairBS, b0 = blockIdx.x * kPairBS;
  const int ta = threadIdx.x / kPairBS, tb = threadIdx.x % kPairBS;
  int acc = 0;
  for (int x0 = 0; x0 < d.NT; x0 += kPairChunk) {
    for (int q = threadIdx.x; q < kPairChunk * kPairBS; q += blockDim.x) {
      const int tt = q / kPairBS, cc = q % kPairBS;
      const int x = x0 + tt;
      const bool inx = x < d.NT;
      As[tt][cc] = (inx && a0 + cc < d.E) ? A[(int64_t)x * d.E + a0 + cc] : 0ull;
      Bs[tt][cc] = (inx && b0 + cc < d.E) ? cur[(int64_t)x * d.E + b0 + cc] : 0ull;
    }
    __syncthreads();
#pragma unroll 8
    for (int tt = 0; tt < kPairChunk; ++tt) acc += __popcll(As[tt][ta] & Bs[tt][tb]);
    __syncthreads();
  }
  const int a = a0 + ta, b = b0 + tb;
  if (a < d.E && b < d.E) out[(int64_t)a * d.E + b] = (!is_trans && a == b) ? 0 : acc;
}

template <int P, int VPL>
hipError_t launch_topk_pv(const Dims& d, const float* logits, const int32_t* prev_topk, int32_t* topk_idx,
                          float* topk_val, uint64_t* tile_mask, uint64_t* prev_mask, int32_t* status,
                          hipStream_t st) {
  const int threads = P * 64 < 1024 ? P * 64 : 1024;
  const size_t lds = sizeof(unsigned long long) * (size_t)d.E * (prev_topk ? 2 : 1);
  hipLaunchKernelGGL((route_topk_kernel<P, VPL>), dim3(d.NT), dim3(threads), lds, st, d, logits, prev_topk,
                     topk_idx, topk_val, tile_mask, prev_mask, status);
  return hipGetLastError();
}

}  // namespace

// Lanes per token P: the smallest power of two (>= 4) that leaves at most 16
// logits per lane; VPL: logits per lane rounded up to a power of two.
hipError_t launch_route_topk(const Dims& d, const float* logits, const int32_t* prev_topk, int32_t* topk_idx,
                             float* topk_val, uint64_t* tile_mask, uint64_t* prev_mask, int32_t* status,
                             hipStream_t st) {
  if (d.NT == 0) return hipSuccess;
#define MOE_TOPK_CASE(P_, V_)                                                                             \
  if (d.E <= (P_) * (V_))                                                                                 \
    return launch_topk_pv<P_, V_>(d, logits, prev_topk, topk_idx, topk_val, tile_mask, prev_mask, status, \
                                  st);
  MOE_TOPK_CASE(4, 4)
  MOE_TOPK_CASE(4, 8)
  MOE_TOPK_CASE(4, 16)
  MOE_TOPK_CASE(8, 16)
  MOE_TOPK_CASE(16, 16)
  MOE_TOPK_CASE(32, 16)
  MOE_TOPK_CASE(64, 16)
  MOE_TOPK_CASE(64, 32)
#undef MOE_TOPK_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_build_masks(const Dims& d, const int32_t* topk_idx, const int32_t* prev_topk,
                              uint64_t* tile_mask, uint64_t* prev_mask, int32_t* status, hipStream_t st) {
  if (d.NT == 0) return hipSuccess;
  const size_t lds = sizeof(unsigned long long) * (size_t)d.E * (prev_topk ? 2 : 1);
  hipLaunchKernelGGL(build_masks_kernel, dim3(d.NT), dim3(256), lds, st, d, topk_idx, prev_topk, tile_mask,
                     prev_mask, status);
  return hipGetLastError();
}

hipError_t launch_scan(const Dims& d, const uint64_t* tile_mask, int32_t* tile_base, int32_t* omega,
                       int32_t* count, hipStream_t st) {
  const int blocks = (d.E + 63) / 64;
  const size_t lds = sizeof(int32_t) * 64 * (size_t)d.R;
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(scan_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(scan_kernel, dim3(blocks), dim3(1024), lds, st, d, tile_mask, tile_base, omega, count);
  return hipGetLastError();
}

hipError_t launch_pairs(const Dims& d, const uint64_t* tile_mask, const uint64_t* prev_mask, int32_t* cooc,
                        int32_t* trans, hipStream_t st) {
  if (!cooc && !trans) return hipSuccess;
  const int nb = (d.E + kPairBS - 1) / kPairBS;
  // slice 0 co-selection, slice 1 transitions; one launch covers the requested ones.
  const int nz = (cooc ? 1 : 0) + (trans ? 1 : 0);
  const int zbase = cooc ? 0 : 1;
  hipLaunchKernelGGL(pair_kernel, dim3(nb, nb, nz), dim3(256), 0, st, d, tile_mask, prev_mask, cooc, trans, zbase);
  return hipGetLastError();
}

}  // namespace moe
