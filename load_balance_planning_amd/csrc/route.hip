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

__device__ __forceinline__ uint32_t float_from_order_key(uint32_t k) {
  return (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
  lo = __shfl(lo, src);
  hi = __shfl(hi, src);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
  lo = __shfl_xor(lo, m);
  hi = __shfl_xor(hi, m);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// DPP lane moves inside a row of 16 lanes (controls: quad_perm [1,0,3,2] = 0xB1,
// quad_perm [2,3,0,1] = 0x4E, row_half_mirror = 0x141, row_mirror = 0x140).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Max over each aligned group of P lanes, result in every lane of the group.
// Within a 16-lane row the butterfly uses DPP (quad swaps, then the half-row
// and row mirrors, which pair every lane with one of the other half); wider
// groups finish with two cross-row exchanges.
template <int P>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) {
  if (P >= 2) v = max_u64(v, dpp_u64<0xB1>(v));
  if (P >= 4) v = max_u64(v, dpp_u64<0x4E>(v));
  if (P >= 8) v = max_u64(v, dpp_u64<0x141>(v));
  if (P >= 16) v = max_u64(v, dpp_u64<0x140>(v));
  if (P >= 32) v = max_u64(v, shfl_xor_u64(v, 16));
  if (P >= 64) v = max_u64(v, shfl_xor_u64(v, 32));
  return v;
}

// Exchange with lane (l ^ J) inside aligned groups: DPP for J < 4, else the
// LDS crossbar.
template <int J>
__device__ __forceinline__ uint64_t xor_lane_u64(uint64_t v) {
  if (J == 1) return dpp_u64<0xB1>(v);
  if (J == 2) return dpp_u64<0x4E>(v);
  return shfl_xor_u64(v, J);
}

template <int P, int SIZE, int J>
__device__ __forceinline__ uint64_t bitonic_step(uint64_t v, int lig) {
  const uint64_t o = xor_lane_u64<J>(v);
  const bool desc = (lig & SIZE) == 0;  // the last stage (SIZE = P) sorts every group descending
  const bool lower = (lig & J) == 0;
  const bool keep_max = lower == desc;
  const uint64_t mx = o > v ? o : v, mn = o > v ? v : o;
  return keep_max ? mx : mn;
}

// Bitonic sort of one 64-bit key per lane over aligned groups of P lanes,
// descending: afterwards lane l of a group holds the group's (l+1)-th largest.
template <int P>
__device__ __forceinline__ uint64_t group_sort_desc(uint64_t v, int lig) {
#define MOE_BSTEP(S, J) if (P >= (S)) v = bitonic_step<P, ((S) >= P ? P : (S)), J>(v, lig);
  MOE_BSTEP(2, 1)
  MOE_BSTEP(4, 2) MOE_BSTEP(4, 1)
  MOE_BSTEP(8, 4) MOE_BSTEP(8, 2) MOE_BSTEP(8, 1)
  MOE_BSTEP(16, 8) MOE_BSTEP(16, 4) MOE_BSTEP(16, 2) MOE_BSTEP(16, 1)
  MOE_BSTEP(32, 16) MOE_BSTEP(32, 8) MOE_BSTEP(32, 4) MOE_BSTEP(32, 2) MOE_BSTEP(32, 1)
  MOE_BSTEP(64, 32) MOE_BSTEP(64, 16) MOE_BSTEP(64, 8) MOE_BSTEP(64, 4) MOE_BSTEP(64, 2) MOE_BSTEP(64, 1)
#undef MOE_BSTEP
  return v;
}

// One workgroup per tile.  A group of P lanes handles one token; lane l holds
// VPL logits as 64-bit keys
//   high word: order key of the logit (-0.0 folded onto +0.0)
//   low word : (0x7fffffff - e) << 1 | (logit is -0.0)
// so the largest key is the largest logit with ties to the lower expert, and
// the key alone gives back the expert and the exact logit bits.  Keys are
// unique, so a descending sort of the candidates (below) gives the top-k in
// order with ties already broken; lane j of the group writes choice j.
// Workgroup size: one wave per token group of a 64-token tile, at most 1024
// threads; 32 keys per lane need more than the 128 VGPRs a 1024-thread
// workgroup allows, so those use 512.
template <int P, int VPL>
constexpr int topk_threads() {
  return (P * 64 < 1024 ? P * 64 : 1024) / (VPL >= 32 ? 2 : 1);
}

template <int P, int VPL, bool VEC4>
__global__ __launch_bounds__((topk_threads<P, VPL>())) void route_topk_kernel(Dims d, const float* __restrict__ logits,
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

  const int lane = tid % P;                  // lane inside the token group
  const int grp_base = (tid & 63) - lane;     // wave lane of the group's first lane
  uint64_t* cand_buf = reinterpret_cast<uint64_t*>(smem_masks + (want_prev ? 2 : 1) * d.E) + (tid & ~63);
  const int ngrp = nthr / P;
  bool bad = false;
  for (int i = tid / P; i < nt; i += ngrp) {
    const int64_t t = t0 + i;
    const float* row = logits + t * d.E;
    uint64_t key[VPL];
    if (VEC4) {
      // lane l reads logits 4(l + P v) .. 4(l + P v) + 3 as one 16-byte load;
      // every load is issued before any is used (out-of-range lanes re-read
      // the row start and mask the keys).
      float4 f4[VPL / 4];
#pragma unroll
      for (int v = 0; v < VPL / 4; ++v) {
        const int e0 = 4 * (lane + P * v);
        f4[v] = *reinterpret_cast<const float4*>(row + (e0 < d.E ? e0 : 0));
      }
#pragma unroll
      for (int v = 0; v < VPL / 4; ++v) {
        const int e0 = 4 * (lane + P * v);
        const float4 f = f4[v];
        const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int e = e0 + q;
          const uint32_t u = __float_as_uint(fv[q]);
          bad |= (e < d.E) && ((u & 0x7fffffffu) > 0x7f800000u);
          key[4 * v + q] = e < d.E ? ((uint64_t)float_order_key(u) << 32) |
                                         (uint64_t)(((0x7fffffffu - (uint32_t)e) << 1) | (u == 0x80000000u ? 1u : 0u))
                                   : 0ull;
        }
      }
    } else {
      uint32_t uv[VPL];
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const int e = lane + v * P;
        uv[v] = __float_as_uint(row[e < d.E ? e : 0]);
      }
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const int e = lane + v * P;
        const uint32_t u = uv[v];
        bad |= (e < d.E) && ((u & 0x7fffffffu) > 0x7f800000u);
        key[v] = e < d.E ? ((uint64_t)float_order_key(u) << 32) |
                               (uint64_t)(((0x7fffffffu - (uint32_t)e) << 1) | (u == 0x80000000u ? 1u : 0u))
                         : 0ull;  // below every real key
      }
    }
    // Threshold: the k-th largest of the group's lane maxima.  At least k
    // keys reach it, so every top-k key does; the keys that reach it are the
    // candidates.  When at most P keys qualify (the usual case) they are
    // sorted once across the group's lanes; otherwise k rounds of group max.
    uint64_t lmax = key[0];
#pragma unroll
    for (int v = 1; v < VPL; ++v) lmax = max_u64(lmax, key[v]);
    bool fast = d.k <= P;
    int total = 0, before = 0, mine = 0;
    if (fast) {
      const uint64_t sorted = group_sort_desc<P>(lmax, lane);
      const uint64_t tau = shfl_u64(sorted, grp_base + d.k - 1);
#pragma unroll
      for (int v = 0; v < VPL; ++v) mine += key[v] >= tau ? 1 : 0;
      int incl = mine;
#pragma unroll
      for (int off = 1; off < P; off <<= 1) {
        const int o = __shfl_up(incl, off, P);
        if (lane >= off) incl += o;
      }
      before = incl - mine;
      total = __shfl(incl, grp_base + P - 1);
      fast = total <= P;
      if (fast) {
        uint64_t* buf = cand_buf + grp_base;
        int w = before;
#pragma unroll
        for (int v = 0; v < VPL; ++v)
          if (key[v] >= tau) buf[w++] = key[v];
        wave_lds_sync();
        uint64_t c = lane < total ? buf[lane] : 0ull;
        wave_lds_sync();
        c = group_sort_desc<P>(c, lane);
        if (lane < d.k) {
          const uint32_t lo = (uint32_t)c;
          const int e = (int)(0x7fffffffu - (lo >> 1));
          if ((unsigned)e < (unsigned)d.E) {
            const uint32_t u = (lo & 1u) ? 0x80000000u : float_from_order_key((uint32_t)(c >> 32));
            topk_idx[t * d.k + lane] = e;
            if (topk_val) topk_val[t * d.k + lane] = __uint_as_float(u);
            atomicOr(&smask[e], 1ull << i);
          } else {
            bad = true;
          }
        }
      }
    }
    if (!fast) {
      for (int j = 0; j < d.k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int v = 1; v < VPL; ++v) best = max_u64(best, key[v]);
        best = group_max_u64<P>(best);
#pragma unroll
        for (int v = 0; v < VPL; ++v) key[v] = key[v] == best ? 0ull : key[v];
        if (lane == 0) {
          const uint32_t lo = (uint32_t)best;
          const int e = (int)(0x7fffffffu - (lo >> 1));
          if ((unsigned)e < (unsigned)d.E) {
            const uint32_t u = (lo & 1u) ? 0x80000000u : float_from_order_key((uint32_t)(best >> 32));
            topk_idx[t * d.k + j] = e;
            if (topk_val) topk_val[t * d.k + j] = __uint_as_float(u);
            atomicOr(&smask[e], 1ull << i);
          } else {
            bad = true;
          }
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

// omega, expert counts and the exclusive tile prefix.  One workgroup per 16
// experts and all source ranks: thread (row, e) with 64 rows; when there are
// fewer than 64 sources each source's tiles are split over several rows.
// Prefixes: over the rows of a source (chunks of tiles), then over sources.
constexpr int kScanEB = 16;
constexpr int kScanRows = 1024 / kScanEB;

__global__ __launch_bounds__(1024) void scan_kernel(Dims d, const uint64_t* __restrict__ tile_mask,
                                                    int32_t* __restrict__ tile_base, int32_t* __restrict__ omega,
                                                    int32_t* __restrict__ count) {
  extern __shared__ int32_t smem_scan[];
  const int el = threadIdx.x % kScanEB, row = threadIdx.x / kScanEB;
  const int e = blockIdx.x * kScanEB + el;
  const bool ok = e < d.E;
  const int R = d.R, C = d.C;
  const int rps = R < kScanRows ? kScanRows / R : 1;      // rows per source
  const int cc = (C + rps - 1) / rps;                     // tiles per row
  int32_t* part = smem_scan;                              // [R][rps][EB] chunk sums -> chunk prefixes
  int32_t* tot = smem_scan + R * rps * kScanEB;           // [R][EB] source sums -> source prefixes
  // rows handle (source, chunk) pairs r = row, row + 64, ... over R * rps pairs
  for (int r = row; r < R * rps; r += kScanRows) {
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
  for (int q = threadIdx.x; q < R * kScanEB; q += blockDim.x) {
    const int src = q / kScanEB, l = q - src * kScanEB;
    int run = 0;
    for (int ch = 0; ch < rps; ++ch) {
      const int v = part[(src * rps + ch) * kScanEB + l];
      part[(src * rps + ch) * kScanEB + l] = run;
      run += v;
    }
    tot[src * kScanEB + l] = run;
    if (blockIdx.x * kScanEB + l < d.E) omega[(int64_t)src * d.E + blockIdx.x * kScanEB + l] = run;
  }
  __syncthreads();
  if (threadIdx.x < kScanEB) {
    int run = 0;
    for (int src = 0; src < R; ++src) {
      const int v = tot[src * kScanEB + el];
      tot[src * kScanEB + el] = run;
      run += v;
    }
    if (ok) count[e] = run;
  }
  __syncthreads();
  for (int r = row; r < R * rps; r += kScanRows) {
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

// Pair counts as a binary product over tiles:
//   out[a][b] = sum_x popcount(A[x][a] & B[x][b]).
// A workgroup owns a 64 x PB block; its 16 waves split the tiles.  Each lane
// holds A[x][a] for its own a; the PB masks B[x][b0..b0+PB) are wave-uniform
// and come in through scalar loads, so one b costs two AND and two popcount
// VALU operations for 64 experts a and 64 tokens.  Partial sums of the waves
// meet in LDS.  The co-selection matrix is symmetric: only blocks touching
// the upper triangle are computed, and each off-diagonal count is written
// to both (a, b) and (b, a).  blockIdx.z + zbase: 0 co-selection (A = B =
// this layer, zero diagonal), 1 transitions (A = previous layer, B = this layer).
template <int PB>
__global__ __launch_bounds__(1024) void pair_kernel(Dims d, const uint64_t* __restrict__ cur,
                                                    const uint64_t* __restrict__ prev, int32_t* __restrict__ cooc,
                                                    int32_t* __restrict__ trans, int zbase) {
  __shared__ int32_t acc_s[64 * PB];
  const bool is_trans = (int)blockIdx.z + zbase == 1;
  const uint64_t* A = is_trans ? prev : cur;
  int32_t* out = is_trans ? trans : cooc;
  const int a0 = blockIdx.x * 64, b0 = blockIdx.y * PB;
  if (!is_trans && b0 + PB - 1 < a0) return;  // strictly below the diagonal: written as mirrors
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), nwave = blockDim.x >> 6;
  for (int q = threadIdx.x; q < 64 * PB; q += blockDim.x) acc_s[q] = 0;
  __syncthreads();
  const int a = a0 + lane;
  const bool a_ok = a < d.E;
  int acc[PB];
#pragma unroll
  for (int bb = 0; bb < PB; ++bb) acc[bb] = 0;
  constexpr int kBatch = 4;
  for (int x0 = wave * kBatch; x0 < d.NT; x0 += nwave * kBatch) {
    uint64_t am[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int x = x0 + u < d.NT ? x0 + u : d.NT - 1;
      am[u] = A[(int64_t)x * d.E + (a_ok ? a : 0)];
      am[u] = (a_ok && x0 + u < d.NT) ? am[u] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int x = x0 + u < d.NT ? x0 + u : d.NT - 1;
      const uint64_t* brow = cur + (int64_t)x * d.E;
      const uint32_t alo = (uint32_t)am[u], ahi = (uint32_t)(am[u] >> 32);
#pragma unroll
      for (int bb = 0; bb < PB; ++bb) {
        const uint64_t bv = brow[b0 + bb < d.E ? b0 + bb : 0];
        acc[bb] += __popc(alo & (uint32_t)bv) + __popc(ahi & (uint32_t)(bv >> 32));
      }
    }
  }
#pragma unroll
  for (int bb = 0; bb < PB; ++bb)
    if (acc[bb] != 0) atomicAdd(&acc_s[lane * PB + bb], acc[bb]);
  __syncthreads();
  for (int q = threadIdx.x; q < 64 * PB; q += blockDim.x) {
    const int al = q / PB, bl = q - al * PB;
    const int aa = a0 + al, bb = b0 + bl;
    if (aa >= d.E || bb >= d.E) continue;
    if (is_trans) {
      out[(int64_t)aa * d.E + bb] = acc_s[q];
    } else if (aa == bb) {
      out[(int64_t)aa * d.E + bb] = 0;
    } else if (aa < bb) {
      out[(int64_t)aa * d.E + bb] = acc_s[q];
      out[(int64_t)bb * d.E + aa] = acc_s[q];
    }
  }
}

template <int P, int VPL>
hipError_t launch_topk_pv(const Dims& d, const float* logits, const int32_t* prev_topk, int32_t* topk_idx,
                          float* topk_val, uint64_t* tile_mask, uint64_t* prev_mask, int32_t* status,
                          hipStream_t st) {
  const int threads = topk_threads<P, VPL>();
  const size_t lds = sizeof(unsigned long long) * ((size_t)d.E * (prev_topk ? 2 : 1) + threads);
  const bool vec4 = (d.E % 4) == 0 && (VPL % 4) == 0 && ((uintptr_t)logits % 16) == 0;
  if (vec4) {
    hipLaunchKernelGGL((route_topk_kernel<P, VPL, true>), dim3(d.NT), dim3(threads), lds, st, d, logits, prev_topk,
                       topk_idx, topk_val, tile_mask, prev_mask, status);
  } else {
    hipLaunchKernelGGL((route_topk_kernel<P, VPL, false>), dim3(d.NT), dim3(threads), lds, st, d, logits, prev_topk,
                       topk_idx, topk_val, tile_mask, prev_mask, status);
  }
  return hipGetLastError();
}

}  // namespace

// Lanes per token P: the smallest power of two (>= 4) that leaves at most 16
// logits per lane and is at least 2k, so that the threshold of the selection
// (the k-th largest lane maximum) rarely admits more than P candidates; VPL:
// logits per lane rounded up to a power of two (>= 4).
hipError_t launch_route_topk(const Dims& d, const float* logits, const int32_t* prev_topk, int32_t* topk_idx,
                             float* topk_val, uint64_t* tile_mask, uint64_t* prev_mask, int32_t* status,
                             hipStream_t st) {
  if (d.NT == 0) return hipSuccess;
  int P = 4;
  while (P < 64 && (P * 16 < d.E || P < 2 * d.k)) P *= 2;
  int V = 4;
  while (P * V < d.E) V *= 2;
#define MOE_TOPK_CASE(P_, V_)                                                                             \
  if (P == (P_) && V == (V_))                                                                             \
    return launch_topk_pv<P_, V_>(d, logits, prev_topk, topk_idx, topk_val, tile_mask, prev_mask, status, \
                                  st);
  MOE_TOPK_CASE(4, 4)
  MOE_TOPK_CASE(4, 8)
  MOE_TOPK_CASE(4, 16)
  MOE_TOPK_CASE(8, 4)
  MOE_TOPK_CASE(8, 8)
  MOE_TOPK_CASE(8, 16)
  MOE_TOPK_CASE(16, 4)
  MOE_TOPK_CASE(16, 8)
  MOE_TOPK_CASE(16, 16)
  MOE_TOPK_CASE(32, 4)
  MOE_TOPK_CASE(32, 8)
  MOE_TOPK_CASE(32, 16)
  MOE_TOPK_CASE(64, 4)
  MOE_TOPK_CASE(64, 8)
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

size_t scan_lds_bytes(const Dims& d) {
  const int rps = d.R < kScanRows ? kScanRows / d.R : 1;
  return sizeof(int32_t) * ((size_t)d.R * rps * kScanEB + (size_t)d.R * kScanEB);
}

hipError_t launch_scan(const Dims& d, const uint64_t* tile_mask, int32_t* tile_base, int32_t* omega,
                       int32_t* count, hipStream_t st) {
  const int blocks = (d.E + kScanEB - 1) / kScanEB;
  const size_t lds = scan_lds_bytes(d);
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
  // slice 0 co-selection, slice 1 transitions; one launch covers the requested ones.
  const int nz = (cooc ? 1 : 0) + (trans ? 1 : 0);
  const int zbase = cooc ? 0 : 1;
  const int na = (d.E + 63) / 64;
  hipLaunchKernelGGL((pair_kernel<8>), dim3(na, (d.E + 7) / 8, nz), dim3(1024), 0, st, d, tile_mask, prev_mask, cooc,
                     trans, zbase);
  return hipGetLastError();
}

}  // namespace moe
