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
#include "pair_count.h"
#include "tile_scan.h"

namespace moe {
namespace {

// Inverse of the order key u ^ (sign ? 0xffffffff : 0x80000000) of IEEE bits u.
__device__ __forceinline__ uint32_t float_from_order_key(uint32_t k) {
  return (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
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

// Exchange with lane (l ^ J) of the same aligned group of 2J lanes, all
// inside the DPP unit for J <= 8: quad permutes for J = 1, 2; for J = 4 a
// row shift left or right by 4 (selected by bit 2 of the lane); for J = 8 a
// row rotate by 8 (inside a row of 16 lanes that is l ^ 8).  J = 16 uses the
// swizzle unit (xor mask mode), J = 32 the LDS crossbar.
template <int J>
__device__ __forceinline__ uint32_t xor_lane_u32(uint32_t v, int lig) {
  if (J == 1) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false);
  if (J == 2) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false);
  if (J == 4) {
    const uint32_t up = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x104, 0xf, 0xf, false);  // row_shl:4
    const uint32_t dn = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
    return (lig & 4) ? dn : up;
  }
  if (J == 8) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false);
  if (J == 16) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (16 << 10) | 0x1F);
  return (uint32_t)__shfl_xor((int)v, J);
}

// Inclusive sum over the lanes 0..lig of each aligned group of P lanes: a DPP
// row scan (row shifts by 1, 2, 4, 8, masked at group borders), then row
// broadcasts for groups wider than a row.
template <int P>
__device__ __forceinline__ int group_incl_scan(int v, int lig) {
  int o;
  if (P >= 2) { o = __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false); v += (lig & 15) >= 1 ? o : 0; }
  if (P >= 4) { o = __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false); v += (lig & 15) >= 2 ? o : 0; }
  if (P >= 8) { o = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false); v += (lig & 15) >= 4 ? o : 0; }
  if (P >= 16) { o = __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false); v += (lig & 15) >= 8 ? o : 0; }
  if (P >= 32) { o = __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false); v += o; }  // row_bcast:15 into rows 1, 3
  if (P >= 64) { o = __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false); v += o; }  // row_bcast:31 into rows 2, 3
  return v;
}

// Value of the last lane of each aligned group of P lanes, in every lane.
template <int P>
__device__ __forceinline__ int group_last(int v) {
  if (P == 64) return __builtin_amdgcn_readlane(v, 63);
  return __builtin_amdgcn_ds_swizzle(v, ((0x1F & ~(P - 1)) << 0) | ((P - 1) << 5));
}

template <int SIZE, int J>
__device__ __forceinline__ uint32_t bitonic_step_u32(uint32_t v, int lig) {
  const uint32_t o = xor_lane_u32<J>(v, lig);
  const bool desc = (lig & SIZE) == 0;  // in the last stage every lane sorts descending
  const bool keep_max = ((lig & J) == 0) == desc;
  return keep_max ? max(o, v) : min(o, v);
}

// Bitonic sort of one 32-bit key per lane over aligned groups of P lanes,
// descending: afterwards lane l of a group holds the group's (l+1)-th largest.
template <int P>
__device__ __forceinline__ uint32_t group_sort_desc_u32(uint32_t v, int lig) {
#define MOE_BSTEP(S, J) if (P >= (S)) v = bitonic_step_u32<((S) >= P ? P : (S)), J>(v, lig);
  MOE_BSTEP(2, 1)
  MOE_BSTEP(4, 2) MOE_BSTEP(4, 1)
  MOE_BSTEP(8, 4) MOE_BSTEP(8, 2) MOE_BSTEP(8, 1)
  MOE_BSTEP(16, 8) MOE_BSTEP(16, 4) MOE_BSTEP(16, 2) MOE_BSTEP(16, 1)
  MOE_BSTEP(32, 16) MOE_BSTEP(32, 8) MOE_BSTEP(32, 4) MOE_BSTEP(32, 2) MOE_BSTEP(32, 1)
  MOE_BSTEP(64, 32) MOE_BSTEP(64, 16) MOE_BSTEP(64, 8) MOE_BSTEP(64, 4) MOE_BSTEP(64, 2) MOE_BSTEP(64, 1)
#undef MOE_BSTEP
  return v;
}

// Tokens per top-k workgroup: one token per group of P lanes, every token of
// the workgroup in a single round (no loop, no prefetch registers).  A 64-token
// tile is split over 64 / TPW workgroups, each of which stores its TPW-bit
// slice (8 bits at least) of every presence mask.  Workgroups are 256 threads
// (512 for 64 lanes per token): the size of a gather workgroup, so that with
// two batches in flight the top-k of one takes the slots the other batch's
// gather frees one workgroup at a time (1024-thread workgroups waited there
// for the whole gather: 755 us instead of 22 on MI355X; alone the two sizes
// run the same).
template <int P, int V>
constexpr int topk_tpw() {
  return 256 / P < 8 ? 8 : (256 / P > 64 ? 64 : 256 / P);
}
template <int P, int V>
constexpr int topk_threads() {
  return topk_tpw<P, V>() * P;
}

// Expert held in key slot v of lane l: 16-byte loads give lane l the experts
// 4(l + P w) .. 4(l + P w) + 3 for w = v / 4; scalar loads give l + P v.
template <int P, bool VEC4>
__device__ __forceinline__ int slot_expert(int l, int v) {
  return VEC4 ? 4 * (l + P * (v >> 2)) + (v & 3) : l + P * v;
}

// Order key of IEEE bits u: the IEEE total order as unsigned integers.
__device__ __forceinline__ uint32_t order_key(uint32_t u) {
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Order keys of the IEEE total order: +inf and -inf.  A NaN's key lies above
// the first (positive NaNs) or below the second (negative NaNs).
constexpr uint32_t kKeyPosInf = 0xFF800000u;
constexpr uint32_t kKeyNegInf = 0x007FFFFFu;
constexpr uint32_t kKeyNegZero = 0x7FFFFFFFu;
constexpr uint32_t kKeyPosZero = 0x80000000u;

// A group of P lanes handles one token, lane l holding V logits as order
// keys.  Selection:
//   1. tau = the k-th largest of the P lane maxima.  k keys reach tau, so
//      every key of the top-k does; the keys >= tau are the candidates.
//   2. The candidates (about k + 2 on average when P >= 2k) are compacted to
//      LDS as 64-bit keys (order key << 32 | (0x7fffffff - e) << 1), unique
//      per expert, so a key's rank among them is its output position: larger
//      logit first, equal logits to the lower expert.
// -0.0 must rank equal to +0.0 (and keep its own bits), which 32-bit order keys
// do not express, and more than P candidates do not fit the group: such tokens
// take k rounds of a group max over 64-bit keys that fold -0.0 onto +0.0 and
// keep the sign in bit 0.
// A NaN shows as a lane maximum above the key of +inf or a lane minimum below
// the key of -inf.  With `full` (P*V == E, 16-byte loads) every slot holds an
// expert and no slot needs masking.
template <int P, int V, bool VEC4>
__global__ __launch_bounds__((topk_threads<P, V>())) void route_topk_kernel(Dims d, bool full,
                                                                        const float* __restrict__ logits,
                                                                        const int32_t* __restrict__ prev_topk,
                                                                        int32_t* __restrict__ topk_idx,
                                                                        float* __restrict__ topk_val,
                                                                        uint64_t* __restrict__ tile_mask,
                                                                        uint64_t* __restrict__ prev_mask,
                                                                        int32_t* __restrict__ omega_acc,
                                                                        int32_t* __restrict__ status) {
  constexpr int TPW = topk_tpw<P, V>();
  constexpr int SLICES = 64 / TPW;
  extern __shared__ unsigned long long smem_masks[];
  unsigned long long* smask = smem_masks;
  unsigned long long* pmask = smem_masks + d.E;
  const int x = blockIdx.x / SLICES, h = blockIdx.x - x * SLICES;
  const int s = x / d.C, c = x - s * d.C;
  const int64_t t0 = (int64_t)s * d.Tr + (int64_t)c * kTile + h * TPW;
  const int nt = max(0, min(TPW, d.Tr - c * kTile - h * TPW));
  const int tid = threadIdx.x, nthr = blockDim.x;
  const bool want_prev = prev_topk != nullptr;
  for (int e = tid; e < d.E; e += nthr) {
    smask[e] = 0ull;
    if (want_prev) pmask[e] = 0ull;
  }
  __syncthreads();

  const int lane = tid % P;                // lane inside the token group
  const int grp_base = (tid & 63) - lane;  // wave lane of the group's first lane
  const uint64_t grp_bits = (P == 64 ? ~0ull : ((1ull << P) - 1ull)) << grp_base;
  uint64_t* cand = reinterpret_cast<uint64_t*>(smem_masks + (want_prev ? 2 : 1) * d.E) + (tid & ~63) + grp_base;
  const int i = tid / P;  // token of this group
  bool bad = false;
  if (i < nt) {
    const int64_t t = t0 + i;
    const float* __restrict__ row = logits + t * d.E;
    uint32_t key[V];
    if (VEC4) {
#pragma unroll
      for (int w = 0; w < V / 4; ++w) {
        const int e0 = slot_expert<P, VEC4>(lane, 4 * w);
        const float4 f = *reinterpret_cast<const float4*>(row + (full || e0 < d.E ? e0 : 0));
        key[4 * w + 0] = __float_as_uint(f.x);
        key[4 * w + 1] = __float_as_uint(f.y);
        key[4 * w + 2] = __float_as_uint(f.z);
        key[4 * w + 3] = __float_as_uint(f.w);
      }
    } else {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int e = slot_expert<P, VEC4>(lane, v);
        key[v] = __float_as_uint(row[e < d.E ? e : 0]);
      }
    }
    uint32_t lmax, lmin;
    if (full) {
#pragma unroll
      for (int v = 0; v < V; ++v) key[v] = order_key(key[v]);
      lmax = key[0];
      lmin = key[0];
#pragma unroll
      for (int v = 1; v < V; ++v) {
        lmax = max(lmax, key[v]);
        lmin = min(lmin, key[v]);
      }
    } else {
      lmax = 0u;
      lmin = ~0u;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        // with 16-byte loads E is a multiple of 4: a vector is valid as a whole
        const bool ok = VEC4 ? 4 * (lane + P * (v >> 2)) < d.E : slot_expert<P, VEC4>(lane, v) < d.E;
        const uint32_t kv = order_key(key[v]);
        key[v] = ok ? kv : 0u;  // 0: below every logit
        lmax = max(lmax, key[v]);
        lmin = min(lmin, ok ? kv : ~0u);
      }
    }
    bad = lmax > kKeyPosInf || lmin < kKeyNegInf;
    bool fast = d.k <= P;
    if (fast) {
      const uint32_t tau = (uint32_t)__shfl((int)group_sort_desc_u32<P>(lmax, lane), grp_base + d.k - 1);
      if ((__ballot(tau <= kKeyPosZero) & grp_bits) != 0ull) {
        // threshold at or below +0.0: a -0.0 may tie with a candidate
        bool nz = false;
#pragma unroll
        for (int v = 0; v < V; ++v) nz |= key[v] == kKeyNegZero;
        fast = (__ballot(nz) & grp_bits) == 0ull;
      }
      int mine = 0;
#pragma unroll
      for (int v = 0; v < V; ++v) mine += key[v] >= tau ? 1 : 0;
      const int incl = group_incl_scan<P>(mine, lane);
      const int total = group_last<P>(incl);
      fast = fast && total <= P;
      if (fast) {
        int w = incl - mine;
#pragma unroll
        for (int v = 0; v < V; ++v) {
          if (key[v] >= tau) {
            const uint32_t e = (uint32_t)slot_expert<P, VEC4>(lane, v);
            cand[w++] = ((uint64_t)key[v] << 32) | (uint64_t)((0x7fffffffu - e) << 1);
          }
        }
        wave_lds_sync();
        const uint64_t my = cand[lane < total ? lane : 0];
        int rank = 0;
        for (int j = 0; j < total; ++j) rank += cand[j] > my ? 1 : 0;
        if (lane < total && rank < d.k) {
          const int e = (int)(0x7fffffffu - ((uint32_t)my >> 1));
          if ((unsigned)e < (unsigned)d.E) {
            topk_idx[t * d.k + rank] = e;
            if (topk_val) topk_val[t * d.k + rank] = __uint_as_float(float_from_order_key((uint32_t)(my >> 32)));
            atomicOr(&smask[e], 1ull << i);
          } else {
            bad = true;
          }
        }
        wave_lds_sync();
      }
    }
    if (!fast) {
      // k rounds of a group max.  -0.0 ranks as +0.0: its key is folded onto
      // +0.0's (the output value is read back from the row, which keeps the
      // sign).  Each round every lane takes its largest key (ties to the
      // lower slot, i.e. the lower expert), the group the largest (key, lower
      // expert) pair, and the lane holding it clears that key.
#pragma unroll
      for (int v = 0; v < V; ++v) key[v] = key[v] == kKeyNegZero ? kKeyPosZero : key[v];
      for (int j = 0; j < d.k; ++j) {
        uint32_t kb = key[0];
        int vb = 0;
#pragma unroll
        for (int v = 1; v < V; ++v) {
          const bool gt = key[v] > kb;
          kb = gt ? key[v] : kb;
          vb = gt ? v : vb;
        }
        const uint32_t eb = (uint32_t)slot_expert<P, VEC4>(lane, vb);
        const uint64_t mine64 = kb == 0u ? 0ull : ((uint64_t)kb << 32) | (uint64_t)(0x7fffffffu - eb);
        const uint64_t gbest = group_max_u64<P>(mine64);
        if (gbest != 0ull && mine64 == gbest) {
#pragma unroll
          for (int v = 0; v < V; ++v) key[v] = v == vb ? 0u : key[v];
        }
        if (lane == 0) {
          const int e = (int)(0x7fffffffu - (uint32_t)gbest);
          if (gbest != 0ull && (unsigned)e < (unsigned)d.E) {
            topk_idx[t * d.k + j] = e;
            if (topk_val) topk_val[t * d.k + j] = row[e];
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
      const int ip = q / d.k;
      const int e = prev_topk[(t0 + ip) * d.k + (q - ip * d.k)];
      if ((unsigned)e < (unsigned)d.E) {
        const unsigned long long old = atomicOr(&pmask[e], 1ull << ip);
        if (old & (1ull << ip)) atomicOr(status, MOE_STATUS_BAD_TOPK);
      } else {
        atomicOr(status, MOE_STATUS_BAD_TOPK);
      }
    }
  }
  if (bad) atomicOr(status, MOE_STATUS_NAN_LOGIT);
  __syncthreads();
  // This workgroup's TPW-bit slice of every mask word of the tile.
  for (int e = tid; e < d.E; e += nthr) {
    const unsigned long long mk = smask[e];
    uint64_t* word = tile_mask + (int64_t)x * d.E + e;
    if (TPW == 64) *word = mk;
    else if (TPW == 32) reinterpret_cast<uint32_t*>(word)[h] = (uint32_t)mk;
    else if (TPW == 16) reinterpret_cast<uint16_t*>(word)[h] = (uint16_t)mk;
    else reinterpret_cast<uint8_t*>(word)[h] = (uint8_t)mk;
    if (want_prev) {
      const unsigned long long pk = pmask[e];
      uint64_t* pw = prev_mask + (int64_t)x * d.E + e;
      if (TPW == 64) *pw = pk;
      else if (TPW == 32) reinterpret_cast<uint32_t*>(pw)[h] = (uint32_t)pk;
      else if (TPW == 16) reinterpret_cast<uint16_t*>(pw)[h] = (uint16_t)pk;
      else reinterpret_cast<uint8_t*>(pw)[h] = (uint8_t)pk;
    }
    if (omega_acc && mk != 0ull) atomicAdd(&omega_acc[(int64_t)s * d.E + e], __popcll(mk));  // Eq. 3
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

// omega, expert counts and the exclusive tile prefix: one workgroup of 1024
// threads per kScanEB experts (tile_scan.h).
__global__ __launch_bounds__(1024) void scan_kernel(Dims d, const uint64_t* __restrict__ tile_mask,
                                                    int32_t* __restrict__ tile_base, int32_t* __restrict__ omega,
                                                    int32_t* __restrict__ count) {
  extern __shared__ __align__(16) int32_t smem_scan[];  // the pair blocks read 64-bit words
  tile_scan_block<1024>(d, tile_mask, tile_base, omega, count, nullptr, nullptr, blockIdx.x, smem_scan);
}

// Sums of the pair-count partials (pair_count.h), 256 threads per workgroup.
constexpr int kPairThreads = 256;

// The staged calls: the scan's workgroups first, then the pair-count
// partials, in one launch of 1024-thread workgroups.
__global__ __launch_bounds__(1024) void scan_pair_kernel(Dims d, const uint64_t* __restrict__ tile_mask,
                                                         int32_t* __restrict__ tile_base, int32_t* __restrict__ omega,
                                                         int32_t* __restrict__ count, PairArgs pa, int n_scan) {
  extern __shared__ __align__(16) int32_t smem_scan[];  // the pair blocks read 64-bit words
  if ((int)blockIdx.x < n_scan) {
    tile_scan_block<1024>(d, tile_mask, tile_base, omega, count, nullptr, nullptr, blockIdx.x, smem_scan);
    return;
  }
  const int q = (int)blockIdx.x - n_scan, nb = pair_blocks(d);
  const int blk = q % nb, rest = q / nb;
  pair_partial_block<1024>(d, pa, rest / pa.splits + pa.zbase, blk, rest % pa.splits, smem_scan);
}

__global__ __launch_bounds__(kPairThreads) void pair_reduce_kernel(Dims d, PairArgs pa) {
  pair_reduce_one(d, pa, (int)blockIdx.z + pa.zbase, blockIdx.x, blockIdx.y * kPairThreads + threadIdx.x);
}

template <int P, int V, bool VEC4>
hipError_t launch_topk_pv(const Dims& d, bool full, const float* logits, const int32_t* prev_topk, int32_t* topk_idx,
                          float* topk_val, uint64_t* tile_mask, uint64_t* prev_mask, int32_t* omega_acc,
                          int32_t* status, hipStream_t st) {
  constexpr int threads = topk_threads<P, V>();
  constexpr int slices = 64 / topk_tpw<P, V>();
  const size_t lds = sizeof(unsigned long long) * ((size_t)d.E * (prev_topk ? 2 : 1) + threads);
  hipLaunchKernelGGL((route_topk_kernel<P, V, VEC4>), dim3((unsigned)(d.NT * slices)), dim3(threads), lds, st, d, full,
                     logits, prev_topk, topk_idx, topk_val, tile_mask, prev_mask, omega_acc, status);
  return hipGetLastError();
}

}  // namespace

// Lanes per token P: the smallest power of two (>= 4) that is at least 2k, so
// that the threshold of the selection (the k-th largest lane maximum) rarely
// admits more than P candidates, and leaves at most 32 logits per lane; V:
// logits per lane, a multiple of 4 (16-byte loads) when E is.
hipError_t launch_route_topk(const Dims& d, const float* logits, const int32_t* prev_topk, int32_t* topk_idx,
                             float* topk_val, uint64_t* tile_mask, uint64_t* prev_mask, int32_t* omega_acc,
                             int32_t* status, hipStream_t st) {
  if (d.NT == 0) return hipSuccess;
  const bool vec4 = (d.E % 4) == 0 && ((uintptr_t)logits % 16) == 0;
  int P = 4;
  while (P < 64 && (P < 2 * d.k || P * 32 < d.E)) P *= 2;
  int V;
  if (vec4) {
    V = (d.E + 4 * P - 1) / (4 * P) * 4;
  } else {
    V = 8;
    while (P * V < d.E) V *= 4;  // 8 or 32
  }
  const bool full = vec4 && P * V == d.E;
#define MOE_TOPK_CASE(P_, V_, VEC_)                                                                          \
  if (P == (P_) && V == (V_) && vec4 == (VEC_))                                                             \
    return launch_topk_pv<P_, V_, VEC_>(d, full, logits, prev_topk, topk_idx, topk_val, tile_mask, prev_mask, \
                                        omega_acc, status, st);
#define MOE_TOPK_VEC(P_)                                                                                     \
  MOE_TOPK_CASE(P_, 4, true) MOE_TOPK_CASE(P_, 8, true) MOE_TOPK_CASE(P_, 12, true) MOE_TOPK_CASE(P_, 16, true) \
  MOE_TOPK_CASE(P_, 20, true) MOE_TOPK_CASE(P_, 24, true) MOE_TOPK_CASE(P_, 28, true) MOE_TOPK_CASE(P_, 32, true) \
  MOE_TOPK_CASE(P_, 8, false) MOE_TOPK_CASE(P_, 32, false)
  MOE_TOPK_VEC(4)
  MOE_TOPK_VEC(8)
  MOE_TOPK_VEC(16)
  MOE_TOPK_VEC(32)
  MOE_TOPK_VEC(64)
#undef MOE_TOPK_VEC
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

size_t scan_lds_bytes(const Dims& d) { return tile_scan_lds_bytes(d, 1024); }

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

size_t pair_part_words(const Dims& d) {
  const int sp = pair_splits(d, kPairThreads);  // bounds the split counts of 512- and 1024-thread workgroups
  return sp > 1 ? (size_t)2 * pair_blocks(d) * sp * kPairBlock : 0;
}

PairArgs pair_args(const Dims& d, const uint64_t* tile_mask, const uint64_t* prev_mask, int32_t* cooc, int32_t* trans,
                   int32_t* part, int nthr) {
  PairArgs pa;
  pa.cur = tile_mask;
  pa.prev = prev_mask;
  pa.cooc = cooc;
  pa.trans = trans;
  pa.part = part;
  pa.splits = pair_splits(d, nthr);
  pa.nz = (cooc ? 1 : 0) + (trans ? 1 : 0);
  pa.zbase = cooc ? 0 : 1;
  return pa;
}

hipError_t launch_scan_pairs(const Dims& d, const uint64_t* tile_mask, int32_t* tile_base, int32_t* omega,
                             int32_t* count, const uint64_t* prev_mask, int32_t* cooc, int32_t* trans, int32_t* part,
                             hipStream_t st) {
  if (!cooc && !trans) return launch_scan(d, tile_mask, tile_base, omega, count, st);
  const PairArgs pa = pair_args(d, tile_mask, prev_mask, cooc, trans, part, 1024);
  const int n_scan = (d.E + kScanEB - 1) / kScanEB;
  const int64_t n_pair = (int64_t)pair_blocks(d) * pa.splits * pa.nz;
  size_t lds = scan_lds_bytes(d);
  if (lds < pair_lds_bytes(1024)) lds = pair_lds_bytes(1024);
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(scan_pair_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(scan_pair_kernel, dim3((unsigned)(n_scan + n_pair)), dim3(1024), lds, st, d, tile_mask, tile_base,
                     omega, count, pa, n_scan);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pa.splits == 1) return e;
  hipLaunchKernelGGL(pair_reduce_kernel, dim3(pair_blocks(d), kPairBlock / kPairThreads, pa.nz), dim3(kPairThreads), 0,
                     st, d, pa);
  return hipGetLastError();
}

}  // namespace moe
