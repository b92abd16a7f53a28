// Correlated expert placement on gfx950.
//
// [Coupling] "Moving Correlated Experts Together": the co-selection counts
// C[a][b] (moe_plan_route's cooc) are the edge weights of a graph on the
// experts; the graph is partitioned over the R ranks with exactly E/R experts
// per rank so that heavily co-selected experts share a rank.  The objective is
//   intra = sum over pairs a < b on one rank of C[a][b]
// (for top-2 routing exactly the rows a deduplicating dispatcher saves),
// maximised by greedy growth and then pair-swap local search:
//   growth      ranks 0..R-1 in order; a rank's first expert is the unplaced
//               one with the largest deg(e) = sum_x C[e][x], each further one
//               the unplaced expert with the largest co-selection with the
//               rank's experts so far; ties to the lower expert id;
//   refinement  swap the pair a < b on different ranks with the largest gain
//                 aff[rb][a] - aff[ra][a] + aff[ra][b] - aff[rb][b] - 2 C[a][b]
//               (aff[r][x] = sum over y on rank r of C[x][y]; ties to the lower
//               a, then b) while the gain is positive, at most max_swaps times.
//
// One workgroup of 1024 threads; the problem is tiny and sequential.  Growth
// takes E steps of one argmax each: every thread holds the affinities of its
// E/1024 experts in registers, a wave's maximum comes from a DPP butterfly
// inside each 16-lane row and four lane reads, and the workgroup's from an LDS
// atomic max into one of three rotating slots -- one barrier per step.  When
// the counts fit 16 bits and E*E*2 bytes fit in LDS (E up to ~270), C is
// copied to LDS during the degree pass and one wave runs the whole growth
// (wave-uniform argmax, no atomic, no barrier per step).
// Refinement keeps, for every rank pair (r1 < r2), the best swap key of the
// pairs between them; a swap between ra and rb changes only the gains of pairs
// with an expert on ra or rb, so an iteration re-evaluates 2R-3 rank pairs
// (about 2*E*E/R expert pairs) instead of all E*E/2.  aff and the rank-pair
// keys live in LDS when they fit, else in the handle's workspace.
#include "internal.h"

namespace moe {
namespace {

constexpr int kPlaceThreads = 1024;
constexpr int kPlaceWaves = kPlaceThreads / 64;
constexpr uint64_t kGainBias = 1ull << 40;  // |gain| < 2^34 for valid counts
constexpr int kPairBits = 22;               // pair index a*E+b < 2048^2
constexpr uint64_t kPairMask = (1ull << kPairBits) - 1;

struct PlaceArgs {
  const int32_t* C;    // [E][E] co-selection counts
  int32_t max_swaps;
  int32_t* expert_rank;
  int32_t* rank_experts;
  int64_t* intra;
  int32_t* n_swaps;
  int32_t* aff_ws;     // [R][E] when aff does not fit in LDS
  uint64_t* key_ws;    // [R][R] when the rank-pair keys do not fit in LDS
  int32_t* status;
};

struct PlaceLds {
  size_t rank_of, mem, pos, deg, own, col, red, aff, key, c16, total;
  bool aff_in_lds, key_in_lds, c_in_lds;
};

constexpr size_t kPlaceAffLds = 64 * 1024;
constexpr size_t kPlaceKeyLds = 32 * 1024;

constexpr size_t kPlaceLdsBudget = 160 * 1024;
constexpr int kWaveGrowMaxE = 384;  // the one-wave growth holds up to 6 experts per lane

// Row stride (16-bit elements) of the LDS copy of C: even, so that a lane's
// two experts 2l, 2l + 1 are one aligned 32-bit word.  A tail pad of 128
// elements covers the last row's reads past E.
__host__ __device__ inline int c16_stride(int E) { return E + (E & 1); }

// LDS: the arrays of the whole kernel first; then a region that the growth
// uses for a 16-bit copy of the co-selection counts (when it fits) and the
// refinement for own, the per-wave columns, aff and the rank-pair keys.
PlaceLds place_lds(const Dims& d) {
  PlaceLds l;
  size_t o = 0;
  auto take = [&](size_t b) { const size_t at = o; o += (b + 15) / 16 * 16; return at; };
  l.rank_of = take(sizeof(int32_t) * d.E);
  l.mem = take(sizeof(int32_t) * d.E);
  l.pos = take(sizeof(int32_t) * d.E);
  l.deg = take(sizeof(int32_t) * d.E);
  l.red = take(sizeof(uint64_t) * (kPlaceWaves + 1));  // also the growth's three argmax slots
  const size_t shared_at = o;
  l.own = take(sizeof(int32_t) * d.E);
  l.col = take(sizeof(int32_t) * kPlaceWaves * (size_t)d.R);
  const size_t aff_b = sizeof(int32_t) * (size_t)d.R * d.E;
  const size_t key_b = sizeof(uint64_t) * (size_t)d.R * d.R;
  l.aff_in_lds = aff_b <= kPlaceAffLds;
  l.key_in_lds = key_b <= kPlaceKeyLds;
  l.aff = l.aff_in_lds ? take(aff_b) : 0;
  l.key = l.key_in_lds ? take(key_b) : 0;
  const size_t c16_b = sizeof(uint16_t) * ((size_t)d.E * c16_stride(d.E) + 128);
  l.c16 = shared_at;
  l.c_in_lds = shared_at + c16_b <= kPlaceLdsBudget && d.E <= kWaveGrowMaxE;
  l.total = l.c_in_lds && shared_at + c16_b > o ? shared_at + c16_b : o;
  return l;
}

// DPP moves inside a 16-lane row (quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror): after the four steps every lane holds its
// row's maximum.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}

__device__ __forceinline__ uint32_t row_max(uint32_t v) {
  v = max(v, dpp32<0xB1>(v));
  v = max(v, dpp32<0x4E>(v));
  v = max(v, dpp32<0x141>(v));
  return max(v, dpp32<0x140>(v));
}

__device__ __forceinline__ uint64_t row_max(uint64_t v) {
  auto step = [](uint64_t x, uint32_t lo, uint32_t hi) {
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    return o > x ? o : x;
  };
  v = step(v, dpp32<0xB1>((uint32_t)v), dpp32<0xB1>((uint32_t)(v >> 32)));
  v = step(v, dpp32<0x4E>((uint32_t)v), dpp32<0x4E>((uint32_t)(v >> 32)));
  v = step(v, dpp32<0x141>((uint32_t)v), dpp32<0x141>((uint32_t)(v >> 32)));
  return step(v, dpp32<0x140>((uint32_t)v), dpp32<0x140>((uint32_t)(v >> 32)));
}

__device__ __forceinline__ uint32_t lane_read(uint32_t v, int l) { return (uint32_t)__builtin_amdgcn_readlane((int)v, l); }
__device__ __forceinline__ uint64_t lane_read(uint64_t v, int l) {
  return ((uint64_t)lane_read((uint32_t)(v >> 32), l) << 32) | lane_read((uint32_t)v, l);
}

// Maximum over the wave, wave-uniform.
template <class K>
__device__ __forceinline__ K wave_max(K v) {
  v = row_max(v);
  const K a = lane_read(v, 0), b = lane_read(v, 16), c = lane_read(v, 32), e = lane_read(v, 48);
  const K x = a > b ? a : b, y = c > e ? c : e;
  return x > y ? x : y;
}

__device__ __forceinline__ int64_t wave_sum(int64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Maximum of v over the workgroup, returned to every thread.
__device__ __forceinline__ uint64_t block_max(uint64_t v, uint64_t* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) red[w] = v;
  __syncthreads();
  if (w == 0) {
    uint64_t x = lane < kPlaceWaves ? red[lane] : 0;
    x = wave_max(x);
    if (lane == 0) red[kPlaceWaves] = x;
  }
  __syncthreads();
  return red[kPlaceWaves];
}

// Rank-pair swap keys live in LDS (ds atomics) or in global memory (device
// atomics at L2; reads bypass the L1).
template <bool LDS>
__device__ __forceinline__ uint64_t key_load(const uint64_t* p) {
  if constexpr (LDS) return *p;
  else return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Swap keys of the pairs (x, y), y on another rank than x, folded into
// key[min(rx, ry)][max(rx, ry)] by atomic max.  A key is the gain, then the
// pair (lower id first) preferring lower ids:
//   gain = aff[ry][x] - own[x] + aff[rx][y] - own[y] - 2 C[x][y],
// own[e] = aff[rank(e)][e].  ALL: every x, with y > x.  Otherwise x runs over
// the experts of ranks ra and rb and y over all experts.  One wave per x:
// the C row and the aff[rx] row are read along y (coalesced); the column
// aff[*][x] goes to the wave's LDS buffer col.
template <bool ALL, bool KEY_LDS>
__device__ __forceinline__ void eval_rows(const Dims& d, const int32_t* __restrict__ C, const int32_t* aff,
                                          const int32_t* own, const int32_t* rank_of, const int32_t* mem,
                                          uint64_t* key, int32_t* col, int ra, int rb) {
  const int E = d.E, R = d.R, Er = d.Er;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nx = ALL ? E : 2 * Er;
  for (int i = wave; i < nx; i += kPlaceWaves) {
    const int x = ALL ? i : (i < Er ? mem[ra * Er + i] : mem[rb * Er + i - Er]);
    const int rx = rank_of[x];
    const int64_t ox = own[x];
    for (int r = lane; r < R; r += 64) col[r] = aff[(int64_t)r * E + x];
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    const int32_t* crow = C + (int64_t)x * E;
    const int32_t* arow = aff + (int64_t)rx * E;
#pragma unroll 2
    for (int y = (ALL ? x + 1 : 0) + lane; y < E; y += 64) {
      const int ry = rank_of[y];
      if (ry == rx) continue;
      const int64_t g = (int64_t)col[ry] - ox + arow[y] - own[y] - 2 * (int64_t)crow[y];
      const uint64_t pair = (uint64_t)min(x, y) * E + max(x, y);
      const uint64_t kk = ((uint64_t)(g + (int64_t)kGainBias) << kPairBits) | (kPairMask - pair);
      atomicMax(&key[min(rx, ry) * R + max(rx, ry)], kk);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // col is rewritten for the next x
  }
}

// Greedy growth in one wave, with C's rows in LDS (16-bit, row stride
// c16_stride(E), even): lane l holds the affinities of experts 2l + 128u and
// 2l + 128u + 1 (u < U), read as one 32-bit word per u and step with no
// bounds branch -- lanes past E read the next row (or the tail pad) into
// experts that are never alive.  The argmax is wave-uniform (DPP and lane
// reads), so a step needs no atomic and no barrier; the picks are kept one
// per lane and written out every 64 steps and at the end of each rank.
template <class K, int U>
__device__ __forceinline__ void grow_wave(const Dims& d, const uint16_t* c16, const int32_t* deg, int32_t* rank_of,
                                          int32_t* mem, int32_t* pos, int32_t* aff) {
  const int E = d.E, R = d.R, Er = d.Er, Es = c16_stride(E);
  const int lane = threadIdx.x & 63;
  constexpr int J = 2 * U;
  constexpr int kShift = 12;
  constexpr K kIdx = ((K)1 << kShift) - 1;
  int32_t dg[J], a[J];
  uint32_t alive = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = 2 * lane + 128 * (j >> 1) + (j & 1);
    dg[j] = e < E ? deg[e] : 0;
    if (e < E) alive |= 1u << j;
  }
  int32_t pk = 0;  // lane i: the pick of step (m - m % 64 + i) of the current rank
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int j = 0; j < J; ++j) a[j] = 0;
    for (int m = 0; m < Er; ++m) {
      K best = 0;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int e = 2 * lane + 128 * (j >> 1) + (j & 1);
        const K kk = ((K)(m == 0 ? dg[j] : a[j]) << kShift) | (K)(kIdx - e);
        best = ((alive >> j) & 1u) && kk > best ? kk : best;
      }
      best = wave_max(best);
      const int pick = (int)(kIdx - (best & kIdx));
      const uint32_t* row = reinterpret_cast<const uint32_t*>(c16 + pick * Es) + lane;
      uint32_t v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = row[64 * u];
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (2 * lane + 128 * (j >> 1) + (j & 1) == pick) alive &= ~(1u << j);
      const int q = m & 63;
      if (lane == q) pk = pick;
      if (q == 63 || m == Er - 1) {
        const int base = r * Er + m - q;
        if (lane <= q) {
          mem[base + lane] = pk;
          rank_of[pk] = r;
          pos[pk] = base + lane;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        a[2 * u] += (int32_t)(v[u] & 0xffffu);
        a[2 * u + 1] += (int32_t)(v[u] >> 16);
      }
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = 2 * lane + 128 * (j >> 1) + (j & 1);
      if (e < E) aff[(int64_t)r * E + e] = a[j];
    }
  }
}

template <class K>
__device__ __forceinline__ void grow_wave_any(const Dims& d, const uint16_t* c16, const int32_t* deg, int32_t* rank_of,
                                              int32_t* mem, int32_t* pos, int32_t* aff) {
  if (d.E <= 128) grow_wave<K, 1>(d, c16, deg, rank_of, mem, pos, aff);
  else if (d.E <= 256) grow_wave<K, 2>(d, c16, deg, rank_of, mem, pos, aff);
  else grow_wave<K, 3>(d, c16, deg, rank_of, mem, pos, aff);
}

// Greedy growth, one expert per step for E steps; thread t holds the
// affinities to the rank being filled of experts t, t + 1024, ... (NPL of
// them).  The step's argmax goes through slot[g % 3]: step g clears the slot
// of step g + 1, whose last readers (step g - 2) all passed barrier g - 1.
template <class K, int NPL>
__device__ __forceinline__ void grow(const Dims& d, const int32_t* __restrict__ C, const int32_t* deg, int32_t* rank_of,
                                     int32_t* mem, int32_t* pos, int32_t* aff, uint64_t* red) {
  const int E = d.E, R = d.R, Er = d.Er;
  const int tid = threadIdx.x, lane = tid & 63;
  constexpr int kShift = 12;  // kIdx - e >= 2048: a candidate's key is never 0
  constexpr K kIdx = ((K)1 << kShift) - 1;
  K* slot = reinterpret_cast<K*>(red);  // three slots
  if (tid < 3) slot[tid] = 0;
  __syncthreads();
  bool placed[NPL];
  int32_t a[NPL];
#pragma unroll
  for (int u = 0; u < NPL; ++u) placed[u] = false;
  int g = 0;
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int u = 0; u < NPL; ++u) a[u] = 0;
    for (int m = 0; m < Er; ++m, ++g) {
      K best = 0;
#pragma unroll
      for (int u = 0; u < NPL; ++u) {
        const int e = tid + kPlaceThreads * u;
        if (e < E && !placed[u]) {
          const int32_t sc = m == 0 ? deg[e] : max(a[u], 0);
          const K kk = ((K)sc << kShift) | (K)(kIdx - e);
          best = kk > best ? kk : best;
        }
      }
      best = wave_max(best);
      if (lane == 0 && best != 0) atomicMax(&slot[g % 3], best);
      if (tid == 0) slot[(g + 1) % 3] = 0;
      __syncthreads();
      const int pick = (int)(kIdx - (slot[g % 3] & kIdx));
#pragma unroll
      for (int u = 0; u < NPL; ++u)
        if (tid + kPlaceThreads * u == pick) placed[u] = true;
      if (tid == 0) {
        rank_of[pick] = r;
        mem[r * Er + m] = pick;
        pos[pick] = r * Er + m;
      }
      const int32_t* row = C + (int64_t)pick * E;  // C[pick][e] = C[e][pick]
#pragma unroll
      for (int u = 0; u < NPL; ++u) {
        const int e = tid + kPlaceThreads * u;
        if (e < E) a[u] += row[e];
      }
    }
#pragma unroll
    for (int u = 0; u < NPL; ++u) {
      const int e = tid + kPlaceThreads * u;
      if (e < E) aff[(int64_t)r * E + e] = a[u];
    }
  }
}

template <int NPL, bool AFF_LDS, bool KEY_LDS, bool C_LDS>
__global__ __launch_bounds__(kPlaceThreads) void place_kernel(Dims d, PlaceLds ly, PlaceArgs pa) {
  extern __shared__ __align__(16) char smem_place[];
  int32_t* rank_of = reinterpret_cast<int32_t*>(smem_place + ly.rank_of);
  int32_t* mem = reinterpret_cast<int32_t*>(smem_place + ly.mem);  // [R][Er] experts of each rank
  int32_t* pos = reinterpret_cast<int32_t*>(smem_place + ly.pos);  // slot of each expert in mem
  int32_t* deg = reinterpret_cast<int32_t*>(smem_place + ly.deg);
  int32_t* own = reinterpret_cast<int32_t*>(smem_place + ly.own);
  int32_t* col = reinterpret_cast<int32_t*>(smem_place + ly.col) + (threadIdx.x >> 6) * d.R;
  uint64_t* red = reinterpret_cast<uint64_t*>(smem_place + ly.red);
  int32_t* aff;
  uint64_t* key;
  if constexpr (AFF_LDS) aff = reinterpret_cast<int32_t*>(smem_place + ly.aff);
  else aff = pa.aff_ws;
  if constexpr (KEY_LDS) key = reinterpret_cast<uint64_t*>(smem_place + ly.key);
  else key = pa.key_ws;
  const int E = d.E, R = d.R, Er = d.Er;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t* __restrict__ C = pa.C;

  // Degrees (column sums, equal to the row sums of a symmetric matrix) and
  // input checks: zero diagonal, no negative count, sums below 2^31
  // (symmetry itself is the caller's contract).  Every thread reads: with E a
  // multiple of 4 and C 16-byte aligned, thread t takes the 16-byte column
  // group t mod (E/4) of the rows congruent to t / (E/4), otherwise one column
  // of the rows congruent to t / E (up to E = 512) or whole columns, and adds
  // its partial sums into 64-bit totals kept in the member and slot tables'
  // space (unused until the growth).
  uint16_t* c16 = reinterpret_cast<uint16_t*>(smem_place + ly.c16);
  int64_t* deg64 = reinterpret_cast<int64_t*>(smem_place + ly.mem);  // spans mem and pos
  const int Es = c16_stride(E);
  for (int e = tid; e < E; e += kPlaceThreads) deg64[e] = 0;
  __syncthreads();
  uint32_t my_max_entry = 0;  // a negative count reads as a large one here
  bool bad = false;
  auto add_deg = [&](int e, int64_t v) {
    atomicAdd(reinterpret_cast<unsigned long long*>(&deg64[e]), (unsigned long long)v);
  };
  if (E % 4 == 0 && ((uintptr_t)C & 15) == 0) {
    const int Q = E / 4, G = kPlaceThreads / Q;  // G >= 2: E <= 2048
    if (tid < G * Q) {
      const int c4 = tid % Q, g = tid / Q, e0 = 4 * c4;
      const int4* C4 = reinterpret_cast<const int4*>(C);
      int64_t s0 = 0, s1 = 0, s2 = 0, s3 = 0;
#pragma unroll 8
      for (int x = g; x < E; x += G) {
        const int4 v = C4[(int64_t)x * Q + c4];
        bad |= v.x < 0 || v.y < 0 || v.z < 0 || v.w < 0;
        if (x >= e0 && x < e0 + 4) bad |= (x == e0 ? v.x : x == e0 + 1 ? v.y : x == e0 + 2 ? v.z : v.w) != 0;
        s0 += v.x;
        s1 += v.y;
        s2 += v.z;
        s3 += v.w;
        if constexpr (C_LDS) {
          my_max_entry = max(my_max_entry, max(max((uint32_t)v.x, (uint32_t)v.y), max((uint32_t)v.z, (uint32_t)v.w)));
          uint2 h;  // used only when every entry fits; Es = E here, so 8-byte aligned
          h.x = ((uint32_t)v.x & 0xffffu) | ((uint32_t)v.y << 16);
          h.y = ((uint32_t)v.z & 0xffffu) | ((uint32_t)v.w << 16);
          *reinterpret_cast<uint2*>(c16 + x * Es + e0) = h;
        }
      }
      add_deg(e0, s0);
      add_deg(e0 + 1, s1);
      add_deg(e0 + 2, s2);
      add_deg(e0 + 3, s3);
    }
  } else {
    const int G = E <= kPlaceThreads / 2 ? kPlaceThreads / E : 1;
    for (int t = tid; t < G * E; t += kPlaceThreads) {
      const int e = t % E, g = t / E;
      int64_t s = 0;
#pragma unroll 8
      for (int x = g; x < E; x += G) {
        const int32_t v = C[(int64_t)x * E + e];
        bad |= v < 0 || (x == e && v != 0);
        s += v;
        if constexpr (C_LDS) {
          my_max_entry = max(my_max_entry, (uint32_t)v);
          c16[x * Es + e] = (uint16_t)v;  // used only when every entry fits
        }
      }
      add_deg(e, s);
    }
  }
  if (bad) atomicOr(pa.status, MOE_STATUS_BAD_PAIRS);
  bool use_c16 = false;
  if constexpr (C_LDS) use_c16 = block_max((uint64_t)my_max_entry, red) <= 0xffffu;
  else __syncthreads();
  int64_t my_max_deg = 0;
  for (int e = tid; e < E; e += kPlaceThreads) {
    const int64_t s = deg64[e];
    if (s > INT32_MAX) atomicOr(pa.status, MOE_STATUS_BAD_PAIRS);
    const int32_t dg = (int32_t)(s < 0 ? 0 : s > INT32_MAX ? INT32_MAX : s);
    deg[e] = dg;
    my_max_deg = max(my_max_deg, (int64_t)dg);
  }
  const uint64_t max_deg = block_max((uint64_t)my_max_deg, red);  // also publishes deg[]; deg64 is free after

  // Greedy growth.  Scores are sums of counts, so never above the largest
  // degree: when that is below 2^20 a 32-bit key (score, then 4095 - e) suffices.
  // With the LDS copy of C the first wave grows alone; as the refinement
  // reuses that LDS space, aff goes to the workspace first and into LDS after.
  if (use_c16) {
    if (wave == 0) {
      if (max_deg < (1u << 20)) grow_wave_any<uint32_t>(d, c16, deg, rank_of, mem, pos, pa.aff_ws);
      else grow_wave_any<uint64_t>(d, c16, deg, rank_of, mem, pos, pa.aff_ws);
    }
    __syncthreads();
    if constexpr (AFF_LDS)
      for (int q = tid; q < R * E; q += kPlaceThreads) aff[q] = pa.aff_ws[q];
  } else if (max_deg < (1u << 20)) {
    grow<uint32_t, NPL>(d, C, deg, rank_of, mem, pos, aff, red);
  } else {
    grow<uint64_t, NPL>(d, C, deg, rank_of, mem, pos, aff, red);
  }
  for (int64_t q = tid; q < (int64_t)R * R; q += kPlaceThreads) key[q] = 0;
  __syncthreads();
  for (int e = tid; e < E; e += kPlaceThreads) own[e] = aff[(int64_t)rank_of[e] * E + e];
  __syncthreads();

  // Best swap of every rank pair.
  eval_rows<true, KEY_LDS>(d, C, aff, own, rank_of, mem, key, col, 0, 0);
  __syncthreads();

  const int cap = pa.max_swaps < 0 ? 4096 : pa.max_swaps;
  int swaps = 0;
  for (;;) {
    uint64_t best = 0;
    for (int q = tid; q < R * R; q += kPlaceThreads) {
      const uint64_t v = key_load<KEY_LDS>(&key[q]);
      best = v > best ? v : best;
    }
    best = block_max(best, red);
    const int64_t gain = (int64_t)(best >> kPairBits) - (int64_t)kGainBias;
    if (best == 0 || gain <= 0 || swaps >= cap) break;
    const int64_t pair = (int64_t)(kPairMask - (best & kPairMask));
    const int xa = (int)(pair / E), xb = (int)(pair - (int64_t)xa * E);
    const int ra = rank_of[xa], rb = rank_of[xb];
    // aff of ranks ra and rb; clear the keys of every rank pair with ra or rb.
    for (int x = tid; x < E; x += kPlaceThreads) {
      const int32_t ca = C[(int64_t)xa * E + x], cb = C[(int64_t)xb * E + x];
      aff[(int64_t)ra * E + x] += cb - ca;
      aff[(int64_t)rb * E + x] += ca - cb;
    }
    for (int q = tid; q < 2 * R; q += kPlaceThreads) {
      const int c = q < R ? ra : rb, o = q < R ? q : q - R;
      if (o != c) key[min(c, o) * R + max(c, o)] = 0;
    }
    __syncthreads();  // every thread has read rank_of[xa], rank_of[xb]
    // The swap: each of the 2*Er slots of ranks ra and rb is rewritten by one
    // thread (xa and xb trade places), with its expert's rank, slot and own.
    for (int q = tid; q < 2 * Er; q += kPlaceThreads) {
      const int r = q < Er ? ra : rb, slot = r * Er + (q < Er ? q : q - Er);
      int e = mem[slot];
      e = e == xa ? xb : e == xb ? xa : e;
      mem[slot] = e;
      rank_of[e] = r;
      pos[e] = slot;
      own[e] = aff[(int64_t)r * E + e];
    }
    __syncthreads();
    eval_rows<false, KEY_LDS>(d, C, aff, own, rank_of, mem, key, col, ra, rb);
    __syncthreads();
    ++swaps;
  }

  // Outputs: ranks, the experts of each rank in ascending order, the kept weight.
  int64_t w = 0;
  for (int e = tid; e < E; e += kPlaceThreads) {
    const int r = rank_of[e];
    int before = 0;
    for (int i = 0; i < Er; ++i) before += mem[r * Er + i] < e;
    pa.expert_rank[e] = r;
    pa.rank_experts[r * Er + before] = e;
    w += own[e];
  }
  w = wave_sum(w);
  __syncthreads();
  if (lane == 0) reinterpret_cast<int64_t*>(red)[wave] = w;
  __syncthreads();
  if (tid == 0) {
    int64_t s = 0;
    for (int i = 0; i < kPlaceWaves; ++i) s += reinterpret_cast<int64_t*>(red)[i];
    *pa.intra = s / 2;  // each pair counted from both sides
    *pa.n_swaps = swaps;
  }
}

template <int NPL, bool AFF_LDS, bool KEY_LDS, bool C_LDS>
hipError_t launch_place_n(const Dims& d, const PlaceLds& ly, const PlaceArgs& pa, hipStream_t st) {
  auto kern = place_kernel<NPL, AFF_LDS, KEY_LDS, C_LDS>;
  if (ly.total > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)ly.total);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(1), dim3(kPlaceThreads), ly.total, st, d, ly, pa);
  return hipGetLastError();
}

template <int NPL, bool C_LDS>
hipError_t launch_place_lds(const Dims& d, const PlaceLds& ly, const PlaceArgs& pa, hipStream_t st) {
  if (ly.aff_in_lds && ly.key_in_lds) return launch_place_n<NPL, true, true, C_LDS>(d, ly, pa, st);
  if (ly.aff_in_lds) return launch_place_n<NPL, true, false, C_LDS>(d, ly, pa, st);
  if (ly.key_in_lds) return launch_place_n<NPL, false, true, C_LDS>(d, ly, pa, st);
  return launch_place_n<NPL, false, false, C_LDS>(d, ly, pa, st);
}

}  // namespace

size_t place_lds_bytes(const Dims& d) { return place_lds(d).total; }

hipError_t launch_place(const Dims& d, const int32_t* cooc, int32_t max_swaps, const moe_place_out& out,
                        const Workspace& ws, hipStream_t st) {
  const PlaceLds ly = place_lds(d);
  const PlaceArgs pa{cooc, max_swaps, out.expert_rank, out.rank_experts, out.intra, out.n_swaps,
                     ws.place_aff, ws.place_key, ws.status};
  if (ly.c_in_lds) return launch_place_lds<1, true>(d, ly, pa, st);  // E <= 384 here
  if (d.E <= kPlaceThreads) return launch_place_lds<1, false>(d, ly, pa, st);
  return launch_place_lds<2, false>(d, ly, pa, st);
}

}  // namespace moe
