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
// Four launches.  The passes over all of C run on the whole chip; the two
// sequential phases run in one workgroup each:
//   prep   one wave per row: the degree (row sum), the input checks, the row's
//          largest entry and a 16-bit copy of the row;
//   grow   one workgroup.  One wave grows alone -- each step a wave-uniform
//          argmax (DPP and one lane read, no atomic, no barrier) and one row
//          read: the 16-bit rows from LDS when every count fits 16 bits and
//          the copy fits there (E <= 282); else, with every degree below
//          2^19, the int32 rows of C from L2; else the 16-bit copy from L2.
//          With degrees below 2^19 a key carries a live bit (a step adds the
//          count << 12, no mask), else a per-slot mask.  The rest (counts past 16 bits with E <= 282, or with a
//          degree of 2^19 or more) takes the whole workgroup: affinities in
//          registers, one LDS atomic max and one barrier per step.  It
//          leaves the ranks, aff and own[e] = aff[rank(e)][e];
//   pass   one wave per expert x: the swap keys of its pairs (x, y > x),
//          folded per rank in LDS, then one device atomic max per rank pair;
//   swap   one workgroup: the refinement.  A swap between ra and rb changes
//          only the gains of pairs with an expert on ra or rb, so an iteration
//          re-evaluates 2R-3 rank pairs (about 2*E*E/R expert pairs) instead
//          of all E*E/2.  aff and the rank-pair keys live in LDS when they fit.
#include <type_traits>
#include <algorithm>

#include "internal.h"

namespace moe {
namespace {

constexpr int kPlaceThreads = 1024;
constexpr int kPlaceWaves = kPlaceThreads / 64;
constexpr int kPassWaves = 4;               // waves per workgroup of the prep and pair passes
constexpr int kGrowThreads = 256;           // the growth's workgroup
constexpr int kGrowWaves = kGrowThreads / 64;
constexpr uint64_t kGainBias = 1ull << 40;  // |gain| < 2^34 for valid counts
constexpr int kPairBits = 22;               // pair index a*E+b < 2048^2
constexpr uint64_t kPairMask = (1ull << kPairBits) - 1;

constexpr size_t kPlaceAffLds = 64 * 1024;
constexpr size_t kPlaceKeyLds = 34 * 1024;  // R up to 64, rows padded by one key
constexpr size_t kPlaceLdsBudget = 160 * 1024;
constexpr int kMaxU = 16;  // 32-bit words of a 16-bit row per lane: E <= 2048
constexpr size_t kGrowRedBytes = 16 * (kGrowWaves + 2);  // the reduction slots and a sink word

// Row stride (16-bit elements) of the 16-bit copy of C: even, so that a lane's
// two experts 2l, 2l + 1 are one aligned 32-bit word.  A tail pad of 128
// elements covers the last row's reads past E.
__host__ __device__ inline int c16_stride(int E) { return E + (E & 1); }
__host__ __device__ inline size_t c16_count(int E) { return (size_t)E * c16_stride(E) + 128; }

// The workspace parts of the placement.
struct PlaceState {
  int32_t* deg;      // [E] row sums, clamped to [0, 2^31)
  int32_t* rowmax;   // [E] largest entry of each row, as unsigned (a negative entry reads as a large one)
  int32_t* rank_of;  // [E]
  int32_t* own;      // [E] aff[rank_of[e]][e]
  int32_t* mem;      // [R][Er] the experts of each rank
  int32_t* aff;      // [R][E]
  uint64_t* key;     // [R][R] best swap key of each rank pair (r1 < r2)
  uint16_t* c16;     // [E][c16_stride(E)] + pad
};

PlaceState place_state(const Dims& d, const Workspace& ws) {
  return PlaceState{ws.place_int,         ws.place_int + d.E, ws.place_int + 2 * d.E, ws.place_int + 3 * d.E,
                    ws.place_mem,         ws.place_aff,       ws.place_key,           ws.place_c16};
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

// Maximum over the wave, wave-uniform, for the growth's per-step argmax: the
// 16-lane row maxima, then row_bcast:15 (rows 1 and 3 take the last lane of
// the row before) and row_bcast:31 (rows 2 and 3 take lane 31), so lane 63
// holds the maximum: one lane read instead of four and their scalar maxima.
// Keys are unsigned, so the 0 that disabled rows read leaves them unchanged.
__device__ __forceinline__ uint32_t bcast_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));
  return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));
}

__device__ __forceinline__ uint64_t bcast_max(uint64_t v) {
  auto step = [](uint64_t x, uint32_t lo, uint32_t hi) {
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    return o > x ? o : x;
  };
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, 0x142, 0xa, 0xf, false),
           (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), 0x142, 0xa, 0xf, false));
  return step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, 0x143, 0xc, 0xf, false),
              (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), 0x143, 0xc, 0xf, false));
}

template <class K>
__device__ __forceinline__ K wave_max63(K v) {
  return lane_read(bcast_max(row_max(v)), 63);
}

__device__ __forceinline__ int64_t wave_sum(int64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Maximum of v over a workgroup of NW waves, returned to every thread
// (red: NW + 1 entries; the next call may follow at once, as it writes
// entries [0, NW) and reads entry NW only after a barrier).
template <int NW>
__device__ __forceinline__ uint64_t block_max(uint64_t v, uint64_t* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) red[w] = v;
  __syncthreads();
  if (w == 0) {
    uint64_t x = lane < NW ? red[lane] : 0;
    x = wave_max(x);
    if (lane == 0) red[NW] = x;
  }
  __syncthreads();
  return red[NW];
}

// Swap key of experts x on rank rx and y on rank ry != rx: the gain
//   aff[ry][x] - own[x] + aff[rx][y] - own[y] - 2 C[x][y]
// biased to be positive, then the pair (lower id first) preferring lower ids.
__device__ __forceinline__ uint64_t swap_key(int64_t gain, int x, int y, int E) {
  const uint64_t pair = (uint64_t)min(x, y) * E + max(x, y);
  return ((uint64_t)(gain + (int64_t)kGainBias) << kPairBits) | (kPairMask - pair);
}

// Brings [p, p + bytes) into this CU's L2 (one dword per 128-byte line, eight
// lines in flight per thread) so that the sequential phase after it reads its
// rows at L2 latency.  The loaded words are folded into *sink (LDS) only to
// keep the loads; the value is meaningless.
template <int NT>
__device__ __forceinline__ void warm_l2(const void* p, size_t bytes, uint32_t* sink) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(p);
  const int64_t lines = (int64_t)(bytes / 128);
  uint32_t acc = 0;
  for (int64_t l0 = threadIdx.x; l0 < lines; l0 += 8 * NT) {
    uint32_t t[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) t[b] = l0 + b * NT < lines ? w[(l0 + b * NT) * 32] : 0;
#pragma unroll
    for (int b = 0; b < 8; ++b) acc ^= t[b];
  }
  if (acc == 0x9e3779b9u) *sink = acc;
}

// ---------------------------------------------------------------------------
// prep: one wave per row e of C.  deg[e] = sum_x C[e][x], the checks (no
// negative count, zero diagonal, row sum below 2^31; symmetry is the caller's
// contract), the row's largest entry and its 16-bit copy (meaningful only
// when every entry fits 16 bits, which the growth checks).
__global__ __launch_bounds__(64 * kPassWaves) void place_prep_kernel(Dims d, const int32_t* __restrict__ C,
                                                                     PlaceState s, int32_t* __restrict__ status) {
  const int E = d.E, Es = c16_stride(E);
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * kPassWaves + (threadIdx.x >> 6);
  if (e >= E) return;  // no barrier below
  const int32_t* row = C + (int64_t)e * E;
  uint16_t* out = s.c16 + (size_t)e * Es;
  int64_t sum = 0;
  uint32_t mx = 0;
  bool bad = false;
  if (E % 4 == 0 && ((uintptr_t)C & 15) == 0) {
    const int4* r4 = reinterpret_cast<const int4*>(row);
#pragma unroll 4
    for (int q = lane; q < E / 4; q += 64) {
      const int4 v = r4[q];
      const int y = 4 * q;
      bad |= v.x < 0 || v.y < 0 || v.z < 0 || v.w < 0;
      if (e >= y && e < y + 4) bad |= (e == y ? v.x : e == y + 1 ? v.y : e == y + 2 ? v.z : v.w) != 0;
      sum += (int64_t)v.x + v.y + v.z + v.w;
      mx = max(mx, max(max((uint32_t)v.x, (uint32_t)v.y), max((uint32_t)v.z, (uint32_t)v.w)));
      uint2 h;  // Es = E here: 8-byte aligned
      h.x = ((uint32_t)v.x & 0xffffu) | ((uint32_t)v.y << 16);
      h.y = ((uint32_t)v.z & 0xffffu) | ((uint32_t)v.w << 16);
      *reinterpret_cast<uint2*>(out + y) = h;
    }
  } else {
    for (int y = lane; y < E; y += 64) {
      const int32_t v = row[y];
      bad |= v < 0 || (y == e && v != 0);
      sum += v;
      mx = max(mx, (uint32_t)v);
      out[y] = (uint16_t)v;
    }
  }
  if (bad) atomicOr(status, MOE_STATUS_BAD_PAIRS);
  sum = wave_sum(sum);
  mx = wave_max(mx);
  if (lane == 0) {
    if (sum > INT32_MAX) atomicOr(status, MOE_STATUS_BAD_PAIRS);
    s.deg[e] = (int32_t)(sum < 0 ? 0 : sum > INT32_MAX ? INT32_MAX : sum);
    s.rowmax[e] = (int32_t)mx;
  }
}

// ---------------------------------------------------------------------------
// grow: the greedy growth.

// One wave, with C's rows as 16-bit counts (row stride c16_stride(E), even):
// lane l holds the affinities of experts 2l + 128u and 2l + 128u + 1 (u < U),
// read as one 32-bit word per u and step with no bounds branch -- lanes past E
// read the next row (or the tail pad) into experts that are never alive.  A
// key is (score, then 4095 - e), masked to 0 once e is placed; the argmax is
// wave-uniform (DPP and one lane read), so a step needs no atomic and no
// barrier.  Step g's pick goes into lane g % 64 of a register, stored with
// its rank every 64 steps.  c16 points to LDS or to global memory.
template <class K, int U>
__device__ __forceinline__ void grow_wave(const Dims& d, const uint16_t* c16, const int32_t* deg, int32_t* rank_of,
                                          int32_t* mem, int32_t* aff) {
  const int E = d.E, R = d.R, Er = d.Er, Es = c16_stride(E);
  const int lane = threadIdx.x & 63;
  constexpr int J = 2 * U;
  constexpr int kShift = 12;
  constexpr K kIdx = ((K)1 << kShift) - 1;
  // live: 0 once placed, else -1 (a key mask); with more than eight slots a
  // vector, so that the slot a step kills is written by a wave-uniform index
  // in registers
  typedef int32_t LiveVec __attribute__((ext_vector_type(J <= 16 ? 16 : 32)));
  std::conditional_t<(J > 8), LiveVec, int32_t[J]> live;
  int32_t dg[J], a[J];
  uint32_t ik[J];  // 4095 - e
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = 2 * lane + 128 * (j >> 1) + (j & 1);
    ik[j] = (uint32_t)(kIdx - (K)e);
    live[j] = e < E ? -1 : 0;
    dg[j] = deg[min(e, E - 1)];  // unguarded: a guarded load waits alone
    a[j] = 0;
  }
  // picks of steps g0 .. g0 + n - 1 in lanes 0 .. n - 1: mem and rank_of
  auto flush = [&](int held, int g0, int n) {
    if (lane < n) {
      mem[g0 + lane] = held;
      rank_of[held] = (g0 + lane) / Er;
    }
  };
  int held = 0, g = 0;
  for (int r = 0; r < R; ++r) {
    for (int m = 0; m < Er; ++m, ++g) {
      K best = 0;
      if (m == 0) {
#pragma unroll
        for (int j = 0; j < J; ++j) best = max(best, (((K)(uint32_t)dg[j] << kShift) | ik[j]) & (K)(int64_t)live[j]);
      } else {
#pragma unroll
        for (int j = 0; j < J; ++j) best = max(best, (((K)(uint32_t)a[j] << kShift) | ik[j]) & (K)(int64_t)live[j]);
      }
      best = wave_max63(best);
      // A live expert always has a key above 0, so the pick is below E; the
      // clamp only keeps the row read inside the copy whatever the input.
      const int pick = min((int)(kIdx - (best & kIdx)), E - 1);
      const uint32_t* row = reinterpret_cast<const uint32_t*>(c16 + pick * Es) + lane;
      uint32_t v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = row[64 * u];
      // placed: slot 2 (pick / 128) + pick % 2 of lane (pick / 2) % 64.  The
      // slot index is wave-uniform: with many slots per lane the one register
      // is read and written by index (four instructions); with few, every slot
      // compares its id with the pick's.
      if constexpr (J > 8) {
        const int jp = 2 * (pick >> 7) + (pick & 1);
        live[jp] = lane == ((pick >> 1) & 63) ? 0 : live[jp];
      } else {
        const uint32_t ikp = (uint32_t)(kIdx - (K)pick);
#pragma unroll
        for (int j = 0; j < J; ++j) live[j] = ik[j] == ikp ? 0 : live[j];
      }
      held = lane == (g & 63) ? pick : held;
      if ((g & 63) == 63) flush(held, g - 63, 64);
      if (m == 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          a[2 * u] = (int32_t)(v[u] & 0xffffu);
          a[2 * u + 1] = (int32_t)(v[u] >> 16);
        }
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          a[2 * u] += (int32_t)(v[u] & 0xffffu);
          a[2 * u + 1] += (int32_t)(v[u] >> 16);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = 2 * lane + 128 * (j >> 1) + (j & 1);
      if (e < E) aff[(int64_t)r * E + e] = a[j];
    }
  }
  if (g & 63) flush(held, g & ~63, g & 63);
}

// grow_wave with the 32-bit live-bit keys of grow_wave_c32 (every degree below
// 2^19): a step adds each 16-bit count << 12 to its key with no mask.
template <int U>
__device__ __forceinline__ void grow_wave_live(const Dims& d, const uint16_t* c16, const int32_t* deg,
                                               int32_t* rank_of, int32_t* mem, int32_t* aff) {
  const int E = d.E, R = d.R, Er = d.Er, Es = c16_stride(E);
  const int lane = threadIdx.x & 63;
  constexpr int J = 2 * U;
  constexpr uint32_t kLive = 0x80000000u, kIdx = 0xfffu;
  uint32_t key[J], dk[J], ik[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = 2 * lane + 128 * (j >> 1) + (j & 1);
    ik[j] = kIdx - (uint32_t)e;
    key[j] = (e < E ? kLive : 0u) | ik[j];
    dk[j] = ((uint32_t)deg[min(e, E - 1)] << 12) | ik[j];  // unguarded: a guarded load waits alone
  }
  // picks of steps g0 .. g0 + n - 1 in lanes 0 .. n - 1: mem and rank_of
  auto flush = [&](int held, int g0, int n) {
    if (lane < n) {
      mem[g0 + lane] = held;
      rank_of[held] = (g0 + lane) / Er;
    }
  };
  int held = 0, g = 0;
  for (int r = 0; r < R; ++r) {
    for (int m = 0; m < Er; ++m, ++g) {
      uint32_t best = 0;
      if (m == 0) {
#pragma unroll
        for (int j = 0; j < J; ++j) best = max(best, (key[j] & kLive) | dk[j]);
      } else {
#pragma unroll
        for (int j = 0; j < J; ++j) best = max(best, key[j]);
      }
      best = wave_max63(best);
      // A live expert always has a key at or above 2^31, so the pick is below
      // E; the clamp only keeps the row read inside the copy whatever the input.
      const int pick = min((int)(kIdx - (best & kIdx)), E - 1);
      const uint32_t* row = reinterpret_cast<const uint32_t*>(c16 + pick * Es) + lane;
      uint32_t v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = row[64 * u];
      // placed: the one (lane, j) whose id part matches (experts past E never do)
      const uint32_t ikp = kIdx - (uint32_t)pick;
#pragma unroll
      for (int j = 0; j < J; ++j) key[j] = ik[j] == ikp ? key[j] & ~kLive : key[j];
      held = lane == (g & 63) ? pick : held;
      if ((g & 63) == 63) flush(held, g - 63, 64);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t lo = (v[u] & 0xffffu) << 12, hi = (v[u] >> 16) << 12;
        if (m == 0) {
          key[2 * u] = (key[2 * u] & (kLive | kIdx)) + lo;
          key[2 * u + 1] = (key[2 * u + 1] & (kLive | kIdx)) + hi;
        } else {
          key[2 * u] += lo;
          key[2 * u + 1] += hi;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = 2 * lane + 128 * (j >> 1) + (j & 1);
      if (e < E) aff[(int64_t)r * E + e] = (int32_t)((key[j] >> 12) & 0x7ffffu);
    }
  }
  if (g & 63) flush(held, g & ~63, g & 63);
}

// grow_wave for U = ceil(E / 128) words per lane (rounded up to an
// instantiated size); UMAX bounds the sizes instantiated.
template <class K, int UMAX>
__device__ __forceinline__ void grow_wave_u(int U, const Dims& d, const uint16_t* c16, const int32_t* deg,
                                            int32_t* rank_of, int32_t* mem, int32_t* aff) {
  if (U <= 1) grow_wave<K, 1>(d, c16, deg, rank_of, mem, aff);
  else if (UMAX <= 2 || U <= 2) grow_wave<K, (UMAX < 2 ? UMAX : 2)>(d, c16, deg, rank_of, mem, aff);
  else if (UMAX <= 3 || U <= 3) grow_wave<K, (UMAX < 3 ? UMAX : 3)>(d, c16, deg, rank_of, mem, aff);
  else if (UMAX <= 4 || U <= 4) grow_wave<K, (UMAX < 4 ? UMAX : 4)>(d, c16, deg, rank_of, mem, aff);
  else if (UMAX <= 5 || U <= 5) grow_wave<K, (UMAX < 5 ? UMAX : 5)>(d, c16, deg, rank_of, mem, aff);
  else if (UMAX <= 6 || U <= 6) grow_wave<K, (UMAX < 6 ? UMAX : 6)>(d, c16, deg, rank_of, mem, aff);
  else if (UMAX <= 7 || U <= 7) grow_wave<K, (UMAX < 7 ? UMAX : 7)>(d, c16, deg, rank_of, mem, aff);
  else if (UMAX <= 8 || U <= 8) grow_wave<K, (UMAX < 8 ? UMAX : 8)>(d, c16, deg, rank_of, mem, aff);
  else if (UMAX <= 10 || U <= 10) grow_wave<K, (UMAX < 10 ? UMAX : 10)>(d, c16, deg, rank_of, mem, aff);
  else if (UMAX <= 12 || U <= 12) grow_wave<K, (UMAX < 12 ? UMAX : 12)>(d, c16, deg, rank_of, mem, aff);
  else grow_wave<K, UMAX>(d, c16, deg, rank_of, mem, aff);
}

// One wave, from the int32 rows of C (L2-resident), when every degree is
// below 2^19: lane l holds experts l + 64 j (j < J), each as one 32-bit key
//   live << 31 | score << 12 | (4095 - e),
// the score (the co-selection with the rank so far, at most the expert's
// degree) never reaching bit 31.  A step adds each row entry << 12 to its key
// (one shift-and-add, no mask): a placed expert's cleared live bit keeps it
// below every live key.  The rank's first step keys the live experts by
// degree instead.  The placed slot is cleared by its wave-uniform index.
template <int J>
__device__ __forceinline__ void grow_wave_c32(const Dims& d, const int32_t* __restrict__ C, const int32_t* deg,
                                              int32_t* rank_of, int32_t* mem, int32_t* aff) {
  const int E = d.E, R = d.R, Er = d.Er;
  const int lane = threadIdx.x & 63;
  constexpr uint32_t kLive = 0x80000000u, kIdx = 0xfffu;
  typedef uint32_t KeyVec __attribute__((ext_vector_type(J <= 16 ? 16 : 32)));
  KeyVec key;
  uint32_t dk[J];  // deg << 12 | (4095 - e)
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + 64 * j;
    const uint32_t ik = kIdx - (uint32_t)e;
    key[j] = (e < E ? kLive : 0u) | ik;
    dk[j] = ((uint32_t)deg[min(e, E - 1)] << 12) | ik;  // unguarded: a guarded load waits alone
  }
  // picks of steps g0 .. g0 + n - 1 in lanes 0 .. n - 1: mem and rank_of
  auto flush = [&](int held, int g0, int n) {
    if (lane < n) {
      mem[g0 + lane] = held;
      rank_of[held] = (g0 + lane) / Er;
    }
  };
  int held = 0, g = 0;
  for (int r = 0; r < R; ++r) {
    for (int m = 0; m < Er; ++m, ++g) {
      uint32_t best = 0;
      if (m == 0) {
#pragma unroll
        for (int j = 0; j < J; ++j) best = max(best, (key[j] & kLive) | dk[j]);
      } else {
#pragma unroll
        for (int j = 0; j < J; ++j) best = max(best, (uint32_t)key[j]);
      }
      best = wave_max63(best);
      // A live expert always has a key at or above 2^31 (its degree key above
      // 0), so the pick is below E; the clamp only keeps the row read inside C.
      const int pick = min((int)(kIdx - (best & kIdx)), E - 1);
      const int32_t* row = C + (int64_t)pick * E;
      uint32_t v[J];
#pragma unroll
      for (int j = 0; j < J; ++j) v[j] = (uint32_t)row[min(64 * j + lane, E - 1)];
      const int jp = pick >> 6;
      key[jp] = lane == (pick & 63) ? key[jp] & ~kLive : key[jp];
      held = lane == (g & 63) ? pick : held;
      if ((g & 63) == 63) flush(held, g - 63, 64);
      if (m == 0) {
#pragma unroll
        for (int j = 0; j < J; ++j) key[j] = (key[j] & (kLive | kIdx)) + (v[j] << 12);
      } else {
#pragma unroll
        for (int j = 0; j < J; ++j) key[j] += v[j] << 12;
      }
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = lane + 64 * j;
      if (e < E) aff[(int64_t)r * E + e] = (int32_t)((key[j] >> 12) & 0x7ffffu);
    }
  }
  if (g & 63) flush(held, g & ~63, g & 63);
}

// grow_wave_c32 with J >= ceil(E / 64) slots per lane, from the sizes
// instantiated for a workgroup of 256 threads holding NPL experts each.
template <int NPL>
__device__ __forceinline__ void grow_wave_c32_e(const Dims& d, const int32_t* C, const int32_t* deg,
                                                int32_t* rank_of, int32_t* mem, int32_t* aff) {
  const int J = (d.E + 63) / 64;
  if constexpr (NPL <= 2) {
    if (J <= 6) grow_wave_c32<6>(d, C, deg, rank_of, mem, aff);
    else grow_wave_c32<8>(d, C, deg, rank_of, mem, aff);
  } else if constexpr (NPL <= 4) {
    if (J <= 10) grow_wave_c32<10>(d, C, deg, rank_of, mem, aff);
    else if (J <= 12) grow_wave_c32<12>(d, C, deg, rank_of, mem, aff);
    else if (J <= 14) grow_wave_c32<14>(d, C, deg, rank_of, mem, aff);
    else grow_wave_c32<16>(d, C, deg, rank_of, mem, aff);
  } else {
    if (J <= 20) grow_wave_c32<20>(d, C, deg, rank_of, mem, aff);
    else if (J <= 24) grow_wave_c32<24>(d, C, deg, rank_of, mem, aff);
    else if (J <= 28) grow_wave_c32<28>(d, C, deg, rank_of, mem, aff);
    else grow_wave_c32<32>(d, C, deg, rank_of, mem, aff);
  }
}

// The whole workgroup, with the int32 counts (any entry size): thread t holds
// the affinities to the rank being filled of experts t, t + 256, ... (NPL of
// them).  The step's argmax goes through slot[g % 3]: step g clears the slot
// of step g + 1, whose last readers (step g - 2) all passed barrier g - 1.
template <class K, int NPL>
__device__ __forceinline__ void grow_block(const Dims& d, const int32_t* __restrict__ C, const int32_t* deg,
                                           int32_t* rank_of, int32_t* mem, int32_t* aff, uint64_t* red) {
  const int E = d.E, R = d.R, Er = d.Er;
  const int tid = threadIdx.x, lane = tid & 63;
  constexpr int kShift = 12;  // kIdx - e >= 2048: a candidate's key is never 0
  constexpr K kIdx = ((K)1 << kShift) - 1;
  K* slot = reinterpret_cast<K*>(red);  // three slots
  if (tid < 3) slot[tid] = 0;
  __syncthreads();
  bool placed[NPL];
  int32_t a[NPL], dg[NPL];
#pragma unroll
  for (int u = 0; u < NPL; ++u) {
    const int e = tid + kGrowThreads * u;
    placed[u] = false;
    dg[u] = deg[min(e, E - 1)];  // unguarded: a guarded load waits alone
  }
  int g = 0;
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int u = 0; u < NPL; ++u) a[u] = 0;
    for (int m = 0; m < Er; ++m, ++g) {
      K best = 0;
#pragma unroll
      for (int u = 0; u < NPL; ++u) {
        const int e = tid + kGrowThreads * u;
        if (e < E && !placed[u]) {
          const int32_t sc = m == 0 ? dg[u] : max(a[u], 0);
          const K kk = ((K)sc << kShift) | (K)(kIdx - e);
          best = kk > best ? kk : best;
        }
      }
      best = wave_max(best);
      if (lane == 0 && best != 0) atomicMax(&slot[g % 3], best);
      if (tid == 0) slot[(g + 1) % 3] = 0;
      __syncthreads();
      const int pick = min((int)(kIdx - (slot[g % 3] & kIdx)), E - 1);  // below E for any live expert
#pragma unroll
      for (int u = 0; u < NPL; ++u)
        if (tid + kGrowThreads * u == pick) placed[u] = true;
      if (tid == 0) {
        rank_of[pick] = r;
        mem[r * Er + m] = pick;
      }
      const int32_t* row = C + (int64_t)pick * E;  // C[pick][e] = C[e][pick]
#pragma unroll
      for (int u = 0; u < NPL; ++u) {
        const int e = tid + kGrowThreads * u;
        if (e < E) a[u] += row[e];
      }
    }
#pragma unroll
    for (int u = 0; u < NPL; ++u) {
      const int e = tid + kGrowThreads * u;
      if (e < E) aff[(int64_t)r * E + e] = a[u];
    }
  }
}

// One workgroup of 256.  Reads the prep results; with every count within 16
// bits the first wave grows alone (from an LDS copy of the 16-bit rows when
// C_LDS, else from the copy in global memory), otherwise the workgroup does.
// Also clears the rank-pair keys for the pair pass and writes own.
template <bool C_LDS, int NPL>
__global__ __launch_bounds__(kGrowThreads) void place_grow_kernel(Dims d, const int32_t* __restrict__ C,
                                                                  PlaceState s) {
  extern __shared__ __align__(16) char smem_grow[];
  uint64_t* red = reinterpret_cast<uint64_t*>(smem_grow);  // kGrowWaves + 1 entries
  const int E = d.E, R = d.R;
  const int tid = threadIdx.x, wave = tid >> 6;
  uint32_t mx = 0, md = 0;
  for (int e = tid; e < E; e += kGrowThreads) {
    mx = max(mx, (uint32_t)s.rowmax[e]);
    md = max(md, (uint32_t)s.deg[e]);
  }
  for (int64_t q = tid; q < (int64_t)R * R; q += kGrowThreads) s.key[q] = 0;
  const bool fit16 = block_max<kGrowWaves>(mx, red) <= 0xffffu;
  const uint32_t mdeg = block_max<kGrowWaves>(md, red);
  const bool key32 = mdeg < (1u << 20);  // scores never exceed the largest degree
  const int U = (E + 127) / 128;
  if (!C_LDS && mdeg < (1u << 19)) {
    // rows too many for LDS, degrees small enough for the live-bit keys: the
    // int32 rows, warmed into this CU's L2
    warm_l2<kGrowThreads>(C, (size_t)E * E * sizeof(int32_t), reinterpret_cast<uint32_t*>(red + kGrowWaves + 1));
    __syncthreads();
    if (wave == 0) grow_wave_c32_e<NPL>(d, C, s.deg, s.rank_of, s.mem, s.aff);
  } else if (fit16) {
    const uint16_t* c16 = s.c16;
    if constexpr (C_LDS) {
      // The 16-bit rows into LDS, sixteen 16-byte loads in flight per thread.
      uint16_t* c16l = reinterpret_cast<uint16_t*>(smem_grow + kGrowRedBytes);
      const int nvec = (int)((size_t)E * c16_stride(E) * 2 / 16) + 1;  // within the pad
      const uint4* src = reinterpret_cast<const uint4*>(s.c16);
      uint4* dst = reinterpret_cast<uint4*>(c16l);
      for (int q0 = tid; q0 < nvec; q0 += 16 * kGrowThreads) {
        uint4 t[16];
#pragma unroll
        for (int b = 0; b < 16; ++b) t[b] = q0 + b * kGrowThreads < nvec ? src[q0 + b * kGrowThreads] : uint4{};
#pragma unroll
        for (int b = 0; b < 16; ++b)
          if (q0 + b * kGrowThreads < nvec) dst[q0 + b * kGrowThreads] = t[b];
      }
      c16 = c16l;
    } else {
      warm_l2<kGrowThreads>(s.c16, c16_count(E) * sizeof(uint16_t), reinterpret_cast<uint32_t*>(red + kGrowWaves + 1));
    }
    __syncthreads();
    // An LDS copy holds at most 282 rows: three words per lane.
    constexpr int UMAX = C_LDS ? 3 : kMaxU;
    if (wave == 0) {
      if (C_LDS && mdeg < (1u << 19)) {
        if (U <= 1) grow_wave_live<1>(d, c16, s.deg, s.rank_of, s.mem, s.aff);
        else if (U <= 2) grow_wave_live<2>(d, c16, s.deg, s.rank_of, s.mem, s.aff);
        else grow_wave_live<3>(d, c16, s.deg, s.rank_of, s.mem, s.aff);
      } else if (key32) {
        grow_wave_u<uint32_t, UMAX>(U, d, c16, s.deg, s.rank_of, s.mem, s.aff);
      } else {
        grow_wave_u<uint64_t, UMAX>(U, d, c16, s.deg, s.rank_of, s.mem, s.aff);
      }
    }
  } else if (key32) {
    grow_block<uint32_t, NPL>(d, C, s.deg, s.rank_of, s.mem, s.aff, red);
  } else {
    grow_block<uint64_t, NPL>(d, C, s.deg, s.rank_of, s.mem, s.aff, red);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kGrowThreads) s.own[e] = s.aff[(int64_t)s.rank_of[e] * E + e];
}

// ---------------------------------------------------------------------------
// pass: one wave per expert x, the keys of its pairs (x, y > x) with y on
// another rank; each wave folds them per rank ry in LDS (atomic max), then
// adds one device atomic max per rank into key[min(rx, ry)][max(rx, ry)].
// rank_of and own are staged in LDS by the workgroup.
__global__ __launch_bounds__(64 * kPassWaves) void place_pass_kernel(Dims d, const int32_t* __restrict__ C,
                                                                     PlaceState s) {
  extern __shared__ __align__(16) char smem_pass[];
  const int E = d.E, R = d.R;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t* kb = reinterpret_cast<uint64_t*>(smem_pass) + (size_t)wave * R;
  int32_t* col = reinterpret_cast<int32_t*>(smem_pass + sizeof(uint64_t) * kPassWaves * R) + (size_t)wave * R;
  int32_t* rk = reinterpret_cast<int32_t*>(smem_pass + (sizeof(uint64_t) + sizeof(int32_t)) * kPassWaves * R);
  int32_t* ow = rk + E;
  for (int e = threadIdx.x; e < E; e += 64 * kPassWaves) {
    rk[e] = s.rank_of[e];
    ow[e] = s.own[e];
  }
  __syncthreads();
  const int x = blockIdx.x * kPassWaves + wave;
  if (x >= E) return;  // no barrier below
  const int rx = rk[x];
  const int64_t ox = ow[x];
  for (int r = lane; r < R; r += 64) {
    col[r] = s.aff[(int64_t)r * E + x];
    kb[r] = 0;
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  const int32_t* crow = C + (int64_t)x * E;
  const int32_t* arow = s.aff + (int64_t)rx * E;
  constexpr int kB = 8;  // entries per lane with their loads in flight together (unguarded, clamped)
  for (int y0 = x + 1 + lane; y0 < E; y0 += 64 * kB) {
    int32_t av[kB], cv[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const int y = min(y0 + 64 * b, E - 1);
      av[b] = arow[y];
      cv[b] = crow[y];
    }
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const int y = y0 + 64 * b;
      if (y >= E) break;
      const int ry = rk[y];
      if (ry == rx) continue;
      const int64_t g = (int64_t)col[ry] - ox + av[b] - ow[y] - 2 * (int64_t)cv[b];
      atomicMax(&kb[ry], swap_key(g, x, y, E));
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  for (int r = lane; r < R; r += 64) {
    const uint64_t v = kb[r];
    if (v != 0) atomicMax(reinterpret_cast<unsigned long long*>(&s.key[min(rx, r) * R + max(rx, r)]),
                          (unsigned long long)v);
  }
}

// ---------------------------------------------------------------------------
// swap: the refinement, one workgroup of 1024.

struct SwapLds {
  size_t rank_of, mem, own, red, col, aff, key, total;
  bool aff_in_lds, key_in_lds;
};

SwapLds swap_lds(const Dims& d) {
  SwapLds l;
  size_t o = 0;
  auto take = [&](size_t b) { const size_t at = o; o += (b + 15) / 16 * 16; return at; };
  l.rank_of = take(sizeof(int32_t) * d.E);
  l.mem = take(sizeof(int32_t) * d.E);
  l.own = take(sizeof(int32_t) * d.E);
  l.red = take(sizeof(uint64_t) * (kPlaceWaves + 3));  // wave partials, a result, two swap-loop maxima
  l.col = take(sizeof(int32_t) * kPlaceWaves * (size_t)d.R);
  const size_t aff_b = sizeof(int32_t) * (size_t)d.R * d.E;
  const size_t key_b = sizeof(uint64_t) * (size_t)d.R * (d.R + 1);
  l.aff_in_lds = aff_b <= kPlaceAffLds;
  l.key_in_lds = key_b <= kPlaceKeyLds;
  l.aff = l.aff_in_lds ? take(aff_b) : 0;
  l.key = l.key_in_lds ? take(key_b) : 0;
  l.total = o;
  return l;
}

// Rank-pair swap keys live in LDS (ds atomics) or in global memory (device
// atomics at L2; reads bypass the L1).
template <bool LDS>
__device__ __forceinline__ uint64_t key_load(const uint64_t* p) {
  if constexpr (LDS) return *p;
  else return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Keys of the pairs (x, y) with x on rank ra or rb and y on another rank than
// x, folded into key[min(rx, ry) * ks + max(rx, ry)] by atomic max.  One wave per
// x: the column aff[*][x] goes to the wave's LDS buffer col; the C row and
// the aff[rx] row are read along y (coalesced), kB entries per lane at a time:
// every read of a batch (C, aff, rank, own; then the column entries of those
// ranks) is issued before its first key is formed and its atomics go out
// (the loads unguarded, at clamped indices: a guarded load gets a basic block
// and a wait of its own).
template <bool C16, int kB>
__device__ __forceinline__ void eval_rows(const Dims& d, const int32_t* __restrict__ C, const uint16_t* __restrict__ c16,
                                          const int32_t* aff, const int32_t* own, const int32_t* rank_of,
                                          const int32_t* mem, uint64_t* key, int ks, int32_t* col, int ra, int rb) {
  const int E = d.E, R = d.R, Er = d.Er, Es = c16_stride(E);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = wave; i < 2 * Er; i += kPlaceWaves) {
    const int x = i < Er ? mem[ra * Er + i] : mem[rb * Er + i - Er];
    const int rx = rank_of[x];
    const int64_t ox = own[x];
    for (int r = lane; r < R; r += 64) col[r] = aff[(int64_t)r * E + x];
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    const int32_t* crow = C + (int64_t)x * E;
    const uint16_t* hrow = c16 + (int64_t)x * Es;
    const int32_t* arow = aff + (int64_t)rx * E;
    for (int y0 = lane; y0 < E; y0 += 64 * kB) {
      // every read of the batch before any atomic: the reads, then the
      // column entries of the ranks just read, then the keys
      int32_t av[kB], cv[kB], ryv[kB], owv[kB], cov[kB];
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        const int y = min(y0 + 64 * b, E - 1);
        av[b] = arow[y];
        cv[b] = C16 ? (int32_t)hrow[y] : crow[y];
        ryv[b] = rank_of[y];
        owv[b] = own[y];
      }
#pragma unroll
      for (int b = 0; b < kB; ++b) cov[b] = col[ryv[b]];
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        const int y = y0 + 64 * b, ry = ryv[b];
        if (y < E && ry != rx) {
          const int64_t g = (int64_t)cov[b] - ox + av[b] - owv[b] - 2 * (int64_t)cv[b];
          atomicMax(&key[min(rx, ry) * ks + max(rx, ry)], swap_key(g, x, y, E));
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // col is rewritten for the next x
  }
}

// The pair swaps, at most max_swaps (< 0: 4096) while the best gain is
// positive; returns their number.  C16: the counts are read from the 16-bit rows.
template <bool C16, bool KEY_LDS>
__device__ __forceinline__ int swap_loop(const Dims& d, const int32_t* __restrict__ C, const uint16_t* __restrict__ c16,
                                         int32_t max_swaps, int32_t* aff, int32_t* own, int32_t* rank_of, int32_t* mem,
                                         uint64_t* key, int ks, int32_t* col, uint64_t* red) {
  const int E = d.E, R = d.R, Er = d.Er, Es = c16_stride(E);
  const int tid = threadIdx.x;
  const int cap = max_swaps < 0 ? 4096 : max_swaps;
  // The largest key of iteration i: each wave's maximum into top[i % 2] by an
  // LDS atomic, one barrier, then read by all.  top[(i + 1) % 2] is cleared
  // in iteration i after that barrier: its last reads (iteration i - 1) were
  // before the barriers that ended iteration i - 1.
  uint64_t* top = red + kPlaceWaves + 1;
  if (tid == 0) top[0] = top[1] = 0;
  __syncthreads();
  int swaps = 0;
  for (int it = 0;; ++it) {
    uint64_t best = 0;
    for (int q = tid; q < R * ks; q += kPlaceThreads) {
      const uint64_t v = key_load<KEY_LDS>(&key[q]);
      best = v > best ? v : best;
    }
    best = wave_max(best);
    if ((tid & 63) == 0) atomicMax(&top[it & 1], best);
    __syncthreads();
    best = top[it & 1];
    const int64_t gain = (int64_t)(best >> kPairBits) - (int64_t)kGainBias;
    if (best == 0 || gain <= 0 || swaps >= cap) break;
    const int64_t pair = (int64_t)(kPairMask - (best & kPairMask));
    const int xa = (int)(pair / E), xb = (int)(pair - (int64_t)xa * E);
    const int ra = rank_of[xa], rb = rank_of[xb];
    if (tid == 0) top[(it + 1) & 1] = 0;
    // aff of ranks ra and rb; clear the keys of every rank pair with ra or rb.
    for (int x = tid; x < E; x += kPlaceThreads) {
      const int32_t ca = C16 ? (int32_t)c16[(int64_t)xa * Es + x] : C[(int64_t)xa * E + x];
      const int32_t cb = C16 ? (int32_t)c16[(int64_t)xb * Es + x] : C[(int64_t)xb * E + x];
      aff[(int64_t)ra * E + x] += cb - ca;
      aff[(int64_t)rb * E + x] += ca - cb;
    }
    for (int q = tid; q < 2 * R; q += kPlaceThreads) {
      const int c = q < R ? ra : rb, o = q < R ? q : q - R;
      if (o != c) key[min(c, o) * ks + max(c, o)] = 0;
    }
    __syncthreads();  // every thread has read rank_of[xa], rank_of[xb]
    // The swap: each of the 2*Er slots of ranks ra and rb is rewritten by one
    // thread (xa and xb trade places), with its expert's rank and own.
    for (int q = tid; q < 2 * Er; q += kPlaceThreads) {
      const int r = q < Er ? ra : rb, slot = r * Er + (q < Er ? q : q - Er);
      int e = mem[slot];
      e = e == xa ? xb : e == xb ? xa : e;
      mem[slot] = e;
      rank_of[e] = r;
      own[e] = aff[(int64_t)r * E + e];
    }
    __syncthreads();
    // entries per lane and batch: E / 64, at most eight (no clamped duplicates when E is small)
    if (E <= 128) eval_rows<C16, 2>(d, C, c16, aff, own, rank_of, mem, key, ks, col, ra, rb);
    else if (E <= 256) eval_rows<C16, 4>(d, C, c16, aff, own, rank_of, mem, key, ks, col, ra, rb);
    else eval_rows<C16, 8>(d, C, c16, aff, own, rank_of, mem, key, ks, col, ra, rb);
    __syncthreads();
    ++swaps;
  }

  return swaps;
}

template <bool AFF_LDS, bool KEY_LDS>
__global__ __launch_bounds__(kPlaceThreads) void place_swap_kernel(Dims d, SwapLds ly, const int32_t* __restrict__ C,
                                                                   int32_t max_swaps, PlaceState s, moe_place_out out) {
  extern __shared__ __align__(16) char smem_swap[];
  int32_t* rank_of = reinterpret_cast<int32_t*>(smem_swap + ly.rank_of);
  int32_t* mem = reinterpret_cast<int32_t*>(smem_swap + ly.mem);  // [R][Er] experts of each rank
  int32_t* own = reinterpret_cast<int32_t*>(smem_swap + ly.own);
  int32_t* col = reinterpret_cast<int32_t*>(smem_swap + ly.col) + (threadIdx.x >> 6) * d.R;
  uint64_t* red = reinterpret_cast<uint64_t*>(smem_swap + ly.red);
  int32_t* aff;
  uint64_t* key;
  const int E = d.E, R = d.R, Er = d.Er;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if constexpr (AFF_LDS) {
    aff = reinterpret_cast<int32_t*>(smem_swap + ly.aff);
    for (int64_t q = tid; q < (int64_t)R * E; q += kPlaceThreads) aff[q] = s.aff[q];
  } else {
    aff = s.aff;
  }
  // In LDS the key table's rows are R + 1 words apart: the entries
  // key[r][rx] of one column then fall in different banks (with R words
  // apart every lane's atomic on a rank below rx hit one bank).
  const int ks = KEY_LDS ? R + 1 : R;
  if constexpr (KEY_LDS) {
    key = reinterpret_cast<uint64_t*>(smem_swap + ly.key);
    for (int q = tid; q < R * ks; q += kPlaceThreads) {
      const int r = q / ks, c = q - r * ks;
      key[q] = c < R ? s.key[r * R + c] : 0;
    }
  } else {
    key = s.key;
  }
  for (int e = tid; e < E; e += kPlaceThreads) {
    rank_of[e] = s.rank_of[e];
    mem[e] = s.mem[e];
    own[e] = s.own[e];
  }
  __syncthreads();

  // The counts as 16-bit rows when they fit (half the bytes).
  uint32_t mx = 0;
  for (int e = tid; e < E; e += kPlaceThreads) mx = max(mx, (uint32_t)s.rowmax[e]);
  const bool fit16 = block_max<kPlaceWaves>(mx, red) <= 0xffffu;
  const int swaps = fit16 ? swap_loop<true, KEY_LDS>(d, C, s.c16, max_swaps, aff, own, rank_of, mem, key, ks, col, red)
                          : swap_loop<false, KEY_LDS>(d, C, s.c16, max_swaps, aff, own, rank_of, mem, key, ks, col, red);

  // Outputs: ranks, the experts of each rank in ascending order, the kept weight.
  int64_t w = 0;
  for (int e = tid; e < E; e += kPlaceThreads) {
    const int r = rank_of[e];
    int before = 0;
    for (int i = 0; i < Er; ++i) before += mem[r * Er + i] < e;
    out.expert_rank[e] = r;
    out.rank_experts[r * Er + before] = e;
    w += own[e];
  }
  w = wave_sum(w);
  if (lane == 0) reinterpret_cast<int64_t*>(red)[wave] = w;
  __syncthreads();
  if (tid == 0) {
    int64_t t = 0;
    for (int i = 0; i < kPlaceWaves; ++i) t += reinterpret_cast<int64_t*>(red)[i];
    *out.intra = t / 2;  // each pair counted from both sides
    *out.n_swaps = swaps;
  }
}

// ---------------------------------------------------------------------------
// Launch shapes.

size_t grow_c16_lds_bytes(const Dims& d) { return c16_count(d.E) * sizeof(uint16_t); }
bool grow_c_in_lds(const Dims& d) { return kGrowRedBytes + grow_c16_lds_bytes(d) <= kPlaceLdsBudget; }
size_t grow_lds_bytes(const Dims& d) { return kGrowRedBytes + (grow_c_in_lds(d) ? grow_c16_lds_bytes(d) : 0); }
size_t pass_lds_bytes(const Dims& d) {
  return (sizeof(uint64_t) + sizeof(int32_t)) * kPassWaves * (size_t)d.R + 2 * sizeof(int32_t) * (size_t)d.E;
}

// Dynamic LDS above 64 KiB must be allowed per kernel.
hipError_t allow_lds(const void* kern, size_t lds) {
  if (lds <= 65536) return hipSuccess;
  return hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

template <bool C_LDS, int NPL>
hipError_t launch_grow(const Dims& d, const int32_t* C, const PlaceState& s, hipStream_t st) {
  auto kern = place_grow_kernel<C_LDS, NPL>;
  const size_t lds = grow_lds_bytes(d);
  const hipError_t e = allow_lds(reinterpret_cast<const void*>(kern), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(1), dim3(kGrowThreads), lds, st, d, C, s);
  return hipGetLastError();
}

template <bool AFF_LDS, bool KEY_LDS>
hipError_t launch_swap(const Dims& d, const SwapLds& ly, const int32_t* C, int32_t max_swaps, const PlaceState& s,
                       const moe_place_out& out, hipStream_t st) {
  auto kern = place_swap_kernel<AFF_LDS, KEY_LDS>;
  const hipError_t e = allow_lds(reinterpret_cast<const void*>(kern), ly.total);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(1), dim3(kPlaceThreads), ly.total, st, d, ly, C, max_swaps, s, out);
  return hipGetLastError();
}

}  // namespace

size_t place_c16_elems(const Dims& d) { return c16_count(d.E); }

size_t place_lds_bytes(const Dims& d) {
  return std::max(std::max(grow_lds_bytes(d), pass_lds_bytes(d)), swap_lds(d).total);
}

hipError_t launch_place(const Dims& d, const int32_t* cooc, int32_t max_swaps, const moe_place_out& out,
                        const Workspace& ws, hipStream_t st) {
  const PlaceState s = place_state(d, ws);
  const unsigned pass_grid = (unsigned)((d.E + kPassWaves - 1) / kPassWaves);
  hipLaunchKernelGGL(place_prep_kernel, dim3(pass_grid), dim3(64 * kPassWaves), 0, st, d, cooc, s, ws.status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (grow_c_in_lds(d)) e = launch_grow<true, 2>(d, cooc, s, st);  // E <= 282 here
  else if (d.E <= 2 * kGrowThreads) e = launch_grow<false, 2>(d, cooc, s, st);
  else if (d.E <= 4 * kGrowThreads) e = launch_grow<false, 4>(d, cooc, s, st);
  else e = launch_grow<false, 8>(d, cooc, s, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(place_pass_kernel, dim3(pass_grid), dim3(64 * kPassWaves), pass_lds_bytes(d), st, d, cooc, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const SwapLds ly = swap_lds(d);
  if (ly.aff_in_lds && ly.key_in_lds) return launch_swap<true, true>(d, ly, cooc, max_swaps, s, out, st);
  if (ly.aff_in_lds) return launch_swap<true, false>(d, ly, cooc, max_swaps, s, out, st);
  if (ly.key_in_lds) return launch_swap<false, true>(d, ly, cooc, max_swaps, s, out, st);
  return launch_swap<false, false>(d, ly, cooc, max_swaps, s, out, st);
}

}  // namespace moe
