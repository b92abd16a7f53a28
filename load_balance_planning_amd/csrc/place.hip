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
// One workgroup of 1024 threads; the problem is tiny and sequential.  The
// growth runs in wave 0 alone (E sequential argmax steps, no barriers: each
// lane holds E/64 affinities in registers).  Refinement keeps, for every rank
// pair (r1 < r2), the best swap key of the pairs between them; a swap between
// ra and rb changes only the gains of pairs with an expert on ra or rb, so an
// iteration re-evaluates 2R-3 rank pairs (about 2*E*E/R expert pairs) instead
// of all E*E/2.  aff and the rank-pair keys live in LDS when they fit, else in
// the handle's workspace.
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
  size_t rank_of, mem, pos, deg, red, aff, key, total;
  bool aff_in_lds, key_in_lds;
};

constexpr size_t kPlaceAffLds = 64 * 1024;
constexpr size_t kPlaceKeyLds = 32 * 1024;

PlaceLds place_lds(const Dims& d) {
  PlaceLds l;
  size_t o = 0;
  auto take = [&](size_t b) { const size_t at = o; o += (b + 15) / 16 * 16; return at; };
  l.rank_of = take(sizeof(int32_t) * d.E);
  l.mem = take(sizeof(int32_t) * d.E);
  l.pos = take(sizeof(int32_t) * d.E);
  l.deg = take(sizeof(int32_t) * d.E);
  l.red = take(sizeof(uint64_t) * (kPlaceWaves + 1));
  const size_t aff_b = sizeof(int32_t) * (size_t)d.R * d.E;
  const size_t key_b = sizeof(uint64_t) * (size_t)d.R * d.R;
  l.aff_in_lds = aff_b <= kPlaceAffLds;
  l.key_in_lds = key_b <= kPlaceKeyLds;
  l.aff = l.aff_in_lds ? take(aff_b) : 0;
  l.key = l.key_in_lds ? take(key_b) : 0;
  l.total = o;
  return l;
}

__device__ __forceinline__ uint64_t wave_max(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = __shfl_xor(v, off);
    v = o > v ? o : v;
  }
  return v;
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

// Swap key of experts x (rank r1) and y (rank r2): the gain, then the pair
// (lower id first) preferring lower ids.
__device__ __forceinline__ uint64_t swap_key(const Dims& d, const int32_t* __restrict__ C, const int32_t* aff,
                                             int x, int y, int r1, int r2) {
  const int64_t g = (int64_t)aff[(int64_t)r2 * d.E + x] - aff[(int64_t)r1 * d.E + x] + aff[(int64_t)r1 * d.E + y] -
                    aff[(int64_t)r2 * d.E + y] - 2 * (int64_t)C[(int64_t)x * d.E + y];
  const int a = min(x, y), b = max(x, y);
  const uint64_t pair = (uint64_t)a * d.E + b;
  return ((uint64_t)(g + (int64_t)kGainBias) << kPairBits) | (kPairMask - pair);
}

// Best swap key of every rank pair in a set of nb candidate pairs: pair_of(b)
// returns the ranks (r1 < r2) of candidate b, or r1 < 0 to skip it.  A group
// of tpb lanes (a power of two within one wave) evaluates one rank pair.
template <class PairOf>
__device__ __forceinline__ void eval_blocks(const Dims& d, const int32_t* __restrict__ C, const int32_t* aff,
                                            const int32_t* mem, uint64_t* key, int nb, PairOf pair_of) {
  int tpb = kPlaceThreads / max(nb, 1);
  tpb = tpb >= 64 ? 64 : tpb >= 32 ? 32 : tpb >= 16 ? 16 : tpb >= 8 ? 8 : tpb >= 4 ? 4 : tpb >= 2 ? 2 : 1;
  const int groups = kPlaceThreads / tpb;
  const int sub = threadIdx.x % tpb;
  const int Er = d.Er, items = Er * Er;
  for (int b = threadIdx.x / tpb; b < nb; b += groups) {
    int r1, r2;
    pair_of(b, r1, r2);
    if (r1 < 0) continue;  // uniform within the group
    uint64_t best = 0;
    for (int it = sub; it < items; it += tpb) {
      const int ix = it / Er, iy = it - ix * Er;
      const int x = mem[r1 * Er + ix], y = mem[r2 * Er + iy];
      const uint64_t kk = swap_key(d, C, aff, x, y, r1, r2);
      best = kk > best ? kk : best;
    }
    for (int off = tpb >> 1; off >= 1; off >>= 1) {
      const uint64_t o = __shfl_xor(best, off, tpb);
      best = o > best ? o : best;
    }
    if (sub == 0) key[(int64_t)r1 * d.R + r2] = best;
  }
}

template <int NPL>
__global__ __launch_bounds__(kPlaceThreads) void place_kernel(Dims d, PlaceLds ly, PlaceArgs pa) {
  extern __shared__ __align__(16) char smem_place[];
  int32_t* rank_of = reinterpret_cast<int32_t*>(smem_place + ly.rank_of);
  int32_t* mem = reinterpret_cast<int32_t*>(smem_place + ly.mem);  // [R][Er] experts of each rank
  int32_t* pos = reinterpret_cast<int32_t*>(smem_place + ly.pos);  // slot of each expert in mem
  int32_t* deg = reinterpret_cast<int32_t*>(smem_place + ly.deg);
  uint64_t* red = reinterpret_cast<uint64_t*>(smem_place + ly.red);
  int32_t* aff = ly.aff_in_lds ? reinterpret_cast<int32_t*>(smem_place + ly.aff) : pa.aff_ws;
  uint64_t* key = ly.key_in_lds ? reinterpret_cast<uint64_t*>(smem_place + ly.key) : pa.key_ws;
  const int E = d.E, R = d.R, Er = d.Er;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t* __restrict__ C = pa.C;

  // Degrees and input checks: zero diagonal, no negative count, row sums
  // below 2^31 (symmetry is the caller's contract).
  for (int e = wave; e < E; e += kPlaceWaves) {
    int64_t s = 0;
    bool bad = false;
    for (int x = lane; x < E; x += 64) {
      const int32_t v = C[(int64_t)e * E + x];
      bad |= v < 0 || (x == e && v != 0);
      s += v;
    }
    s = wave_sum(s);
    bad = __any(bad);
    if (lane == 0) {
      if (bad || s > INT32_MAX) atomicOr(pa.status, MOE_STATUS_BAD_PAIRS);
      deg[e] = (int32_t)(s < 0 ? 0 : s > INT32_MAX ? INT32_MAX : s);
    }
  }
  for (int64_t q = tid; q < (int64_t)R * R; q += kPlaceThreads) key[q] = 0;
  __syncthreads();

  // Greedy growth in wave 0: lane l holds experts l, l+64, ...
  if (wave == 0) {
    uint32_t placed = 0;
    int32_t a[NPL];
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int u = 0; u < NPL; ++u) a[u] = 0;
      for (int m = 0; m < Er; ++m) {
        uint64_t best = 0;
#pragma unroll
        for (int u = 0; u < NPL; ++u) {
          const int e = lane + 64 * u;
          if (e < E && !(placed >> u & 1u)) {
            const int32_t sc = m == 0 ? deg[e] : max(a[u], 0);
            const uint64_t kk = ((uint64_t)sc << 12) | (uint64_t)(4095 - e);
            best = kk > best ? kk : best;
          }
        }
        best = wave_max(best);
        const int pick = 4095 - (int)(best & 4095);
        if ((pick & 63) == lane) placed |= 1u << (pick >> 6);
        if (lane == 0) {
          rank_of[pick] = r;
          mem[r * Er + m] = pick;
          pos[pick] = r * Er + m;
        }
        const int32_t* row = C + (int64_t)pick * E;  // C[pick][e] = C[e][pick]
#pragma unroll
        for (int u = 0; u < NPL; ++u) {
          const int e = lane + 64 * u;
          if (e < E) a[u] += row[e];
        }
      }
#pragma unroll
      for (int u = 0; u < NPL; ++u) {
        const int e = lane + 64 * u;
        if (e < E) aff[(int64_t)r * E + e] = a[u];
      }
    }
  }
  __syncthreads();

  // Best swap of every rank pair.
  eval_blocks(d, C, aff, mem, key, R * R, [&](int b, int& r1, int& r2) {
    r1 = b / R;
    r2 = b - r1 * R;
    if (r1 >= r2) r1 = -1;
  });
  __syncthreads();

  const int cap = pa.max_swaps < 0 ? 4096 : pa.max_swaps;
  int swaps = 0;
  for (;;) {
    uint64_t best = 0;
    for (int64_t q = tid; q < (int64_t)R * R; q += kPlaceThreads) best = key[q] > best ? key[q] : best;
    best = block_max(best, red);
    const int64_t gain = (int64_t)(best >> kPairBits) - (int64_t)kGainBias;
    if (best == 0 || gain <= 0 || swaps >= cap) break;
    const int64_t pair = (int64_t)(kPairMask - (best & kPairMask));
    const int xa = (int)(pair / E), xb = (int)(pair - (int64_t)xa * E);
    const int ra = rank_of[xa], rb = rank_of[xb];
    for (int x = tid; x < E; x += kPlaceThreads) {
      const int32_t ca = C[(int64_t)xa * E + x], cb = C[(int64_t)xb * E + x];
      aff[(int64_t)ra * E + x] += cb - ca;
      aff[(int64_t)rb * E + x] += ca - cb;
    }
    __syncthreads();  // every thread has read rank_of[xa], rank_of[xb]
    if (tid == 0) {
      const int pa_ = pos[xa], pb_ = pos[xb];
      rank_of[xa] = rb;
      rank_of[xb] = ra;
      mem[pa_] = xb;
      mem[pb_] = xa;
      pos[xa] = pb_;
      pos[xb] = pa_;
    }
    __syncthreads();
    // The rank pairs with ra or rb on one side; (ra, rb) once.
    eval_blocks(d, C, aff, mem, key, 2 * R, [&](int b, int& r1, int& r2) {
      const int c = b < R ? ra : rb, o = b < R ? b : b - R;
      if (o == c || (b >= R && o == ra)) {
        r1 = -1;
        return;
      }
      r1 = min(c, o);
      r2 = max(c, o);
    });
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
    w += aff[(int64_t)r * E + e];
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

template <int NPL>
hipError_t launch_place_n(const Dims& d, const PlaceLds& ly, const PlaceArgs& pa, hipStream_t st) {
  if (ly.total > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(place_kernel<NPL>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)ly.total);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(place_kernel<NPL>, dim3(1), dim3(kPlaceThreads), ly.total, st, d, ly, pa);
  return hipGetLastError();
}

}  // namespace

size_t place_lds_bytes(const Dims& d) { return place_lds(d).total; }

hipError_t launch_place(const Dims& d, const int32_t* cooc, int32_t max_swaps, const moe_place_out& out,
                        const Workspace& ws, hipStream_t st) {
  const PlaceLds ly = place_lds(d);
  const PlaceArgs pa{cooc, max_swaps, out.expert_rank, out.rank_experts, out.intra, out.n_swaps,
                     ws.place_aff, ws.place_key, ws.status};
  const int npl = (d.E + 63) / 64;
  if (npl <= 1) return launch_place_n<1>(d, ly, pa, st);
  if (npl <= 2) return launch_place_n<2>(d, ly, pa, st);
  if (npl <= 4) return launch_place_n<4>(d, ly, pa, st);
  if (npl <= 8) return launch_place_n<8>(d, ly, pa, st);
  if (npl <= 16) return launch_place_n<16>(d, ly, pa, st);
  return launch_place_n<32>(d, ly, pa, st);
}

}  // namespace moe
