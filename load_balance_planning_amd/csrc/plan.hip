// Replica placement, token re-routing, quotas and per-slot instances on gfx950.
//
// [TopoEP] section 4.3 (two-stage solver, Eqs. 9 and 10) with the quota and
// slot rules documented in moe_plan.h.  Three kernels:
//   plan_kernel    one workgroup of 16 waves holding the solver state in LDS.
//                  The domains are independent in both stages, so wave w plans
//                  domains w, w+16, ...; each refinement iteration is a
//                  wave-wide argmin over packed candidate keys followed by one
//                  update -- the page's one-update-per-iteration rule.
//   quota_kernel   one workgroup per replicated expert computes its three-pass
//                  transport in closed form (interval overlaps of cumulative
//                  demand and capacity); other workgroups copy the routing
//                  matrix into the quota columns of single-instance experts,
//                  and one derives the dispatch offsets from the instance loads.
//   assign_kernel  one thread per slot: stable rank inside its (source,
//                  expert) pair from the tile masks, then instance and position.
// All arithmetic is integer and every selection has a total order, so the plan
// is bitwise reproducible.
#include <algorithm>

#include "internal.h"
#include "pair_count.h"
#include "slot_assign.h"
#include "tile_scan.h"

namespace moe {
namespace {

// Dynamic LDS of the plan kernel; the solver helpers index it by the offsets
// of PlanLayout so that every access compiles to an LDS instruction.
// 16-byte aligned: parts of it are read as 64- and 128-bit words, and the
// dynamic region starts after the static LDS, whatever its size.
extern __shared__ __align__(16) int32_t plan_lds[];

// Solver launch workgroups: 512 threads (one wave per domain of up to eight
// in both stages) when the launch runs alone, 256 -- the row copy's size --
// when it must be placed beside another batch's running copy, which frees
// one 256-thread slot at a time.
constexpr int kPlanThreadsAlone = 512;
constexpr int kPlanThreadsBeside = 256;
constexpr int kPlanMaxWaves = kPlanThreadsAlone / 64;
constexpr int kDemandLdsMax = 16384;  // M*E int32 entries kept in LDS when they fit
constexpr int kQuotaThreads = 256;     // >= kMaxR: one source (and one instance) per thread
constexpr int kFillCells = 1024;       // quota cells per fill workgroup

// Offsets (int32 units) of the plan kernel's LDS arrays.
struct PlanLayout {
  int L, nrep, inst_base, rep_dom, Umain, eoff, rl, misc, hm, rep_e, rep_U, rep_id, wave_tot, D;
  int RW;     // 64-bit words per host mask (ranks / 64, rounded up)
  int NS;     // replica slots per rank held in LDS
  int total;
};

// The layer dimensions and the LDS layout, copied to LDS once per launch: the
// solver helpers are separate functions (one variant per shape, so the
// kernel's registers stay bounded), and reading these from LDS spares each
// call the round trip through the stack that by-value structs would take.
__shared__ Dims plan_dims;
__shared__ PlanLayout plan_ly;

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

// Maximum over the wave, returned in every lane.  Inside each 16-lane row a
// DPP butterfly (quad swaps, half-row and row mirrors); the four row results
// are then read out with readlane.  All 64 lanes must be active.
__device__ __forceinline__ uint64_t wave_allmax_u64(uint64_t v) {
  uint64_t o;
  o = dpp_u64<0xB1>(v); v = o > v ? o : v;
  o = dpp_u64<0x4E>(v); v = o > v ? o : v;
  o = dpp_u64<0x141>(v); v = o > v ? o : v;
  o = dpp_u64<0x140>(v); v = o > v ? o : v;
  uint64_t r = readlane_u64(v, 0);
  o = readlane_u64(v, 16); r = o > r ? o : r;
  o = readlane_u64(v, 32); r = o > r ? o : r;
  o = readlane_u64(v, 48); r = o > r ? o : r;
  return r;
}

// Lexicographic minimum of (hi, lo) over the wave, in every lane (branch-free).
__device__ __forceinline__ void wave_allmin_key(uint64_t& hi, uint32_t& lo) {
#define MOE_MIN_STEP(CTRL)                                              \
  {                                                                     \
    const uint64_t oh = dpp_u64<CTRL>(hi);                              \
    const uint32_t ol = dpp_u32<CTRL>(lo);                              \
    const bool take = (oh < hi) | ((oh == hi) & (ol < lo));             \
    hi = take ? oh : hi;                                                \
    lo = take ? ol : lo;                                                \
  }
  MOE_MIN_STEP(0xB1)
  MOE_MIN_STEP(0x4E)
  MOE_MIN_STEP(0x141)
  MOE_MIN_STEP(0x140)
#undef MOE_MIN_STEP
  uint64_t rh = readlane_u64(hi, 0);
  uint32_t rl = (uint32_t)__builtin_amdgcn_readlane((int)lo, 0);
#pragma unroll
  for (int row = 1; row < 4; ++row) {
    const uint64_t oh = readlane_u64(hi, row * 16);
    const uint32_t ol = (uint32_t)__builtin_amdgcn_readlane((int)lo, row * 16);
    const bool take = (oh < rh) | ((oh == rh) & (ol < rl));
    rh = take ? oh : rh;
    rl = take ? ol : rl;
  }
  hi = rh;
  lo = rl;
}

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  return v;
}

// In-place exclusive scan of a[0..n) in LDS by the whole plan workgroup (NT
// threads); returns the total.
template <int NT>
__device__ int block_excl_scan(int* a, int n, int* wave_tot) {
  constexpr int kWaves = NT / 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  __syncthreads();
  const int per = (n + NT - 1) / NT;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int sum = 0;
  for (int q = lo; q < hi; ++q) sum += a[q];
  const int incl = wave_incl_scan(sum);
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int v = wave_tot[w];
      wave_tot[w] = run;
      run += v;
    }
    wave_tot[kWaves] = run;
  }
  __syncthreads();
  int run = wave_tot[wave] + incl - sum;
  for (int q = lo; q < hi; ++q) {
    const int v = a[q];
    a[q] = run;
    run += v;
  }
  const int total = wave_tot[kWaves];
  __syncthreads();
  return total;
}

__device__ __forceinline__ int overlap(int a0, int a1, int b0, int b1) {
  const int lo = a0 > b0 ? a0 : b0, hi = a1 < b1 ? a1 : b1;
  return hi > lo ? hi - lo : 0;
}

__device__ __forceinline__ int domain_budget(Dims d, int m) {
  return d.B / d.M + (m < d.B % d.M ? 1 : 0);
}


// Stage 1 of one domain with the candidate keys in registers: lane l holds
// the keys of experts l, l+64, ... (at most 64*KMAX experts).
template <int KMAX>
__device__ __noinline__ void stage1_domain(int m, const int32_t* Dglobal) {
  const Dims d = plan_dims;
  const PlanLayout ly = plan_ly;
  int32_t* nrep = plan_lds + ly.nrep;
  int32_t* rep_e = plan_lds + ly.rep_e;
  int32_t* rep_U = plan_lds + ly.rep_U;
  int32_t* rep_dom = plan_lds + ly.rep_dom;
  unsigned long long* hm = reinterpret_cast<unsigned long long*>(plan_lds + ly.hm);
  const int RW = ly.RW, NS = ly.NS;
  const int lane = threadIdx.x & 63;
  const int E = d.E, G = d.G, Er = d.Er;
  const int Bd = domain_budget(d, m);
  uint64_t key[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    const int e = lane + 64 * i;
    key[i] = 0ull;
    if (e < E) {
      const int rm = e / Er;
      const int64_t Dv = ly.D >= 0 ? plan_lds[ly.D + m * E + e] : Dglobal[m * E + e];
      // Remote experts with positive benefit (Eq. 9); S > 0, so larger benefit
      // is larger demand; ties to the lower expert.
      if (rm / G != m && 2 * Dv * d.S - d.W > 0) key[i] = ((uint64_t)Dv << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
    }
  }
  int my_nrep = 0, placed = 0;
  while (placed < Bd) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < KMAX; ++i) best = key[i] > best ? key[i] : best;
    best = wave_allmax_u64(best);
    if (best == 0ull) break;
    const int ebest = (int)(0xffffffffu - (uint32_t)best);
#pragma unroll
    for (int i = 0; i < KMAX; ++i) key[i] = key[i] == best ? 0ull : key[i];
    // Least-occupied rank with a free slot, ties to the lower rank.
    uint64_t rk = (lane < G && my_nrep < d.n_slot) ? ((uint64_t)(uint32_t)my_nrep << 32) | (uint32_t)lane : ~0ull;
    uint32_t unused = 0;
    wave_allmin_key(rk, unused);
    if (rk == ~0ull) break;
    if (lane == (int)(uint32_t)rk) {
      const int r = m * G + lane;
      rep_e[r * NS + my_nrep] = ebest;
      rep_U[r * NS + my_nrep] = 0;
      atomicOr(&hm[ebest * RW + (r >> 6)], 1ull << (r & 63));
      my_nrep += 1;
    }
    placed += 1;
  }
  if (lane < G) nrep[m * G + lane] = my_nrep;
  if (lane == 0) rep_dom[m] = placed;
}

// Max over aligned groups of GS lanes (GS <= 16) with DPP, in every lane.
template <int GS>
__device__ __forceinline__ uint64_t group_allmax_u64(uint64_t v) {
  uint64_t o;
  if (GS >= 2) { o = dpp_u64<0xB1>(v); v = o > v ? o : v; }
  if (GS >= 4) { o = dpp_u64<0x4E>(v); v = o > v ? o : v; }
  if (GS >= 8) { o = dpp_u64<0x141>(v); v = o > v ? o : v; }
  if (GS >= 16) { o = dpp_u64<0x140>(v); v = o > v ? o : v; }
  return v;
}

// Stage 2 of one domain for G <= GS <= 16.  The wave is 64/GS groups of GS
// lanes; lane (g, t) stands for rank r0 + t of the domain and every group
// keeps the same copy of the rank loads, so the busiest rank comes out of a
// DPP max inside the group.  Lane (g, t) then evaluates the moves of hosted
// entries c = g, g + 64/GS, ... of the busiest rank to target t: all
// candidates of an iteration are evaluated at once and one wave-wide argmin
// picks the move.  The winning key also carries the entry index, so the
// update needs no search.
template <int GS>
__device__ __noinline__ void stage2_grouped(int m) {
  const Dims d = plan_dims;
  const PlanLayout ly = plan_ly;
  constexpr int NG = 64 / GS;
  int32_t* L = plan_lds + ly.L;
  int32_t* nrep = plan_lds + ly.nrep;
  int32_t* Umain = plan_lds + ly.Umain;
  int32_t* rep_e = plan_lds + ly.rep_e;
  int32_t* rep_U = plan_lds + ly.rep_U;
  int32_t* rep_dom = plan_lds + ly.rep_dom;
  unsigned long long* hm = reinterpret_cast<unsigned long long*>(plan_lds + ly.hm);
  const int RW = ly.RW, NS = ly.NS;
  const int lane = threadIdx.x & 63;
  const int t = lane % GS, g = lane / GS;
  const int G = d.G, Er = d.Er, E = d.E;
  const int Bd = domain_budget(d, m);
  const int r0 = m * G;
  const bool in_dom = t < G;
  const int r = r0 + (in_dom ? t : 0);
  int Lr = in_dom ? L[r] : 0;
  int nr = in_dom ? nrep[r] : 0;
  int repdom = rep_dom[m];
  const int hw = r >> 6;
  const uint64_t hbit = 1ull << (r & 63);
  for (int it = 0; it < d.max_iters; ++it) {
    const uint64_t kb = group_allmax_u64<GS>(in_dom ? ((uint64_t)(uint32_t)Lr << 32) |
                                                        (uint64_t)(0xffffffffu - (uint32_t)t) : 0ull);
    const int lb = __builtin_amdgcn_readfirstlane((int)(0xffffffffu - (uint32_t)kb));
    const int rb = r0 + lb;
    const int Lb = __builtin_amdgcn_readfirstlane((int)(kb >> 32));
    const int nh = Er + __builtin_amdgcn_readlane(nr, lb);
    const int half = (Lb - Lr) >> 1;
    const bool cand = in_dom && t != lb;
    const bool can_add = nr < d.n_slot && repdom < Bd;
    uint64_t best_hi = ~0ull;
    uint32_t best_lo = ~0u;
    for (int c = g; c < nh; c += NG) {
      const bool is_main = c < Er;
      const int jr = rb * NS + (is_main ? 0 : c - Er);
      const int em = rb * Er + (is_main ? c : 0);
      const int er = rep_e[jr];
      const int Ur = rep_U[jr];
      const int Um = Umain[em];
      const int e = is_main ? em : er;
      const int Ub = is_main ? Um : Ur;
      const bool hosted = (hm[(e < E ? e : 0) * RW + hw] & hbit) != 0ull;
      const int delta = Ub < half ? Ub : half;
      const bool ok = cand & (Ub > 0) & (hosted | can_add) & (delta >= 1);
      // Key: largest delta, lowest target load, existing instance first, lower e, lower r_t.
      const uint64_t hi = ok ? ((uint64_t)(uint32_t)(0x7fffffff - delta) << 32) | (uint64_t)(uint32_t)Lr : ~0ull;
      const uint32_t lo = ((uint32_t)(hosted ? 0 : 1) << 31) | ((uint32_t)e << 20) | ((uint32_t)r << 12) | (uint32_t)c;
      const bool take = (hi < best_hi) | ((hi == best_hi) & (lo < best_lo));
      best_hi = take ? hi : best_hi;
      best_lo = take ? lo : best_lo;
    }
    wave_allmin_key(best_hi, best_lo);
    if (best_hi == ~0ull) break;
    const int delta = 0x7fffffff - (int)(uint32_t)(best_hi >> 32);
    const bool is_new = (best_lo >> 31) != 0u;
    const int e = (int)((best_lo >> 20) & 0x7ffu);
    const int rt = (int)((best_lo >> 12) & 0xffu);
    const int cb = (int)(best_lo & 0xfffu);
    const int lt = rt - r0;
    const int nrt = __builtin_amdgcn_readlane(nr, lt);
    const bool main_t = e >= rt * Er && e < rt * Er + Er;
    if (lane == 0) {
      if (cb < Er) Umain[e] -= delta;
      else rep_U[rb * NS + (cb - Er)] -= delta;
      if (is_new) {
        rep_e[rt * NS + nrt] = e;
        rep_U[rt * NS + nrt] = delta;
        nrep[rt] = nrt + 1;
        atomicOr(&hm[e * RW + (rt >> 6)], 1ull << (rt & 63));
      } else if (main_t) {
        Umain[e] += delta;
      }
    }
    if (!is_new && !main_t && lane < nrt && rep_e[rt * NS + lane] == e) rep_U[rt * NS + lane] += delta;
    Lr += (in_dom && t == lt) ? delta : 0;
    Lr -= (in_dom && t == lb) ? delta : 0;
    nr += (in_dom && t == lt && is_new) ? 1 : 0;
    repdom += is_new ? 1 : 0;
    wave_sync();
  }
  if (g == 0 && in_dom) { L[r] = Lr; nrep[r] = nr; }
  if (lane == 0) rep_dom[m] = repdom;
}

// Max over aligned groups of GS lanes (GS <= 16) of 32-bit keys, in every lane.
template <int GS>
__device__ __forceinline__ uint32_t group_allmax_u32(uint32_t v) {
  if (GS >= 2) v = max(v, dpp_u32<0xB1>(v));
  if (GS >= 4) v = max(v, dpp_u32<0x4E>(v));
  if (GS >= 8) v = max(v, dpp_u32<0x141>(v));
  if (GS >= 16) v = max(v, dpp_u32<0x140>(v));
  return v;
}

// Minimum of a 64-bit key over the wave, in every lane (branch-free).
__device__ __forceinline__ uint64_t wave_allmin_u64(uint64_t v) {
  uint64_t o;
  o = dpp_u64<0xB1>(v); v = o < v ? o : v;
  o = dpp_u64<0x4E>(v); v = o < v ? o : v;
  o = dpp_u64<0x141>(v); v = o < v ? o : v;
  o = dpp_u64<0x140>(v); v = o < v ? o : v;
  uint64_t r = readlane_u64(v, 0);
  o = readlane_u64(v, 16); r = o < r ? o : r;
  o = readlane_u64(v, 32); r = o < r ? o : r;
  o = readlane_u64(v, 48); r = o < r ? o : r;
  return r;
}

// Stage 2 of one domain with every hosted entry in registers (G <= GS <= 16,
// at most J*64/GS entries -- mains plus replica slots -- per rank, every rank
// load below 2^24).  Lane (g, t) stands for rank r0 + t and holds entries
// c = g + (64/GS) j of that rank: eR[j] its expert (-1 for an empty slot) and
// UR[j] its load U[e][r].  An iteration takes the busiest rank from a DPP max
// of (L << 4 | 15 - t) inside the group, reads the busiest rank's entries
// from the lanes of the group that hold them (one cross-lane read per
// register), evaluates moving each of them to target t, and picks the move
// with one wave-wide minimum of a 64-bit key
//   (2^24 - 1 - delta) << 40 | L_t << 16 | new << 15 | e << 4 | t,
// the same order as the LDS solver: largest delta, lowest target load,
// existing instance first, lower expert, lower target rank.  The two lanes
// involved update their registers; only the host bitmask lives in LDS.  The
// state is written back at the end.
template <int GS, int J>
__device__ __noinline__ void stage2_regs(int m) {
  const Dims d = plan_dims;
  const PlanLayout ly = plan_ly;
  constexpr int NG = 64 / GS;
  int32_t* L = plan_lds + ly.L;
  int32_t* nrep = plan_lds + ly.nrep;
  int32_t* Umain = plan_lds + ly.Umain;
  int32_t* rep_e = plan_lds + ly.rep_e;
  int32_t* rep_U = plan_lds + ly.rep_U;
  int32_t* rep_dom = plan_lds + ly.rep_dom;
  unsigned long long* hm = reinterpret_cast<unsigned long long*>(plan_lds + ly.hm);
  const int RW = ly.RW, NS = ly.NS;
  const int lane = threadIdx.x & 63;
  const int t = lane % GS, g = lane / GS;
  const int G = d.G, Er = d.Er;
  const int Bd = domain_budget(d, m);
  const int r0 = m * G;
  const bool in_dom = t < G;
  const int r = r0 + (in_dom ? t : 0);
  int Lr = in_dom ? L[r] : 0;
  int nr = in_dom ? nrep[r] : 0;
  int repdom = rep_dom[m];
  const int hw = r >> 6;
  const uint64_t hbit = 1ull << (r & 63);
  int eR[J], UR[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = g + NG * j;
    eR[j] = -1;
    UR[j] = 0;
    if (in_dom && c < Er) {
      eR[j] = r * Er + c;
      UR[j] = Umain[r * Er + c];
    } else if (in_dom && c - Er < nr) {
      eR[j] = rep_e[r * NS + (c - Er)];
      UR[j] = rep_U[r * NS + (c - Er)];
    }
  }
  for (int it = 0; it < d.max_iters; ++it) {
    const uint32_t kb = group_allmax_u32<GS>(in_dom ? ((uint32_t)Lr << 4) | (uint32_t)(15 - t) : 0u);
    const int lb = 15 - (int)(__builtin_amdgcn_readfirstlane(kb) & 15u);
    const int Lb = (int)(__builtin_amdgcn_readfirstlane(kb) >> 4);
    const int nh = Er + __builtin_amdgcn_readlane(nr, lb);
    const int half = (Lb - Lr) >> 1;
    const bool cand = in_dom && t != lb;
    const bool can_add = nr < d.n_slot && repdom < Bd;
    const int src = g * GS + lb;  // the lane of this group holding the busiest rank's entries
    uint64_t best = ~0ull;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = g + NG * j;
      const int eb = __shfl(eR[j], src);
      const int Ub = __shfl(UR[j], src);
      const bool exists = c < nh && eb >= 0;
      const int es = exists ? eb : 0;
      const bool hosted = (hm[es * RW + hw] & hbit) != 0ull;
      const int delta = Ub < half ? Ub : half;
      const bool ok = exists & cand & (Ub > 0) & (hosted | can_add) & (delta >= 1);
      const uint64_t key = ((uint64_t)(0xffffffu - (uint32_t)delta) << 40) | ((uint64_t)(uint32_t)Lr << 16) |
                           ((uint64_t)(hosted ? 0u : 1u) << 15) | ((uint64_t)(uint32_t)es << 4) | (uint64_t)t;
      best = ok && key < best ? key : best;
    }
    best = wave_allmin_u64(best);
    if (best == ~0ull) break;
    const int delta = (int)(0xffffffu - (uint32_t)(best >> 40));
    const bool is_new = ((best >> 15) & 1ull) != 0ull;
    const int e = (int)((best >> 4) & 0x7ffull);
    const int lt = (int)(best & 15ull);
    const int rt = r0 + lt;
    const int nrt = __builtin_amdgcn_readlane(nr, lt);
    const int cn = Er + nrt;  // slot of a new replica on the target
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = g + NG * j;
      const bool from = in_dom && t == lb && eR[j] == e;
      const bool to_new = is_new && in_dom && t == lt && c == cn;
      const bool to_old = !is_new && in_dom && t == lt && eR[j] == e;
      UR[j] += ((to_new | to_old) ? delta : 0) - (from ? delta : 0);
      UR[j] = to_new ? delta : UR[j];
      eR[j] = to_new ? e : eR[j];
    }
    if (is_new && lane == 0) atomicOr(&hm[e * RW + (rt >> 6)], 1ull << (rt & 63));
    Lr += (in_dom && t == lt) ? delta : 0;
    Lr -= (in_dom && t == lb) ? delta : 0;
    nr += (in_dom && t == lt && is_new) ? 1 : 0;
    repdom += is_new ? 1 : 0;
    wave_sync();
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = g + NG * j;
    if (in_dom && c < Er) {
      Umain[r * Er + c] = UR[j];
    } else if (in_dom && c - Er < nr) {
      rep_e[r * NS + (c - Er)] = eR[j];
      rep_U[r * NS + (c - Er)] = UR[j];
    }
  }
  if (g == 0 && in_dom) { L[r] = Lr; nrep[r] = nr; }
  if (lane == 0) rep_dom[m] = repdom;
}

// Register-resident stage 2 when a rank's entries fit in 4 registers per lane
// and the loads in the narrow key (the largest load of a domain never grows
// during refinement), else the LDS version.
template <int GS>
__device__ void stage2_domain(const Dims& d, const PlanLayout& ly, int m) {
  constexpr int NG = 64 / GS;
  const int ent = d.Er + ly.NS;
  const int lane = threadIdx.x & 63;
  const int32_t* L = plan_lds + ly.L;
  int lmax = lane < d.G ? L[m * d.G + lane] : 0;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lmax = max(lmax, __shfl_xor(lmax, off));
  const bool narrow = lmax < (1 << 24);
  if (narrow && ent <= NG) stage2_regs<GS, 1>(m);
  else if (narrow && ent <= 2 * NG) stage2_regs<GS, 2>(m);
  else if (narrow && ent <= 4 * NG) stage2_regs<GS, 4>(m);
  else stage2_grouped<GS>(m);
}

// Solver state in LDS:
//   hm[e][w]        64-bit words of the set of ranks hosting an instance of e
//   rep_e/rep_U[r][j] expert and load of replica slot j < nrep[r] of rank r
//   Umain[e]        load of e's main instance;  L[r] rank loads
// Workgroup 0 is the solver; it reads the routing matrix from omega.
// Workgroups 1.. (when scan.mask is given) run on the CUs the solver leaves
// idle: for kScanEB experts each, the scan job of tile_scan.h (the tile
// prefix of the presence masks; the routing matrix and expert counts, or a
// comparison of the routing matrix with the solver's input).
template <int NT>
__global__ __launch_bounds__(NT) void plan_kernel(Dims d, PlanLayout ly, const int32_t* __restrict__ omega,
                                                            ScanJob scan, moe_plan_out out, Workspace ws, PairArgs pa,
                                                            int n_scan) {
  if (blockIdx.x > 0) {
    const int blk = blockIdx.x - 1;
    if (blk < n_scan) {
      tile_scan_block<NT>(d, scan.mask, scan.base, scan.omega, scan.count, scan.check, ws.status, blk,
                                    plan_lds);
      return;
    }
    // pair-count partials (pair_count.h), summed by the quota launch
    const int q = blk - n_scan, nb = pair_blocks(d);
    pair_partial_block<NT>(d, pa, (q / nb) / pa.splits + pa.zbase, q % nb, (q / nb) % pa.splits, plan_lds);
    return;
  }
  int32_t* lds = plan_lds;
  int32_t* L = lds + ly.L;
  int32_t* nrep = lds + ly.nrep;
  int32_t* inst_base = lds + ly.inst_base;
  int32_t* rep_dom = lds + ly.rep_dom;
  int32_t* Umain = lds + ly.Umain;
  int32_t* eoff = lds + ly.eoff;
  int32_t* rl = lds + ly.rl;
  int32_t* misc = lds + ly.misc;  // [1] experts replicated in stage 1, [2] replicated at the end
  unsigned long long* hm = reinterpret_cast<unsigned long long*>(lds + ly.hm);
  int32_t* rep_e = lds + ly.rep_e;
  int32_t* rep_U = lds + ly.rep_U;
  int32_t* rep_id = lds + ly.rep_id;
  int32_t* wave_tot = lds + ly.wave_tot;
  int32_t* D = ly.D >= 0 ? lds + ly.D : ws.demand;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (tid == 0) {  // read by the solver helpers after the first barrier
    plan_dims = d;
    plan_ly = ly;
  }
  const int E = d.E, R = d.R, G = d.G, M = d.M, Er = d.Er, RW = ly.RW, NS = ly.NS;
  auto host_bit = [&](int e, int r) -> bool { return (hm[e * RW + (r >> 6)] >> (r & 63)) & 1ull; };
  // Slot of expert e among the replicas of rank r (-1 if none).
  auto rep_slot = [&](int r, int e) -> int {
    for (int j = 0; j < nrep[r]; ++j)
      if (rep_e[r * NS + j] == e) return j;
    return -1;
  };

  // ---- domain demand D[m][e] (Eq. 4), expert loads, main placement (C5) ----
  // Four entries per thread at a time, so that their G loads each are in
  // flight together (the routing matrix comes from L2 or HBM: one entry at a
  // time left the Kimi-K2-shaped solver ~10 us in this loop).
  for (int i0 = tid; i0 < M * E; i0 += 4 * NT) {
    const int32_t* o[4];
    int sum[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = min(i0 + u * NT, M * E - 1);
      const int m = idx / E, e = idx - m * E;
      o[u] = omega + (int64_t)m * G * E + e;
      sum[u] = 0;
    }
#pragma unroll 8
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int u = 0; u < 4; ++u) sum[u] += o[u][(int64_t)g * E];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i0 + u * NT < M * E) D[i0 + u * NT] = sum[u];
  }
  for (int q = tid; q < E * RW; q += NT) {
    const int e = q / RW, w = q - e * RW;
    const int rm = e / Er;
    hm[q] = (rm >> 6) == w ? (1ull << (rm & 63)) : 0ull;
  }
  for (int r = tid; r < R; r += NT) nrep[r] = 0;
  if (tid == 0) { misc[0] = 0; misc[1] = 0; misc[2] = 0; misc[3] = 0; }
  __syncthreads();
  for (int e = tid; e < E; e += NT) {
    int cnt = 0;
    for (int m = 0; m < M; ++m) cnt += D[m * E + e];
    Umain[e] = cnt;  // every assignment on the main instance until replicas exist
  }

  // ---- stage 1: inter-node placement (Eq. 9), one wave per domain ----------
  for (int m = wave; m < M; m += (NT / 64)) {
    if (E <= 64 * 2) stage1_domain<2>(m, ws.demand);
    else if (E <= 64 * 4) stage1_domain<4>(m, ws.demand);
    else if (E <= 64 * 16) stage1_domain<16>(m, ws.demand);
    else stage1_domain<32>(m, ws.demand);
  }
  __syncthreads();

  // ---- stage-1 routing --------------------------------------------------------
  // Experts without replicas keep every assignment on the main instance.
  // Replicated experts are routed per source: to the instance in the source's
  // domain if there is one (at most one after stage 1), else split evenly over
  // all instances in rank order.
  for (int e = tid; e < E; e += NT) {
    int n = 0;
    for (int w = 0; w < RW; ++w) n += __popcll(hm[e * RW + w]);
    if (n > 1) {
      rl[atomicAdd(&misc[1], 1)] = e;
      Umain[e] = 0;
    }
  }
  __syncthreads();
  const int nr1 = misc[1];
  for (int idx = tid; idx < nr1 * R; idx += NT) {
    const int q = idx / R, s = idx - q * R;
    const int e = rl[q];
    const int w = omega[(int64_t)s * E + e];
    if (w == 0) continue;
    const int ms = s / G, rm = e / Er;
    int local = -1;
    for (int r = ms * G; r < (ms + 1) * G; ++r)
      if (host_bit(e, r)) { local = r; break; }
    if (local >= 0) {
      if (local == rm) {
        atomicAdd(&Umain[e], w);
      } else {
        const int j = rep_slot(local, e);
        if (j >= 0) atomicAdd(&rep_U[local * NS + j], w);
      }
      continue;
    }
    int n = 0;
    for (int ww = 0; ww < RW; ++ww) n += __popcll(hm[e * RW + ww]);
    int pos = 0;
    for (int ww = 0; ww < RW; ++ww) {
      unsigned long long bits = hm[e * RW + ww];
      while (bits) {
        const int r = ww * 64 + __ffsll((long long)bits) - 1;
        bits &= bits - 1;
        const int share = w / n + (pos < w % n ? 1 : 0);
        ++pos;
        if (share == 0) continue;
        if (r == rm) {
          atomicAdd(&Umain[e], share);
        } else {
          const int j = rep_slot(r, e);
          if (j >= 0) atomicAdd(&rep_U[r * NS + j], share);
        }
      }
    }
  }
  __syncthreads();
  for (int r = tid; r < R; r += NT) {
    int sum = 0;
    for (int h = 0; h < Er; ++h) sum += Umain[r * Er + h];
    for (int j = 0; j < nrep[r]; ++j) sum += rep_U[r * NS + j];
    L[r] = sum;
  }
  __syncthreads();

  // ---- stage 2: intra-node refinement (Eq. 10), one wave per domain --------
  // Lane l < G is rank r = m*G + l: it holds L_r and its replica count in
  // registers, evaluates itself as the target of every expert hosted on the
  // busiest rank, and applies its own side of the chosen move.
  const bool grouped = G <= 16;
  if (grouped) {
    for (int m = wave; m < M; m += (NT / 64)) {
      if (G <= 2) stage2_domain<2>(d, ly, m);
      else if (G <= 4) stage2_domain<4>(d, ly, m);
      else if (G <= 8) stage2_domain<8>(d, ly, m);
      else stage2_domain<16>(d, ly, m);
    }
  } else
  for (int m = wave; m < M; m += (NT / 64)) {
    const int Bd = domain_budget(d, m);
    const int r0 = m * G;
    const bool in_dom = lane < G;
    const int r = r0 + (in_dom ? lane : 0);
    int Lr = in_dom ? L[r] : 0;
    int nr = in_dom ? nrep[r] : 0;
    int repdom = rep_dom[m];
    for (int it = 0; it < d.max_iters; ++it) {
      const uint64_t kb = wave_allmax_u64(in_dom ? ((uint64_t)(uint32_t)Lr << 32) |
                                                     (uint64_t)(0xffffffffu - (uint32_t)lane) : 0ull);
      const int lb = (int)(0xffffffffu - (uint32_t)kb);
      const int rb = r0 + lb;
      const int Lb = (int)(kb >> 32);
      const int nh = Er + __builtin_amdgcn_readlane(nr, lb);
      uint64_t best_hi = ~0ull;
      uint32_t best_lo = ~0u;
      if (in_dom && lane != lb) {
        const int half = (Lb - Lr) >> 1;
        const bool can_add = nr < d.n_slot && repdom < Bd;
        for (int h = 0; h < nh; ++h) {
          int e, Ub;
          if (h < Er) {
            e = rb * Er + h;
            Ub = Umain[e];
          } else {
            e = rep_e[rb * NS + (h - Er)];
            Ub = rep_U[rb * NS + (h - Er)];
          }
          if (Ub <= 0) continue;
          const bool hosted = host_bit(e, r);
          if (!hosted && !can_add) continue;
          const int delta = Ub < half ? Ub : half;
          if (delta < 1) continue;
          // Key: largest delta, lowest target load, existing instance first, lower e, lower r_t.
          const uint64_t hi = ((uint64_t)(uint32_t)(0x7fffffff - delta) << 32) | (uint64_t)(uint32_t)Lr;
          const uint32_t lo = ((uint32_t)(hosted ? 0 : 1) << 31) | ((uint32_t)e << 16) | (uint32_t)r;
          if (hi < best_hi || (hi == best_hi && lo < best_lo)) {
            best_hi = hi;
            best_lo = lo;
          }
        }
      }
      wave_allmin_key(best_hi, best_lo);
      if (best_hi == ~0ull) break;
      const int delta = 0x7fffffff - (int)(uint32_t)(best_hi >> 32);
      const bool is_new = (best_lo >> 31) != 0u;
      const int e = (int)((best_lo >> 16) & 0x7fffu);
      const int rt = (int)(best_lo & 0xffffu);
      if (in_dom && lane == lb) {
        Lr -= delta;
        if (e / Er == rb) {
          Umain[e] -= delta;
        } else {
          const int j = rep_slot(rb, e);
          if (j >= 0) rep_U[rb * NS + j] -= delta;
        }
      }
      if (in_dom && r == rt) {
        Lr += delta;
        if (is_new) {
          rep_e[rt * NS + nr] = e;
          rep_U[rt * NS + nr] = delta;
          nr += 1;
          nrep[rt] = nr;
          atomicOr(&hm[e * RW + (rt >> 6)], 1ull << (rt & 63));
        } else if (e / Er == rt) {
          Umain[e] += delta;
        } else {
          const int j = rep_slot(rt, e);
          if (j >= 0) rep_U[rt * NS + j] += delta;
        }
      }
      if (is_new) repdom += 1;
      wave_sync();
    }
    if (in_dom) { L[r] = Lr; nrep[r] = nr; }
    if (lane == 0) rep_dom[m] = repdom;
  }
  __syncthreads();

  // ---- instance table -------------------------------------------------------
  for (int q = tid; q < R; q += NT) inst_base[q] = Er + nrep[q];
  const int n_inst = block_excl_scan<NT>(inst_base, R, wave_tot);
  if (tid == 0) inst_base[R] = n_inst;
  // Replicas of rank q: ids after its mains, ordered by expert.
  for (int q = tid; q < R; q += NT) {
    const int n = nrep[q];
    for (int j = 0; j < n; ++j) {
      const int e = rep_e[q * NS + j];
      int pos = 0;
      for (int j2 = 0; j2 < n; ++j2) pos += rep_e[q * NS + j2] < e ? 1 : 0;
      const int id = inst_base[q] + Er + pos;
      rep_id[q * NS + j] = id;
      out.inst_expert[id] = e; out.inst_rank[id] = q; out.inst_load[id] = rep_U[q * NS + j];
    }
  }
  for (int e = tid; e < E; e += NT) {
    const int q = e / Er;
    const int id = inst_base[q] + (e - q * Er);
    out.inst_expert[id] = e; out.inst_rank[id] = q; out.inst_load[id] = Umain[e];
    int n = 0;
    for (int w = 0; w < RW; ++w) n += __popcll(hm[e * RW + w]);
    eoff[e] = n;
  }
  for (int i = n_inst + tid; i < d.cap; i += NT) {
    out.inst_expert[i] = -1; out.inst_rank[i] = -1; out.inst_load[i] = -1;
  }
  for (int q = tid; q < R; q += NT) out.rank_load[q] = L[q];
  if (tid == 0) out.n_inst[0] = n_inst;
  const int total_inst = block_excl_scan<NT>(eoff, E, wave_tot);
  if (tid == 0) eoff[E] = total_inst;
  __syncthreads();
  for (int e = tid; e <= E; e += NT) ws.einst_off[e] = eoff[e];
  // Per-expert instance lists in rank order (the set bits of the host mask),
  // and the experts with more than one instance.
  for (int e = tid; e < E; e += NT) {
    const int rm = e / Er;
    int pos = eoff[e];
    if (eoff[e + 1] - pos > 1) ws.rlist[atomicAdd(&misc[2], 1)] = e;
    for (int w = 0; w < RW; ++w) {
      unsigned long long bits = hm[e * RW + w];
      while (bits) {
        const int q = w * 64 + __ffsll((long long)bits) - 1;
        bits &= bits - 1;
        const int j = q == rm ? 0 : rep_slot(q, e);
        ws.einst_list[pos++] = q == rm ? inst_base[q] + (e - q * Er) : (j >= 0 ? rep_id[q * NS + j] : 0);
      }
    }
  }
  __syncthreads();
  if (tid == 0) ws.rlist[E] = misc[2];
}

// Exclusive scan over the quota workgroup (kQuotaThreads threads, one value each).
__device__ int quota_block_excl_scan(int v, int* wtot) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int incl = wave_incl_scan(v);
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wtot[w];
  __syncthreads();
  return base + incl - v;
}

// Dispatch offsets: exclusive prefix of the instance loads (the receive
// counts of every instance) and, since instances are rank-major, each rank's
// first row.  One workgroup; thread j sums a contiguous run of instances.  A
// rank with no instance (impossible in a plan of this library: every rank
// keeps its main experts) gets the offset of the next rank that has one.
__device__ void offsets_block(const Dims& d, const moe_plan_out& plan, int32_t* inst_offset, int32_t* rank_offset,
                              int32_t* status) {
  __shared__ int wtot_o[kQuotaThreads / 64];
  const int tid = threadIdx.x;
  int n = plan.n_inst[0];
  if (n < 0 || n > d.cap) {
    if (tid == 0) atomicOr(status, MOE_STATUS_PLAN_CHECK);
    n = 0;
  }
  for (int r = tid; r < d.R; r += kQuotaThreads) rank_offset[r] = -1;
  const int per = (n + kQuotaThreads - 1) / kQuotaThreads;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int sum = 0;
  for (int q = lo; q < hi; ++q) sum += plan.inst_load[q];
  const int before = quota_block_excl_scan(sum, wtot_o);
  int total = 0;
  for (int w = 0; w < kQuotaThreads / 64; ++w) total += wtot_o[w];
  int run = before;
  for (int q = lo; q < hi; ++q) {
    inst_offset[q] = run;
    const int r = plan.inst_rank[q];
    if ((unsigned)r < (unsigned)d.R && (q == 0 || plan.inst_rank[q - 1] != r)) rank_offset[r] = run;
    run += plan.inst_load[q];
  }
  for (int i = n + tid; i <= d.cap; i += kQuotaThreads) inst_offset[i] = i == n ? total : -1;
  __syncthreads();
  if (tid == 0) {
    int next = total;
    for (int r = d.R - 1; r >= 0; --r) {
      if (rank_offset[r] < 0) rank_offset[r] = next;
      next = rank_offset[r];
    }
    rank_offset[d.R] = total;
  }
}

// Quotas.  Workgroups [0, n_transport): replicated expert rlist[b]; then
// n_fill workgroups fill the columns of single-instance experts (all demand
// on the one instance) and zero the unused columns; then, with inst_offset
// given, one workgroup computes the dispatch offsets; then the pair-count
// sums.
__global__ __launch_bounds__(kQuotaThreads) void quota_kernel(Dims d, const int32_t* __restrict__ omega,
                                                              moe_plan_out out, int32_t* inst_offset,
                                                              int32_t* rank_offset, Workspace ws, int n_transport,
                                                              int n_fill, PairArgs pa) {
  const int E = d.E, R = d.R, G = d.G, cap = d.cap;
  const int tid = threadIdx.x;
  const int n_off = inst_offset ? 1 : 0;
  if ((int)blockIdx.x >= n_transport + n_fill + n_off) {  // the pair counts: sums of the solver launch's partials
    constexpr int kChunks = kPairBlock / kQuotaThreads;
    const int r = (int)blockIdx.x - (n_transport + n_fill + n_off), nb = pair_blocks(d);
    const int rest = r / nb;
    pair_reduce_one(d, pa, rest / kChunks + pa.zbase, r % nb, (rest % kChunks) * kQuotaThreads + tid);
    return;
  }
  if ((int)blockIdx.x == n_transport + n_fill) {
    offsets_block(d, out, inst_offset, rank_offset, ws.status);
    return;
  }
  if ((int)blockIdx.x >= n_transport) {
    const int n = out.n_inst[0];
    const int64_t c0 = (int64_t)(blockIdx.x - n_transport) * kFillCells;
    for (int64_t c = c0 + tid; c < c0 + kFillCells && c < (int64_t)R * cap; c += kQuotaThreads) {
      const int s = (int)(c / cap), i = (int)(c - (int64_t)s * cap);
      if (i >= n) {
        out.quota[c] = 0;
      } else {
        const int e = out.inst_expert[i];
        if ((unsigned)e < (unsigned)E && ws.einst_off[e + 1] - ws.einst_off[e] == 1)
          out.quota[c] = omega[(int64_t)s * E + e];
      }
    }
    return;
  }
  const int q = blockIdx.x;
  if (q >= ws.rlist[E]) return;
  const int e = ws.rlist[q];
  if ((unsigned)e >= (unsigned)E) return;
  const int off = ws.einst_off[e], ne = ws.einst_off[e + 1] - off;
  if (ne < 2 || ne > R || off < 0 || off + ne > cap) {
    if (tid == 0) atomicOr(ws.status, MOE_STATUS_PLAN_CHECK);
    return;
  }
  // Sources: one per thread.  Instances (rank order): one per thread.
  __shared__ int dem0[kMaxR], fA[kMaxR], demA[kMaxR], pfxB[kMaxR], demB[kMaxR], pfxC[kMaxR], onr[kMaxR];
  __shared__ int iid[kMaxR], irank[kMaxR], cap0[kMaxR], capA[kMaxR], cpfxB[kMaxR], capB[kMaxR], cpfxC[kMaxR];
  __shared__ int wtot[kQuotaThreads / 64];
  if (tid < R) { dem0[tid] = omega[(int64_t)tid * E + e]; onr[tid] = -1; }
  if (tid < ne) {
    int i = ws.einst_list[off + tid];
    if ((unsigned)i >= (unsigned)cap) i = 0;  // cannot happen for a plan written by plan_kernel
    int r = out.inst_rank[i];
    if ((unsigned)r >= (unsigned)R) r = 0;
    iid[tid] = i; irank[tid] = r; cap0[tid] = out.inst_load[i];
  }
  __syncthreads();
  if (tid < ne) onr[irank[tid]] = tid;
  __syncthreads();
  // Pass A: the instance on the source's own rank.
  if (tid < R) {
    const int a = onr[tid];
    const int f = a >= 0 ? min(dem0[tid], cap0[a]) : 0;
    fA[tid] = f;
    demA[tid] = dem0[tid] - f;
  }
  __syncthreads();
  if (tid < ne) capA[tid] = cap0[tid] - fA[irank[tid]];
  __syncthreads();
  // Pass B: within each domain, sources ascending against instances in rank
  // order: the greedy fill equals the overlap of the cumulative intervals.
  if (tid < R) {
    const int m = tid / G;
    int run = 0;
    for (int s2 = m * G; s2 < tid; ++s2) run += demA[s2];
    pfxB[tid] = run;
    int capd = 0;
    for (int a = 0; a < ne; ++a) capd += (irank[a] / G == m) ? capA[a] : 0;
    demB[tid] = demA[tid] - min(demA[tid], max(0, capd - run));
  }
  if (tid < ne) {
    const int m = irank[tid] / G;
    int run = 0;
    for (int a2 = tid - 1; a2 >= 0 && irank[a2] / G == m; --a2) run += capA[a2];
    cpfxB[tid] = run;
    int demd = 0;
    for (int s2 = m * G; s2 < (m + 1) * G; ++s2) demd += demA[s2];
    capB[tid] = capA[tid] - overlap(run, run + capA[tid], 0, demd);
  }
  __syncthreads();
  // Pass C: all sources against all instances.
  const int pC = quota_block_excl_scan(tid < R ? demB[tid] : 0, wtot);
  const int cC = quota_block_excl_scan(tid < ne ? capB[tid] : 0, wtot);
  if (tid < R) pfxC[tid] = pC;
  if (tid < ne) cpfxC[tid] = cC;
  __syncthreads();
  if (tid == 0) {
    // Every remaining assignment must find a remaining slot.
    const int dt = pfxC[R - 1] + demB[R - 1], ct = cpfxC[ne - 1] + capB[ne - 1];
    if (dt != ct) atomicOr(ws.status, MOE_STATUS_PLAN_CHECK);
  }
  // Quota of (s, a) = the three passes' flows; column prefix over sources.
  const int wave = tid >> 6, lane = tid & 63;
  for (int a = wave; a < ne; a += kQuotaThreads / 64) {
    const int i = iid[a], ra = irank[a], ma = ra / G;
    int carry = 0;
    for (int s0 = 0; s0 < R; s0 += 64) {
      const int s = s0 + lane;
      int v = 0;
      if (s < R) {
        v = (ra == s ? fA[s] : 0) +
            (ma == s / G ? overlap(pfxB[s], pfxB[s] + demA[s], cpfxB[a], cpfxB[a] + capA[a]) : 0) +
            overlap(pfxC[s], pfxC[s] + demB[s], cpfxC[a], cpfxC[a] + capB[a]);
        out.quota[(int64_t)s * cap + i] = v;
      }
      const int incl = wave_incl_scan(v);
      if (s < R) ws.colpre[(int64_t)i * R + s] = carry + incl - v;
      carry += __shfl(incl, 63);
    }
  }
}

// Instance and in-instance position of every slot.
__global__ __launch_bounds__(256) void assign_kernel(Dims d, const int32_t* __restrict__ topk,
                                                     const uint64_t* __restrict__ tile_mask,
                                                     const int32_t* __restrict__ tile_base,
                                                     const int32_t* __restrict__ quota, Workspace ws,
                                                     int32_t* __restrict__ slot_inst, int32_t* __restrict__ slot_rank,
                                                     int32_t* __restrict__ clear, int64_t clear_n) {
  const int64_t sigma = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t N = (int64_t)d.T * d.k;
  for (int64_t i = sigma; i < clear_n; i += (int64_t)gridDim.x * blockDim.x) clear[i] = 0;
  if (sigma >= N) return;
  int inst, rank;
  assign_slot(d, sigma, topk, tile_mask, tile_base, quota, ws, inst, rank);
  slot_inst[sigma] = inst;
  slot_rank[sigma] = rank;
}

// beside: the launch must fit beside another batch's resident row copy.
PlanLayout plan_layout(const Dims& d, bool beside) {
  PlanLayout ly;
  int o = 0;
  auto take = [&](int n) { const int at = o; o += (n + 3) & ~3; return at; };
  ly.RW = (d.R + 63) / 64;
  const int max_bd = (d.B + d.M - 1) / d.M;
  ly.NS = d.n_slot < max_bd ? d.n_slot : max_bd;
  if (ly.NS < 1) ly.NS = 1;
  ly.L = take(d.R);
  ly.nrep = take(d.R);
  ly.inst_base = take(d.R + 1);
  ly.rep_dom = take(d.M);
  ly.Umain = take(d.E);
  ly.eoff = take(d.E + 1);
  ly.rl = take(d.E + 1);
  ly.misc = take(4);
  ly.hm = take(2 * d.E * ly.RW);
  ly.rep_e = take(d.R * ly.NS);
  ly.rep_U = take(d.R * ly.NS);
  ly.rep_id = take(d.R * ly.NS);
  ly.wave_tot = take(kPlanMaxWaves + 1);
  // The domain demand lives in LDS when the whole layout then still fits --
  // beside another batch's resident row copy, within what that copy leaves
  // free (measured on the Kimi-K2-sized layer: with D in LDS, 48 KB, the
  // solver launch waited for the other copy's end; with D in global memory
  // the solver takes ~10 us more alone).
  // (one LDS block is left for the kernel's static LDS, the layer dimensions)
  const size_t budget = (beside ? kBesideGatherLds : kCuLdsBytes) - kLdsBlock;
  const bool d_fits = d.M * d.E <= kDemandLdsMax && (size_t)(o + d.M * d.E) * 4 <= budget;
  ly.D = d_fits ? take(d.M * d.E) : -1;
  ly.total = o;
  return ly;
}

}  // namespace

size_t plan_lds_bytes(const Dims& d) { return sizeof(int32_t) * (size_t)plan_layout(d, false).total; }

namespace {

template <int NT>
hipError_t launch_plan_nt(const Dims& d, const int32_t* omega, const ScanJob& scan, const uint64_t* prev_mask,
                          int32_t* cooc, int32_t* trans, int32_t* part, const moe_plan_out& out, const Workspace& ws,
                          bool beside, PairArgs* pa_out, hipStream_t st) {
  const PlanLayout ly = plan_layout(d, beside);
  size_t lds = sizeof(int32_t) * (size_t)ly.total;
  const int n_scan = scan.mask ? (d.E + kScanEB - 1) / kScanEB : 0;
  if (n_scan > 0) lds = std::max(lds, tile_scan_lds_bytes(d, NT));
  // Pair counts from the masks: partials on the CUs the solver leaves idle,
  // their sums in the quota launch (with one split the partials are final).
  PairArgs pa = pair_args(d, scan.mask, prev_mask, cooc, trans, part, NT);
  if (!scan.mask) pa.nz = 0;
  const int64_t n_pair = (int64_t)pair_blocks(d) * pa.splits * pa.nz;
  if (n_pair > 0) lds = std::max(lds, pair_lds_bytes(NT));
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(plan_kernel<NT>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(plan_kernel<NT>, dim3((unsigned)(1 + n_scan + n_pair)), dim3(NT), lds, st, d, ly, omega, scan,
                     out, ws, pa, n_scan);
  *pa_out = pa;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_plan(const Dims& d, const int32_t* omega, const ScanJob& scan, const uint64_t* prev_mask,
                       int32_t* cooc, int32_t* trans, int32_t* part, const moe_plan_out& out, int32_t* inst_offset,
                       int32_t* rank_offset, const Workspace& ws, bool beside, hipStream_t st) {
  PairArgs pa;
  hipError_t e = beside ? launch_plan_nt<kPlanThreadsBeside>(d, omega, scan, prev_mask, cooc, trans, part, out, ws,
                                                            true, &pa, st)
                        : launch_plan_nt<kPlanThreadsAlone>(d, omega, scan, prev_mask, cooc, trans, part, out, ws,
                                                           false, &pa, st);
  if (e != hipSuccess) return e;
  const int64_t n_reduce = pa.splits > 1 ? (int64_t)pair_blocks(d) * (kPairBlock / kQuotaThreads) * pa.nz : 0;
  const int n_transport = d.B < d.E ? d.B : d.E;  // each replicated expert owns at least one replica
  const int n_fill = (int)(((int64_t)d.R * d.cap + kFillCells - 1) / kFillCells);
  const int n_off = inst_offset ? 1 : 0;
  hipLaunchKernelGGL(quota_kernel, dim3((unsigned)(n_transport + n_fill + n_off + n_reduce)), dim3(kQuotaThreads), 0,
                     st, d, omega, out, inst_offset, rank_offset, ws, n_transport, n_fill, pa);
  return hipGetLastError();
}

namespace {

__global__ __launch_bounds__(256) void zero_kernel(int32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0;
}

}  // namespace

hipError_t launch_zero(int32_t* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

hipError_t launch_assign(const Dims& d, const int32_t* topk_idx, const uint64_t* tile_mask,
                         const int32_t* tile_base, const moe_plan_out& out, const Workspace& ws, int32_t* clear,
                         int64_t clear_n, hipStream_t st) {
  const int64_t N = (int64_t)d.T * d.k;
  if (N == 0) return hipSuccess;
  const int64_t blocks = (N + 255) / 256;
  hipLaunchKernelGGL(assign_kernel, dim3((unsigned)blocks), dim3(256), 0, st, d, topk_idx, tile_mask, tile_base,
                     out.quota, ws, out.slot_inst, out.slot_rank, clear, clear ? clear_n : 0);
  return hipGetLastError();
}

}  // namespace moe
