// Replica placement, token re-routing, quotas and per-slot instances on gfx950.
//
// [TopoEP] section 4.3 (two-stage solver, Eqs. 9 and 10) with the quota and
// slot rules documented in moe_plan.h.  The solver runs in one workgroup of
// 16 waves with its whole state in LDS: the domains are independent in both
// stages, so wave w plans domains w, w+16, ...; each stage-2 iteration is a
// wave-wide argmin over packed candidate keys followed by one update, the
// one-update-per-iteration rule of the page.  All arithmetic is integer and
// every selection has a total order, so the plan is bitwise reproducible.
#include "internal.h"

namespace moe {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kTransportWaves = 8;  // waves with LDS scratch for the per-expert quota transport

// Offsets (in int32 units) of the plan kernel's LDS arrays.
struct PlanLayout {
  int L, nrep, inst_base, rep_dom, base_d, Umain, ereps, eoff, rlist, misc;
  int rep_e, rep_r, rep_U, rep_inst, inst_e, inst_r, inst_u, wave_tot, scratch;
  int scratch_per_wave;
  int total;
};

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
  lo = __shfl_xor(lo, m);
  hi = __shfl_xor(hi, m);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint64_t o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}

// Lexicographic minimum of (hi, lo) over the wave.
__device__ __forceinline__ void wave_min_key(uint64_t& hi, uint32_t& lo) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint64_t oh = shfl_xor_u64(hi, m);
    const uint32_t ol = (uint32_t)__shfl_xor((int)lo, m);
    if (oh < hi || (oh == hi && ol < lo)) {
      hi = oh;
      lo = ol;
    }
  }
}

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  return v;
}

// In-place exclusive scan of a[0..n) in LDS by the whole workgroup; returns the total.
// wave_tot: kPlanWaves + 1 ints of LDS.
__device__ int block_excl_scan(int* a, int n, int* wave_tot) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  __syncthreads();
  const int per = (n + kPlanThreads - 1) / kPlanThreads;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int sum = 0;
  for (int q = lo; q < hi; ++q) sum += a[q];
  const int incl = wave_incl_scan(sum);
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < kPlanWaves; ++w) {
      const int v = wave_tot[w];
      wave_tot[w] = run;
      run += v;
    }
    wave_tot[kPlanWaves] = run;
  }
  __syncthreads();
  int run = wave_tot[wave] + incl - sum;
  for (int q = lo; q < hi; ++q) {
    const int v = a[q];
    a[q] = run;
    run += v;
  }
  const int total = wave_tot[kPlanWaves];
  __syncthreads();
  return total;
}

__device__ __forceinline__ int64_t overlap(int64_t a0, int64_t a1, int64_t b0, int64_t b1) {
  const int64_t lo = a0 > b0 ? a0 : b0, hi = a1 < b1 ? a1 : b1;
  return hi > lo ? hi - lo : 0;
}

__device__ __forceinline__ int domain_budget(const Dims& d, int m) {
  return d.B / d.M + (m < d.B % d.M ? 1 : 0);
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(Dims d, PlanLayout ly, const int32_t* __restrict__ omega,
                                                            moe_plan_out out, Workspace ws) {
  extern __shared__ int32_t lds[];
  int32_t* L = lds + ly.L;
  int32_t* nrep = lds + ly.nrep;
  int32_t* inst_base = lds + ly.inst_base;
  int32_t* rep_dom = lds + ly.rep_dom;
  int32_t* base_d = lds + ly.base_d;
  int32_t* Umain = lds + ly.Umain;
  int32_t* ereps = lds + ly.ereps;
  int32_t* eoff = lds + ly.eoff;
  int32_t* rlist = lds + ly.rlist;
  int32_t* misc = lds + ly.misc;  // [0] n_inst, [1] replicated experts, [2] check flag
  int32_t* rep_e = lds + ly.rep_e;
  int32_t* rep_r = lds + ly.rep_r;
  int32_t* rep_U = lds + ly.rep_U;
  int32_t* rep_inst = lds + ly.rep_inst;
  int32_t* inst_e = lds + ly.inst_e;
  int32_t* inst_r = lds + ly.inst_r;
  int32_t* inst_u = lds + ly.inst_u;
  int32_t* wave_tot = lds + ly.wave_tot;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int E = d.E, R = d.R, G = d.G, M = d.M, Er = d.Er;

  // ---- init ---------------------------------------------------------------
  for (int e = tid; e < E; e += kPlanThreads) { Umain[e] = 0; ereps[e] = 0; }
  for (int r = tid; r < R; r += kPlanThreads) nrep[r] = 0;
  for (int m = tid; m < M; m += kPlanThreads) rep_dom[m] = 0;
  if (tid == 0) {
    int run = 0;
    for (int m = 0; m < M; ++m) { base_d[m] = run; run += domain_budget(d, m); }
    base_d[M] = run;
    misc[0] = 0; misc[1] = 0; misc[2] = 0;
  }
  // Domain demand D[m][e] (Eq. 4), int64 in the workspace.
  for (int idx = tid; idx < M * E; idx += kPlanThreads) {
    const int m = idx / E, e = idx - m * E;
    int64_t sum = 0;
    for (int g = 0; g < G; ++g) sum += omega[(int64_t)(m * G + g) * E + e];
    ws.demand[idx] = sum;
  }
  __syncthreads();

  // ---- stage 1: inter-node placement (Eq. 9), one wave per domain ----------
  for (int m = wave; m < M; m += kPlanWaves) {
    const int Bd = base_d[m + 1] - base_d[m];
    uint32_t taken = 0;  // bit i: expert lane + 64 i already placed in this domain
    while (rep_dom[m] < Bd) {
      uint64_t best = 0ull;
      for (int i = 0, e = lane; e < E; ++i, e += 64) {
        if ((taken >> i) & 1u) continue;
        if ((e / Er) / G == m) continue;
        const int64_t D = ws.demand[(int64_t)m * E + e];
        if (2 * D * d.S - d.W <= 0) continue;
        // Largest benefit first; S > 0 so that is the largest demand; ties to the lower expert.
        const uint64_t key = ((uint64_t)D << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
        best = key > best ? key : best;
      }
      best = wave_max_u64(best);
      if (best == 0ull) break;
      const int ebest = (int)(0xffffffffu - (uint32_t)best);
      if ((ebest & 63) == lane) taken |= 1u << (ebest >> 6);
      int stop = 0;
      if (lane == 0) {
        int rbest = -1;  // least-occupied rank with a free slot, ties to the lower rank
        for (int r = m * G; r < (m + 1) * G; ++r)
          if (nrep[r] < d.n_slot && (rbest < 0 || nrep[r] < nrep[rbest])) rbest = r;
        if (rbest < 0) {
          stop = 1;
        } else {
          const int j = base_d[m] + rep_dom[m];
          rep_e[j] = ebest; rep_r[j] = rbest; rep_U[j] = 0;
          nrep[rbest] += 1;
          rep_dom[m] += 1;
          atomicAdd(&ereps[ebest], 1);
        }
      }
      stop = __shfl(stop, 0);
      wave_sync();
      if (stop) break;
    }
  }
  __syncthreads();

  // ---- stage-1 routing: even split over the selected instances -------------
  for (int idx = tid; idx < R * E; idx += kPlanThreads) {
    const int s = idx / E, e = idx - s * E;
    const int w = omega[idx];
    if (w == 0) continue;
    const int ms = s / G, mm = (e / Er) / G;
    if (ereps[e] == 0 || mm == ms) {
      atomicAdd(&Umain[e], w);
      continue;
    }
    int local = -1;
    for (int j = base_d[ms]; j < base_d[ms] + rep_dom[ms]; ++j)
      if (rep_e[j] == e) local = j;
    if (local >= 0) {
      atomicAdd(&rep_U[local], w);
      continue;
    }
    // No instance in the source's domain: all instances of e, in rank order.
    // After stage 1 each domain holds at most one instance of e and the
    // domains are rank-ordered, so walking the domains visits them in order.
    const int n = 1 + ereps[e];
    int pos = 0;
    for (int m = 0; m < M; ++m) {
      int target = -2;
      if (m == mm) {
        target = -1;
      } else {
        for (int j = base_d[m]; j < base_d[m] + rep_dom[m]; ++j)
          if (rep_e[j] == e) target = j;
      }
      if (target == -2) continue;
      const int share = w / n + (pos < w % n ? 1 : 0);
      ++pos;
      if (share == 0) continue;
      if (target == -1) atomicAdd(&Umain[e], share);
      else atomicAdd(&rep_U[target], share);
    }
  }
  __syncthreads();
  for (int r = tid; r < R; r += kPlanThreads) {
    int sum = 0;
    for (int h = 0; h < Er; ++h) sum += Umain[r * Er + h];
    const int m = r / G;
    for (int j = base_d[m]; j < base_d[m] + rep_dom[m]; ++j)
      if (rep_r[j] == r) sum += rep_U[j];
    L[r] = sum;
  }
  __syncthreads();

  // ---- stage 2: intra-node refinement (Eq. 10), one wave per domain --------
  for (int m = wave; m < M; m += kPlanWaves) {
    const int Bd = base_d[m + 1] - base_d[m];
    const int bj = base_d[m];
    const int r0 = m * G;
    for (int it = 0; it < d.max_iters; ++it) {
      uint64_t kb = 0ull;
      if (lane < G) kb = ((uint64_t)(uint32_t)L[r0 + lane] << 32) | (uint64_t)(0xffffffffu - (uint32_t)lane);
      kb = wave_max_u64(kb);
      const int rb = r0 + (int)(0xffffffffu - (uint32_t)kb);
      const int Lb = (int)(kb >> 32);
      const int nh = Er + rep_dom[m];
      uint64_t best_hi = ~0ull;
      uint32_t best_lo = ~0u;
      for (int cidx = lane; cidx < nh * G; cidx += 64) {
        const int h = cidx / G, rt = r0 + (cidx - h * G);
        if (rt == rb) continue;
        int e, Ub;
        if (h < Er) {
          e = rb * Er + h;
          Ub = Umain[e];
        } else {
          const int j = bj + (h - Er);
          if (rep_r[j] != rb) continue;
          e = rep_e[j];
          Ub = rep_U[j];
        }
        if (Ub <= 0) continue;
        bool hosted = (e / Er) == rt;
        for (int j = bj; j < bj + rep_dom[m] && !hosted; ++j) hosted = rep_e[j] == e && rep_r[j] == rt;
        if (!hosted && !(nrep[rt] < d.n_slot && rep_dom[m] < Bd)) continue;
        const int Lt = L[rt];
        const int half = (Lb - Lt) >> 1;
        const int delta = Ub < half ? Ub : half;
        if (delta < 1) continue;
        // Key: largest delta, lowest target load, existing instance first, lower e, lower r_t.
        const uint64_t hi = ((uint64_t)(uint32_t)(0x7fffffff - delta) << 32) | (uint64_t)(uint32_t)Lt;
        const uint32_t lo = ((uint32_t)(hosted ? 0 : 1) << 31) | ((uint32_t)e << 16) | (uint32_t)rt;
        if (hi < best_hi || (hi == best_hi && lo < best_lo)) {
          best_hi = hi;
          best_lo = lo;
        }
      }
      wave_min_key(best_hi, best_lo);
      if (best_hi == ~0ull) break;
      if (lane == 0) {
        const int delta = 0x7fffffff - (int)(uint32_t)(best_hi >> 32);
        const bool is_new = (best_lo >> 31) != 0u;
        const int e = (int)((best_lo >> 16) & 0x7fffu);
        const int rt = (int)(best_lo & 0xffffu);
        if ((e / Er) == rb) {
          Umain[e] -= delta;
        } else {
          for (int j = bj; j < bj + rep_dom[m]; ++j)
            if (rep_e[j] == e && rep_r[j] == rb) rep_U[j] -= delta;
        }
        if (is_new) {
          const int j = bj + rep_dom[m];
          rep_e[j] = e; rep_r[j] = rt; rep_U[j] = delta;
          rep_dom[m] += 1;
          nrep[rt] += 1;
          atomicAdd(&ereps[e], 1);
        } else if ((e / Er) == rt) {
          Umain[e] += delta;
        } else {
          for (int j = bj; j < bj + rep_dom[m]; ++j)
            if (rep_e[j] == e && rep_r[j] == rt) rep_U[j] += delta;
        }
        L[rb] -= delta;
        L[rt] += delta;
      }
      wave_sync();
    }
  }
  __syncthreads();

  // ---- instance table -------------------------------------------------------
  for (int r = tid; r < R; r += kPlanThreads) inst_base[r] = Er + nrep[r];
  const int n_inst = block_excl_scan(inst_base, R, wave_tot);
  if (tid == 0) { inst_base[R] = n_inst; misc[0] = n_inst; }
  const int nregion = base_d[M];
  for (int j = tid; j < nregion; j += kPlanThreads) {
    int m = 0;
    while (base_d[m + 1] <= j) ++m;
    rep_inst[j] = -1;
    if (j - base_d[m] >= rep_dom[m]) continue;
    const int r = rep_r[j], e = rep_e[j];
    int pos = 0;
    for (int q = base_d[m]; q < base_d[m] + rep_dom[m]; ++q) pos += (rep_r[q] == r && rep_e[q] < e) ? 1 : 0;
    const int id = inst_base[r] + Er + pos;
    rep_inst[j] = id;
    inst_e[id] = e; inst_r[id] = r; inst_u[id] = rep_U[j];
  }
  for (int e = tid; e < E; e += kPlanThreads) {
    const int r = e / Er;
    const int id = inst_base[r] + (e - r * Er);
    inst_e[id] = e; inst_r[id] = r; inst_u[id] = Umain[e];
    eoff[e] = 1 + ereps[e];
  }
  for (int r = tid; r < R; r += kPlanThreads) out.rank_load[r] = L[r];
  if (tid == 0) out.n_inst[0] = n_inst;
  __syncthreads();
  for (int i = tid; i < d.cap; i += kPlanThreads) {
    const bool live = i < n_inst;
    out.inst_expert[i] = live ? inst_e[i] : -1;
    out.inst_rank[i] = live ? inst_r[i] : -1;
    out.inst_load[i] = live ? inst_u[i] : -1;
    if (!live) inst_e[i] = -1;
  }
  const int total_inst = block_excl_scan(eoff, E, wave_tot);
  if (tid == 0) eoff[E] = total_inst;
  __syncthreads();
  for (int e = tid; e <= E; e += kPlanThreads) ws.einst_off[e] = eoff[e];
  // Per-expert instance lists in rank order.
  for (int e = tid; e < E; e += kPlanThreads) {
    const int rm = e / Er;
    int pos = 0;
    if (ereps[e] > 0) {
      for (int m = 0; m < M; ++m)
        for (int j = base_d[m]; j < base_d[m] + rep_dom[m]; ++j) pos += (rep_e[j] == e && rep_r[j] < rm) ? 1 : 0;
      const int q = atomicAdd(&misc[1], 1);
      rlist[q] = e;
    }
    ws.einst_list[eoff[e] + pos] = inst_base[rm] + (e - rm * Er);
  }
  for (int j = tid; j < nregion; j += kPlanThreads) {
    if (rep_inst[j] < 0) continue;
    const int e = rep_e[j], r = rep_r[j];
    int pos = (e / Er) < r ? 1 : 0;
    for (int m = 0; m < M; ++m)
      for (int q = base_d[m]; q < base_d[m] + rep_dom[m]; ++q) pos += (rep_e[q] == e && rep_r[q] < r) ? 1 : 0;
    ws.einst_list[eoff[e] + pos] = rep_inst[j];
  }
  __syncthreads();

  // ---- quotas of replicated experts: three-pass transport, one wave each ---
  const int nrepl = misc[1];
  if (wave < kTransportWaves) {
    int32_t* sc = lds + ly.scratch + wave * ly.scratch_per_wave;
    int32_t* dem = sc;           // [R]
    int32_t* pfx = sc + R;       // [R]
    int32_t* onr = sc + 2 * R;   // [R] list index of the instance on rank s, or -1
    int32_t* caps = sc + 3 * R;  // [R] remaining capacity of list entry a
    int32_t* cpfx = sc + 4 * R;  // [R]
    int32_t* ilst = sc + 5 * R;  // [R] instance id of list entry a
    int32_t* irank = sc + 6 * R; // [R] rank of list entry a
    for (int q = wave; q < nrepl; q += kTransportWaves) {
      const int e = rlist[q];
      const int off = eoff[e], ne = eoff[e + 1] - eoff[e];
      for (int a = lane; a < ne; a += 64) {
        const int i = ws.einst_list[off + a];
        ilst[a] = i; irank[a] = inst_r[i]; caps[a] = inst_u[i];
      }
      for (int s = lane; s < R; s += 64) { onr[s] = -1; dem[s] = omega[(int64_t)s * E + e]; }
      wave_sync();
      for (int a = lane; a < ne; a += 64) onr[irank[a]] = a;
      // Every access to qrep[.][s] below is made by the lane that owns source s.
      for (int s = lane; s < R; s += 64)
        for (int a = 0; a < ne; ++a) ws.qrep[(int64_t)ilst[a] * R + s] = 0;
      wave_sync();
      // Pass A: the instance on the source's own rank.
      for (int s = lane; s < R; s += 64) {
        const int a = onr[s];
        if (a < 0) continue;
        const int f = min(dem[s], caps[a]);
        if (f <= 0) continue;
        dem[s] -= f; caps[a] -= f;
        ws.qrep[(int64_t)ilst[a] * R + s] += f;
      }
      wave_sync();
      // Pass B: instances in the source's domain.  Sources ascending and
      // instances in rank order: the greedy fill is the overlap of the two
      // cumulative intervals, computed per domain.
      for (int s = lane; s < R; s += 64) {
        int run = 0;
        for (int s2 = (s / G) * G; s2 < s; ++s2) run += dem[s2];
        pfx[s] = run;
      }
      for (int a = lane; a < ne; a += 64) {
        int run = 0;
        for (int a2 = a - 1; a2 >= 0 && irank[a2] / G == irank[a] / G; --a2) run += caps[a2];
        cpfx[a] = run;
      }
      wave_sync();
      {
        int newdem[4], newcap[4];
        int u = 0;
        for (int s = lane; s < R; s += 64, ++u) {
          const int m = s / G;
          int left = dem[s];
          for (int a = 0; a < ne && left > 0; ++a) {
            if (irank[a] / G != m) continue;
            const int f = (int)overlap(pfx[s], pfx[s] + dem[s], cpfx[a], cpfx[a] + caps[a]);
            if (f > 0) { ws.qrep[(int64_t)ilst[a] * R + s] += f; left -= f; }
          }
          newdem[u] = left;
        }
        u = 0;
        for (int a = lane; a < ne; a += 64, ++u) {
          const int m = irank[a] / G;
          const int last = (m + 1) * G - 1;
          const int dtot = pfx[last] + dem[last];
          newcap[u] = caps[a] - (int)overlap(cpfx[a], cpfx[a] + caps[a], 0, dtot);
        }
        wave_sync();
        u = 0;
        for (int s = lane; s < R; s += 64, ++u) dem[s] = newdem[u];
        u = 0;
        for (int a = lane; a < ne; a += 64, ++u) caps[a] = newcap[u];
        wave_sync();
      }
      // Pass C: all instances, all sources.
      {
        int carry = 0;
        for (int s0 = 0; s0 < R; s0 += 64) {
          const int s = s0 + lane;
          const int v = s < R ? dem[s] : 0;
          const int incl = wave_incl_scan(v);
          if (s < R) pfx[s] = carry + incl - v;
          carry += __shfl(incl, 63);
        }
        carry = 0;
        for (int a0 = 0; a0 < ne; a0 += 64) {
          const int a = a0 + lane;
          const int v = a < ne ? caps[a] : 0;
          const int incl = wave_incl_scan(v);
          if (a < ne) cpfx[a] = carry + incl - v;
          carry += __shfl(incl, 63);
        }
        wave_sync();
        bool left_over = false;
        for (int s = lane; s < R; s += 64) {
          int left = dem[s];
          for (int a = 0; a < ne && left > 0; ++a) {
            const int f = (int)overlap(pfx[s], pfx[s] + dem[s], cpfx[a], cpfx[a] + caps[a]);
            if (f > 0) { ws.qrep[(int64_t)ilst[a] * R + s] += f; left -= f; }
          }
          left_over |= left != 0;
        }
        if (left_over) misc[2] = 1;
      }
      wave_sync();
      // Exclusive prefix of each instance's quotas over the sources.
      for (int a = 0; a < ne; ++a) {
        const int64_t base = (int64_t)ilst[a] * R;
        int carry = 0;
        for (int s0 = 0; s0 < R; s0 += 64) {
          const int s = s0 + lane;
          const int v = s < R ? ws.qrep[base + s] : 0;
          const int incl = wave_incl_scan(v);
          if (s < R) ws.colpre[base + s] = carry + incl - v;
          carry += __shfl(incl, 63);
        }
      }
      wave_sync();
    }
  }
  __syncthreads();

  // ---- dense quota matrix ----------------------------------------------------
  const int cap = d.cap;
  for (int64_t idx = tid; idx < (int64_t)R * cap; idx += kPlanThreads) {
    const int s = (int)(idx / cap), i = (int)(idx - (int64_t)s * cap);
    int q = 0;
    if (i < n_inst) {
      const int e = inst_e[i];
      q = ereps[e] == 0 ? omega[(int64_t)s * E + e] : ws.qrep[(int64_t)i * R + s];
    }
    out.quota[idx] = q;
  }
  if (tid == 0 && misc[2]) atomicOr(ws.status, MOE_STATUS_PLAN_CHECK);
}

// Instance and in-instance position of every slot.
__global__ __launch_bounds__(256) void assign_kernel(Dims d, const int32_t* __restrict__ topk,
                                                     const uint64_t* __restrict__ tile_mask,
                                                     const int32_t* __restrict__ tile_base,
                                                     const int32_t* __restrict__ quota, Workspace ws,
                                                     int32_t* __restrict__ slot_inst, int32_t* __restrict__ slot_rank) {
  const int64_t sigma = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t N = (int64_t)d.T * d.k;
  if (sigma >= N) return;
  const int64_t t = sigma / d.k;
  const int s = (int)(t / d.Tr);
  const int tl = (int)(t - (int64_t)s * d.Tr);
  const int x = s * d.C + (tl >> 6);
  const int bit = tl & 63;
  const int e = topk[sigma];
  int inst = -1, rank = -1;
  if ((unsigned)e < (unsigned)d.E) {
    const uint64_t m = tile_mask[(int64_t)x * d.E + e];
    const int low = __popcll(m & ((1ull << bit) - 1ull));
    const int base = tile_base[(int64_t)x * d.E + e];
    const int o0 = ws.einst_off[e], o1 = ws.einst_off[e + 1];
    if (o1 - o0 == 1) {
      // One instance: its segment holds the expert's slots of all sources in token order.
      inst = ws.einst_list[o0];
      rank = base + low;
    } else {
      const int p = base - tile_base[(int64_t)s * d.C * d.E + e] + low;
      int cum = 0;
      for (int a = o0; a < o1; ++a) {
        const int i = ws.einst_list[a];
        if ((unsigned)i >= (unsigned)d.cap) break;
        const int qv = quota[(int64_t)s * d.cap + i];
        if (p < cum + qv) {
          inst = i;
          rank = ws.colpre[(int64_t)i * d.R + s] + (p - cum);
          break;
        }
        cum += qv;
      }
    }
  }
  if (inst < 0) atomicOr(ws.status, MOE_STATUS_PLAN_CHECK);
  slot_inst[sigma] = inst;
  slot_rank[sigma] = rank;
}

PlanLayout plan_layout(const Dims& d) {
  PlanLayout ly;
  int o = 0;
  auto take = [&](int n) { const int at = o; o += (n + 3) & ~3; return at; };
  ly.L = take(d.R);
  ly.nrep = take(d.R);
  ly.inst_base = take(d.R + 1);
  ly.rep_dom = take(d.M);
  ly.base_d = take(d.M + 1);
  ly.Umain = take(d.E);
  ly.ereps = take(d.E);
  ly.eoff = take(d.E + 1);
  ly.rlist = take(d.E + 1);
  ly.misc = take(4);
  const int nb = d.B > 0 ? d.B : 1;
  ly.rep_e = take(nb);
  ly.rep_r = take(nb);
  ly.rep_U = take(nb);
  ly.rep_inst = take(nb);
  ly.inst_e = take(d.cap);
  ly.inst_r = take(d.cap);
  ly.inst_u = take(d.cap);
  ly.wave_tot = take(kPlanWaves + 1);
  ly.scratch_per_wave = 7 * d.R;
  ly.scratch = take(kTransportWaves * ly.scratch_per_wave);
  ly.total = o;
  return ly;
}

}  // namespace

size_t plan_lds_bytes(const Dims& d) { return sizeof(int32_t) * (size_t)plan_layout(d).total; }

hipError_t launch_plan(const Dims& d, const int32_t* omega, const moe_plan_out& out, const Workspace& ws,
                       hipStream_t st) {
  const PlanLayout ly = plan_layout(d);
  const size_t lds = sizeof(int32_t) * (size_t)ly.total;
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(plan_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), lds, st, d, ly, omega, out, ws);
  return hipGetLastError();
}

hipError_t launch_assign(const Dims& d, const int32_t* topk_idx, const uint64_t* tile_mask,
                         const int32_t* tile_base, const moe_plan_out& out, const Workspace& ws, hipStream_t st) {
  const int64_t N = (int64_t)d.T * d.k;
  if (N == 0) return hipSuccess;
  const int64_t blocks = (N + 255) / 256;
  hipLaunchKernelGGL(assign_kernel, dim3((unsigned)blocks), dim3(256), 0, st, d, topk_idx, tile_mask, tile_base,
                     out.quota, ws, out.slot_inst, out.slot_rank);
  return hipGetLastError();
}

}  // namespace moe
