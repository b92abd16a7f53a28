// CPU oracle for the MoE dispatch-planning path -- TEST INFRASTRUCTURE ONLY.
//
// Plain, slow, single-threaded and written for checking by eye against the
// pages.  Only the tests, the smoke check and the benchmark's CPU-baseline
// leg load it; it shares no code with the HIP library.  The function-level
// comments cite the passage each step follows:
//   [TopoEP]   "TopoEP: Topology-Aware Load Balancing for Expert-Parallel MoE
//              Training" (sections 2.1, 3.1, 4.1-4.3; Eqs. 3, 4, 9, 10; Fig. 9)
//   [Coupling] "Expert Coupling in MoE Pretraining" (sections "Experts Are
//              Correlated Within a Layer", "Routing Is Also Correlated Across
//              Layers")
// Where the pages leave a choice open, the reading taken is stated at the
// step that needs it.
//
// Build without fast-math, FTZ or DAZ: the top-k order relies on exact IEEE
// comparisons.

#include "moe_oracle.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <numeric>
#include <vector>

namespace {

struct Derived {
  int64_t M, Tr, Er, n_slot, S, W, max_iters;
};

bool valid(const oracle_cfg* c) {
  if (!c) return false;
  if (c->T < 0 || c->E < 1 || c->k < 1 || c->k > c->E || c->R < 1 || c->G < 1 || c->H < 1) return false;
  if (c->R % c->G != 0 || c->T % c->R != 0 || c->E % c->R != 0 || c->B < 0) return false;
  return true;
}

Derived derive(const oracle_cfg* c) {
  Derived d;
  d.M = c->R / c->G;
  d.Tr = c->T / c->R;
  d.Er = c->E / c->R;
  // Replica slots per rank: the configured value, else enough for the
  // largest per-domain share of the budget spread over the domain's ranks.
  int64_t per_dom = (c->B + d.M - 1) / d.M;
  d.n_slot = c->n_slot > 0 ? c->n_slot : (per_dom + c->G - 1) / c->G;
  // More slots than the whole budget can never be filled.
  if (d.n_slot > c->B) d.n_slot = c->B;
  // S_tok: one bf16 activation row.  ||W_e||: three H x I bf16 matrices with
  // I = 3H/8, i.e. 9H^2/4 bytes (9 MiB at H = 2048, the TopoEP Fig. 3 example).
  d.S = c->S > 0 ? c->S : 2LL * c->H;
  d.W = c->W >= 0 ? c->W : 9LL * c->H * c->H / 4;
  d.max_iters = c->max_iters > 0 ? c->max_iters : 4096;
  return d;
}

// Fixed contiguous layouts (the pages leave them open):
//   source rank of token t: contiguous blocks of T/R tokens;
//   NVLink domain of rank r: contiguous blocks of G ranks;
//   main rank of expert e: contiguous blocks of E/R experts.
inline int64_t src_of(const Derived& d, int64_t t) { return t / d.Tr; }
inline int64_t dom_of(const oracle_cfg* c, int64_t r) { return r / c->G; }
inline int64_t main_of(const Derived& d, int64_t e) { return e / d.Er; }

int64_t domain_budget(const oracle_cfg* c, const Derived& d, int64_t dom) {
  // The budget B counts extra instances of the whole layer; each domain gets
  // an equal share, the remainder going to the lowest domains, so that the
  // domains can be planned independently (TopoEP section 4.3).
  return c->B / d.M + (dom < c->B % d.M ? 1 : 0);
}

}  // namespace

extern "C" int oracle_params(const oracle_cfg* c, int64_t* out) {
  if (!valid(c) || !out) return -1;
  Derived d = derive(c);
  out[0] = d.M; out[1] = d.Tr; out[2] = d.Er; out[3] = d.n_slot;
  out[4] = d.S; out[5] = d.W; out[6] = d.max_iters; out[7] = c->B;
  return 0;
}

extern "C" int oracle_domain_budget(const oracle_cfg* c, int32_t* out_bd) {
  if (!valid(c) || !out_bd) return -1;
  Derived d = derive(c);
  for (int64_t m = 0; m < d.M; ++m) out_bd[m] = (int32_t)domain_budget(c, d, m);
  return 0;
}

// ---------------------------------------------------------------------------
// Top-k gating and histograms.
//
// [TopoEP] section 2.1: the router of each rank selects the top-k experts of
// each of its local tokens.  The order of the k picks and the treatment of
// equal logits are not given; here the picks are listed by logit, largest
// first, equal logits ordered by lower expert index, -0.0 equal to +0.0, and
// a NaN logit is an error.
//
// [TopoEP] Eq. 3: omega[s][e] counts the token-expert assignments of source
// rank s that select expert e; count[e] is its column sum (the expert load).
// [Coupling] "Experts Are Correlated Within a Layer": cooc[a][b] counts the
// tokens selecting both a and b, a != b; the diagonal is masked (zero).
// [Coupling] "Routing Is Also Correlated Across Layers": trans[a][b] counts
// the tokens that select a in the previous layer and b in this one.
// ---------------------------------------------------------------------------
extern "C" int oracle_route(const oracle_cfg* c, const float* logits, const int32_t* prev_topk,
                            int32_t* topk_idx, float* topk_val, int32_t* count, int32_t* omega,
                            int32_t* cooc, int32_t* trans) {
  if (!valid(c) || (c->T > 0 && (!logits || !topk_idx)) || !count || !omega) return -1;
  Derived d = derive(c);
  const int64_t T = c->T, E = c->E, k = c->k, R = c->R;
  int status = 0;
  std::vector<int32_t> order(E);
  for (int64_t t = 0; t < T; ++t) {
    const float* row = logits + t * E;
    bool has_nan = false;
    for (int64_t e = 0; e < E; ++e) has_nan |= std::isnan(row[e]);
    if (has_nan) {
      status = -4;
      for (int64_t j = 0; j < k; ++j) {
        topk_idx[t * k + j] = (int32_t)j;
        if (topk_val) topk_val[t * k + j] = row[j];
      }
      continue;
    }
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return row[a] > row[b]; });
    for (int64_t j = 0; j < k; ++j) {
      topk_idx[t * k + j] = order[j];
      if (topk_val) topk_val[t * k + j] = row[order[j]];
    }
  }
  std::fill(count, count + E, 0);
  std::fill(omega, omega + R * E, 0);
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < k; ++j) {
      int32_t e = topk_idx[t * k + j];
      count[e] += 1;
      omega[src_of(d, t) * E + e] += 1;
    }
  if (cooc) {
    std::fill(cooc, cooc + E * E, 0);
    for (int64_t t = 0; t < T; ++t)
      for (int64_t i = 0; i < k; ++i)
        for (int64_t j = 0; j < k; ++j) {
          int32_t a = topk_idx[t * k + i], b = topk_idx[t * k + j];
          if (a != b) cooc[(int64_t)a * E + b] += 1;
        }
  }
  if (trans && prev_topk) {
    std::fill(trans, trans + E * E, 0);
    for (int64_t t = 0; t < T; ++t)
      for (int64_t i = 0; i < k; ++i)
        for (int64_t j = 0; j < k; ++j) {
          int32_t a = prev_topk[t * k + i], b = topk_idx[t * k + j];
          trans[(int64_t)a * E + b] += 1;
        }
  }
  return status;
}

// ---------------------------------------------------------------------------
// Replica placement and token routing: [TopoEP] section 4.3.
// ---------------------------------------------------------------------------
extern "C" int oracle_plan(const oracle_cfg* c, const int32_t* omega, const int32_t* topk_idx,
                           int32_t* n_inst_out, int32_t* inst_expert, int32_t* inst_rank,
                           int32_t* inst_load, int32_t* rank_load, int32_t* quota, int32_t* slot_inst,
                           int32_t* rank_load_stage1, int32_t* trace, int32_t trace_cap, int32_t* n_trace) {
  if (!valid(c) || !omega || (c->T > 0 && (!topk_idx || !slot_inst)) || !n_inst_out || !inst_expert ||
      !inst_rank || !inst_load || !rank_load || !quota)
    return -1;
  Derived d = derive(c);
  const int64_t T = c->T, E = c->E, k = c->k, R = c->R, G = c->G, M = d.M;
  const int64_t cap = E + c->B;  // instance-table capacity
  auto om = [&](int64_t s, int64_t e) -> int64_t { return omega[s * E + e]; };

  // Placement x[e][r] (1 if rank r hosts an instance of e), per-instance
  // load U[e][r], rank load L[r], replicas per rank and per domain.
  std::vector<uint8_t> x(E * R, 0);
  std::vector<int64_t> U(E * R, 0), L(R, 0), nrep(R, 0), rep_dom(M, 0);
  auto X = [&](int64_t e, int64_t r) -> uint8_t& { return x[e * R + r]; };
  auto Uer = [&](int64_t e, int64_t r) -> int64_t& { return U[e * R + r]; };

  // Fixed main placement (constraint C5).
  for (int64_t e = 0; e < E; ++e) X(e, main_of(d, e)) = 1;

  // Domain demand D[dom][e], Eq. 4: assignments of expert e whose source rank
  // lies in the domain.
  std::vector<int64_t> D(M * E, 0);
  for (int64_t s = 0; s < R; ++s)
    for (int64_t e = 0; e < E; ++e) D[dom_of(c, s) * E + e] += om(s, e);

  // Stage 1, inter-node placement, each domain on its own.  Benefit Eq. 9:
  // b = 2 * D * S_tok - ||W_e||, kept only for experts whose main instance is
  // outside the domain and with b > 0 (this is criterion C4).  Candidates are
  // taken in descending benefit (equal benefits: lower expert first).  Each
  // goes to the least-occupied rank of the domain with a free slot (fewest
  // replicas; equal: lower rank), until the domain's budget share is spent or
  // no rank has a free slot.
  for (int64_t m = 0; m < M; ++m) {
    std::vector<std::pair<int64_t, int64_t>> cand;  // (benefit, expert)
    for (int64_t e = 0; e < E; ++e) {
      if (dom_of(c, main_of(d, e)) == m) continue;
      int64_t b = 2 * D[m * E + e] * d.S - d.W;
      if (b > 0) cand.push_back({b, e});
    }
    std::stable_sort(cand.begin(), cand.end(), [](const std::pair<int64_t, int64_t>& a,
                                                  const std::pair<int64_t, int64_t>& b) {
      if (a.first != b.first) return a.first > b.first;
      return a.second < b.second;
    });
    const int64_t Bd = domain_budget(c, d, m);
    for (const auto& ce : cand) {
      if (rep_dom[m] >= Bd) break;
      int64_t best = -1;
      for (int64_t r = m * G; r < (m + 1) * G; ++r) {
        if (nrep[r] >= d.n_slot) continue;
        if (best < 0 || nrep[r] < nrep[best]) best = r;
      }
      if (best < 0) break;
      X(ce.second, best) = 1;
      nrep[best] += 1;
      rep_dom[m] += 1;
    }
  }

  // Stage-1 token routing.  For each (s, e) use the instances of e in the
  // source's domain if there are any, else every instance of e; split
  // omega[s][e] evenly: each selected instance (in rank order) gets the floor
  // share and the first (omega mod m) of them one more.  Then the instance
  // loads U and rank loads L.
  for (int64_t s = 0; s < R; ++s)
    for (int64_t e = 0; e < E; ++e) {
      int64_t w = om(s, e);
      if (w == 0) continue;
      std::vector<int64_t> sel;
      for (int64_t r = 0; r < R; ++r)
        if (X(e, r) && dom_of(c, r) == dom_of(c, s)) sel.push_back(r);
      if (sel.empty())
        for (int64_t r = 0; r < R; ++r)
          if (X(e, r)) sel.push_back(r);
      int64_t m = (int64_t)sel.size();
      for (int64_t i = 0; i < m; ++i) Uer(e, sel[i]) += w / m + (i < w % m ? 1 : 0);
    }
  for (int64_t r = 0; r < R; ++r) {
    L[r] = 0;
    for (int64_t e = 0; e < E; ++e) L[r] += Uer(e, r);
  }
  if (rank_load_stage1)
    for (int64_t r = 0; r < R; ++r) rank_load_stage1[r] = (int32_t)L[r];

  // Stage 2, intra-node refinement, each domain on its own (Eq. 10).  Every
  // iteration: the busiest rank r_b (equal loads: lower rank); candidates are
  // the experts e hosted on r_b with U[e][r_b] > 0 and the other ranks r_t of
  // the domain that host e or still have a free slot (and the domain still
  // has budget); the transfer is delta = min(U[e][r_b], floor((L_b - L_t)/2)),
  // kept if delta >= 1.  The chosen candidate has the largest delta, then the
  // lowest target load, then prefers an existing instance over a new replica
  // (a new replica costs a parameter transfer), then lower e, then lower r_t.
  // One update per iteration; stop when no candidate remains or after
  // max_iters iterations.
  int32_t ntr = 0;
  for (int64_t m = 0; m < M; ++m) {
    const int64_t Bd = domain_budget(c, d, m);
    for (int64_t it = 0; it < d.max_iters; ++it) {
      int64_t rb = m * G;
      for (int64_t r = m * G; r < (m + 1) * G; ++r)
        if (L[r] > L[rb]) rb = r;
      bool found = false;
      int64_t bd = 0, blt = 0, bnew = 0, be = 0, brt = 0;
      for (int64_t e = 0; e < E; ++e) {
        if (!X(e, rb) || Uer(e, rb) <= 0) continue;
        for (int64_t rt = m * G; rt < (m + 1) * G; ++rt) {
          if (rt == rb) continue;
          int64_t is_new = X(e, rt) ? 0 : 1;
          if (is_new && !(nrep[rt] < d.n_slot && rep_dom[m] < Bd)) continue;
          int64_t delta = std::min(Uer(e, rb), (L[rb] - L[rt]) / 2);
          if (delta < 1) continue;
          bool better;
          if (!found) better = true;
          else if (delta != bd) better = delta > bd;
          else if (L[rt] != blt) better = L[rt] < blt;
          else if (is_new != bnew) better = is_new < bnew;
          else if (e != be) better = e < be;
          else better = rt < brt;
          if (better) { found = true; bd = delta; blt = L[rt]; bnew = is_new; be = e; brt = rt; }
        }
      }
      if (!found) break;
      if (bnew) { X(be, brt) = 1; nrep[brt] += 1; rep_dom[m] += 1; }
      Uer(be, rb) -= bd; Uer(be, brt) += bd;
      L[rb] -= bd; L[brt] += bd;
      if (trace && ntr < trace_cap) {
        int32_t* rec = trace + 7 * (int64_t)ntr;
        rec[0] = (int32_t)m; rec[1] = (int32_t)it; rec[2] = (int32_t)rb; rec[3] = (int32_t)be;
        rec[4] = (int32_t)brt; rec[5] = (int32_t)bd; rec[6] = (int32_t)bnew;
      }
      ++ntr;
    }
  }
  if (n_trace) *n_trace = ntr;

  // Instance table: rank-major; on each rank its main experts (ascending),
  // then its replicas (ascending expert).
  std::vector<int64_t> inst_of(E * R, -1);
  int64_t n = 0;
  for (int64_t r = 0; r < R; ++r) {
    for (int64_t e = 0; e < E; ++e)
      if (main_of(d, e) == r) inst_of[e * R + r] = n++;
    for (int64_t e = 0; e < E; ++e)
      if (X(e, r) && main_of(d, e) != r) inst_of[e * R + r] = n++;
  }
  if (n > cap) return -5;
  for (int64_t i = 0; i < cap; ++i) { inst_expert[i] = -1; inst_rank[i] = -1; inst_load[i] = -1; }
  for (int64_t e = 0; e < E; ++e)
    for (int64_t r = 0; r < R; ++r)
      if (inst_of[e * R + r] >= 0) {
        int64_t i = inst_of[e * R + r];
        inst_expert[i] = (int32_t)e; inst_rank[i] = (int32_t)r; inst_load[i] = (int32_t)Uer(e, r);
      }
  *n_inst_out = (int32_t)n;
  for (int64_t r = 0; r < R; ++r) rank_load[r] = (int32_t)L[r];

  // Quotas q[s][i]: how many of source s's assignments of expert e run on
  // instance i.  Stage 2 fixes only the instance loads; the quotas are then
  // a transport of the demands omega[s][e] onto the capacities U of e's
  // instances (rank order), filled in three passes so that assignments stay
  // as close to their source as the loads allow: the source's own rank,
  // then its own domain, then anywhere.
  std::fill(quota, quota + R * cap, 0);
  for (int64_t e = 0; e < E; ++e) {
    std::vector<int64_t> insts;
    for (int64_t r = 0; r < R; ++r)
      if (inst_of[e * R + r] >= 0) insts.push_back(inst_of[e * R + r]);
    std::vector<int64_t> dem(R), capi(insts.size());
    for (int64_t s = 0; s < R; ++s) dem[s] = om(s, e);
    for (size_t a = 0; a < insts.size(); ++a) capi[a] = inst_load[insts[a]];
    for (int pass = 0; pass < 3; ++pass)
      for (int64_t s = 0; s < R; ++s)
        for (size_t a = 0; a < insts.size(); ++a) {
          int64_t r = inst_rank[insts[a]];
          bool ok = pass == 0 ? (r == s) : pass == 1 ? (dom_of(c, r) == dom_of(c, s)) : true;
          if (!ok) continue;
          int64_t amt = std::min(dem[s], capi[a]);
          quota[s * cap + insts[a]] += (int32_t)amt;
          dem[s] -= amt; capi[a] -= amt;
        }
    for (int64_t s = 0; s < R; ++s) if (dem[s] != 0) return -5;
    for (size_t a = 0; a < capi.size(); ++a) if (capi[a] != 0) return -5;
  }

  // Instance of every slot (t, j).  Within each (source, expert) pair the
  // slots are taken in token order; the p-th one goes to the first instance
  // (rank order) whose running quota sum exceeds p.
  std::vector<int64_t> seen(E, 0);
  for (int64_t t = 0; t < T; ++t) {
    if (t % d.Tr == 0) std::fill(seen.begin(), seen.end(), 0);
    int64_t s = src_of(d, t);
    for (int64_t j = 0; j < k; ++j) {
      int64_t e = topk_idx[t * k + j];
      int64_t p = seen[e]++;
      int64_t run = 0, chosen = -1;
      for (int64_t r = 0; r < R && chosen < 0; ++r) {
        int64_t i = inst_of[e * R + r];
        if (i < 0) continue;
        run += quota[s * cap + i];
        if (run > p) chosen = i;
      }
      if (chosen < 0) return -5;
      slot_inst[t * k + j] = (int32_t)chosen;
    }
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Dispatch layout and row copy.  TopoEP section 5: the communication manager
// derives receive counts on the GPU from the device-resident routing; here
// the slots are stably sorted by instance (ties in slot order t*k + j), which
// gives each instance a contiguous segment of the dispatch buffer, with
// per-instance and per-rank counts as exclusive prefix sums.
// ---------------------------------------------------------------------------
extern "C" int oracle_dispatch(const oracle_cfg* c, int32_t n_inst, const int32_t* inst_rank,
                               const int32_t* slot_inst, const uint16_t* hidden,
                               int32_t* perm, int32_t* slot_pos, int32_t* inst_offset, int32_t* rank_offset,
                               int32_t* slot_rank, uint16_t* dispatch) {
  if (!valid(c) || !inst_rank || !inst_offset || !rank_offset) return -1;
  const int64_t T = c->T, k = c->k, R = c->R, H = c->H;
  const int64_t cap = c->E + c->B, N = T * k;
  if (n_inst < 0 || n_inst > cap) return -1;
  if (N > 0 && (!slot_inst || !perm || !slot_pos)) return -1;
  for (int64_t q = 0; q < N; ++q)
    if (slot_inst[q] < 0 || slot_inst[q] >= n_inst) return -1;

  std::vector<int32_t> order(N);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return slot_inst[a] < slot_inst[b]; });
  for (int64_t pos = 0; pos < N; ++pos) { perm[pos] = order[pos]; slot_pos[order[pos]] = (int32_t)pos; }

  std::vector<int64_t> icount(n_inst, 0), rcount(R, 0);
  for (int64_t q = 0; q < N; ++q) icount[slot_inst[q]] += 1;
  for (int64_t i = 0; i <= cap; ++i) inst_offset[i] = -1;
  int64_t run = 0;
  for (int64_t i = 0; i < n_inst; ++i) { inst_offset[i] = (int32_t)run; run += icount[i]; }
  inst_offset[n_inst] = (int32_t)run;
  for (int64_t i = 0; i < n_inst; ++i) rcount[inst_rank[i]] += icount[i];
  run = 0;
  for (int64_t r = 0; r < R; ++r) { rank_offset[r] = (int32_t)run; run += rcount[r]; }
  rank_offset[R] = (int32_t)run;
  if (slot_rank)
    for (int64_t q = 0; q < N; ++q) slot_rank[q] = slot_pos[q] - inst_offset[slot_inst[q]];

  if (dispatch && hidden)
    for (int64_t pos = 0; pos < N; ++pos)
      std::memcpy(dispatch + pos * H, hidden + (int64_t)(perm[pos] / k) * H, (size_t)H * sizeof(uint16_t));
  return 0;
}

// Gate-weighted combine -- the return path of the dispatch ([TopoEP] section
// 2.1, Fig. 1: each token's expert outputs come back and are summed).  The
// pages do not define the weights; the reading taken is the softmax of the k
// selected logits, subtracting their maximum before exp.  In double:
//   w[t][j]   = exp(v[t][j] - max_j v[t][j]) / sum_j' exp(v[t][j'] - max)
//   out[t][h] = sum over j = 0..k-1 of w[t][j] * expert_out[slot_pos[t*k+j]][h]
// A non-finite selected logit is a precondition violation (-4).
extern "C" int oracle_combine(const oracle_cfg* c, const float* topk_val, const int32_t* slot_pos,
                              const uint16_t* expert_out, double* out) {
  if (!valid(c)) return -1;
  const int64_t T = c->T, k = c->k, H = c->H, N = T * k;
  if (T > 0 && (!topk_val || !slot_pos || !expert_out || !out)) return -1;
  for (int64_t q = 0; q < N; ++q)
    if (slot_pos[q] < 0 || slot_pos[q] >= N) return -1;
  std::vector<double> w(k);
  for (int64_t t = 0; t < T; ++t) {
    double m = -INFINITY;
    for (int64_t j = 0; j < k; ++j) {
      const double v = topk_val[t * k + j];
      if (!std::isfinite(v)) return -4;
      m = std::max(m, v);
    }
    double s = 0.0;
    for (int64_t j = 0; j < k; ++j) {
      w[j] = std::exp((double)topk_val[t * k + j] - m);
      s += w[j];
    }
    for (int64_t j = 0; j < k; ++j) w[j] /= s;
    for (int64_t h = 0; h < H; ++h) {
      double acc = 0.0;
      for (int64_t j = 0; j < k; ++j) {
        const uint32_t bits = (uint32_t)expert_out[(int64_t)slot_pos[t * k + j] * H + h] << 16;
        float x;
        std::memcpy(&x, &bits, sizeof(x));
        acc += w[j] * (double)x;
      }
      out[t * H + h] = acc;
    }
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Correlated expert placement ([Coupling] "Moving Correlated Experts
// Together"): experts are the nodes of a graph whose edge weights are the
// co-selection counts C[a][b]; the graph is partitioned over the R ranks with
// exactly E/R experts on every rank, keeping heavily co-selected experts on one
// rank.  The page names the goal and the constraint but no algorithm; the
// reading taken here is the objective "co-selection weight inside the ranks"
//   intra = sum over pairs a < b on the same rank of C[a][b]
// (for top-2 routing this is exactly the number of rows a deduplicating
// dispatcher saves), maximised by greedy graph growth followed by pair-swap
// local search:
//   growth: ranks are filled in order 0..R-1.  The first expert of a rank is
//     the unplaced expert with the largest total co-selection deg(e) =
//     sum_x C[e][x]; each further one is the unplaced expert with the largest
//     co-selection with the experts already on the rank.  Ties: lower e.
//   refinement: repeatedly swap the two experts a < b on different ranks whose
//     exchange raises intra the most (ties: lower a, then lower b), while the
//     gain is positive, at most max_swaps times (max_swaps < 0: 4096).
// The gain of exchanging a (rank ra) and b (rank rb), with
// aff[r][x] = sum over y on rank r of C[x][y], is
//   aff[rb][a] - aff[ra][a] + aff[ra][b] - aff[rb][b] - 2 C[a][b].
// cooc must be symmetric with a zero diagonal, entries >= 0, every row sum
// below 2^31 (what oracle_route writes); otherwise -1.
// ---------------------------------------------------------------------------
namespace {

bool cooc_valid(int64_t E, const int32_t* C) {
  for (int64_t a = 0; a < E; ++a) {
    int64_t sum = 0;
    if (C[a * E + a] != 0) return false;
    for (int64_t b = 0; b < E; ++b) {
      if (C[a * E + b] < 0 || C[a * E + b] != C[b * E + a]) return false;
      sum += C[a * E + b];
    }
    if (sum > INT32_MAX) return false;
  }
  return true;
}

}  // namespace

extern "C" int oracle_place(const oracle_cfg* c, const int32_t* cooc, int32_t max_swaps, int32_t* expert_rank,
                            int32_t* rank_experts, int64_t* intra, int32_t* n_swaps) {
  if (!valid(c) || !cooc || !expert_rank || !rank_experts || !intra || !n_swaps) return -1;
  const int64_t E = c->E, R = c->R, Er = E / R;
  if (!cooc_valid(E, cooc)) return -1;
  const int64_t cap = max_swaps < 0 ? 4096 : max_swaps;
  auto C = [&](int64_t a, int64_t b) { return (int64_t)cooc[a * E + b]; };

  std::vector<int64_t> rank(E, -1), deg(E, 0), aff(R * E, 0);
  for (int64_t e = 0; e < E; ++e)
    for (int64_t x = 0; x < E; ++x) deg[e] += C(e, x);

  // Greedy growth, one rank after the other.
  for (int64_t r = 0; r < R; ++r) {
    for (int64_t m = 0; m < Er; ++m) {
      int64_t pick = -1, best = -1;
      for (int64_t e = 0; e < E; ++e) {
        if (rank[e] >= 0) continue;
        const int64_t score = m == 0 ? deg[e] : aff[r * E + e];
        if (score > best) { best = score; pick = e; }
      }
      rank[pick] = r;
      for (int64_t x = 0; x < E; ++x) aff[r * E + x] += C(x, pick);
    }
  }

  // Pair-swap refinement.
  int64_t swaps = 0;
  while (swaps < cap) {
    int64_t ba = -1, bb = -1, bg = 0;
    for (int64_t a = 0; a < E; ++a)
      for (int64_t b = a + 1; b < E; ++b) {
        const int64_t ra = rank[a], rb = rank[b];
        if (ra == rb) continue;
        const int64_t g = aff[rb * E + a] - aff[ra * E + a] + aff[ra * E + b] - aff[rb * E + b] - 2 * C(a, b);
        if (g > bg) { bg = g; ba = a; bb = b; }
      }
    if (ba < 0) break;
    const int64_t ra = rank[ba], rb = rank[bb];
    for (int64_t x = 0; x < E; ++x) {
      aff[ra * E + x] += C(x, bb) - C(x, ba);
      aff[rb * E + x] += C(x, ba) - C(x, bb);
    }
    rank[ba] = rb;
    rank[bb] = ra;
    ++swaps;
  }

  int64_t w = 0;
  for (int64_t a = 0; a < E; ++a)
    for (int64_t b = a + 1; b < E; ++b)
      if (rank[a] == rank[b]) w += C(a, b);
  std::vector<int64_t> fill(R, 0);
  for (int64_t e = 0; e < E; ++e) {
    expert_rank[e] = (int32_t)rank[e];
    rank_experts[rank[e] * Er + fill[rank[e]]++] = (int32_t)e;  // e ascending within each rank
  }
  *intra = w;
  *n_swaps = (int32_t)swaps;
  return 0;
}

// ---------------------------------------------------------------------------
// Deduplicated dispatch ([Coupling] "Moving Correlated Experts Together",
// Fig. 3): a token whose selected experts share a destination rank is sent
// there once, with the list of its slots that rank serves.  The rank of slot
// q = t*k+j is key_rank[slot_key[q]] -- slot_key holds top-k expert ids with
// key_rank a placement (expert -> rank), or instance ids with the planner's
// instance ranks; key_rank = NULL means the contiguous placement
// slot_key[q] / (E/R).  Token t comes from source rank t / (T/R).
//   tok_ranks[t]     distinct destination ranks of token t
//   rank_rows[s][r]  rows sent from source s to rank r: tokens of s with at
//                    least one slot on r (the deduplicated count)
//   rank_slots[s][r] slots of source s on rank r (one row each without
//                    deduplication); nullable
// Keys outside [0, n_keys) (or [0, E) without a table) and table entries
// outside [0, R) are -1.
// ---------------------------------------------------------------------------
namespace {

int slot_ranks(const oracle_cfg* c, const int32_t* slot_key, const int32_t* key_rank, int32_t n_keys,
               std::vector<int64_t>& rank) {
  const int64_t N = (int64_t)c->T * c->k, Er = c->E / c->R;
  rank.assign(N, 0);
  for (int64_t q = 0; q < N; ++q) {
    const int64_t key = slot_key[q];
    if (key_rank) {
      if (key < 0 || key >= n_keys) return -1;
      rank[q] = key_rank[key];
    } else {
      if (key < 0 || key >= c->E) return -1;
      rank[q] = key / Er;
    }
    if (rank[q] < 0 || rank[q] >= c->R) return -1;
  }
  return 0;
}

}  // namespace

extern "C" int oracle_dedup(const oracle_cfg* c, const int32_t* slot_key, const int32_t* key_rank, int32_t n_keys,
                            int32_t* tok_ranks, int32_t* rank_rows, int32_t* rank_slots) {
  if (!valid(c) || !tok_ranks || !rank_rows) return -1;
  const int64_t T = c->T, k = c->k, R = c->R, Tr = T / R;
  if (T > 0 && !slot_key) return -1;
  std::vector<int64_t> rank;
  if (slot_ranks(c, slot_key, key_rank, n_keys, rank) != 0) return -1;
  for (int64_t i = 0; i < R * R; ++i) {
    rank_rows[i] = 0;
    if (rank_slots) rank_slots[i] = 0;
  }
  for (int64_t t = 0; t < T; ++t) {
    const int64_t s = t / Tr;
    int64_t distinct = 0;
    for (int64_t j = 0; j < k; ++j) {
      const int64_t r = rank[t * k + j];
      if (rank_slots) rank_slots[s * R + r] += 1;
      bool seen = false;
      for (int64_t i = 0; i < j; ++i) seen = seen || rank[t * k + i] == r;
      if (!seen) {
        ++distinct;
        rank_rows[s * R + r] += 1;
      }
    }
    tok_ranks[t] = (int32_t)distinct;
  }
  return 0;
}

// The deduplicated dispatch layout and row copy: one row per (destination
// rank, token) pair that has at least one slot, ordered by rank, then token.
//   n_rows[0]          number of rows (the sum of tok_ranks)
//   row_token[p]       token of row p
//   row_slots[p]       bit j set when slot j of that token goes to that rank
//   rank_row_offset[r] first row of rank r; entry R is n_rows
//   slot_row[q]        row carrying slot q
//   ddispatch[p][:]    = hidden[row_token[p]][:] (nullable)
// Capacity T*k rows; entries from n_rows on are -1 (ddispatch rows untouched).
extern "C" int oracle_dedup_dispatch(const oracle_cfg* c, const int32_t* slot_key, const int32_t* key_rank,
                                     int32_t n_keys, const uint16_t* hidden, int32_t* n_rows, int32_t* row_token,
                                     int32_t* row_slots, int32_t* rank_row_offset, int32_t* slot_row,
                                     uint16_t* ddispatch) {
  if (!valid(c) || !n_rows || !row_token || !row_slots || !rank_row_offset || !slot_row) return -1;
  const int64_t T = c->T, k = c->k, R = c->R, H = c->H, N = T * k;
  if (k > 32 || (T > 0 && !slot_key)) return -1;
  std::vector<int64_t> rank;
  if (slot_ranks(c, slot_key, key_rank, n_keys, rank) != 0) return -1;
  int64_t p = 0;
  for (int64_t r = 0; r < R; ++r) {
    rank_row_offset[r] = (int32_t)p;
    for (int64_t t = 0; t < T; ++t) {
      uint32_t mask = 0;
      for (int64_t j = 0; j < k; ++j)
        if (rank[t * k + j] == r) mask |= 1u << j;
      if (mask == 0) continue;
      row_token[p] = (int32_t)t;
      row_slots[p] = (int32_t)mask;
      for (int64_t j = 0; j < k; ++j)
        if (mask >> j & 1u) slot_row[t * k + j] = (int32_t)p;
      if (ddispatch && hidden) std::memcpy(ddispatch + p * H, hidden + t * H, (size_t)H * sizeof(uint16_t));
      ++p;
    }
  }
  rank_row_offset[R] = (int32_t)p;
  *n_rows = (int32_t)p;
  for (int64_t q = p; q < N; ++q) row_token[q] = row_slots[q] = -1;
  return 0;
}

// ---------------------------------------------------------------------------
// Plan quality ([TopoEP] section 6.2 Fig. 10 and section 6.4 Fig. 13(b): the
// rank-load imbalance, the largest per-rank token-expert load over the mean;
// section 6.6 Fig. 16: the share of assignments executed on another node than
// their source, and the share executed by replicas).  From a plan:
//   out[0] assignments             sum of q[s][i]
//   out[1] same rank               sum of q[s][i] with rank(i) = s
//   out[2] same node               sum of q[s][i] with dom(rank(i)) = dom(s)
//   out[3] other node              out[0] - out[2]
//   out[4] served by replicas      sum of q[s][i] with rank(i) != main(expert(i))
//   out[5] largest rank load       max_r rank_load[r]
//   out[6] smallest rank load      min_r rank_load[r]
//   out[7] replicas                n_inst - E
// The imbalance of Fig. 10 is out[5] * R / out[0].
// ---------------------------------------------------------------------------
extern "C" int oracle_quality(const oracle_cfg* c, int32_t n_inst, const int32_t* inst_expert,
                              const int32_t* inst_rank, const int32_t* rank_load, const int32_t* quota,
                              int64_t* out) {
  if (!valid(c) || !inst_expert || !inst_rank || !rank_load || !quota || !out) return -1;
  const Derived d = derive(c);
  const int64_t R = c->R, cap = (int64_t)c->E + c->B;
  if (n_inst < c->E || n_inst > cap) return -1;
  for (int k = 0; k < 8; ++k) out[k] = 0;
  for (int64_t s = 0; s < R; ++s)
    for (int64_t i = 0; i < n_inst; ++i) {
      const int64_t q = quota[s * cap + i], r = inst_rank[i], e = inst_expert[i];
      if (r < 0 || r >= R || e < 0 || e >= c->E) return -1;
      out[0] += q;
      if (r == s) out[1] += q;
      if (dom_of(c, r) == dom_of(c, s)) out[2] += q;
      if (r != main_of(d, e)) out[4] += q;
    }
  out[3] = out[0] - out[2];
  out[5] = rank_load[0];
  out[6] = rank_load[0];
  for (int64_t r = 1; r < R; ++r) {
    out[5] = std::max<int64_t>(out[5], rank_load[r]);
    out[6] = std::min<int64_t>(out[6], rank_load[r]);
  }
  out[7] = n_inst - c->E;
  return 0;
}

// ---------------------------------------------------------------------------
// Token-shuffle prediction ([Coupling] "Moving Tokens Toward Their Next
// Experts": a token's experts at this layer predict which GPU holds most of
// its next-layer experts; the token is moved there before the next router).
// The page gives no formula; the reading taken is that each of the token's
// experts a votes with its empirical next-layer distribution:
//   P[a][r]   = (sum over experts b on rank r of X[a][b]) / count[a]
//               (X: this layer -> next layer transition counts, count[a]:
//               this layer's assignments of a; 0 when count[a] = 0)
//   score[r]  = P[a_0][r] + P[a_1][r] + ... + P[a_{k-1}][r]   (slot order)
//   pred[t]   = argmax_r score[r], ties to the lower rank
// score[r] / k is the expected share of the token's next-layer experts on r.
// All of it in IEEE double, in this order.  The rank of b is key_rank[b]
// (NULL: contiguous b / (E/R)).  With topk_next given, local[0] counts the
// next layer's slots on the predicted rank and local[1] those on the token's
// own source rank t / (T/R) (no shuffling).  rank_tokens[r]: tokens predicted
// for rank r.
// ---------------------------------------------------------------------------
extern "C" int oracle_predict(const oracle_cfg* c, const int32_t* topk_cur, const int32_t* trans,
                              const int32_t* count_cur, const int32_t* key_rank, const int32_t* topk_next,
                              int32_t* pred, int32_t* rank_tokens, int64_t* local) {
  if (!valid(c) || !trans || !count_cur || !pred || !rank_tokens) return -1;
  const int64_t T = c->T, E = c->E, k = c->k, R = c->R, Tr = T / R, Er = E / R;
  if (T > 0 && !topk_cur) return -1;
  std::vector<int64_t> rank_of(E);
  for (int64_t b = 0; b < E; ++b) {
    rank_of[b] = key_rank ? key_rank[b] : b / Er;
    if (rank_of[b] < 0 || rank_of[b] >= R) return -1;
  }
  std::vector<double> P(E * R, 0.0);
  for (int64_t a = 0; a < E; ++a) {
    if (count_cur[a] < 0) return -1;
    std::vector<int64_t> n(R, 0);
    for (int64_t b = 0; b < E; ++b) n[rank_of[b]] += trans[a * E + b];
    for (int64_t r = 0; r < R; ++r) P[a * R + r] = count_cur[a] > 0 ? (double)n[r] / (double)count_cur[a] : 0.0;
  }
  for (int64_t r = 0; r < R; ++r) rank_tokens[r] = 0;
  if (local) local[0] = local[1] = 0;
  std::vector<double> score(R);
  for (int64_t t = 0; t < T; ++t) {
    std::fill(score.begin(), score.end(), 0.0);
    for (int64_t j = 0; j < k; ++j) {
      const int64_t a = topk_cur[t * k + j];
      if (a < 0 || a >= E) return -1;
      for (int64_t r = 0; r < R; ++r) score[r] += P[a * R + r];
    }
    int64_t best = 0;
    for (int64_t r = 1; r < R; ++r)
      if (score[r] > score[best]) best = r;
    pred[t] = (int32_t)best;
    rank_tokens[best] += 1;
    if (local && topk_next)
      for (int64_t j = 0; j < k; ++j) {
        const int64_t b = topk_next[t * k + j];
        if (b < 0 || b >= E) return -1;
        if (rank_of[b] == best) local[0] += 1;
        if (rank_of[b] == t / Tr) local[1] += 1;
      }
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Replica slots ([TopoEP] section 3.2, Replica Buffer Management, and Fig. 6:
// every rank keeps N_slot replica slots; the plan maps each occupied slot to
// an expert and so to its main rank, the source of the BF16 parameters pulled
// in the forward pass and the destination of the gradients returned in the
// backward pass; the main instance keeps the optimizer state).  Reading: the
// replicas of rank r, in instance order (ascending expert), fill its slots
// 0, 1, ...; the remaining slots are empty (-1).
//   slot_expert [R][N_slot], slot_main [R][N_slot] = main(expert), inst_slot [E+B]
//   (the slot of each replica instance; -1 for main and unused instances).
// Parameter pull: replica_params[r][j][:] = main_params[slot_expert[r][j]][:]
// (main_params [E][P]: rank m owns rows m*E/R ... (m+1)*E/R - 1).
// Gradient return: grad_accum[m][r][e - m*E/R][:] = replica_grads[r][j][:]
// for the expert e in slot j of rank r and m = main(e) -- the main rank's
// buffer split by source rank.  Empty slots move nothing.
// ---------------------------------------------------------------------------
extern "C" int oracle_slot_map(const oracle_cfg* c, int32_t n_inst, const int32_t* inst_expert,
                               const int32_t* inst_rank, int32_t* slot_expert, int32_t* slot_main, int32_t* inst_slot) {
  if (!valid(c) || !inst_expert || !inst_rank || !slot_expert || !slot_main || !inst_slot) return -1;
  const Derived d = derive(c);
  const int64_t R = c->R, cap = (int64_t)c->E + c->B, ns = d.n_slot;
  if (n_inst < c->E || n_inst > cap) return -1;
  for (int64_t q = 0; q < R * ns; ++q) slot_expert[q] = slot_main[q] = -1;
  for (int64_t i = 0; i < cap; ++i) inst_slot[i] = -1;
  std::vector<int64_t> used(R, 0);
  for (int64_t i = 0; i < n_inst; ++i) {  // instances are rank-major
    const int64_t r = inst_rank[i], e = inst_expert[i];
    if (r < 0 || r >= R || e < 0 || e >= c->E) return -1;
    if (main_of(d, e) == r) continue;
    if (used[r] >= ns) return -5;
    slot_expert[r * ns + used[r]] = (int32_t)e;
    slot_main[r * ns + used[r]] = (int32_t)main_of(d, e);
    inst_slot[i] = (int32_t)used[r];
    ++used[r];
  }
  return 0;
}

extern "C" int oracle_replica_pull(const oracle_cfg* c, const int32_t* slot_expert, const uint16_t* main_params,
                                   int64_t P, uint16_t* replica_params) {
  if (!valid(c) || !slot_expert || !main_params || !replica_params || P < 0) return -1;
  const Derived d = derive(c);
  for (int64_t q = 0; q < (int64_t)c->R * d.n_slot; ++q) {
    const int64_t e = slot_expert[q];
    if (e < 0) continue;
    if (e >= c->E) return -1;
    std::memcpy(replica_params + q * P, main_params + e * P, (size_t)P * sizeof(uint16_t));
  }
  return 0;
}

extern "C" int oracle_replica_push(const oracle_cfg* c, const int32_t* slot_expert, const uint16_t* replica_grads,
                                   int64_t P, uint16_t* grad_accum) {
  if (!valid(c) || !slot_expert || !replica_grads || !grad_accum || P < 0) return -1;
  const Derived d = derive(c);
  const int64_t R = c->R, ns = d.n_slot, Er = d.Er;
  for (int64_t r = 0; r < R; ++r)
    for (int64_t j = 0; j < ns; ++j) {
      const int64_t e = slot_expert[r * ns + j];
      if (e < 0) continue;
      if (e >= c->E) return -1;
      const int64_t m = main_of(d, e);
      std::memcpy(grad_accum + ((m * R + r) * Er + (e - m * Er)) * P, replica_grads + (r * ns + j) * P,
                  (size_t)P * sizeof(uint16_t));
    }
  return 0;
}
