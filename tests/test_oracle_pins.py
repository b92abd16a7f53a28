"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these checks re-types the oracle's own arithmetic: they use brute
force (counting ranks, one-hot matrix products, subset enumeration), the
worked examples on the pages (tests/golden/), closed forms and invariants
(TopoEP constraints C1-C5 of section 4.2, the refinement properties of
section 4.3).
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from tests import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def cfg_from(d, **over):
    d = dict(d)
    d.update(over)
    return oracle.make_cfg(d["T"], d["E"], d["k"], d["R"], d["G"], d["H"], d["B"], d.get("n_slot", 0),
                           d.get("W", -1), d.get("S", 0), d.get("max_iters", 0))


# ---------------------------------------------------------------------------
# Top-k gating
# ---------------------------------------------------------------------------

def brute_topk(row: np.ndarray, k: int) -> list:
    """Rank of e = number of experts that beat it (larger value, or equal value and lower index)."""
    E = len(row)
    v = row.astype(np.float64)  # -0.0 == +0.0 in float comparison
    rank = [sum(1 for f in range(E) if v[f] > v[e] or (v[f] == v[e] and f < e)) for e in range(E)]
    inv = [None] * E
    for e, r in enumerate(rank):
        inv[r] = e
    return inv[:k]


@pytest.mark.parametrize("ties", [False, True])
def test_topk_matches_counting_ranks(ties):
    T, E, k, R = 48, 12, 5, 4
    logits = inputs.random_logits(11 + ties, T, E, ties=ties)
    logits[0, :] = np.float32(0.5)
    logits[1, 3], logits[1, 7] = np.float32(np.inf), np.float32(-np.inf)
    logits[2, :] = np.float32(-0.0)
    logits[2, ::3] = np.float32(0.0)
    cfg = oracle.make_cfg(T, E, k, R, 2, 8, 0)
    out = oracle.route(cfg, logits)
    assert out["status"] == 0
    for t in range(T):
        assert list(out["topk_idx"][t]) == brute_topk(logits[t], k), t
        np.testing.assert_array_equal(out["topk_val"][t].view(np.uint32),
                                      logits[t, out["topk_idx"][t]].view(np.uint32))


def test_topk_closed_forms():
    T, E, R = 16, 8, 2
    # all logits equal: the lowest k indices, in order
    cfg = oracle.make_cfg(T, E, 3, R, 1, 8, 0)
    out = oracle.route(cfg, np.full((T, E), 1.25, np.float32))
    assert (out["topk_idx"] == np.arange(3)).all()
    # k = E: a full permutation sorted by descending logit
    cfg = oracle.make_cfg(T, E, E, R, 1, 8, 0)
    lg = inputs.random_logits(3, T, E)
    out = oracle.route(cfg, lg)
    for t in range(T):
        assert sorted(out["topk_idx"][t]) == list(range(E))
        assert (np.diff(lg[t, out["topk_idx"][t]]) <= 0).all()


def test_topk_nan_is_an_error():
    cfg = oracle.make_cfg(8, 4, 2, 2, 1, 8, 0)
    lg = np.zeros((8, 4), np.float32)
    lg[5, 2] = np.nan
    assert oracle.route(cfg, lg)["status"] == -4


# ---------------------------------------------------------------------------
# Histograms: routing matrix, co-selection, transitions
# ---------------------------------------------------------------------------

def onehot(topk: np.ndarray, E: int) -> np.ndarray:
    T = topk.shape[0]
    Y = np.zeros((T, E), np.int64)
    for t in range(T):
        Y[t, topk[t]] = 1
    return Y


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_histograms_match_onehot_products(seed):
    T, E, k, R = 120, 12, 4, 4
    lg = inputs.random_logits(seed, T, E, ties=(seed == 2))
    prev = inputs.random_topk(seed + 50, T, E, k)
    cfg = oracle.make_cfg(T, E, k, R, 2, 8, 0)
    out = oracle.route(cfg, lg, prev_topk=prev)
    Y = onehot(out["topk_idx"], E)
    Yp = onehot(prev, E)
    Tr = T // R
    omega = np.stack([Y[s * Tr:(s + 1) * Tr].sum(0) for s in range(R)])
    np.testing.assert_array_equal(out["omega"], omega)
    np.testing.assert_array_equal(out["count"], Y.sum(0))
    C = Y.T @ Y
    np.fill_diagonal(C, 0)
    np.testing.assert_array_equal(out["cooc"], C)
    np.testing.assert_array_equal(out["trans"], Yp.T @ Y)
    # invariants named in the build contract
    assert out["count"].sum() == T * k
    assert (out["omega"].sum(1) == Tr * k).all()
    assert (out["cooc"] == out["cooc"].T).all() and (np.diag(out["cooc"]) == 0).all()
    np.testing.assert_array_equal(out["cooc"].sum(1), out["count"] * (k - 1))
    np.testing.assert_array_equal(out["trans"].sum(1), Yp.sum(0) * k)
    np.testing.assert_array_equal(out["trans"].sum(0), out["count"] * k)
    assert out["trans"].sum() == T * k * k


# ---------------------------------------------------------------------------
# Worked examples of the pages
# ---------------------------------------------------------------------------

def run_plan_from_omega(cfgd, omega, topk=None, trace_cap=256, **over):
    cfg = cfg_from(cfgd, **over)
    T, k = cfg.T, cfg.k
    topk = np.zeros((T, k), np.int32) if topk is None else np.asarray(topk, np.int32).reshape(T, k)
    return cfg, oracle.plan(cfg, np.asarray(omega, np.int32), topk, trace_cap=trace_cap)


def moves(plan):
    return [dict(domain=int(r[0]), r_busy=int(r[2]), expert=int(r[3]), r_target=int(r[4]), delta=int(r[5]),
                 new_replica=int(r[6])) for r in plan["trace"]]


def quota_nonzero(plan):
    q = plan["quota"]
    return [[int(s), int(i), int(q[s, i])] for s, i in zip(*np.nonzero(q))]


def test_fig9_two_stage_example():
    g = json.load(open(os.path.join(GOLDEN, "fig9_example.json")))
    cfg, p = run_plan_from_omega(g["config"], g["omega"])
    ex = g["expected"]
    assert list(p["rank_load_stage1"]) == ex["rank_load_stage1"]
    assert list(p["rank_load"]) == ex["rank_load"]
    assert moves(p) == ex["refinement_moves"]
    assert int(p["n_inst"][0]) == ex["n_inst"]
    assert list(p["inst_expert"]) == ex["inst_expert"]
    assert list(p["inst_rank"]) == ex["inst_rank"]
    assert list(p["inst_load"]) == ex["inst_load"]
    assert quota_nonzero(p) == ex["quota_nonzero"]
    G = cfg.G
    cross = sum(int(p["quota"][s, i]) for s in range(cfg.R) for i in range(int(p["n_inst"][0]))
                if s // G != p["inst_rank"][i] // G)
    assert cross == ex["cross_domain_assignments"]
    for v in g["variants"]:
        cfg2, p2 = run_plan_from_omega(g["config"], g["omega"], **v["override"])
        assert list(p2["rank_load_stage1"]) == v["rank_load_stage1"], v["what"]
        assert list(p2["rank_load"]) == v["rank_load"], v["what"]
        assert moves(p2) == v["refinement_moves"], v["what"]


def test_even_split_example():
    g = json.load(open(os.path.join(GOLDEN, "even_split_example.json")))
    c = g["config"]
    cfg = cfg_from(c)
    topk = np.asarray(g["topk"], np.int32).reshape(c["T"], c["k"])
    lg = np.zeros((c["T"], c["E"]), np.float32)
    lg[np.arange(c["T"]), topk[:, 0]] = 1.0
    r = oracle.route(cfg, lg)
    ex = g["expected"]
    np.testing.assert_array_equal(r["topk_idx"], topk)
    assert r["omega"].tolist() == ex["omega"]
    p = oracle.plan(cfg, r["omega"], r["topk_idx"], trace_cap=16)
    assert list(p["rank_load_stage1"]) == ex["rank_load_stage1"]
    assert list(p["rank_load"]) == ex["rank_load"]
    assert int(p["n_inst"][0]) == ex["n_inst"]
    assert list(p["inst_expert"]) == ex["inst_expert"]
    assert list(p["inst_rank"]) == ex["inst_rank"]
    assert list(p["inst_load"]) == ex["inst_load"]
    assert quota_nonzero(p) == ex["quota_nonzero"]
    assert list(p["slot_inst"]) == ex["slot_inst"]
    d = oracle.dispatch(cfg, int(p["n_inst"][0]), p["inst_rank"], p["slot_inst"], None)
    assert list(d["inst_offset"]) == ex["inst_offset"]
    assert list(d["rank_offset"]) == ex["rank_offset"]


def check_golden_plan(cfg, p, ex):
    assert oracle.params(cfg)["n_slot"] == ex["n_slot"]
    assert list(p["rank_load_stage1"]) == ex["rank_load_stage1"]
    assert list(p["rank_load"]) == ex["rank_load"]
    assert moves(p) == ex["refinement_moves"]
    assert int(p["n_inst"][0]) == ex["n_inst"]
    assert list(p["inst_expert"]) == ex["inst_expert"]
    assert list(p["inst_rank"]) == ex["inst_rank"]
    assert list(p["inst_load"]) == ex["inst_load"]
    assert quota_nonzero(p) == ex["quota_nonzero"]


def test_stage1_spread_example():
    """TopoEP section 4.3: inter-node replicas go to the least occupied rank with a free slot.
    With two slots per rank, three replicas of one domain spread over its two ranks (hand-derived)."""
    g = json.load(open(os.path.join(GOLDEN, "stage1_spread_example.json")))
    cfg, p = run_plan_from_omega(g["config"], g["omega"])
    ex = g["expected"]
    check_golden_plan(cfg, p, ex)
    assert [list(x) for x in sorted(stage1_replicas(cfg, p))] == ex["stage1_replicas"]
    for v in g["variants"]:
        cfg2, p2 = run_plan_from_omega(g["config"], g["omega"], **v["override"])
        assert [list(x) for x in sorted(stage1_replicas(cfg2, p2))] == v["stage1_replicas"], v["what"]
        assert list(p2["rank_load_stage1"]) == v["rank_load_stage1"], v["what"]
        assert list(p2["rank_load"]) == v["rank_load"], v["what"]
        assert moves(p2) == v["refinement_moves"], v["what"]


def test_quota_order_example():
    """Quota transport (the reading of TopoEP section 4.3's routing): two sources of a domain
    compete for residual capacity on two instances in the same-domain pass, and two sources of
    another domain for two instances in the cross-domain pass (hand-derived)."""
    g = json.load(open(os.path.join(GOLDEN, "quota_order_example.json")))
    cfg, p = run_plan_from_omega(g["config"], g["omega"])
    ex = g["expected"]
    check_golden_plan(cfg, p, ex)
    G = cfg.G
    cross = sum(int(p["quota"][s, i]) for s in range(cfg.R) for i in range(int(p["n_inst"][0]))
                if s // G != p["inst_rank"][i] // G)
    assert cross == ex["cross_domain_assignments"]
    check_quota_passes(cfg, {"omega": np.asarray(g["omega"], np.int32)}, p)


def test_fig3_traffic_arithmetic_and_benefit_sign():
    """TopoEP section 2.3, Fig. 3: N = 4096 tokens of 2,048-wide bf16 activations, 9 MiB of
    parameters per expert; 64 MiB of token traffic versus 18 MiB + 9 MiB (about 2.4x).
    Eq. 9 must then favour the replica (b > 0); the break-even demand is 9H/16 tokens."""
    H = 2048
    cfg = oracle.make_cfg(0, 2, 1, 2, 1, H, 1)
    prm = oracle.params(cfg)
    MiB = 1 << 20
    assert prm["S"] == 2 * H and prm["W"] == 9 * MiB
    N = 4096
    token_traffic = 4 * N * prm["S"]          # dispatch + combine, forward + backward
    replica_traffic = 2 * prm["W"] + prm["W"]  # two parameter fetches + one gradient
    assert token_traffic == 64 * MiB and replica_traffic == 27 * MiB
    assert round(token_traffic / replica_traffic, 1) == 2.4
    # two single-rank domains, expert 1 lives on rank 1; rank 0 sends D assignments to it
    for D, placed in [(4096, True), (1153, True), (1152, False), (0, False)]:
        omega = np.array([[0, D], [0, 0]], np.int32)
        p = oracle.plan(cfg, omega, np.zeros((0, 1), np.int32))
        has_replica = int(p["n_inst"][0]) == 3
        assert has_replica == placed, D
        if placed:
            assert list(p["inst_expert"][:2]) == [0, 1] and p["inst_rank"][1] == 0


# ---------------------------------------------------------------------------
# Plan properties on random small layers
# ---------------------------------------------------------------------------

def random_case(cfgd, seed):
    cfg = cfg_from(cfgd)
    topk = inputs.random_topk(seed, cfg.T, cfg.E, cfg.k, skew=1.5)
    lg = np.zeros((cfg.T, cfg.E), np.float32)
    for j in range(cfg.k):
        lg[np.arange(cfg.T), topk[:, j]] = np.float32(cfg.k - j)
    r = oracle.route(cfg, lg)
    np.testing.assert_array_equal(r["topk_idx"], topk)
    p = oracle.plan(cfg, r["omega"], r["topk_idx"], trace_cap=100000)
    return cfg, r, p


def placement(cfg, p):
    n = int(p["n_inst"][0])
    return {(int(p["inst_expert"][i]), int(p["inst_rank"][i])) for i in range(n)}


def check_plan_invariants(cfg, r, p):
    prm = oracle.params(cfg)
    T, E, k, R, G = cfg.T, cfg.E, cfg.k, cfg.R, cfg.G
    M, Er = prm["M"], prm["Er"]
    n = int(p["n_inst"][0])
    X = placement(cfg, p)
    omega = r["omega"].astype(np.int64)
    D = np.stack([omega[m * G:(m + 1) * G].sum(0) for m in range(M)])
    # C5: every expert keeps its main instance
    for e in range(E):
        assert (e, e // Er) in X
    reps = [(e, rr) for (e, rr) in X if rr != e // Er]
    assert n == E + len(reps)
    # C3: replicas per rank; per-domain budget
    for rr in range(R):
        assert sum(1 for (_, x) in reps if x == rr) <= prm["n_slot"]
    for m in range(M):
        assert sum(1 for (_, x) in reps if x // G == m) <= prm["Bd"][m]
    # C4: a cross-domain replica only where one parameter transfer beats the exposed token bytes
    for (e, rr) in reps:
        if rr // G != (e // Er) // G:
            assert prm["W"] < 2 * D[rr // G, e] * prm["S"]
    # instance table order: rank-major, mains then replicas, experts ascending
    keys = [(int(p["inst_rank"][i]), int(p["inst_expert"][i]) // Er != int(p["inst_rank"][i]),
             int(p["inst_expert"][i])) for i in range(n)]
    assert keys == sorted(keys)
    assert (p["inst_expert"][n:] == -1).all() and (p["inst_load"][n:] == -1).all()
    q = p["quota"].astype(np.int64)
    assert (q[:, n:] == 0).all()
    # C1 conservation and C2 reachability through the quotas
    for e in range(E):
        cols = [i for i in range(n) if p["inst_expert"][i] == e]
        np.testing.assert_array_equal(q[:, cols].sum(1), omega[:, e])
    np.testing.assert_array_equal(q[:, :n].sum(0), p["inst_load"][:n])
    assert (p["inst_load"][:n] >= 0).all()
    # rank load is the sum of its instance loads; total is T*k
    L = np.zeros(R, np.int64)
    for i in range(n):
        L[p["inst_rank"][i]] += p["inst_load"][i]
    np.testing.assert_array_equal(L, p["rank_load"])
    assert L.sum() == T * k
    assert L.max(initial=0) >= math.ceil(T * k / R)
    assert p["rank_load"].max(initial=0) <= p["rank_load_stage1"].max(initial=0)
    # every slot runs on an instance of its own expert; per (source, instance) counts are the quotas
    si = p["slot_inst"].reshape(T, k)
    assert (p["inst_expert"][si] == r["topk_idx"]).all()
    Tr = T // R if R else 0
    cnt = np.zeros_like(q)
    for t in range(T):
        for j in range(k):
            cnt[t // Tr, si[t, j]] += 1
    np.testing.assert_array_equal(cnt, q)
    # within a (source, expert) pair the instance index never decreases along the tokens
    for s in range(R):
        for e in range(E):
            seq = [si[t, j] for t in range(s * Tr, (s + 1) * Tr) for j in range(k) if r["topk_idx"][t, j] == e]
            assert seq == sorted(seq)


def check_quota_locality(cfg, r, p):
    """Same-rank flow is the largest possible and cross-domain flow the smallest possible."""
    G, R = cfg.G, cfg.R
    n = int(p["n_inst"][0])
    q = p["quota"].astype(np.int64)
    omega = r["omega"].astype(np.int64)
    for e in range(cfg.E):
        cols = [i for i in range(n) if p["inst_expert"][i] == e]
        U = {int(p["inst_rank"][i]): int(p["inst_load"][i]) for i in cols}
        same = sum(int(q[int(p["inst_rank"][i]), i]) for i in cols)
        assert same == sum(min(int(omega[s, e]), U.get(s, 0)) for s in range(R))
        cross = sum(int(q[s, i]) for s in range(R) for i in cols if s // G != p["inst_rank"][i] // G)
        want = 0
        for m in range(R // G):
            dem = int(omega[m * G:(m + 1) * G, e].sum())
            cap = sum(u for rr, u in U.items() if rr // G == m)
            want += max(0, dem - cap)
        assert cross == want


def comonotone_ok(F, dem, cap) -> bool:
    """F is the north-west-corner (comonotone) coupling of dem and cap in the given orders: the flow
    from the first a sources to the first b sinks is min(sum of their demands, sum of their capacities)."""
    F = np.asarray(F, np.int64)
    if F.size == 0:
        return True
    want = np.minimum.outer(np.cumsum(dem), np.cumsum(cap))
    return bool((F >= 0).all() and np.array_equal(F.cumsum(0).cumsum(1), want))


def check_quota_passes(cfg, r, p):
    """The quota reading, pass by pass, from the final quota matrix alone.  Flows on the source's own
    rank are pass A; other flows inside a domain pass B; flows across domains pass C (a pass cannot
    add to a pair whose demand or capacity an earlier pass emptied).  Pass A takes min(demand,
    load) on the source's own rank; passes B (per domain) and C (all) are the comonotone couplings
    of the residual demands, sources ascending, with the residual loads, instances in rank order."""
    G, R = cfg.G, cfg.R
    M = R // G
    n = int(p["n_inst"][0])
    q = p["quota"].astype(np.int64)
    omega = np.asarray(r["omega"]).astype(np.int64)
    for e in range(cfg.E):
        cols = [i for i in range(n) if p["inst_expert"][i] == e]
        ranks = [int(p["inst_rank"][i]) for i in cols]
        assert ranks == sorted(ranks)
        dem = omega[:, e].copy()
        cap = np.array([int(p["inst_load"][i]) for i in cols], np.int64)
        for a, rr in enumerate(ranks):  # pass A
            f = int(q[rr, cols[a]])
            assert f == min(dem[rr], cap[a])
            dem[rr] -= f
            cap[a] -= f
        for m in range(M):  # pass B, domain by domain
            S = list(range(m * G, (m + 1) * G))
            A = [a for a in range(len(cols)) if ranks[a] // G == m]
            F = np.array([[0 if s == ranks[a] else int(q[s, cols[a]]) for a in A] for s in S], np.int64)
            assert comonotone_ok(F, dem[S], cap[A]), (e, m)
            dem[S] -= F.sum(1)
            cap[A] -= F.sum(0)
        F = np.array([[int(q[s, cols[a]]) if s // G != ranks[a] // G else 0 for a in range(len(cols))]
                      for s in range(R)], np.int64)  # pass C
        assert comonotone_ok(F, dem, cap), e
        assert (dem - F.sum(1) == 0).all() and (cap - F.sum(0) == 0).all()


def replay_refinement(cfg, r, p):
    """Undo the recorded refinement moves from the final state, then replay them forward and
    check each against a brute-force enumeration of the candidates of Eq. 10."""
    prm = oracle.params(cfg)
    E, R, G, M, Er = cfg.E, cfg.R, cfg.G, prm["M"], prm["Er"]
    n = int(p["n_inst"][0])
    U = np.zeros((E, R), np.int64)
    X = np.zeros((E, R), bool)
    for i in range(n):
        U[p["inst_expert"][i], p["inst_rank"][i]] = p["inst_load"][i]
        X[p["inst_expert"][i], p["inst_rank"][i]] = True
    L = p["rank_load"].astype(np.int64).copy()
    tr = p["trace"]
    assert len(tr) == p["n_iters"]
    for rec in tr[::-1]:
        m, it, rb, e, rt, delta, new = (int(x) for x in rec)
        U[e, rb] += delta; U[e, rt] -= delta; L[rb] += delta; L[rt] -= delta
        if new:
            assert U[e, rt] == 0
            X[e, rt] = False
    np.testing.assert_array_equal(L, p["rank_load_stage1"])
    # Stage-1 routing keeps a domain's demand inside the domain whenever the domain hosts the
    # expert (TopoEP 4.3: "selects instances in the source domain whenever they are available").
    omega = r["omega"].astype(np.int64)
    for e in range(E):
        for m in range(M):
            ranks = list(range(m * G, (m + 1) * G))
            if X[e, ranks].any():
                assert U[e, ranks].sum() >= omega[m * G:(m + 1) * G, e].sum()
            else:
                assert U[e, ranks].sum() == 0
    nrep = np.array([sum(1 for e in range(E) if X[e, rr] and e // Er != rr) for rr in range(R)])
    rep_dom = np.array([nrep[m * G:(m + 1) * G].sum() for m in range(M)])

    def candidates(m):
        ranks = range(m * G, (m + 1) * G)
        rb = max(ranks, key=lambda x: (L[x], -x))
        out = []
        for e in range(E):
            if not X[e, rb] or U[e, rb] <= 0:
                continue
            for rt in ranks:
                if rt == rb:
                    continue
                new = not X[e, rt]
                if new and not (nrep[rt] < prm["n_slot"] and rep_dom[m] < prm["Bd"][m]):
                    continue
                d = min(U[e, rb], (L[rb] - L[rt]) // 2)
                if d >= 1:
                    out.append(((-d, L[rt], int(new), e, rt), rb))
        return rb, sorted(out)

    by_dom = {}
    for rec in tr:
        by_dom.setdefault(int(rec[0]), []).append(rec)
    for m in range(M):
        for rec in by_dom.get(m, []):
            _, it, rb, e, rt, delta, new = (int(x) for x in rec)
            rb_ref, cands = candidates(m)
            assert rb == rb_ref
            assert cands, "a move was recorded with no feasible candidate"
            (key, _) = cands[0]
            assert key == (-delta, L[rt], new, e, rt)
            before = (L ** 2).sum()
            U[e, rb] -= delta; U[e, rt] += delta; L[rb] -= delta; L[rt] += delta
            if new:
                X[e, rt] = True; nrep[rt] += 1; rep_dom[m] += 1
            assert L[rb] >= L[rt]            # the half-gap bound never reverses the order
            assert (L ** 2).sum() < before   # every move strictly improves balance
        if len(by_dom.get(m, [])) < prm["max_iters"]:
            assert not candidates(m)[1]      # refinement stops only when no candidate remains
    np.testing.assert_array_equal(L, p["rank_load"])


@pytest.mark.parametrize("case", range(40))
def test_plan_properties_random(case):
    cfgd = inputs.small_configs(1000 + case, 1)[0]
    cfg, r, p = random_case(cfgd, case)
    check_plan_invariants(cfg, r, p)
    check_quota_locality(cfg, r, p)
    check_quota_passes(cfg, r, p)
    replay_refinement(cfg, r, p)


def stage1_replicas(cfg, p):
    prm = oracle.params(cfg)
    created = {(int(rec[3]), int(rec[4])) for rec in p["trace"] if rec[6]}
    return {(e, rr) for (e, rr) in placement(cfg, p) if rr != e // prm["Er"]} - created


@pytest.mark.parametrize("case", range(40))
def test_stage1_exhaustive(case):
    """Inter-node placement: positive-benefit remote experts only, budget and slots respected,
    and the chosen set has the largest total benefit of any admissible set (enumerated).  With
    several ranks per domain and up to three slots per rank, "least occupied rank with a free
    slot, ties to the lower rank" starting from empty ranks is a round robin: the j-th replica of
    a domain (descending benefit, ties to the lower expert) lands on the domain's rank j mod G."""
    g = inputs.rng(500 + case)
    G = int(g.choice([1, 2, 3, 4])); M = int(g.choice([2, 3])); R = G * M
    Er = int(g.choice([1, 2])); E = R * Er
    k = int(g.integers(1, min(E, 4) + 1)); Tr = int(g.integers(4, 20)); T = Tr * R
    n_slot = int(g.choice([0, 1, 2, 3]))
    B = int(g.integers(0, 3 * R + 1)); W = int(g.choice([0, 3, 9]))
    stacked = case >= 30  # domains that must place more replicas than they have ranks
    if stacked:
        G, Er = max(G, 2), 2; R = G * M; E = R * Er; T = max(Tr, 10) * R; k = min(4, E)
        n_slot, B, W = int(g.choice([2, 3])), 3 * R, 0
    cfg = oracle.make_cfg(T, E, k, R, G, 4, B, n_slot, W, 1, 0)
    topk = inputs.random_topk(case, T, E, k, skew=0.3 if stacked else 2.0)
    lg = np.zeros((T, E), np.float32)
    for j in range(k):
        lg[np.arange(T), topk[:, j]] = np.float32(k - j)
    r = oracle.route(cfg, lg)
    p = oracle.plan(cfg, r["omega"], r["topk_idx"], trace_cap=100000)
    prm = oracle.params(cfg)
    S1 = stage1_replicas(cfg, p)
    omega = r["omega"].astype(np.int64)
    placed_beyond_ranks = False
    for m in range(M):
        Dm = omega[m * G:(m + 1) * G].sum(0)
        b = {e: 2 * int(Dm[e]) * prm["S"] - prm["W"] for e in range(E) if (e // Er) // G != m}
        pos = [e for e in b if b[e] > 0]
        cap = min(int(prm["Bd"][m]), G * prm["n_slot"])
        chosen = [e for (e, rr) in S1 if rr // G == m]
        assert all(e in pos for e in chosen)
        assert len(chosen) == min(cap, len(pos))
        # the largest total benefit over every admissible subset (greedy by benefit is optimal
        # under a cardinality cap; the enumeration confirms it on these small domains)
        top = sorted(pos, key=lambda e: -b[e])[:cap]
        if len(pos) <= 14:
            best = max((sum(b[e] for e in sub) for size in range(0, cap + 1)
                        for sub in itertools.combinations(pos, min(size, len(pos)))), default=0)
            assert best == sum(b[e] for e in top)
        assert sum(b[e] for e in chosen) == sum(b[e] for e in top)
        # where each replica went: round robin over the domain's ranks in placement order
        order = sorted(chosen, key=lambda e: (-b[e], e))
        where = {e: rr for (e, rr) in S1 if rr // G == m}
        assert [where[e] for e in order] == [m * G + j % G for j in range(len(order))]
        assert max([sum(1 for (_, rr) in S1 if rr == x) for x in range(m * G, (m + 1) * G)]) <= prm["n_slot"]
        placed_beyond_ranks = placed_beyond_ranks or len(order) > G
    if stacked:
        assert placed_beyond_ranks  # a second slot of some rank was used


def test_single_domain_has_no_inter_node_stage():
    """TopoEP section 6.3: with all ranks in one NVLink domain there is no inter-node placement."""
    cfgd = dict(T=256, E=16, k=4, R=8, G=8, H=8, B=8, W=0, S=1)
    cfg, r, p = random_case(cfgd, 7)
    assert not stage1_replicas(cfg, p)
    check_plan_invariants(cfg, r, p)


def test_default_slots_let_every_domain_spend_its_share():
    """Default N_slot is the smallest per-rank slot count with which every domain can place its
    whole share of the budget (G * N_slot >= max B_d); the workloads give 1, 2, 1, 1, 1."""
    for case in range(200):
        g = inputs.rng(case)
        G = int(g.integers(1, 9)); M = int(g.integers(1, 9)); B = int(g.integers(0, 100))
        cfg = oracle.make_cfg(0, G * M, 1, G * M, G, 8, B)
        prm = oracle.params(cfg)
        assert sum(prm["Bd"]) == B and max(prm["Bd"]) - min(prm["Bd"]) <= 1
        assert list(prm["Bd"]) == sorted(prm["Bd"], reverse=True)
        assert G * prm["n_slot"] >= max(prm["Bd"])
        assert prm["n_slot"] == 0 or G * (prm["n_slot"] - 1) < max(prm["Bd"])
    for (B, M, G, want) in [(2, 2, 2, 1), (16, 2, 4, 2), (32, 8, 8, 1), (64, 8, 8, 1), (16, 4, 8, 1)]:
        assert oracle.params(oracle.make_cfg(0, G * M, 1, G * M, G, 8, B))["n_slot"] == want


def test_no_budget_is_static_placement():
    cfgd = dict(T=512, E=16, k=4, R=4, G=2, H=8, B=0, W=0, S=1)
    cfg, r, p = random_case(cfgd, 8)
    assert int(p["n_inst"][0]) == cfg.E
    Er = cfg.E // cfg.R
    static = np.array([r["count"][x * Er:(x + 1) * Er].sum() for x in range(cfg.R)])
    np.testing.assert_array_equal(p["rank_load"], static)


def test_iteration_cap_and_empty_layer():
    cfgd = dict(T=512, E=16, k=4, R=4, G=4, H=8, B=8, W=0, S=1, max_iters=1)
    cfg, r, p = random_case(cfgd, 9)
    assert p["n_iters"] <= 1
    check_plan_invariants(cfg, r, p)
    cfg0 = oracle.make_cfg(0, 8, 2, 4, 2, 8, 4, 0, 0, 1, 0)
    out = oracle.run_all(cfg0, np.zeros((0, 8), np.float32), np.zeros((0, 8), np.uint16))
    assert int(out["n_inst"][0]) == 8 and out["rank_load"].sum() == 0
    assert list(out["inst_offset"][:9]) == [0] * 9 and list(out["rank_offset"]) == [0] * 5


# ---------------------------------------------------------------------------
# Dispatch layout and row copy
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", range(10))
def test_dispatch_layout_properties(case):
    cfgd = inputs.small_configs(2000 + case, 1)[0]
    cfg, r, p = random_case(cfgd, case)
    T, k, H, R = cfg.T, cfg.k, cfg.H, cfg.R
    hid = inputs.random_hidden(case, T, H)
    n = int(p["n_inst"][0])
    d = oracle.dispatch(cfg, n, p["inst_rank"], p["slot_inst"], hid)
    N = T * k
    perm, pos = d["perm"], d["slot_pos"]
    assert sorted(perm.tolist()) == list(range(N))
    assert (perm[pos] == np.arange(N)).all()
    si = p["slot_inst"]
    keys = si[perm]
    assert (np.diff(keys) >= 0).all()
    for i in range(n):  # stable: slot ids increase inside each instance segment
        seg = perm[d["inst_offset"][i]:d["inst_offset"][i + 1]]
        assert (np.diff(seg) > 0).all() and len(seg) == p["inst_load"][i]
        assert (si[seg] == i).all()
    assert d["inst_offset"][n] == N and (d["inst_offset"][n + 1:] == -1).all()
    for x in range(R):
        lo, hi = d["rank_offset"][x], d["rank_offset"][x + 1]
        assert hi - lo == p["rank_load"][x]
        assert (p["inst_rank"][si[perm[lo:hi]]] == x).all()
    np.testing.assert_array_equal(d["slot_rank"], pos - d["inst_offset"][si])
    for q in range(N):
        np.testing.assert_array_equal(d["dispatch"][pos[q]], hid[q // k])


def test_oracle_is_deterministic():
    cfgd = dict(T=640, E=32, k=4, R=8, G=4, H=16, B=8, W=0, S=1)
    cfg = cfg_from(cfgd)
    lg = inputs.random_logits(4, cfg.T, cfg.E)
    hid = inputs.random_hidden(4, cfg.T, cfg.H)
    a = oracle.run_all(cfg, lg, hid)
    b = oracle.run_all(cfg, lg, hid)
    for key, v in a.items():
        if isinstance(v, np.ndarray):
            np.testing.assert_array_equal(v, b[key])
