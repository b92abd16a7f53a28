"""Pins of the placement and deduplication oracle ([Coupling] "Moving
Correlated Experts Together", Fig. 3).

What fixes the results without restating the oracle:
  * the page's chance-level row savings of deduplication alone (6 % for top-2,
    25 % for top-6 at EP8 with 128 experts; tests/golden/coupling_dedup_chance.json)
    against exact enumeration and the hypergeometric closed form;
  * for top-2 routing the rows saved by deduplication equal the co-selection
    weight the placement keeps inside ranks (an exact identity);
  * zero or uniform co-selection gives the contiguous placement; a planted
    partition is recovered; the result admits no improving swap (brute force
    over all swaps); it never beats the exhaustive optimum; relabelling the
    experts relabels the result;
  * the deduplicated layout agrees with the counts, carries every slot once,
    and without anything to deduplicate equals the instance-ordered dispatch.
"""
from __future__ import annotations

import itertools
import json
import os
from math import comb

import numpy as np
import pytest

import oracle
import synth
from tests import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "coupling_dedup_chance.json")


def cfg_of(T, E, k, R, G=1, H=4, B=0):
    return oracle.make_cfg(T, E, k, R, G, H, B)


def sym(a: np.ndarray) -> np.ndarray:
    u = np.triu(a, 1)
    return (u + u.T).astype(np.int32)


def intra_of(C: np.ndarray, rank: np.ndarray) -> int:
    same = rank[:, None] == rank[None, :]
    return int(np.triu(np.where(same, C, 0), 1).sum())


def balanced_partitions(E: int, R: int):
    """Every partition of range(E) into R unlabelled blocks of E/R (as rank arrays)."""
    Er = E // R

    def rec(left, blocks):
        if not left:
            yield blocks
            return
        first, rest = left[0], left[1:]
        for others in itertools.combinations(rest, Er - 1):
            remain = [x for x in rest if x not in others]
            yield from rec(remain, blocks + [(first,) + others])

    for blocks in rec(list(range(E)), []):
        rank = np.empty(E, np.int64)
        for r, b in enumerate(blocks):
            rank[list(b)] = r
        yield rank


def partition_sets(rank: np.ndarray):
    return sorted(tuple(np.flatnonzero(rank == r)) for r in np.unique(rank))


# ---------------------------------------------------------------- deduplication


def test_top2_chance_level_matches_the_page():
    """Every expert pair of a 128-expert top-2 layer once, contiguous EP8:
    the rows saved are the same-rank pairs, 8 * C(16, 2) = 960 of 2 * 8128."""
    g = json.load(open(GOLDEN))
    E, R = g["experts"], g["ep"]
    pairs = np.array(list(itertools.combinations(range(E), 2)), np.int32)
    T = len(pairs)
    assert T == 8128 and T % R == 0
    d = oracle.dedup(cfg_of(T, E, 2, R), pairs)
    slots = 2 * T
    saved = slots - int(d["tok_ranks"].sum())
    assert saved == R * comb(E // R, 2) == 960
    assert round(100 * saved / slots) == g["rows_removed_percent"]["top2"]


def test_top6_every_subset_matches_the_hypergeometric_expectation():
    """All C(12, 6) = 924 six-expert sets, 4 ranks of 3: a rank is hit unless
    all six experts avoid it, so the rows total 924 * 4 * (1 - C(9,6)/C(12,6))."""
    E, R, k = 12, 4, 6
    sets = np.array(list(itertools.combinations(range(E), k)), np.int32)
    d = oracle.dedup(cfg_of(len(sets), E, k, R), sets)
    assert int(d["tok_ranks"].sum()) == len(sets) * R - R * comb(E - E // R, k) == 3360
    assert d["rank_slots"].sum() == len(sets) * k


def test_top6_chance_level_matches_the_page():
    g = json.load(open(GOLDEN))
    E, R, k = g["experts"], g["ep"], 6
    exact = 1 - R * (1 - comb(E - E // R, k) / comb(E, k)) / k
    assert round(100 * exact) == g["rows_removed_percent"]["top6"]
    T = 16384
    rng = inputs.rng(61)
    topk = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)  # uniform 6-subsets
    d = oracle.dedup(cfg_of(T, E, k, R), topk)
    per_tok = 1 - d["tok_ranks"] / k
    f = per_tok.mean()
    sd = per_tok.std() / np.sqrt(T)
    page = g["rows_removed_percent"]["top6"] / 100
    assert abs(f - page) <= 0.005 + 4 * sd, (f, page, sd)
    assert abs(f - exact) <= 4 * sd


def test_dedup_special_cases():
    T, E, k = 96, 12, 4
    topk = inputs.random_topk(3, T, E, k)
    one = oracle.dedup(cfg_of(T, E, k, 1), topk)  # one rank: one row per token
    assert (one["tok_ranks"] == 1).all() and one["rank_rows"].tolist() == [[T]]
    each = oracle.dedup(cfg_of(T, E, k, E), topk)  # one expert per rank: nothing to merge
    assert (each["tok_ranks"] == k).all()
    np.testing.assert_array_equal(each["rank_rows"], each["rank_slots"])
    # a table that sends every expert to rank 2
    c = cfg_of(T, E, k, 4)
    two = oracle.dedup(c, topk, np.full(E, 2, np.int32))
    assert (two["tok_ranks"] == 1).all() and two["rank_rows"][:, 2].sum() == T


def test_dedup_brute_force_and_invariants():
    for seed in range(6):
        g = inputs.rng(seed)
        R = int(g.choice([2, 3, 4]))
        E = R * int(g.integers(1, 5))
        k = int(g.integers(1, min(E, 7) + 1))
        T = R * int(g.integers(0, 40))
        topk = inputs.random_topk(seed, T, E, k) if T else np.zeros((0, k), np.int32)
        table = g.integers(0, R, E).astype(np.int32)
        c = cfg_of(T, E, k, R)
        d = oracle.dedup(c, topk, table)
        Tr = T // R if R else 0
        want_rows = np.zeros((R, R), np.int64)
        want_slots = np.zeros((R, R), np.int64)
        for t in range(T):
            ranks = [int(table[e]) for e in topk[t]]
            assert d["tok_ranks"][t] == len(set(ranks))
            for r in set(ranks):
                want_rows[t // Tr, r] += 1
            for r in ranks:
                want_slots[t // Tr, r] += 1
        np.testing.assert_array_equal(d["rank_rows"], want_rows)
        np.testing.assert_array_equal(d["rank_slots"], want_slots)
        assert (d["rank_rows"] <= d["rank_slots"]).all()


def test_dedup_slot_counts_are_the_routing_matrix_on_contiguous_ranks():
    c = oracle.make_cfg(256, 16, 3, 4, 2, 4, 0)
    r = oracle.route(c, inputs.random_logits(5, 256, 16))
    d = oracle.dedup(c, r["topk_idx"])
    np.testing.assert_array_equal(d["rank_slots"], r["omega"].reshape(4, 4, 4).sum(axis=2))


def test_dedup_rejects_bad_keys():
    c = cfg_of(8, 8, 2, 4)
    topk = np.tile(np.array([[0, 1]], np.int32), (8, 1))
    with pytest.raises(ValueError):
        oracle.dedup(c, np.where(np.arange(16).reshape(8, 2) == 5, 8, topk))
    with pytest.raises(ValueError):
        oracle.dedup(c, topk, np.array([0, 4, 0, 0, 0, 0, 0, 0], np.int32))


# -------------------------------------------------------------------- placement


def test_zero_and_uniform_coselection_give_the_contiguous_placement():
    E, R = 12, 4
    c = cfg_of(4, E, 2, R)
    for C, w in ((np.zeros((E, E), np.int32), 0), (sym(np.full((E, E), 7)), 7)):
        p = oracle.place(c, C)
        np.testing.assert_array_equal(p["expert_rank"], np.arange(E) // (E // R))
        np.testing.assert_array_equal(p["rank_experts"], np.arange(E).reshape(R, E // R))
        assert p["n_swaps"] == 0 and p["intra"] == R * comb(E // R, 2) * w


def test_planted_partition_is_recovered():
    for seed, (E, R) in enumerate([(16, 4), (24, 3), (12, 6), (32, 8)]):
        g = inputs.rng(100 + seed)
        perm = g.permutation(E)
        group = np.empty(E, np.int64)
        group[perm] = np.arange(E) // (E // R)
        same = group[:, None] == group[None, :]
        C = sym(np.where(same, g.integers(100, 121, (E, E)), g.integers(0, 6, (E, E))))
        p = oracle.place(cfg_of(R, E, 2, R), C)
        assert partition_sets(p["expert_rank"]) == partition_sets(group)
        assert p["intra"] == intra_of(C, group)


def test_no_improving_swap_remains_and_the_optimum_bounds_the_result():
    gaps = []
    for seed, (E, R) in enumerate([(8, 4), (8, 2), (9, 3), (6, 3), (10, 5), (12, 3)]):
        g = inputs.rng(200 + seed)
        C = sym(g.integers(0, 30, (E, E)))
        p = oracle.place(cfg_of(R, E, 2, R), C)
        rank = p["expert_rank"].astype(np.int64)
        assert np.bincount(rank, minlength=R).tolist() == [E // R] * R
        w = intra_of(C, rank)
        assert p["intra"] == w
        for a in range(E):
            for b in range(a + 1, E):
                if rank[a] != rank[b]:
                    q = rank.copy()
                    q[a], q[b] = rank[b], rank[a]
                    assert intra_of(C, q) <= w, "swap %d,%d improves" % (a, b)
        best = max(intra_of(C, q) for q in balanced_partitions(E, R))
        assert w <= best
        gaps.append(best - w)
    assert min(gaps) == 0  # the local search reaches the optimum on some of them


def test_relabelling_the_experts_relabels_the_placement():
    """With tie-free weights nothing depends on expert ids: permuting the
    experts permutes the result (ranks keep their numbers)."""
    for seed, (E, R) in enumerate([(12, 3), (16, 4), (20, 5)]):
        g = inputs.rng(300 + seed)
        C = sym(g.integers(0, 1 << 20, (E, E)))
        pi = g.permutation(E)  # new expert i is old expert pi[i]
        Cp = C[np.ix_(pi, pi)]
        c = cfg_of(R, E, 2, R)
        for cap in (0, -1):
            p = oracle.place(c, C, cap)
            q = oracle.place(c, Cp, cap)
            np.testing.assert_array_equal(q["expert_rank"], p["expert_rank"][pi])
            assert q["intra"] == p["intra"] and q["n_swaps"] == p["n_swaps"]


def test_swap_cap():
    E, R = 24, 4
    C = sym(inputs.rng(7).integers(0, 50, (E, E)))
    c = cfg_of(R, E, 2, R)
    p0, p1, pd = oracle.place(c, C, 0), oracle.place(c, C, 1), oracle.place(c, C, -1)
    assert p0["n_swaps"] == 0 and p1["n_swaps"] <= 1
    assert p0["intra"] <= p1["intra"] <= pd["intra"]
    assert pd["n_swaps"] > 1
    assert oracle.place(c, C, pd["n_swaps"])["intra"] == pd["intra"]


def test_top2_rows_saved_equal_the_weight_kept_inside_ranks():
    """A top-2 token saves one row exactly when both its experts share a rank,
    and cooc counts each such token once for that pair."""
    w = synth.Workload("pairs", T=2048, E=32, k=2, R=8, G=2, H=8, B=0, zipf_s=0.8, beta=2.5, group_size=4)
    c = oracle.make_cfg(w.T, w.E, w.k, w.R, w.G, w.H, 0)
    r = oracle.route(c, synth.logits(w))
    for cap in (0, -1):
        p = oracle.place(c, r["cooc"], cap)
        d = oracle.dedup(c, r["topk_idx"], p["expert_rank"])
        assert w.T * 2 - int(d["tok_ranks"].sum()) == p["intra"]
    base = oracle.dedup(c, r["topk_idx"])
    assert int(d["tok_ranks"].sum()) < int(base["tok_ranks"].sum())


def test_latent_expert_groups_are_recovered():
    """Synthetic routing whose co-selection comes from latent expert groups of
    size E/R: with a strong group boost the placement puts each group on one rank."""
    w = synth.Workload("groups", T=4096, E=32, k=4, R=8, G=2, H=8, B=0, beta=4.0, group_size=4)
    c = oracle.make_cfg(w.T, w.E, w.k, w.R, w.G, w.H, 0)
    r = oracle.route(c, synth.logits(w))
    p = oracle.place(c, r["cooc"])
    perm = synth.permutation(w.seed, 0, 2, w.E)  # the generator's group layout (its stream 2)
    group = np.empty(w.E, np.int64)
    group[perm] = np.arange(w.E) // w.group_size
    assert partition_sets(p["expert_rank"]) == partition_sets(group)


def test_place_rejects_invalid_coselection():
    c = cfg_of(4, 8, 2, 4)
    C = sym(inputs.rng(1).integers(0, 9, (8, 8)))
    for bad in (C + np.eye(8, dtype=np.int32), np.where(np.arange(64).reshape(8, 8) == 3, 5, C), -C):
        with pytest.raises(ValueError):
            oracle.place(c, bad)


# --------------------------------------------------------- deduplicated layout


def check_layout(c, topk, table, hidden, lay):
    T, k, R = c.T, c.k, c.R
    d = oracle.dedup(c, topk, table)
    n = lay["n_rows"]
    assert n == int(d["tok_ranks"].sum())
    off = lay["rank_row_offset"]
    np.testing.assert_array_equal(np.diff(off), d["rank_rows"].sum(axis=0))
    assert off[0] == 0 and off[R] == n
    rt, rs = lay["row_token"], lay["row_slots"]
    assert (rt[n:] == -1).all() and (rs[n:] == -1).all()
    rank_of = (topk // (c.E // R)) if table is None else table[topk]
    for r in range(R):
        seg = rt[off[r]:off[r + 1]]
        assert (np.diff(seg) > 0).all()  # tokens ascending, each once
    covered = np.zeros(T * k, np.int64)
    for p in range(n):
        r = int(np.searchsorted(off, p, side="right") - 1)
        t = int(rt[p])
        js = [j for j in range(k) if rs[p] >> j & 1]
        assert js and all(rank_of[t, j] == r for j in js)
        assert [j for j in range(k) if rank_of[t, j] == r] == js
        covered[[t * k + j for j in js]] += 1
    assert (covered == 1).all()
    q = np.arange(T * k)
    np.testing.assert_array_equal(rt[lay["slot_row"]], q // k)
    assert ((rs[lay["slot_row"]] >> (q % k)) & 1).all()
    if hidden is not None:
        np.testing.assert_array_equal(lay["ddispatch"], hidden[rt[:n]])


def test_dedup_layout_properties():
    for seed in range(5):
        g = inputs.rng(40 + seed)
        R = int(g.choice([1, 2, 4]))
        E = R * int(g.integers(1, 5))
        k = int(g.integers(1, min(E, 6) + 1))
        T = R * int(g.integers(0, 30))
        c = cfg_of(T, E, k, R, H=5)
        topk = inputs.random_topk(seed, T, E, k) if T else np.zeros((0, k), np.int32)
        hid = inputs.random_hidden(seed, T, 5)
        for table in (None, g.integers(0, R, E).astype(np.int32)):
            check_layout(c, topk, table, hid, oracle.dedup_dispatch(c, topk, table, hid))


def test_dedup_layout_without_merges_is_the_instance_dispatch():
    """One expert per rank and no replicas: every slot is its own row, and the
    rows come in the order of the planner's dispatch (instances = experts)."""
    T, E, k = 128, 8, 3
    c = oracle.make_cfg(T, E, k, E, 2, 6, 0)
    o = oracle.run_all(c, inputs.random_logits(9, T, E), inputs.random_hidden(9, T, 6))
    lay = oracle.dedup_dispatch(c, o["slot_inst"], o["inst_rank"][:E], inputs.random_hidden(9, T, 6))
    assert lay["n_rows"] == T * k
    np.testing.assert_array_equal(lay["row_token"], o["perm"] // k)
    np.testing.assert_array_equal(lay["row_slots"], 1 << (o["perm"] % k))
    np.testing.assert_array_equal(lay["ddispatch"], o["dispatch"])


def test_dedup_layout_one_rank():
    T, E, k = 40, 6, 3
    c = cfg_of(T, E, k, 1, H=3)
    topk = inputs.random_topk(2, T, E, k)
    lay = oracle.dedup_dispatch(c, topk)
    assert lay["n_rows"] == T
    np.testing.assert_array_equal(lay["row_token"][:T], np.arange(T))
    assert (lay["row_slots"][:T] == (1 << k) - 1).all()
