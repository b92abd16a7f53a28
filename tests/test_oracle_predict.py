"""Pins of the token-shuffle predictor ([Coupling] "Moving Tokens Toward Their
Next Experts"; scoring rule read as each current expert voting with its
empirical next-layer distribution over ranks).

What fixes the result without restating the oracle: a one-expert token whose
next expert is a fixed successor of its current one is always predicted
right; exact rational arithmetic (fractions) on random small layers gives the
same argmax wherever it is not a near-tie; scaling one expert's transition
row together with its count changes nothing (each expert votes with a
distribution); ties (one rank, uniform transitions) go to rank 0; the
unshuffled locality equals the next layer's routing matrix summed over each
source's own experts.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import oracle
import synth
from tests import inputs


def trans_of(cur: np.ndarray, nxt: np.ndarray, E: int) -> np.ndarray:
    """Transition counts X[a][b] = #tokens with a now and b next (the definition, by brute force)."""
    X = np.zeros((E, E), np.int64)
    for a_row, b_row in zip(cur, nxt):
        for a in a_row:
            for b in b_row:
                X[a, b] += 1
    return X.astype(np.int32)


def test_fixed_successor_is_always_predicted():
    T, E, R = 504, 24, 6
    g = inputs.rng(1)
    phi = g.permutation(E)
    cur = g.integers(0, E, (T, 1)).astype(np.int32)
    nxt = phi[cur].astype(np.int32)
    c = oracle.make_cfg(T, E, 1, R, 2, 8, 0)
    cnt = np.bincount(cur[:, 0], minlength=E).astype(np.int32)
    p = oracle.predict(c, cur, trans_of(cur, nxt, E), cnt, topk_next=nxt)
    np.testing.assert_array_equal(p["pred"], phi[cur[:, 0]] // (E // R))
    assert p["local_predicted"] == T
    np.testing.assert_array_equal(p["rank_tokens"], np.bincount(p["pred"], minlength=R))


def exact_scores(cur_row, X, cnt, rank_of, R):
    s = [Fraction(0)] * R
    for a in cur_row:
        if cnt[a] == 0:
            continue
        for b in range(len(rank_of)):
            s[rank_of[b]] += Fraction(int(X[a, b]), int(cnt[a]))
    return s


def test_argmax_against_exact_rationals():
    for seed in range(8):
        g = inputs.rng(50 + seed)
        R = int(g.choice([2, 3, 4, 6]))
        E = R * int(g.integers(1, 5))
        k = int(g.integers(1, min(E, 5) + 1))
        T = R * int(g.integers(4, 30))
        cur = inputs.random_topk(seed, T, E, k)
        nxt = inputs.random_topk(seed + 100, T, E, k)
        X = trans_of(cur, nxt, E)
        cnt = np.bincount(cur.reshape(-1), minlength=E).astype(np.int32)
        table = g.integers(0, R, E).astype(np.int32)
        c = oracle.make_cfg(T, E, k, R, 1, 8, 0)
        p = oracle.predict(c, cur, X, cnt, table, nxt)
        local = 0
        for t in range(T):
            s = exact_scores(cur[t], X, cnt, table, R)
            best = max(s)
            got = int(p["pred"][t])
            assert abs(float(s[got] - best)) <= 1e-12 * k, (seed, t)
            if s.count(best) == 1 and all(float(best - v) > 1e-9 for v in s if v != best):
                assert got == s.index(best), (seed, t)
            if s.count(best) > 1 and all(float(best - v) > 1e-9 for v in s if v != best):
                assert got == s.index(best)  # exact ties: the lower rank (doubles agree on them here)
            local += int((table[nxt[t]] == got).sum())
        assert p["local_predicted"] == local


def test_scaling_one_experts_row_and_count_changes_nothing():
    T, E, k, R = 400, 16, 3, 4
    cur = inputs.random_topk(7, T, E, k, skew=0.0)
    nxt = inputs.random_topk(8, T, E, k, skew=0.0)
    X = trans_of(cur, nxt, E)
    cnt = np.bincount(cur.reshape(-1), minlength=E).astype(np.int32)
    c = oracle.make_cfg(T, E, k, R, 2, 8, 0)
    base = oracle.predict(c, cur, X, cnt)["pred"]
    assert len(set(base.tolist())) > 1
    for a, f in ((0, 2), (5, 8), (11, 3)):
        X2, c2 = X.copy(), cnt.copy()
        X2[a] *= f
        c2[a] *= f
        np.testing.assert_array_equal(oracle.predict(c, cur, X2, c2)["pred"], base)
    X3 = X.copy()
    X3[3] *= 50  # the row alone: expert 3's vote outweighs the others
    assert not np.array_equal(oracle.predict(c, cur, X3, cnt)["pred"], base)


def test_ties_go_to_rank_zero():
    T, E, k = 64, 12, 2
    cur = inputs.random_topk(3, T, E, k)
    c1 = oracle.make_cfg(T, E, k, 1, 1, 8, 0)
    assert (oracle.predict(c1, cur, np.ones((E, E), np.int32), np.full(E, 5, np.int32))["pred"] == 0).all()
    c4 = oracle.make_cfg(T, E, k, 4, 2, 8, 0)
    p = oracle.predict(c4, cur, np.full((E, E), 3, np.int32), np.full(E, 7, np.int32))
    assert (p["pred"] == 0).all() and p["rank_tokens"].tolist() == [T, 0, 0, 0]


def test_unshuffled_locality_is_the_routing_matrix_on_own_experts():
    w = synth.WORKLOADS["coupled_4layer"]
    T = 4096
    lg = synth.all_logits(w, T)
    c = oracle.make_cfg(T, w.E, w.k, w.R, w.G, w.H, 0)
    r0 = oracle.route(c, lg[0])
    r1 = oracle.route(c, lg[1], prev_topk=r0["topk_idx"])
    p = oracle.predict(c, r0["topk_idx"], r1["trans"], r0["count"], topk_next=r1["topk_idx"])
    Er = w.E // w.R
    own = sum(int(r1["omega"][s, s * Er:(s + 1) * Er].sum()) for s in range(w.R))
    assert p["local_source"] == own
    # the coupled routing is predictable: far above the 1/R of staying put
    assert p["local_predicted"] > 2 * p["local_source"]
