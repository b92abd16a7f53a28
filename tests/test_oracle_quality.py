"""Pins of the plan-quality oracle ([TopoEP] section 6.2 Fig. 10, section 6.4
Fig. 13(b), section 6.6 Fig. 16).

What fixes the counts without restating the oracle: the Fig. 9 example (the
eight GPU-0 assignments of E4 are served by the two new replicas, nothing
crosses a domain, every rank ends at 10); the static placement (B = 0) in
closed form from the routing matrix; balanced uniform routing without
replicas, where a share (M-1)/M of the assignments leaves its node -- 50 % and
75 % for two and four nodes, the endpoints the page reports for Megatron-LM;
and a recount slot by slot from the per-slot instances on random layers.
"""
from __future__ import annotations

import json
import os

import numpy as np

import oracle
from tests import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def fig9():
    g = json.load(open(os.path.join(GOLDEN, "fig9_example.json")))
    c = g["config"]
    cfg = oracle.make_cfg(c["T"], c["E"], c["k"], c["R"], c["G"], c["H"], c["B"], c["n_slot"], c["W"], c["S"],
                          c["max_iters"])
    return cfg, np.array(g["omega"], np.int32)


def test_fig9_example():
    cfg, om = fig9()
    p = oracle.plan(cfg, om, np.zeros((0, cfg.k), np.int32))
    q = oracle.quality(cfg, p)
    assert q["assignments"] == int(om.sum()) == 40
    assert q["replica_served"] == 8          # E4 of GPU 0: 4 on E4', 4 on E4''
    assert q["other_node"] == 0 and q["same_node"] == 40
    assert q["same_rank"] == 36               # all but the 4 moved to GPU 1
    assert q["max_rank_load"] == q["min_rank_load"] == 10 and q["imbalance"] == 1.0
    assert q["replicas"] == 2


def test_static_placement_closed_form():
    for seed in range(4):
        g = inputs.rng(seed)
        G, M, Er = int(g.choice([1, 2, 4])), int(g.choice([1, 2, 3])), int(g.integers(1, 4))
        R, E = G * M, G * M * Er
        om = g.integers(0, 30, (R, E)).astype(np.int32)
        cfg = oracle.make_cfg(0, E, 1, R, G, 8, 0)
        q = oracle.quality(cfg, oracle.plan(cfg, om, np.zeros((0, 1), np.int32)))
        main = np.arange(E) // Er
        src = np.arange(R)[:, None]
        assert q["replica_served"] == 0 and q["replicas"] == 0
        assert q["same_rank"] == int(om[main[None, :] == src].sum())
        assert q["same_node"] == int(om[(main[None, :] // G) == (src // G)].sum())
        load = np.bincount(main, weights=om.sum(0), minlength=R)
        assert q["max_rank_load"] == int(load.max()) and q["min_rank_load"] == int(load.min())


def test_uniform_routing_leaves_its_node_m_minus_one_over_m_of_the_time():
    for M, want in ((2, 0.50), (4, 0.75), (1, 0.0), (8, 0.875)):
        G, Er = 8, 2
        R, E = G * M, G * M * Er
        cfg = oracle.make_cfg(0, E, 1, R, G, 8, 2 * R, 0, 1 << 40)  # replicas never pay off
        q = oracle.quality(cfg, oracle.plan(cfg, np.full((R, E), 6, np.int32), np.zeros((0, 1), np.int32)))
        assert q["other_node"] / q["assignments"] == want
        assert q["imbalance"] == 1.0


def test_recount_from_the_slots():
    for i, c in enumerate(inputs.small_configs(17, 24)):
        cfg = oracle.make_cfg(**c)
        lg = inputs.random_logits(i, c["T"], c["E"])
        o = oracle.run_all(cfg, lg, None, want_cooc=False)
        q = oracle.quality(cfg, o)
        inst = o["slot_inst"]
        r = o["inst_rank"][inst]
        e = o["inst_expert"][inst]
        s = np.repeat(np.arange(c["T"]) // (c["T"] // c["R"]) if c["T"] else np.zeros(0, np.int64), c["k"])
        Er = c["E"] // c["R"]
        assert q["assignments"] == c["T"] * c["k"]
        assert q["same_rank"] == int((r == s).sum())
        assert q["same_node"] == int((r // c["G"] == s // c["G"]).sum())
        assert q["other_node"] == q["assignments"] - q["same_node"]
        assert q["replica_served"] == int((r != e // Er).sum())
        assert q["max_rank_load"] == int(o["rank_load"].max()) and q["min_rank_load"] == int(o["rank_load"].min())
        assert q["replicas"] == int(o["n_inst"][0]) - c["E"]
        if c["T"]:
            assert q["max_rank_load"] >= -(-c["T"] * c["k"] // c["R"])


def test_replication_lowers_the_imbalance_on_skewed_routing():
    """Skewed synthetic routing: with replica slots the planner's imbalance is no worse
    than the static placement's (its refinement only ever narrows load gaps)."""
    T, E, k, R, G = 4096, 64, 4, 16, 4
    lg = inputs.random_logits(3, T, E)
    base = None
    for slots in (0, 1, 2):
        cfg = oracle.make_cfg(T, E, k, R, G, 64, slots * R, slots, 0)
        q = oracle.quality(cfg, oracle.run_all(cfg, lg, None, want_cooc=False))
        if base is None:
            base = q["imbalance"]
        assert q["imbalance"] <= base
