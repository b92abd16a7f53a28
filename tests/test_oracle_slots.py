"""Pins of the replica slot map and the parameter / gradient transfers
([TopoEP] section 3.2, Replica Buffer Management; Fig. 6).

What fixes them: the Fig. 9 example (E4's replicas E4' on GPU 0 and E4'' on
GPU 1, both pulling from E4's main rank, GPU 2; the other GPUs' slots empty);
the plan's own replica instances, each in exactly one slot of its rank, never
of a rank's own expert; the pull copying each slot's expert row byte for
byte; the return writing each slot's row into its main rank's buffer region
for that source rank, so that a pull followed by a return puts every
replicated expert's parameters back into exactly the (main, source, expert)
regions the plan names and nowhere else.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle
from tests import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_fig9_slots():
    g = json.load(open(os.path.join(GOLDEN, "fig9_example.json")))
    c = g["config"]
    cfg = oracle.make_cfg(c["T"], c["E"], c["k"], c["R"], c["G"], c["H"], c["B"], c["n_slot"], c["W"], c["S"],
                          c["max_iters"])
    p = oracle.plan(cfg, np.array(g["omega"], np.int32), np.zeros((0, 1), np.int32))
    m = oracle.slot_map(cfg, p)
    assert oracle.params(cfg)["n_slot"] == 1
    assert m["slot_expert"].tolist() == [[4], [4], [-1], [-1]]
    assert m["slot_main"].tolist() == [[2], [2], [-1], [-1]]
    # instance 2 is E4' on GPU 0, instance 5 is E4'' on GPU 1
    assert m["inst_slot"].tolist()[:10] == [-1, -1, 0, -1, -1, 0, -1, -1, -1, -1]


def test_every_replica_in_one_slot():
    for i, c in enumerate(inputs.small_configs(23, 30)):
        cfg = oracle.make_cfg(**c)
        o = oracle.run_all(cfg, inputs.random_logits(i, c["T"], c["E"]), None, want_cooc=False)
        m = oracle.slot_map(cfg, o)
        ns = oracle.params(cfg)["n_slot"]
        Er = c["E"] // c["R"]
        n = int(o["n_inst"][0])
        ie, ir = o["inst_expert"][:n], o["inst_rank"][:n]
        replicas = [(int(ir[i]), int(ie[i])) for i in range(n) if ie[i] // Er != ir[i]]
        occupied = [(r, int(e)) for r in range(c["R"]) for e in m["slot_expert"][r] if e >= 0]
        assert sorted(occupied) == sorted(replicas)
        for r in range(c["R"]):
            row = m["slot_expert"][r]
            k = int((row >= 0).sum())
            assert (row[:k] >= 0).all() and (row[k:] == -1).all()      # filled from slot 0
            assert (np.diff(row[:k]) > 0).all()                          # instance order: ascending expert
            assert ((row[:k] // Er) != r).all()                          # never the rank's own expert
            np.testing.assert_array_equal(m["slot_main"][r][:k], row[:k] // Er)
            assert k <= ns
        for i in range(n):
            if m["inst_slot"][i] >= 0:
                assert m["slot_expert"][ir[i], m["inst_slot"][i]] == ie[i]


def test_pull_then_return_round_trip():
    for i, c in enumerate(inputs.small_configs(29, 12)):
        cfg = oracle.make_cfg(**c)
        o = oracle.run_all(cfg, inputs.random_logits(i, c["T"], c["E"]), None, want_cooc=False)
        m = oracle.slot_map(cfg, o)
        ns = oracle.params(cfg)["n_slot"]
        R, E, Er, P = c["R"], c["E"], c["E"] // c["R"], 5
        main = inputs.random_hidden(i, E, P)
        rep = np.full((R, ns, P), 0xDEAD, np.uint16)
        oracle.replica_pull(cfg, m["slot_expert"], main, rep)
        for r in range(R):
            for j in range(ns):
                e = m["slot_expert"][r, j]
                if e >= 0:
                    np.testing.assert_array_equal(rep[r, j], main[e])
                else:
                    assert (rep[r, j] == 0xDEAD).all()
        acc = np.zeros((R, R, Er, P), np.uint16)
        oracle.replica_push(cfg, m["slot_expert"], rep, acc)
        want = np.zeros_like(acc)
        for r in range(R):
            for e in m["slot_expert"][r]:
                if e >= 0:
                    want[e // Er, r, e % Er] = main[e]
        np.testing.assert_array_equal(acc, want)


def test_bad_instance_is_rejected():
    cfg = oracle.make_cfg(0, 8, 1, 4, 2, 8, 4)
    p = dict(n_inst=np.array([8], np.int32), inst_expert=np.arange(12, dtype=np.int32) % 8,
             inst_rank=np.r_[np.arange(8) // 2, [0] * 4].astype(np.int32))
    p["inst_rank"][3] = 9
    with pytest.raises(ValueError):
        oracle.slot_map(cfg, p)


def test_slots_per_rank_never_exceed_the_budget():
    """A rank can hold at most B replicas (the whole layer's budget), so a configured
    slot count above B is clamped to B; with B = 0 there are no slots at all."""
    assert oracle.params(oracle.make_cfg(8, 4, 2, 2, 1, 8, 0, 2))["n_slot"] == 0
    assert oracle.params(oracle.make_cfg(8, 4, 2, 2, 1, 8, 3, 5))["n_slot"] == 3
    assert oracle.params(oracle.make_cfg(8, 4, 2, 2, 1, 8, 3, 2))["n_slot"] == 2
