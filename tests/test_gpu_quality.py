"""GPU parity of the plan-quality counters (moe_plan_quality) against the
oracle, and of the whole plan at the shapes of [TopoEP] Figs. 10 and 11
(640 experts over 8-128 ranks; 128-2048 experts over 32 ranks) under the
section 6.4 synthetic skew.  Integer results: exact.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mp():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import load_balance_planning_amd as m
    m.lib()
    return m


def gpu_plan_quality(mp, w, lg):
    layer = mp.Layer(mp.make_config(w.T, w.E, w.k, w.R, w.G, w.H, w.B), cooc=False)
    layer.route(torch.from_numpy(lg).cuda())
    layer.plan()
    q = layer.quality()
    torch.cuda.synchronize()
    assert layer.status() == 0
    got = dict(zip(mp.QUALITY_FIELDS, (int(v) for v in q.cpu().numpy())))
    plan = {k: getattr(layer.plan_out, k).cpu().numpy() for k in
            ("n_inst", "inst_expert", "inst_rank", "inst_load", "rank_load", "quota", "slot_inst")}
    layer.close()
    return got, plan


def check(mp, w, full_plan=True):
    lg = synth.logits(w)
    c = oracle.make_cfg(w.T, w.E, w.k, w.R, w.G, w.H, w.B)
    o = oracle.run_all(c, lg, None, want_cooc=False)
    want = oracle.quality(c, o)
    got, plan = gpu_plan_quality(mp, w, lg)
    for k in mp.QUALITY_FIELDS:
        assert got[k] == want[k], (w.name, k, got[k], want[k])
    if full_plan:
        for k, v in plan.items():
            np.testing.assert_array_equal(v.reshape(-1), np.asarray(o[k]).reshape(-1), err_msg="%s %s" % (w.name, k))
    return want


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_quality_on_each_workload(mp, name):
    print("quality %s" % name, flush=True)
    check(mp, synth.WORKLOADS[name], full_plan=False)


@pytest.mark.parametrize("skew,slots", [(0, 0), (0, 2), (-2, 1), (-2, 4), (-4, 0), (-4, 2), (-4, 3)])
def test_plan_and_quality_on_the_skew_sweep(mp, skew, slots):
    w = synth.skew_layer(skew, slots)
    print("skew sweep %s" % w.name, flush=True)
    q = check(mp, w)
    if slots == 0:
        assert q["replicas"] == 0


@pytest.mark.parametrize("E,R", [(640, 8), (640, 16), (640, 128), (128, 32), (2048, 32)])
def test_plan_at_the_solver_scaling_shapes(mp, E, R):
    w = synth.skew_layer(-4, 2, E=E, R=R)
    print("solver shape %s" % w.name, flush=True)
    check(mp, w)
