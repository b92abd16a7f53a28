"""GPU parity of the replica slot map and the parameter pull / gradient return
(moe_plan_slot_map, moe_plan_replica_pull, moe_plan_replica_push) against the
oracle: the map exactly, the copied rows byte for byte, untouched rows
untouched."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
from tests import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mp():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import load_balance_planning_amd as m
    m.lib()
    return m


def dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).cuda()


def host16(t):
    return t.cpu().numpy().view(np.uint16)


def check_layer(mp, cfgd, logits, P):
    T, E, k, R, G, H, B = (cfgd[x] for x in ("T", "E", "k", "R", "G", "H", "B"))
    extra = {kk: cfgd[kk] for kk in ("n_slot", "W", "S", "max_iters") if kk in cfgd}
    oc = oracle.make_cfg(T, E, k, R, G, H, B, extra.get("n_slot", 0), extra.get("W", -1), extra.get("S", 0),
                         extra.get("max_iters", 0))
    o = oracle.run_all(oc, logits, None, want_cooc=False)
    want = oracle.slot_map(oc, o)
    cfg = mp.make_config(T, E, k, R, G, H, B, extra.get("n_slot", 0), extra.get("W", -1), extra.get("S", 0),
                         extra.get("max_iters", 0))
    layer = mp.Layer(cfg, cooc=False)
    layer.route(torch.from_numpy(np.ascontiguousarray(logits)).cuda())
    layer.plan()
    se, sm, isl = layer.slot_map()
    ns = int(layer.sizes.n_slot)
    g = inputs.rng(T + E + P)
    main = g.integers(0, 1 << 16, (E, P), dtype=np.uint16)
    rep = torch.full((R, ns, P), 0x5A5A, dtype=torch.int16, device=layer.device)
    layer.replica_pull(dev16(main), rep)
    grads = g.integers(0, 1 << 16, (R, ns, P), dtype=np.uint16)
    acc = torch.full((R, R, E // R, P), 0x1234, dtype=torch.int16, device=layer.device)
    layer.replica_push(dev16(grads), acc)
    torch.cuda.synchronize()
    assert layer.status() == 0
    np.testing.assert_array_equal(se.cpu().numpy(), want["slot_expert"])
    np.testing.assert_array_equal(sm.cpu().numpy(), want["slot_main"])
    np.testing.assert_array_equal(isl.cpu().numpy(), want["inst_slot"])
    rep_want = np.full((R, ns, P), 0x5A5A, np.uint16)
    oracle.replica_pull(oc, want["slot_expert"], main, rep_want)
    np.testing.assert_array_equal(host16(rep), rep_want)
    acc_want = np.full((R, R, E // R, P), 0x1234, np.uint16)
    oracle.replica_push(oc, want["slot_expert"], grads, acc_want)
    np.testing.assert_array_equal(host16(acc), acc_want)
    layer.close()
    return int((want["slot_expert"] >= 0).sum())


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
@pytest.mark.parametrize("P", [1000, 8192])
def test_each_workload(mp, name, P):
    w = synth.WORKLOADS[name]
    print("slots %s P=%d" % (name, P), flush=True)
    n = check_layer(mp, dict(T=w.T, E=w.E, k=w.k, R=w.R, G=w.G, H=w.H, B=w.B), synth.logits(w), P)
    assert n > 0


@pytest.mark.parametrize("case", range(12))
def test_small_random_layers(mp, case):
    c = inputs.small_configs(4000 + case, 1)[0]
    print("slots small %s" % c, flush=True)
    check_layer(mp, c, inputs.random_logits(case, c["T"], c["E"]), int(inputs.rng(case).choice([1, 7, 8, 24, 20000])))


def test_skew_sweep_point_with_many_slots(mp):
    w = synth.skew_layer(-4, 4)
    print("slots %s" % w.name, flush=True)
    check_layer(mp, dict(T=w.T, E=w.E, k=w.k, R=w.R, G=w.G, H=w.H, B=w.B), synth.logits(w), 64)
