"""GPU parity of the token-shuffle predictor (moe_plan_predict) against the
oracle: predicted ranks, tokens per rank and the locality counts, exactly
(both sides score in IEEE double in slot order, so the argmax is the same
decision)."""
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


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run(mp, cfg_args, cur, X, cnt, table, nxt):
    T, E, k, R, G, H, B = cfg_args
    layer = mp.Layer(mp.make_config(T, E, k, R, G, H, B), cooc=False)
    pred, rt, loc = layer.predict(dev(cur.astype(np.int32)), dev(X.astype(np.int32)), dev(cnt.astype(np.int32)),
                                  None if table is None else dev(table.astype(np.int32)),
                                  None if nxt is None else dev(nxt.astype(np.int32)))
    torch.cuda.synchronize()
    st = layer.status()
    res = pred.cpu().numpy().copy(), rt.cpu().numpy().copy(), loc.cpu().numpy().copy(), st
    layer.close()
    return res


def compare(mp, cfg_args, cur, X, cnt, table, nxt):
    T, E, k, R, G, H, B = cfg_args
    want = oracle.predict(oracle.make_cfg(T, E, k, R, G, H, B), cur, X, cnt, table, nxt)
    pred, rt, loc, st = run(mp, cfg_args, cur, X, cnt, table, nxt)
    assert st == 0
    np.testing.assert_array_equal(pred, want["pred"])
    np.testing.assert_array_equal(rt, want["rank_tokens"])
    if nxt is not None:
        assert (int(loc[0]), int(loc[1])) == (want["local_predicted"], want["local_source"])
    return want


@pytest.mark.parametrize("layer", [0, 1, 2])
def test_coupled_stack_full_size(mp, layer):
    """The 4-layer coupled workload: GPU transition counts feed the GPU predictor."""
    w = synth.WORKLOADS["coupled_4layer"]
    print("predict coupled layer %d -> %d" % (layer, layer + 1), flush=True)
    lg = synth.all_logits(w)
    c = oracle.make_cfg(w.T, w.E, w.k, w.R, w.G, w.H, w.B)
    r0 = oracle.route(c, lg[layer], want_cooc=False)
    r1 = oracle.route(c, lg[layer + 1], prev_topk=r0["topk_idx"], want_cooc=False)
    want = oracle.predict(c, r0["topk_idx"], r1["trans"], r0["count"], None, r1["topk_idx"])
    cfg = mp.make_config(w.T, w.E, w.k, w.R, w.G, w.H, w.B)
    a = mp.Layer(cfg, cooc=False)
    b = mp.Layer(cfg, cooc=False, trans=True)
    a.route(dev(lg[layer]))
    b.route(dev(lg[layer + 1]), prev_topk=a.route_out.topk_idx)
    pred, rt, loc = b.predict(a.route_out.topk_idx, b.route_out.trans, a.route_out.expert_count,
                              topk_next=b.route_out.topk_idx)
    torch.cuda.synchronize()
    assert a.status() == 0 and b.status() == 0
    np.testing.assert_array_equal(pred.cpu().numpy(), want["pred"])
    np.testing.assert_array_equal(rt.cpu().numpy(), want["rank_tokens"])
    assert (int(loc[0]), int(loc[1])) == (want["local_predicted"], want["local_source"])
    print("  locality predicted %.3f, unshuffled %.3f" % (want["local_predicted"] / (w.T * w.k),
                                                          want["local_source"] / (w.T * w.k)), flush=True)
    a.close()
    b.close()


@pytest.mark.parametrize("shape", [(640, 24, 3, 4, 2), (4096, 128, 8, 32, 8), (1024, 2048, 32, 256, 8),
                                   (512, 64, 1, 64, 8), (300, 10, 10, 10, 5), (0, 8, 2, 4, 2), (2048, 896, 16, 64, 8)])
@pytest.mark.parametrize("tabled", [False, True])
def test_random_layers(mp, shape, tabled):
    T, E, k, R, G = shape
    print("predict random T=%d E=%d k=%d R=%d table=%s" % (T, E, k, R, tabled), flush=True)
    g = inputs.rng(T + E + k + R)
    cur = inputs.random_topk(T + 1, T, E, k) if T else np.zeros((0, k), np.int32)
    nxt = inputs.random_topk(T + 2, T, E, k) if T else np.zeros((0, k), np.int32)
    # transitions from an unrelated batch, as when they are gathered earlier
    X = g.integers(0, 40, (E, E)).astype(np.int32)
    cnt = g.integers(0, 60, E).astype(np.int32)
    cnt[::7] = 0
    table = g.integers(0, R, E).astype(np.int32) if tabled else None
    compare(mp, (T, E, k, R, G, 8, 0), cur, X, cnt, table, nxt)


def test_equal_votes_tie_to_the_lowest_rank(mp):
    T, E, k, R = 256, 16, 4, 8
    cur = inputs.random_topk(1, T, E, k)
    pred, rt, _, st = run(mp, (T, E, k, R, 2, 8, 0), cur, np.full((E, E), 3, np.int32), np.full(E, 9, np.int32),
                          None, None)
    assert st == 0 and (pred == 0).all() and rt[0] == T


def test_bad_inputs_set_status(mp):
    T, E, k, R = 128, 16, 2, 4
    cur = inputs.random_topk(2, T, E, k)
    cur[5, 1] = E
    *_, st = run(mp, (T, E, k, R, 2, 8, 0), cur, np.ones((E, E), np.int32), np.ones(E, np.int32), None, None)
    assert st & mp.MOE_STATUS_BAD_TOPK
    table = np.zeros(E, np.int32)
    table[3] = R
    *_, st = run(mp, (T, E, k, R, 2, 8, 0), inputs.random_topk(3, T, E, k), np.ones((E, E), np.int32),
                 np.ones(E, np.int32), table, None)
    assert st & mp.MOE_STATUS_BAD_KEY
