"""Parity in the launch configuration bench.py times: two handles on two
streams, consecutive steps alternating between them with no synchronisation
in between, at full size (the DeepSeek-V3-shaped layer with and without the
copies taking turns, the Kimi-K2-shaped one and the 4-layer stack with them).

The two handles plan two different batches (the workload's logits and those
of the same recipe with another seed), so a handle that read the other's
buffers would show.  After every step its outputs are copied aside on its own
stream (the integers whole, 4096 sampled rows of the dispatch buffer), and
afterwards every copy is checked against the oracle: the integers byte for
byte, each sampled row against its definition, hidden[perm[p] / k].
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth

pytestmark = pytest.mark.gpu

INT_OUTPUTS = ("topk_idx", "expert_count", "omega", "cooc", "n_inst", "inst_expert", "inst_rank", "inst_load",
               "rank_load", "quota", "slot_inst", "slot_rank", "inst_offset", "rank_offset", "perm", "slot_pos")


@pytest.fixture(scope="module")
def mp():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import load_balance_planning_amd as m
    m.lib()
    return m


def small_outputs(layer):
    r, p, d = layer.route_out, layer.plan_out, layer.dispatch_out
    out = dict(topk_idx=r.topk_idx, expert_count=r.expert_count, omega=r.omega, cooc=r.cooc, n_inst=p.n_inst,
               inst_expert=p.inst_expert, inst_rank=p.inst_rank, inst_load=p.inst_load, rank_load=p.rank_load,
               quota=p.quota, slot_inst=p.slot_inst, slot_rank=p.slot_rank, inst_offset=d.inst_offset,
               rank_offset=d.rank_offset, perm=d.perm, slot_pos=d.slot_pos)
    if r.trans is not None:
        out["trans"] = r.trans
    return out


_EXPECTED = {}


def expected(name):
    """The oracle's outputs of every layer of two batches of the workload (the second with
    another seed); a layer after the first also gets the previous layer's top-k."""
    if name in _EXPECTED:
        return _EXPECTED[name]
    w = synth.WORKLOADS[name]
    batches = [w, dataclasses.replace(w, seed=1)]
    ocfg = oracle.make_cfg(w.T, w.E, w.k, w.R, w.G, w.H, w.B)
    logits = [synth.all_logits(b) for b in batches]
    want = []
    for i, lgs in enumerate(logits):
        print("pipeline: oracle for batch %d (%d layers)" % (i, w.L), flush=True)
        layers = []
        for l, lg in enumerate(lgs):
            prev = layers[l - 1]["topk_idx"] if l > 0 else None
            layers.append(oracle.run_all(ocfg, lg, None, prev_topk=prev, want_cooc=True))
        want.append(layers)
    assert not np.array_equal(want[0][0]["slot_pos"], want[1][0]["slot_pos"])
    _EXPECTED[name] = (w, logits, synth.hidden(w), want)
    return _EXPECTED[name]


@pytest.mark.parametrize("name,ordered", [("deepseek_v3_layer", False), ("deepseek_v3_layer", True),
                                          ("kimi_layer", True), ("coupled_4layer", True)])
def test_two_stream_pipeline_full_size(mp, name, ordered):
    """With ordered, the two handles' row copies take turns (moe_plan_set_gather_order), as
    bench.py runs them, and their solver launches take the workgroup size and LDS budget meant
    for running beside the other handle's copy (on the Kimi-K2-shaped layer the domain demand
    then lives in global memory).  The 4-layer stack runs every layer per step, each after the
    first with the previous layer's top-k and transition counts, as bench.py does."""
    w, logits, hidden, want = expected(name)
    cfg = mp.make_config(w.T, w.E, w.k, w.R, w.G, w.H, w.B)
    dev = torch.device("cuda", torch.cuda.current_device())
    hid = torch.from_numpy(hidden.view(np.int16)).to(dev)
    lgs = [[torch.from_numpy(lg).to(dev) for lg in b] for b in logits]
    sets = [[mp.Layer(cfg, device=dev, cooc=True, trans=(l > 0)) for l in range(w.L)] for _ in range(2)]
    streams = [torch.cuda.current_stream(dev), torch.cuda.Stream(dev)]
    turn = [torch.cuda.Event(), torch.cuda.Event()]
    for ev in turn:
        ev.record(streams[0])
    if ordered:
        for i in range(2):
            for layer in sets[i]:
                layer.order_gather(wait=turn[1 - i], done=turn[i])
    rng = np.random.default_rng(11)
    rows = torch.from_numpy(rng.choice(w.T * w.k, 4096, replace=False).astype(np.int64)).to(dev)
    torch.cuda.synchronize()
    copies = []
    n_steps = 6
    print("pipeline: %d alternating steps on two streams (ordered copies: %s)" % (n_steps, ordered), flush=True)
    for s in range(n_steps):
        i = s % 2
        with torch.cuda.stream(streams[i]):
            for l, layer in enumerate(sets[i]):
                prev = sets[i][l - 1].route_out.topk_idx if l > 0 else None
                layer.step(lgs[i][l], hid, prev)
                snap = {k: v.clone() for k, v in small_outputs(layer).items()}
                snap["rows"] = layer.dispatch_out.dispatch.index_select(0, rows)
                copies.append((i, l, snap))
    torch.cuda.synchronize()
    for layer in sets[0] + sets[1]:
        layer.order_gather()
        assert layer.status() == 0
    rows_np = rows.cpu().numpy()
    for s, (i, l, snap) in enumerate(copies):
        o = want[i][l]
        for k in INT_OUTPUTS + (("trans",) if l > 0 else ()):
            ok = "count" if k == "expert_count" else k
            np.testing.assert_array_equal(snap[k].cpu().numpy().reshape(-1), np.asarray(o[ok]).reshape(-1),
                                          err_msg="copy %d (handle %d, layer %d): %s" % (s, i, l, k))
        expect = hidden[o["perm"][rows_np] // w.k]
        np.testing.assert_array_equal(snap["rows"].cpu().numpy().view(np.uint16), expect,
                                      err_msg="copy %d (handle %d, layer %d): dispatch rows" % (s, i, l))
    for layer in sets[0] + sets[1]:
        layer.close()
