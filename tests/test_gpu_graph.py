"""moe_plan_step captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

The call keeps no state in its handle between calls, so a graph of it can
stand in for the call.  Every replay -- with eager work (the outputs
overwritten with -1) and synchronisations between replays -- must give the
bytes of an eager call on another handle, and leave no status flag.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mp():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import load_balance_planning_amd as m
    m.lib()
    return m


def outputs(layer):
    r, p, d = layer.route_out, layer.plan_out, layer.dispatch_out
    named = dict(topk_idx=r.topk_idx, topk_val=r.topk_val, expert_count=r.expert_count, omega=r.omega,
                 cooc=r.cooc, trans=r.trans, n_inst=p.n_inst,
                 inst_expert=p.inst_expert, inst_rank=p.inst_rank, inst_load=p.inst_load, rank_load=p.rank_load,
                 quota=p.quota, slot_inst=p.slot_inst, slot_rank=p.slot_rank, inst_offset=d.inst_offset,
                 rank_offset=d.rank_offset, perm=d.perm, slot_pos=d.slot_pos, dispatch=d.dispatch)
    return {k: v for k, v in named.items() if v is not None}


@pytest.mark.parametrize("name,H", [("qwen3_layer", 2048), ("deepseek_v3_layer", 256), ("coupled_4layer", 64)])
def test_step_graph_replays_match_the_eager_call(mp, name, H):
    w = synth.WORKLOADS[name]
    print("graph %s H=%d" % (name, H), flush=True)
    cfg = mp.make_config(w.T, w.E, w.k, w.R, w.G, H, w.B)
    dev = torch.device("cuda", torch.cuda.current_device())
    lg = [torch.from_numpy(x).to(dev) for x in synth.all_logits(w)]
    hid = torch.from_numpy(synth.hidden(w, H=H).view(np.int16)).to(dev)
    trans = w.L > 1
    # the last layer of the stack, with the previous layer's top-k when there is one
    prev_layer = mp.Layer(cfg, cooc=False) if trans else None
    prev = None
    if trans:
        prev_layer.step(lg[-2], hid)
        prev = prev_layer.route_out.topk_idx
    eager = mp.Layer(cfg, cooc=True, trans=trans)
    eager.step(lg[-1], hid, prev)
    torch.cuda.synchronize()
    assert eager.status() == 0
    want = {k: v.clone() for k, v in outputs(eager).items()}

    layer = mp.Layer(cfg, cooc=True, trans=trans)
    layer.step(lg[-1], hid, prev)  # one eager call first: kernel attributes are set outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.step(lg[-1], hid, prev)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outputs(layer).values():
            t.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = outputs(layer)
        for k, v in want.items():
            assert torch.equal(got[k], v), "replay %d: %s differs" % (rep, k)
    assert layer.status() == 0
    # and the eager call still gives the same bytes after the replays
    layer.step(lg[-1], hid, prev)
    torch.cuda.synchronize()
    for k, v in want.items():
        assert torch.equal(outputs(layer)[k], v), "eager after replays: %s differs" % k
    del graph
    for l in (layer, eager, prev_layer):
        if l is not None:
            l.close()
