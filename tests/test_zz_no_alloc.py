"""moe_plan_step_static, the step that allocates nothing (its workspace is a fixed
device array of the library), called through the C ABI and checked against
moe_plan_step on a handle: every output byte for byte, on calls in a row with
shrinking inputs (the array keeps each call's leftovers for the next)."""
from __future__ import annotations

import ctypes

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


def tensors(layer):
    r, p, d = layer.route_out, layer.plan_out, layer.dispatch_out
    named = dict(topk_idx=r.topk_idx, topk_val=r.topk_val, expert_count=r.expert_count, omega=r.omega,
                 cooc=r.cooc, trans=r.trans, n_inst=p.n_inst, inst_expert=p.inst_expert, inst_rank=p.inst_rank,
                 inst_load=p.inst_load, rank_load=p.rank_load, quota=p.quota, slot_inst=p.slot_inst,
                 slot_rank=p.slot_rank, perm=d.perm, slot_pos=d.slot_pos, inst_offset=d.inst_offset,
                 rank_offset=d.rank_offset, dispatch=d.dispatch)
    return {k: v for k, v in named.items() if v is not None}


def outputs(layer):
    return {k: v.cpu().numpy() for k, v in tensors(layer).items()}


def one_layer(mp, w, H, layer_index=0):
    """Outputs of moe_plan_step (handle) and of moe_plan_step_static (no handle) on the same
    inputs; with layer_index > 0 the previous layer's top-k gives the transition counts."""
    cfg = mp.make_config(w.T, w.E, w.k, w.R, w.G, H, w.B)
    lgs = synth.all_logits(w)
    dev = torch.device("cuda", torch.cuda.current_device())
    lg = torch.from_numpy(lgs[layer_index]).to(dev)
    hid = torch.from_numpy(synth.hidden(w, H=H).view(np.int16)).to(dev)
    trans = layer_index > 0
    prev = None
    if trans:
        first = mp.Layer(cfg, cooc=False)
        first.route(torch.from_numpy(lgs[layer_index - 1]).to(dev))
        prev = first.route_out.topk_idx
    ref = mp.Layer(cfg, trans=trans)
    ref.step(lg, hid, prev)
    got = mp.Layer(cfg, trans=trans)  # caller-owned output buffers for the static call
    for t in tensors(got).values():  # so that every byte compared below is one the call wrote
        t.view(torch.int16).fill_(-7)
    status = torch.full((1,), -1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    mp.moe_plan_step_static(cfg, ptr(lg), ptr(prev), ptr(hid), got.route_out.struct(), got.plan_out.struct(),
                            got.dispatch_out.struct(), ptr(status), stream)
    torch.cuda.synchronize()
    want, have = outputs(ref), outputs(got)
    assert int(status.item()) == 0
    assert ref.status() == 0
    for k in want:
        assert np.array_equal(have[k], want[k]), "%s: %s differs" % (w.name, k)
    for l in (ref, got):
        l.close()
    return int(want["n_inst"][0])


def test_static_step_matches_the_handle_step(mp):
    # Calls in a row, each smaller than the one before: the 4-layer stack's second layer
    # (with transition counts), the DeepSeek-V3-shaped layer, the Mixtral-shaped layer.
    for name, H, li in (("coupled_4layer", 64, 1), ("deepseek_v3_layer", 128, 0), ("mixtral_tiny", 64, 0)):
        w = synth.WORKLOADS[name]
        print("static step %s T=%d E=%d H=%d layer %d" % (name, w.T, w.E, H, li), flush=True)
        n = one_layer(mp, w, H, li)
        assert n >= w.E
