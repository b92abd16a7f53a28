"""GPU parity: the HIP path against the CPU oracle, byte for byte (tolerance 0).

Every output of every call is compared element by element on the same seeded
inputs: top-k indices and values, expert counts, the routing matrix,
co-selection and transition counts, the instance table, rank loads, quotas,
per-slot instances and positions, the dispatch permutation and offsets, and
the gathered bf16 rows.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
from tests import inputs

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def mp():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import load_balance_planning_amd as m
    m.lib()
    return m


def npy(t):
    return None if t is None else t.detach().cpu().numpy()


def ocfg(c):
    return oracle.make_cfg(c.T, c.E, c.k, c.R, c.G, c.H, c.replica_budget, c.slots_per_rank, c.expert_bytes,
                           c.token_bytes, c.max_refine_iters)


def gpu_layer(mp, cfg, logits=None, topk=None, hidden=None, prev_topk=None, trans=False, cooc=True, fused=False):
    """Run route (or hist) -> plan -> dispatch on the GPU -- as three calls, or as the single
    moe_plan_step call when `fused` -- and return host copies of every output."""
    layer = mp.Layer(cfg, cooc=cooc, trans=trans)
    dev = layer.device
    prev = None if prev_topk is None else torch.from_numpy(np.ascontiguousarray(prev_topk, np.int32)).to(dev)
    hid = torch.from_numpy(np.ascontiguousarray(hidden).view(np.int16)).to(dev)
    if fused:
        assert logits is not None
        layer.step(torch.from_numpy(np.ascontiguousarray(logits)).to(dev), hid, prev)
    else:
        if logits is not None:
            layer.route(torch.from_numpy(np.ascontiguousarray(logits)).to(dev), prev)
            layer.plan()
        else:
            tk = torch.from_numpy(np.ascontiguousarray(topk, np.int32)).to(dev)
            layer.hist(tk, prev)
            layer.plan(topk_idx=tk)  # the route output's routing matrix with the given top-k
        layer.dispatch(hid)
    torch.cuda.synchronize()
    r, p, d = layer.route_out, layer.plan_out, layer.dispatch_out
    out = dict(topk_idx=npy(r.topk_idx), topk_val=npy(r.topk_val), count=npy(r.expert_count), omega=npy(r.omega),
               cooc=npy(r.cooc), trans=npy(r.trans), n_inst=npy(p.n_inst), inst_expert=npy(p.inst_expert),
               inst_rank=npy(p.inst_rank), inst_load=npy(p.inst_load), rank_load=npy(p.rank_load),
               quota=npy(p.quota), slot_inst=npy(p.slot_inst), slot_rank=npy(p.slot_rank), perm=npy(d.perm),
               slot_pos=npy(d.slot_pos), inst_offset=npy(d.inst_offset), rank_offset=npy(d.rank_offset),
               dispatch=npy(d.dispatch).view(np.uint16))
    out["status"] = layer.status()
    layer.close()
    return out


def compare(g, o, what="", check_dispatch=True):
    keys = ["count", "omega", "n_inst", "inst_expert", "inst_rank", "inst_load", "rank_load", "quota",
            "slot_inst", "slot_rank", "perm", "slot_pos", "inst_offset", "rank_offset"]
    if o.get("topk_idx") is not None and g.get("topk_val") is not None and o.get("topk_val") is not None:
        np.testing.assert_array_equal(g["topk_idx"], o["topk_idx"], err_msg=what + " topk_idx")
        np.testing.assert_array_equal(g["topk_val"].view(np.uint32), o["topk_val"].view(np.uint32),
                                      err_msg=what + " topk_val")
    for k in ("cooc", "trans"):
        if o.get(k) is not None and g.get(k) is not None:
            np.testing.assert_array_equal(g[k], o[k], err_msg=what + " " + k)
    for k in keys:
        np.testing.assert_array_equal(np.asarray(g[k]).reshape(-1), np.asarray(o[k]).reshape(-1),
                                      err_msg=what + " " + k)
    if check_dispatch:
        assert np.array_equal(g["dispatch"], o["dispatch"]), what + " dispatch rows differ"
    assert g["status"] == 0, what + " status %d" % g["status"]


def oracle_layer(cfg, logits=None, topk=None, hidden=None, prev_topk=None, want_cooc=True):
    oc = ocfg(cfg)
    if logits is None:
        lg = np.zeros((cfg.T, cfg.E), np.float32)
        for j in range(cfg.k):
            lg[np.arange(cfg.T), topk[:, j]] = np.float32(cfg.k - j)
        r = oracle.route(oc, lg, prev_topk, want_cooc)
        r["topk_val"] = None
    else:
        r = oracle.route(oc, logits, prev_topk, want_cooc)
    p = oracle.plan(oc, r["omega"], r["topk_idx"])
    d = oracle.dispatch(oc, int(p["n_inst"][0]), p["inst_rank"], p["slot_inst"], hidden)
    out = dict(r)
    out.update(p)
    out.update(d)
    return out


# ---------------------------------------------------------------------------
# The five workloads at full size
# ---------------------------------------------------------------------------

def workload_cfg(mp, w, expert_bytes=-1):
    return mp.make_config(w.T, w.E, w.k, w.R, w.G, w.H, w.B, expert_bytes=expert_bytes)


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_workload_full_size_parity(mp, name):
    w = synth.WORKLOADS[name]
    cfg = workload_cfg(mp, w)
    hidden = synth.hidden(w)
    prev = None
    for layer, lg in enumerate(synth.all_logits(w)):
        print("workload %s layer %d T=%d E=%d k=%d R=%d H=%d" % (name, layer, w.T, w.E, w.k, w.R, w.H), flush=True)
        o = oracle_layer(cfg, logits=lg, hidden=hidden, prev_topk=prev)
        g = gpu_layer(mp, cfg, logits=lg, hidden=hidden, prev_topk=prev, trans=prev is not None)
        compare(g, o, "%s layer %d" % (name, layer))
        print("workload %s layer %d, single-call step" % (name, layer), flush=True)
        g = gpu_layer(mp, cfg, logits=lg, hidden=hidden, prev_topk=prev, trans=prev is not None, fused=True)
        compare(g, o, "%s layer %d (moe_plan_step)" % (name, layer))
        prev = o["topk_idx"]


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_workload_forced_inter_node_stage(mp, name):
    """||W|| = 0 makes every remote demand worth a replica, so the inter-node stage always fires."""
    w = synth.WORKLOADS[name]
    cfg = workload_cfg(mp, w, expert_bytes=0)
    cfg.H = 64  # the layout is what this case checks; a narrow row keeps the copy small
    hidden = synth.hidden(w, H=64)
    lg = synth.all_logits(w)[0]
    print("workload %s W=0" % name, flush=True)
    g = gpu_layer(mp, cfg, logits=lg, hidden=hidden)
    o = oracle_layer(cfg, logits=lg, hidden=hidden)
    assert int(o["n_inst"][0]) > w.E
    compare(g, o, name + " W=0")


# ---------------------------------------------------------------------------
# Worked examples and edge cases
# ---------------------------------------------------------------------------

def run_plan_only(mp, cfg, omega):
    """Plan from a given routing matrix (no tokens): T = 0 layers."""
    layer = mp.Layer(cfg, cooc=False, topk_val=False)
    om = torch.from_numpy(np.asarray(omega, np.int32)).to(layer.device)
    layer.plan(om, torch.zeros((0, cfg.k), dtype=torch.int32, device=layer.device))
    torch.cuda.synchronize()
    p = layer.plan_out
    out = {k: npy(getattr(p, k)) for k in ("n_inst", "inst_expert", "inst_rank", "inst_load", "rank_load", "quota")}
    out["status"] = layer.status()
    layer.close()
    return out


def test_fig9_example_on_gpu(mp):
    g = json.load(open(os.path.join(GOLDEN, "fig9_example.json")))
    c = g["config"]
    for over in [{}] + [v["override"] for v in g["variants"]]:
        cc = dict(c, **over)
        cfg = mp.make_config(cc["T"], cc["E"], cc["k"], cc["R"], cc["G"], cc["H"], cc["B"], cc["n_slot"], cc["W"],
                             cc["S"], cc["max_iters"])
        got = run_plan_only(mp, cfg, g["omega"])
        want = oracle.plan(ocfg(cfg), np.asarray(g["omega"], np.int32), np.zeros((0, cc["k"]), np.int32))
        for k in ("n_inst", "inst_expert", "inst_rank", "inst_load", "rank_load", "quota"):
            np.testing.assert_array_equal(got[k].reshape(-1), want[k].reshape(-1), err_msg=str(over) + k)
        assert got["status"] == 0
    ex = g["expected"]
    cfg = mp.make_config(c["T"], c["E"], c["k"], c["R"], c["G"], c["H"], c["B"], c["n_slot"], c["W"], c["S"])
    got = run_plan_only(mp, cfg, g["omega"])
    assert list(got["rank_load"]) == ex["rank_load"] and list(got["inst_expert"]) == ex["inst_expert"]


@pytest.mark.parametrize("fixture", ["stage1_spread_example.json", "quota_order_example.json"])
def test_hand_derived_examples_on_gpu(mp, fixture):
    """The hand-derived stage-1 spreading and quota-order examples, planned on the GPU from their
    routing matrices (no tokens): equal to the oracle and to the fixture's expected values."""
    g = json.load(open(os.path.join(GOLDEN, fixture)))
    c = g["config"]
    for over in [{}] + [v["override"] for v in g.get("variants", [])]:
        cc = dict(c, **over)
        cfg = mp.make_config(cc["T"], cc["E"], cc["k"], cc["R"], cc["G"], cc["H"], cc["B"], cc["n_slot"], cc["W"],
                             cc["S"], cc["max_iters"])
        got = run_plan_only(mp, cfg, g["omega"])
        want = oracle.plan(ocfg(cfg), np.asarray(g["omega"], np.int32), np.zeros((0, cc["k"]), np.int32))
        for k in ("n_inst", "inst_expert", "inst_rank", "inst_load", "rank_load", "quota"):
            np.testing.assert_array_equal(got[k].reshape(-1), want[k].reshape(-1), err_msg=str(over) + k)
        assert got["status"] == 0
        if not over:
            ex = g["expected"]
            assert list(got["rank_load"]) == ex["rank_load"] and list(got["inst_expert"]) == ex["inst_expert"]
            q = got["quota"]
            assert [[int(s), int(i), int(q[s, i])] for s, i in zip(*np.nonzero(q))] == ex["quota_nonzero"]


def test_even_split_example_on_gpu(mp):
    g = json.load(open(os.path.join(GOLDEN, "even_split_example.json")))
    c = g["config"]
    cfg = mp.make_config(c["T"], c["E"], c["k"], c["R"], c["G"], c["H"], c["B"], c["n_slot"], c["W"], c["S"])
    topk = np.asarray(g["topk"], np.int32).reshape(c["T"], c["k"])
    hid = inputs.random_hidden(5, c["T"], c["H"])
    got = gpu_layer(mp, cfg, topk=topk, hidden=hid)
    want = oracle_layer(cfg, topk=topk, hidden=hid)
    compare(got, want, "even split")
    assert list(got["slot_inst"]) == g["expected"]["slot_inst"]


@pytest.mark.parametrize("case", range(24))
def test_small_random_layers(mp, case):
    cfgd = inputs.small_configs(3000 + case, 1)[0]
    cfg = mp.make_config(cfgd["T"], cfgd["E"], cfgd["k"], cfgd["R"], cfgd["G"], cfgd["H"], cfgd["B"],
                         cfgd["n_slot"], cfgd["W"], cfgd["S"], cfgd["max_iters"])
    print("small case %d %s" % (case, cfgd), flush=True)
    hid = inputs.random_hidden(case, cfg.T, cfg.H)
    if case % 2 == 0:
        lg = inputs.random_logits(case, cfg.T, cfg.E, ties=(case % 4 == 0))
        prev = inputs.random_topk(case + 7, cfg.T, cfg.E, cfg.k) if cfg.T > 0 else None
        # every other logits case goes through the single-call step
        got = gpu_layer(mp, cfg, logits=lg, hidden=hid, prev_topk=prev, trans=prev is not None, fused=(case % 4 == 2))
        want = oracle_layer(cfg, logits=lg, hidden=hid, prev_topk=prev)
    else:
        topk = inputs.random_topk(case, cfg.T, cfg.E, cfg.k, skew=1.5)
        got = gpu_layer(mp, cfg, topk=topk, hidden=hid)
        want = oracle_layer(cfg, topk=topk, hidden=hid)
    compare(got, want, "small case %d" % case)


@pytest.mark.parametrize("shape", [(640, 8, 2, 4, 2), (2048, 64, 8, 8, 4), (1536, 128, 6, 32, 8),
                                   (1152, 896, 16, 64, 8), (100 * 8, 256, 8, 8, 8)])
def test_ragged_tiles_and_odd_hidden(mp, shape):
    """Token counts per rank that are not multiples of the 64-token tile, odd hidden sizes."""
    T, E, k, R, G = shape
    for H in (8, 13):
        cfg = mp.make_config(T, E, k, R, G, H, max(2, R // 2), expert_bytes=H)
        lg = inputs.random_logits(T + H, T, E)
        hid = inputs.random_hidden(T, T, H)
        got = gpu_layer(mp, cfg, logits=lg, hidden=hid)
        want = oracle_layer(cfg, logits=lg, hidden=hid)
        compare(got, want, "shape %s H=%d" % (shape, H))


@pytest.mark.parametrize("H", [2048, 2056, 8200])
@pytest.mark.parametrize("fused", [False, True])
def test_row_rounds_of_the_gather(mp, H, fused):
    """Rows at the edges of the gather's store rounds: 256 vectors (one round, the
    one-vector-per-thread instantiation), 257 (the four-vector one with a ragged
    second vector) and 1025 (two passes of four vectors, the second one vector
    long), through the staged dispatch and the assigning gather of the step."""
    T, E, k, R, G = 704, 64, 8, 8, 4
    cfg = mp.make_config(T, E, k, R, G, H, 8)
    lg = inputs.random_logits(H + fused, T, E)
    hid = inputs.random_hidden(H, T, H)
    print("row rounds H=%d fused=%s" % (H, fused), flush=True)
    compare(gpu_layer(mp, cfg, logits=lg, hidden=hid, fused=fused), oracle_layer(cfg, logits=lg, hidden=hid),
            "H=%d fused=%s" % (H, fused))


@pytest.mark.parametrize("k,H,fused", [(8, 7168, True), (8, 7168, False), (16, 7168, True), (12, 2056, True),
                                       (12, 2056, False), (32, 2056, True), (9, 8200, True), (32, 8200, True),
                                       (8, 16400, False), (16, 2048, True)])
def test_row_copy_in_parts(mp, k, H, fused):
    """The row copy in one to four parts per token (about 3584 16-byte vectors written per
    workgroup): column halves of 7168- and 8200-wide rows (an odd 1025 vectors), destination
    halves of short rows at k = 32, both at k >= 16 with long rows (and the four-part cap at
    k = 32), two load rounds per column half at H = 16400; through the staged dispatch and
    the single call, which assigns the slots in a kernel of its own before a copy in parts
    and inside the copy otherwise."""
    T, E, R, G = 640, 64, 8, 4
    cfg = mp.make_config(T, E, k, R, G, H, 8)
    lg = inputs.random_logits(k * 100 + H, T, E)
    hid = inputs.random_hidden(k, T, H)
    print("row copy parts k=%d H=%d fused=%s" % (k, H, fused), flush=True)
    compare(gpu_layer(mp, cfg, logits=lg, hidden=hid, fused=fused), oracle_layer(cfg, logits=lg, hidden=hid),
            "k=%d H=%d fused=%s" % (k, H, fused))


def test_ties_signed_zero_and_infinities(mp):
    T, E, k, R, G = 256, 64, 8, 4, 2
    lg = inputs.random_logits(9, T, E, ties=True)
    lg[0, :] = np.float32(1.0)
    lg[1, ::2] = np.float32(-0.0)
    lg[2, 5], lg[2, 9], lg[2, 40] = np.float32(np.inf), np.float32(-np.inf), np.float32(np.inf)
    cfg = mp.make_config(T, E, k, R, G, 8, 4)
    hid = inputs.random_hidden(9, T, 8)
    compare(gpu_layer(mp, cfg, logits=lg, hidden=hid), oracle_layer(cfg, logits=lg, hidden=hid), "ties")


def test_nan_logit_sets_status(mp):
    T, E, k, R, G = 128, 16, 2, 2, 1
    lg = inputs.random_logits(1, T, E)
    lg[77, 3] = np.float32(np.nan)
    cfg = mp.make_config(T, E, k, R, G, 8, 2)
    layer = mp.Layer(cfg)
    layer.route(torch.from_numpy(lg).to(layer.device))
    assert layer.status() & mp.MOE_STATUS_NAN_LOGIT
    assert layer.status() == 0  # reading clears the word
    layer.close()


def test_degenerate_layers(mp):
    cases = [
        dict(T=0, E=8, k=2, R=4, G=2, H=16, B=4),            # no tokens
        dict(T=512, E=16, k=4, R=4, G=2, H=16, B=0),         # no replica budget: static placement
        dict(T=512, E=8, k=8, R=4, G=2, H=16, B=4),          # k = E
        dict(T=1024, E=32, k=4, R=8, G=8, H=16, B=8),        # one domain: no inter-node stage
        dict(T=1024, E=32, k=4, R=8, G=1, H=16, B=8),        # one rank per domain: no refinement
        dict(T=1024, E=32, k=4, R=8, G=4, H=16, B=8, it=1),  # refinement capped at one move
    ]
    for c in cases:
        cfg = mp.make_config(c["T"], c["E"], c["k"], c["R"], c["G"], c["H"], c["B"], expert_bytes=0,
                             max_refine_iters=c.get("it", 0))
        lg = inputs.random_logits(c["T"], c["T"], c["E"])
        hid = inputs.random_hidden(1, c["T"], c["H"])
        compare(gpu_layer(mp, cfg, logits=lg, hidden=hid), oracle_layer(cfg, logits=lg, hidden=hid), str(c))


@pytest.mark.parametrize("shape", [(2048, 2048, 32, 256, 8, 1024, -1, False), (2048, 2048, 32, 256, 64, 1024, 0, True),
                                   (1024, 256, 8, 256, 1, 1024, 0, False), (4096, 2048, 32, 256, 64, 512, 0, True)])
def test_maximum_supported_sizes(mp, shape):
    """The library's limits: E = 2048, k = 32, R = 256, G up to 64, B = 1024 (expert_bytes 0 makes
    stage 1 spend the whole budget); with the layer-to-layer transition counts."""
    T, E, k, R, G, B, W, fused = shape
    H = 8
    cfg = mp.make_config(T, E, k, R, G, H, B, expert_bytes=W)
    print("max sizes T=%d E=%d k=%d R=%d G=%d B=%d W=%d fused=%s" % shape, flush=True)
    lg = inputs.random_logits(E + R, T, E)
    hid = inputs.random_hidden(T, T, H)
    prev = inputs.random_topk(G, T, E, k)
    got = gpu_layer(mp, cfg, logits=lg, hidden=hid, prev_topk=prev, trans=True, fused=fused)
    want = oracle_layer(cfg, logits=lg, hidden=hid, prev_topk=prev)
    compare(got, want, "max sizes %s" % (shape,))


def test_gpu_runs_are_bitwise_identical(mp):
    w = synth.WORKLOADS["qwen3_layer"]
    cfg = mp.make_config(w.T, w.E, w.k, w.R, w.G, 64, w.B, expert_bytes=0)
    lg = synth.logits(w)
    hid = synth.hidden(w, H=64)
    a = gpu_layer(mp, cfg, logits=lg, hidden=hid)
    b = gpu_layer(mp, cfg, logits=lg, hidden=hid)
    for k, v in a.items():
        if isinstance(v, np.ndarray):
            assert np.array_equal(v, b[k]), k


# ---------------------------------------------------------------------------
# The plan call on its own inputs: a routing matrix and the top-k it counts
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["qwen3_layer", "deepseek_v3_layer", "kimi_layer"])
def test_plan_from_a_given_routing_matrix(mp, name):
    """moe_plan_plan takes the routing matrix and the top-k from the caller (here the oracle's,
    as a gathered matrix would arrive), with no route call on the handle: the plan and the
    dispatch that follows it match the oracle byte for byte."""
    w = synth.WORKLOADS[name]
    cfg = workload_cfg(mp, w, expert_bytes=0)
    cfg.H = 64
    lg = synth.all_logits(w)[0]
    hid = synth.hidden(w, H=64)
    o = oracle_layer(cfg, logits=lg, hidden=hid)
    print("plan from a given matrix: %s" % name, flush=True)
    layer = mp.Layer(cfg, cooc=False, topk_val=False)
    dev = layer.device
    om = torch.from_numpy(np.ascontiguousarray(o["omega"], np.int32)).to(dev)
    tk = torch.from_numpy(np.ascontiguousarray(o["topk_idx"], np.int32)).to(dev)
    layer.plan(om, tk)
    layer.dispatch(torch.from_numpy(hid.view(np.int16)).to(dev))
    torch.cuda.synchronize()
    p, d = layer.plan_out, layer.dispatch_out
    got = {k: npy(getattr(p, k)) for k in ("n_inst", "inst_expert", "inst_rank", "inst_load", "rank_load", "quota",
                                            "slot_inst", "slot_rank")}
    got.update({k: npy(getattr(d, k)) for k in ("perm", "slot_pos", "inst_offset", "rank_offset")})
    for k, v in got.items():
        np.testing.assert_array_equal(v.reshape(-1), np.asarray(o[k]).reshape(-1), err_msg=name + " " + k)
    assert np.array_equal(npy(d.dispatch).view(np.uint16), o["dispatch"]), name + " dispatch rows"
    assert layer.status() == 0
    layer.close()


def test_plan_flags_a_routing_matrix_that_does_not_match_the_top_k(mp):
    """A routing matrix that is not the top-k's own sets MOE_STATUS_BAD_OMEGA (the outputs are
    then unspecified, but every write stays in its buffer); a consistent pair sets nothing."""
    T, E, k, R, G, H = 1024, 32, 4, 8, 4, 8
    cfg = mp.make_config(T, E, k, R, G, H, 8, expert_bytes=0)
    topk = inputs.random_topk(77, T, E, k, skew=1.2)
    o = oracle_layer(cfg, topk=topk, hidden=inputs.random_hidden(3, T, H))
    layer = mp.Layer(cfg, cooc=False, topk_val=False)
    dev = layer.device
    tk = torch.from_numpy(topk).to(dev)
    om = torch.from_numpy(np.ascontiguousarray(o["omega"], np.int32)).to(dev)
    layer.plan(om, tk)
    torch.cuda.synchronize()
    assert layer.status() == 0
    bad = o["omega"].copy()
    bad[3, 5] += 1
    bad[3, 6] -= 1 if bad[3, 6] > 0 else -1
    layer.plan(torch.from_numpy(np.ascontiguousarray(bad, np.int32)).to(dev), tk)
    torch.cuda.synchronize()
    assert layer.status() & mp.MOE_STATUS_BAD_OMEGA
    layer.close()


def test_step_after_a_stale_hip_error(mp):
    """A HIP error left by the caller's own earlier call (here a host-side one: selecting device
    -1) is not reported by the next step, and the step after it plans from the right routing
    matrix: the workspace accumulator the step uses is clean before and after."""
    import ctypes
    w = synth.WORKLOADS["qwen3_layer"]
    cfg = workload_cfg(mp, w)
    cfg.H = 64
    lg = synth.logits(w)
    hid = synth.hidden(w, H=64)
    o = oracle_layer(cfg, logits=lg, hidden=hid)
    layer = mp.Layer(cfg, cooc=False)
    dev = layer.device
    lg_d = torch.from_numpy(lg).to(dev)
    hid_d = torch.from_numpy(hid.view(np.int16)).to(dev)
    torch.cuda.synchronize()
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    assert hip.hipSetDevice(-1) != 0  # leaves a host-side error behind, touches no device state
    for rep in range(2):
        layer.step(lg_d, hid_d)
        torch.cuda.synchronize()
        p, d = layer.plan_out, layer.dispatch_out
        for k in ("n_inst", "inst_expert", "inst_load", "rank_load", "quota", "slot_inst"):
            np.testing.assert_array_equal(npy(getattr(p, k)).reshape(-1), np.asarray(o[k]).reshape(-1),
                                          err_msg="step %d %s" % (rep, k))
        np.testing.assert_array_equal(npy(d.perm), o["perm"], err_msg="step %d perm" % rep)
        assert layer.status() == 0
    layer.close()
