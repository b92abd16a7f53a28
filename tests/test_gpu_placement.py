"""GPU parity of correlated placement (moe_plan_place) and the deduplicated
dispatch (moe_plan_dedup_count / moe_plan_dedup_dispatch) against the CPU
oracle.  Integer results: every output byte-equal; the dispatched rows are
bit copies.
"""
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


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def sym(a):
    u = np.triu(a, 1)
    return (u + u.T).astype(np.int32)


def gpu_place(mp, E, R, C, max_swaps=-1):
    layer = mp.Layer(mp.make_config(R, E, 1, R, 1, 8, 0), cooc=False)
    out = layer.place(dev(C), max_swaps)
    torch.cuda.synchronize()
    st = layer.status()
    res = dict(expert_rank=out.expert_rank.cpu().numpy(), rank_experts=out.rank_experts.cpu().numpy(),
               intra=int(out.intra.item()), n_swaps=int(out.n_swaps.item()), status=st)
    layer.close()
    return res


def check_place(got, want, what):
    assert got["status"] == 0, what
    np.testing.assert_array_equal(got["expert_rank"], want["expert_rank"], err_msg=what)
    np.testing.assert_array_equal(got["rank_experts"], want["rank_experts"], err_msg=what)
    assert got["intra"] == want["intra"], what
    assert got["n_swaps"] == want["n_swaps"], what


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_place_on_each_workload(mp, name):
    w = synth.WORKLOADS[name]
    print("place %s E=%d R=%d" % (name, w.E, w.R), flush=True)
    c = oracle.make_cfg(w.T, w.E, w.k, w.R, w.G, w.H, w.B)
    C = oracle.route(c, synth.logits(w))["cooc"]
    want = oracle.place(c, C)
    check_place(gpu_place(mp, w.E, w.R, C), want, name)


@pytest.mark.parametrize("E,R,hi", [(8, 4, 3), (12, 3, 2), (64, 8, 5), (96, 32, 4), (130, 10, 50), (256, 64, 9),
                                    (512, 16, 3), (1024, 128, 6), (2048, 256, 4), (2048, 8, 1000), (40, 40, 9),
                                    (40, 1, 9), (99, 9, 7), (255, 5, 4), (270, 10, 6), (200, 2, 5), (128, 1, 3),
                                    (384, 12, 5), (1280, 64, 5), (1536, 128, 3)])
def test_place_random_coselection_with_ties(mp, E, R, hi):
    """Small integer weights: many equal gains and scores, so the tie rules decide."""
    print("place random E=%d R=%d" % (E, R), flush=True)
    C = sym(inputs.rng(E * 7 + R).integers(0, hi, (E, E)))
    c = oracle.make_cfg(R, E, 1, R, 1, 8, 0)
    for cap in (-1, 0, 1, 3):
        check_place(gpu_place(mp, E, R, C, cap), oracle.place(c, C, cap), "E=%d R=%d cap=%d" % (E, R, cap))


def sparse_large(E, seed, big, per_row):
    """Small counts plus a few large ones (up to per_row per row, each below big)."""
    g = inputs.rng(seed)
    C = g.integers(0, 3, (E, E))
    for _ in range(E * per_row // 2):
        a, b = g.integers(0, E, 2)
        C[a, b] = g.integers(big // 2, big)
    return sym(C)


@pytest.mark.parametrize("case", ["sparse_past_16_bits", "degrees_past_2^19", "ragged_E", "one_slot_per_lane",
                                  "lds_degrees_past_2^19"])
def test_place_growth_paths_many_experts(mp, case):
    """More experts than an LDS copy holds: the one-wave growth from the int32 rows (degrees below
    2^19, also with single counts past 16 bits and E not a multiple of 64), the one from the 16-bit
    copy (degrees past 2^19, counts within 16 bits), and ranks of three experts; with the rows in
    LDS, degrees between 2^19 and 2^20 (the masked 32-bit keys)."""
    E, R, C = {
        "lds_degrees_past_2^19": lambda: (200, 8, sym(inputs.rng(15).integers(3000, 5000, (200, 200)))),
        "sparse_past_16_bits": lambda: (384, 12, sparse_large(384, 11, 200000, 1)),
        "degrees_past_2^19": lambda: (512, 16, sym(inputs.rng(12).integers(0, 3000, (512, 512)))),
        "ragged_E": lambda: (1000, 8, sym(inputs.rng(13).integers(0, 20, (1000, 1000)))),
        "one_slot_per_lane": lambda: (768, 256, sym(inputs.rng(14).integers(0, 50, (768, 768)))),
    }[case]()
    print("place paths %s E=%d R=%d max deg %d max count %d" % (case, E, R, C.sum(1).max(), C.max()), flush=True)
    c = oracle.make_cfg(R, E, 1, R, 1, 8, 0)
    for cap in (0, 4):
        check_place(gpu_place(mp, E, R, C, cap), oracle.place(c, C, cap), "%s cap=%d" % (case, cap))


@pytest.mark.parametrize("lo,hi", [(10000, 30000), (60000, 70000), (0, 1 << 20)])
def test_place_large_counts(mp, lo, hi):
    """Counts near and past 16 bits, degrees past 2^20 (the 64-bit growth keys)."""
    for E, R in [(64, 8), (130, 13)]:
        print("place large E=%d R=%d lo=%d hi=%d" % (E, R, lo, hi), flush=True)
        C = sym(inputs.rng(E + lo).integers(lo, hi, (E, E)))
        c = oracle.make_cfg(R, E, 1, R, 1, 8, 0)
        check_place(gpu_place(mp, E, R, C), oracle.place(c, C), "E=%d R=%d lo=%d" % (E, R, lo))


@pytest.mark.parametrize("E,R", [(1024, 16), (2048, 64)])
def test_place_large_counts_many_experts(mp, E, R):
    """Counts past 16 bits with many experts: the workgroup growth with four and eight experts
    per thread, the refinement on the 32-bit counts (swaps capped to keep the oracle quick)."""
    print("place large E=%d R=%d" % (E, R), flush=True)
    C = sym(inputs.rng(E + R).integers(30000, 70000, (E, E)))
    c = oracle.make_cfg(R, E, 1, R, 1, 8, 0)
    for cap in (0, 6):
        check_place(gpu_place(mp, E, R, C, cap), oracle.place(c, C, cap), "E=%d R=%d cap=%d" % (E, R, cap))


def test_place_flags_invalid_counts(mp):
    E, R = 32, 4
    C = sym(inputs.rng(3).integers(0, 9, (E, E)))
    C[5, 5] = 2
    got = gpu_place(mp, E, R, C)
    assert got["status"] & mp.MOE_STATUS_BAD_PAIRS
    assert sorted(np.bincount(got["expert_rank"], minlength=R).tolist()) == [E // R] * R


def dedup_case(mp, T, E, k, R, G, H, B, logits, hidden, table_kind):
    c = oracle.make_cfg(T, E, k, R, G, H, B)
    o = oracle.run_all(c, logits, hidden, want_cooc=table_kind == "placed")
    if table_kind == "contiguous":
        keys, table = o["topk_idx"], None
    elif table_kind == "placed":
        keys, table = o["topk_idx"], oracle.place(c, o["cooc"])["expert_rank"]
    elif table_kind == "instances":
        keys, table = o["slot_inst"], o["inst_rank"]
    else:
        keys, table = o["topk_idx"], inputs.rng(T + E).integers(0, R, E).astype(np.int32)
    return c, keys, table


def run_dedup(mp, layer, keys, table, hidden):
    kt = dev(keys.reshape(-1).astype(np.int32))
    tt = None if table is None else dev(table.astype(np.int32))
    if hidden is None:
        return layer.dedup_count(kt, tt)
    return layer.dedup_dispatch(dev(hidden, torch.int16), kt, tt)


@pytest.mark.parametrize("shape", [(256, 16, 3, 4, 2, 8, 2), (640, 24, 4, 8, 4, 13, 4), (4096, 64, 8, 8, 4, 64, 8),
                                   (1152, 96, 16, 32, 8, 24, 16), (192, 8, 8, 4, 2, 16, 0), (0, 8, 2, 4, 2, 8, 1),
                                   (130, 10, 3, 1, 1, 8, 0), (300, 10, 2, 10, 5, 8, 3), (2048, 2048, 32, 256, 8, 8, 1024),
                                   # rows of 256, 257 and 1025 vectors: the edges of the store rounds
                                   (704, 64, 8, 8, 4, 2048, 8), (704, 64, 8, 8, 4, 2056, 8), (320, 64, 8, 8, 4, 8200, 8)])
@pytest.mark.parametrize("kind", ["contiguous", "placed", "instances", "random"])
def test_dedup_against_the_oracle(mp, shape, kind):
    T, E, k, R, G, H, B = shape
    print("dedup %s T=%d E=%d k=%d R=%d H=%d" % (kind, T, E, k, R, H), flush=True)
    lg = inputs.random_logits(T + E + k, T, E)
    hid = inputs.random_hidden(T + 1, T, H)
    c, keys, table = dedup_case(mp, T, E, k, R, G, H, B, lg, hid, kind)
    want = oracle.dedup(c, keys, table)
    lay = oracle.dedup_dispatch(c, keys, table, hid)
    layer = mp.Layer(mp.make_config(T, E, k, R, G, H, B), cooc=False)
    got = run_dedup(mp, layer, keys, table, None)
    torch.cuda.synchronize()
    assert layer.status() == 0
    np.testing.assert_array_equal(got.tok_ranks.cpu().numpy(), want["tok_ranks"])
    np.testing.assert_array_equal(got.rank_rows.cpu().numpy(), want["rank_rows"])
    np.testing.assert_array_equal(got.rank_slots.cpu().numpy(), want["rank_slots"])
    got = run_dedup(mp, layer, keys, table, hid)
    torch.cuda.synchronize()
    assert layer.status() == 0
    n = lay["n_rows"]
    assert int(got.n_rows.item()) == n
    for f in ("row_token", "row_slots", "rank_row_offset", "slot_row"):
        np.testing.assert_array_equal(getattr(got, f).cpu().numpy(), lay[f], err_msg=f)
    np.testing.assert_array_equal(got.ddispatch[:n].cpu().numpy().view(np.uint16), lay["ddispatch"])
    np.testing.assert_array_equal(got.tok_ranks.cpu().numpy(), want["tok_ranks"])
    layer.close()


@pytest.mark.parametrize("name", ["qwen3_layer", "deepseek_v3_layer", "kimi_layer"])
def test_dedup_full_size_with_the_placement(mp, name):
    """Full-size layer: GPU route -> GPU place -> GPU dedup dispatch; the
    layout in full and 256 sampled rows against the oracle."""
    w = synth.WORKLOADS[name]
    print("dedup full size %s" % name, flush=True)
    c = oracle.make_cfg(w.T, w.E, w.k, w.R, w.G, w.H, w.B)
    lg = synth.logits(w)
    o = oracle.route(c, lg)
    pl = oracle.place(c, o["cooc"])
    layer = mp.Layer(mp.make_config(w.T, w.E, w.k, w.R, w.G, w.H, w.B), cooc=True)
    hid = synth.hidden(w)
    hid_t = dev(hid, torch.int16)
    layer.route(dev(lg))
    p = layer.place()
    out = layer.dedup_dispatch(hid_t, key_rank=p.expert_rank)
    torch.cuda.synchronize()
    assert layer.status() == 0
    np.testing.assert_array_equal(p.expert_rank.cpu().numpy(), pl["expert_rank"])
    assert int(p.intra.item()) == pl["intra"]
    want = oracle.dedup(c, o["topk_idx"], pl["expert_rank"])
    lay = oracle.dedup_dispatch(c, o["topk_idx"], pl["expert_rank"], None)
    np.testing.assert_array_equal(out.rank_rows.cpu().numpy(), want["rank_rows"])
    np.testing.assert_array_equal(out.tok_ranks.cpu().numpy(), want["tok_ranks"])
    n = lay["n_rows"]
    assert int(out.n_rows.item()) == n
    for f in ("row_token", "row_slots", "rank_row_offset", "slot_row"):
        np.testing.assert_array_equal(getattr(out, f).cpu().numpy(), lay[f], err_msg=f)
    rows = np.random.default_rng(1).choice(n, 256, replace=False)
    got = out.ddispatch[torch.from_numpy(rows).cuda()].cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, hid[lay["row_token"][rows]])
    layer.close()


def test_dedup_flags_bad_keys(mp):
    T, E, k, R = 128, 16, 2, 4
    layer = mp.Layer(mp.make_config(T, E, k, R, 2, 8, 0), cooc=False)
    keys = inputs.random_topk(1, T, E, k)
    keys[3, 1] = E + 5
    got = layer.dedup_dispatch(dev(inputs.random_hidden(2, T, 8), torch.int16), dev(keys))
    torch.cuda.synchronize()
    assert layer.status() & mp.MOE_STATUS_BAD_KEY
    assert int(got.slot_row[3 * k + 1].item()) == -1
    table = np.zeros(E, np.int32)
    table[4] = R
    layer.dedup_count(dev(inputs.random_topk(2, T, E, k)), dev(table))
    torch.cuda.synchronize()
    assert layer.status() & mp.MOE_STATUS_BAD_KEY
    layer.close()
