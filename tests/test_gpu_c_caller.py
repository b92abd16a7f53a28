"""The C ABI from a caller with no Python and no torch (tests/c_abi_caller.cpp:
hipMalloc'd buffers, its own stream), run as a child process.  It runs the path
three ways on one handle -- moe_plan_step; route, plan and dispatch as three
calls; plan and dispatch from a routing matrix and top-k it is handed -- and
every output of every way must equal the oracle's byte for byte."""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

import oracle
from tests import inputs

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi_caller")
OUTPUTS = {"topk_idx": np.int32, "topk_val": np.float32, "count": np.int32, "omega": np.int32, "cooc": np.int32,
           "n_inst": np.int32, "inst_expert": np.int32, "inst_rank": np.int32, "inst_load": np.int32,
           "rank_load": np.int32, "quota": np.int32, "slot_inst": np.int32, "slot_rank": np.int32,
           "inst_offset": np.int32, "rank_offset": np.int32, "perm": np.int32, "slot_pos": np.int32,
           "dispatch": np.uint16}


PLAN_DISPATCH = ("n_inst", "inst_expert", "inst_rank", "inst_load", "rank_load", "quota", "slot_inst", "slot_rank",
                 "inst_offset", "rank_offset", "perm", "slot_pos", "dispatch")


@pytest.mark.parametrize("shape", [(4096, 64, 4, 8, 4, 64, 8), (1600, 256, 8, 16, 8, 24, 16)])
def test_c_caller_matches_the_oracle(tmp_path, shape):
    if not os.path.exists(EXE):  # built by __graft_entry__.build(); built here only when missing
        import load_balance_planning_amd as m
        from tests import c_caller_build
        m.lib()  # the library it links against
        c_caller_build.build()
    T, E, k, R, G, H, B = shape
    print("C caller T=%d E=%d k=%d R=%d G=%d H=%d B=%d" % shape, flush=True)
    lg = inputs.random_logits(T + E, T, E)
    hid = inputs.random_hidden(T + H, T, H)
    o = oracle.run_all(oracle.make_cfg(T, E, k, R, G, H, B), lg, hid)
    (tmp_path / "cfg.txt").write_text("%d %d %d %d %d %d %d\n" % shape)
    lg.astype(np.float32).tofile(tmp_path / "logits.f32")
    hid.astype(np.uint16).tofile(tmp_path / "hidden.u16")
    np.ascontiguousarray(o["omega"], np.int32).tofile(tmp_path / "omega.i32")
    np.ascontiguousarray(o["topk_idx"], np.int32).tofile(tmp_path / "topk.i32")
    r = subprocess.run([EXE, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
    for way, names in (("step", tuple(OUTPUTS)), ("staged", tuple(OUTPUTS)), ("given", PLAN_DISPATCH)):
        for name in names:
            dt = OUTPUTS[name]
            got = np.fromfile(tmp_path / ("%s_%s.bin" % (way, name)), dtype=dt)
            want = np.ascontiguousarray(o[name]).astype(dt).reshape(-1)
            if dt is np.float32:
                got, want = got.view(np.uint32), want.view(np.uint32)
            np.testing.assert_array_equal(got, want, err_msg="%s %s" % (way, name))
