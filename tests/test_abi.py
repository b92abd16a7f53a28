"""The C ABI library loads (no GPU needed) and exports every entry point include/*.h declares;
the host-only size query follows the header's contract."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:int|void)\s+(moe_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


def test_header_declares_the_path():
    assert set(declared_functions()) >= {"moe_plan_create", "moe_plan_route", "moe_plan_plan", "moe_plan_dispatch"}


def test_library_exports_every_declared_symbol():
    import load_balance_planning_amd as m
    lib = m.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", m.lib_path()], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(declared_functions()) <= exported
    assert set(m.EXPORTS) == set(declared_functions())


def test_query_sizes_and_validation():
    import load_balance_planning_amd as m
    s = m.moe_plan_query(m.make_config(32768, 256, 8, 64, 8, 7168, 32))
    assert (s.topk, s.omega, s.pair, s.inst_cap, s.quota) == (262144, 16384, 65536, 288, 64 * 288)
    assert (s.inst_offset, s.rank_offset) == (289, 65)
    # the handle's workspace holds the presence masks and tile prefixes: 512 tiles of 64 tokens, 12 bytes each
    assert s.workspace_bytes >= 512 * 256 * 12
    assert s.dispatch_elems == 32768 * 8 * 7168 and s.n_slot == 1
    assert s.token_bytes == 2 * 7168 and s.expert_bytes == 9 * 7168 * 7168 // 4
    s = m.moe_plan_query(m.make_config(16384, 128, 8, 8, 4, 2048, 16))
    assert s.n_slot == 2
    s = m.moe_plan_query(m.make_config(800, 256, 8, 8, 8, 13, 4))   # 100 tokens per rank: 2 tiles each
    assert s.workspace_bytes >= 16 * 256 * 12
    bad = [m.make_config(100, 8, 2, 3, 1, 16, 0),      # T % R
           m.make_config(96, 9, 2, 3, 2, 16, 0),       # R % G
           m.make_config(96, 8, 9, 4, 2, 16, 0),       # k > E
           m.make_config(96, 8, 2, 4, 2, 0, 0),        # H
           m.make_config(96, 8, 2, 4, 2, 16, -1)]      # B
    for c in bad:
        with pytest.raises(m.MoePlanError) as ei:
            m.moe_plan_query(c)
        assert ei.value.code == m.MOE_ERR_INVALID_ARG
    for c in [m.make_config(1024, 4096, 2, 4, 2, 16, 0), m.make_config(1024, 64, 33, 4, 2, 16, 0),
              m.make_config(1024, 512, 2, 512, 2, 16, 0), m.make_config(1 << 22, 8, 1, 4, 2, 16, 0)]:
        with pytest.raises(m.MoePlanError) as ei:
            m.moe_plan_query(c)
        assert ei.value.code == m.MOE_ERR_UNSUPPORTED


def test_every_call_rejects_a_null_handle_synchronously():
    """Argument errors return MOE_ERR_INVALID_ARG before any device work (so this runs without a GPU)."""
    import load_balance_planning_amd as m
    lib = m.lib()
    calls = {
        "moe_plan_route": (None, None, None, None, None),
        "moe_plan_hist": (None, None, None, None, None),
        "moe_plan_plan": (None, None, None, None, None),
        "moe_plan_dispatch": (None, None, None, None, None),
        "moe_plan_step": (None,) * 8,
        "moe_plan_step_static": (None,) * 9,
        "moe_plan_combine": (None,) * 6,
        "moe_plan_place": (None, None, -1, None, None),
        "moe_plan_dedup_count": (None, None, None, 0, None, None),
        "moe_plan_dedup_dispatch": (None, None, None, 0, None, None, None),
        "moe_plan_quality": (None, None, None, None),
        "moe_plan_predict": (None,) * 8,
        "moe_plan_slot_map": (None, None, None, None),
        "moe_plan_replica_pull": (None, None, None, 0, None, None),
        "moe_plan_replica_push": (None, None, None, 0, None, None),
        "moe_plan_status": (None, None),
        "moe_plan_create": (None, None),
        "moe_plan_query": (None, None),
        "moe_plan_device_info": (0, None),
        "moe_plan_set_events": (None, None, None),
        "moe_plan_set_gather_order": (None, None, None),
    }
    assert set(calls) | {"moe_plan_destroy"} == set(declared_functions())
    for name, args in calls.items():
        assert getattr(lib, name)(*args) == m.MOE_ERR_INVALID_ARG, name
    lib.moe_plan_destroy(None)  # a no-op


def test_static_step_rejects_a_workspace_beyond_its_array():
    """moe_plan_step_static checks, on the host and before any device work, that the
    configuration's workspace fits its fixed 32 MiB array."""
    import ctypes
    import load_balance_planning_amd as m
    lib = m.lib()
    big = m.make_config(1 << 20, 2048, 1, 256, 8, 8, 0)   # 16 384 tiles x 2048 experts of masks
    bufs = [ctypes.c_void_p(16)] * 6
    route = m.moe_route_out(*bufs)
    plan = m.moe_plan_out(*([ctypes.c_void_p(16)] * 8))
    disp = m.moe_dispatch_out(*([ctypes.c_void_p(16)] * 5))
    rc = lib.moe_plan_step_static(ctypes.byref(big), ctypes.c_void_p(16), None, ctypes.c_void_p(16),
                                  ctypes.byref(route), ctypes.byref(plan), ctypes.byref(disp), ctypes.c_void_p(16),
                                  None)
    assert rc == m.MOE_ERR_UNSUPPORTED
