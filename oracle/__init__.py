"""CPU oracle of the MoE dispatch-planning path -- TEST INFRASTRUCTURE ONLY.

A ctypes wrapper around oracle/libmoe_oracle.so (plain single-threaded C++).
Only tests/, the smoke check and the benchmark's CPU-baseline leg may use it.
The product library never imports it and shares no code with it.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


class OracleCfg(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("R", ctypes.c_int32), ("G", ctypes.c_int32), ("H", ctypes.c_int32),
                ("B", ctypes.c_int32), ("n_slot", ctypes.c_int32),
                ("W", ctypes.c_int64), ("S", ctypes.c_int64), ("max_iters", ctypes.c_int32)]


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def lib(path: str | None = None):
    global _LIB
    if path is not None:
        return _setup(ctypes.CDLL(path))
    if _LIB is None:
        alt = os.environ.get("MOE_ORACLE_LIB")  # a mutant build, used by the pin self-test
        if alt:
            _LIB = _setup(ctypes.CDLL(alt))
            return _LIB
        if not os.path.exists(_build.LIB):
            _build.build()
        _LIB = _setup(ctypes.CDLL(_build.LIB))
    return _LIB


def _setup(l):
    vp = ctypes.c_void_p
    l.oracle_params.argtypes = [vp, vp]
    l.oracle_domain_budget.argtypes = [vp, vp]
    l.oracle_route.argtypes = [vp] * 9
    l.oracle_plan.argtypes = [vp] * 12 + [ctypes.c_int32, vp]
    l.oracle_dispatch.argtypes = [vp, ctypes.c_int32] + [vp] * 9
    l.oracle_combine.argtypes = [vp] * 5
    l.oracle_place.argtypes = [vp, vp, ctypes.c_int32, vp, vp, vp, vp]
    l.oracle_dedup.argtypes = [vp, vp, vp, ctypes.c_int32, vp, vp, vp]
    l.oracle_dedup_dispatch.argtypes = [vp, vp, vp, ctypes.c_int32] + [vp] * 7
    l.oracle_quality.argtypes = [vp, ctypes.c_int32] + [vp] * 5
    l.oracle_predict.argtypes = [vp] * 9
    l.oracle_slot_map.argtypes = [vp, ctypes.c_int32] + [vp] * 5
    l.oracle_replica_pull.argtypes = [vp, vp, vp, ctypes.c_int64, vp]
    l.oracle_replica_push.argtypes = [vp, vp, vp, ctypes.c_int64, vp]
    for f in (l.oracle_params, l.oracle_domain_budget, l.oracle_route, l.oracle_plan, l.oracle_dispatch,
              l.oracle_combine, l.oracle_place, l.oracle_dedup, l.oracle_dedup_dispatch, l.oracle_quality,
              l.oracle_predict, l.oracle_slot_map, l.oracle_replica_pull, l.oracle_replica_push):
        f.restype = ctypes.c_int
    return l


def make_cfg(T, E, k, R, G, H, B, n_slot=0, W=-1, S=0, max_iters=0) -> OracleCfg:
    return OracleCfg(T, E, k, R, G, H, B, n_slot, W, S, max_iters)


def params(cfg: OracleCfg, l=None) -> dict:
    l = l or lib()
    out = np.zeros(8, dtype=np.int64)
    rc = l.oracle_params(ctypes.byref(cfg), _p(out))
    if rc != 0:
        raise ValueError("invalid oracle configuration (%d)" % rc)
    M = int(out[0])
    bd = np.zeros(M, dtype=np.int32)
    l.oracle_domain_budget(ctypes.byref(cfg), _p(bd))
    return dict(M=M, Tr=int(out[1]), Er=int(out[2]), n_slot=int(out[3]), S=int(out[4]), W=int(out[5]),
                max_iters=int(out[6]), B=int(out[7]), Bd=bd)


def route(cfg: OracleCfg, logits: np.ndarray, prev_topk: np.ndarray | None = None,
          want_cooc: bool = True, l=None) -> dict:
    l = l or lib()
    T, E, k, R = cfg.T, cfg.E, cfg.k, cfg.R
    logits = np.ascontiguousarray(logits, dtype=np.float32).reshape(T, E)
    out = dict(topk_idx=np.zeros((T, k), np.int32), topk_val=np.zeros((T, k), np.float32),
               count=np.zeros(E, np.int32), omega=np.zeros((R, E), np.int32))
    out["cooc"] = np.zeros((E, E), np.int32) if want_cooc else None
    if prev_topk is not None:
        prev_topk = np.ascontiguousarray(prev_topk, dtype=np.int32).reshape(T, k)
        out["trans"] = np.zeros((E, E), np.int32)
    else:
        out["trans"] = None
    rc = l.oracle_route(ctypes.byref(cfg), _p(logits), _p(prev_topk), _p(out["topk_idx"]), _p(out["topk_val"]),
                        _p(out["count"]), _p(out["omega"]), _p(out["cooc"]), _p(out["trans"]))
    out["status"] = rc
    if rc not in (0, -4):
        raise ValueError("oracle_route failed (%d)" % rc)
    return out


def plan(cfg: OracleCfg, omega: np.ndarray, topk_idx: np.ndarray, trace_cap: int = 0, l=None) -> dict:
    l = l or lib()
    T, E, k, R, B = cfg.T, cfg.E, cfg.k, cfg.R, cfg.B
    cap = E + B
    omega = np.ascontiguousarray(omega, dtype=np.int32).reshape(R, E)
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32).reshape(T, k)
    out = dict(n_inst=np.zeros(1, np.int32), inst_expert=np.zeros(cap, np.int32),
               inst_rank=np.zeros(cap, np.int32), inst_load=np.zeros(cap, np.int32),
               rank_load=np.zeros(R, np.int32), quota=np.zeros((R, cap), np.int32),
               slot_inst=np.zeros(T * k, np.int32), rank_load_stage1=np.zeros(R, np.int32))
    trace = np.zeros((max(trace_cap, 1), 7), np.int32)
    ntr = np.zeros(1, np.int32)
    rc = l.oracle_plan(ctypes.byref(cfg), _p(omega), _p(topk_idx), _p(out["n_inst"]), _p(out["inst_expert"]),
                       _p(out["inst_rank"]), _p(out["inst_load"]), _p(out["rank_load"]), _p(out["quota"]),
                       _p(out["slot_inst"]), _p(out["rank_load_stage1"]),
                       _p(trace) if trace_cap > 0 else None, trace_cap, _p(ntr))
    if rc != 0:
        raise ValueError("oracle_plan failed (%d)" % rc)
    out["n_iters"] = int(ntr[0])
    out["trace"] = trace[:min(int(ntr[0]), trace_cap)] if trace_cap > 0 else None
    return out


def dispatch(cfg: OracleCfg, n_inst: int, inst_rank: np.ndarray, slot_inst: np.ndarray,
             hidden: np.ndarray | None, l=None) -> dict:
    l = l or lib()
    T, k, R, H, cap = cfg.T, cfg.k, cfg.R, cfg.H, cfg.E + cfg.B
    N = T * k
    inst_rank = np.ascontiguousarray(inst_rank, dtype=np.int32)
    slot_inst = np.ascontiguousarray(slot_inst, dtype=np.int32).reshape(N)
    out = dict(perm=np.zeros(N, np.int32), slot_pos=np.zeros(N, np.int32),
               inst_offset=np.zeros(cap + 1, np.int32), rank_offset=np.zeros(R + 1, np.int32),
               slot_rank=np.zeros(N, np.int32))
    disp = None
    if hidden is not None:
        hidden = np.ascontiguousarray(hidden, dtype=np.uint16).reshape(T, H)
        disp = np.zeros((N, H), np.uint16)
    rc = l.oracle_dispatch(ctypes.byref(cfg), int(n_inst), _p(inst_rank), _p(slot_inst), _p(hidden),
                           _p(out["perm"]), _p(out["slot_pos"]), _p(out["inst_offset"]), _p(out["rank_offset"]),
                           _p(out["slot_rank"]), _p(disp))
    if rc != 0:
        raise ValueError("oracle_dispatch failed (%d)" % rc)
    out["dispatch"] = disp
    return out


def combine(cfg: OracleCfg, topk_val: np.ndarray, slot_pos: np.ndarray, expert_out: np.ndarray, l=None) -> np.ndarray:
    """Gate-weighted combine in float64 (see oracle_combine); expert_out holds bf16 bit patterns."""
    l = l or lib()
    T, k, H = cfg.T, cfg.k, cfg.H
    v = np.ascontiguousarray(topk_val, np.float32).reshape(T, k)
    sp = np.ascontiguousarray(slot_pos, np.int32).reshape(T * k)
    x = np.ascontiguousarray(expert_out).view(np.uint16).reshape(T * k, H)
    out = np.zeros((T, H), np.float64)
    rc = l.oracle_combine(ctypes.byref(cfg), _p(v), _p(sp), _p(x), _p(out))
    if rc != 0:
        raise ValueError("oracle_combine failed (%d)" % rc)
    return out


def place(cfg: OracleCfg, cooc: np.ndarray, max_swaps: int = -1, l=None) -> dict:
    """Correlated expert placement (see oracle_place)."""
    l = l or lib()
    E, R = cfg.E, cfg.R
    C = np.ascontiguousarray(cooc, np.int32).reshape(E, E)
    out = dict(expert_rank=np.zeros(E, np.int32), rank_experts=np.zeros((R, E // R), np.int32))
    intra = np.zeros(1, np.int64)
    ns = np.zeros(1, np.int32)
    rc = l.oracle_place(ctypes.byref(cfg), _p(C), int(max_swaps), _p(out["expert_rank"]), _p(out["rank_experts"]),
                        _p(intra), _p(ns))
    if rc != 0:
        raise ValueError("oracle_place failed (%d)" % rc)
    out["intra"] = int(intra[0])
    out["n_swaps"] = int(ns[0])
    return out


def _keys(cfg, slot_key, key_rank):
    sk = np.ascontiguousarray(slot_key, np.int32).reshape(cfg.T * cfg.k)
    kr = None if key_rank is None else np.ascontiguousarray(key_rank, np.int32).reshape(-1)
    return sk, kr, (0 if kr is None else int(kr.size))


def dedup(cfg: OracleCfg, slot_key: np.ndarray, key_rank: np.ndarray | None = None, l=None) -> dict:
    """Deduplicated row counts (see oracle_dedup)."""
    l = l or lib()
    T, R = cfg.T, cfg.R
    sk, kr, nk = _keys(cfg, slot_key, key_rank)
    out = dict(tok_ranks=np.zeros(T, np.int32), rank_rows=np.zeros((R, R), np.int32),
               rank_slots=np.zeros((R, R), np.int32))
    rc = l.oracle_dedup(ctypes.byref(cfg), _p(sk), _p(kr), nk, _p(out["tok_ranks"]), _p(out["rank_rows"]),
                        _p(out["rank_slots"]))
    if rc != 0:
        raise ValueError("oracle_dedup failed (%d)" % rc)
    return out


def dedup_dispatch(cfg: OracleCfg, slot_key: np.ndarray, key_rank: np.ndarray | None = None,
                   hidden: np.ndarray | None = None, l=None) -> dict:
    """Deduplicated dispatch layout and row copy (see oracle_dedup_dispatch)."""
    l = l or lib()
    T, k, R, H = cfg.T, cfg.k, cfg.R, cfg.H
    N = T * k
    sk, kr, nk = _keys(cfg, slot_key, key_rank)
    out = dict(n_rows=np.zeros(1, np.int32), row_token=np.zeros(N, np.int32), row_slots=np.zeros(N, np.int32),
               rank_row_offset=np.zeros(R + 1, np.int32), slot_row=np.zeros(N, np.int32))
    disp = None
    if hidden is not None:
        hidden = np.ascontiguousarray(hidden, np.uint16).reshape(T, H)
        disp = np.zeros((N, H), np.uint16)
    rc = l.oracle_dedup_dispatch(ctypes.byref(cfg), _p(sk), _p(kr), nk, _p(hidden), _p(out["n_rows"]),
                                 _p(out["row_token"]), _p(out["row_slots"]), _p(out["rank_row_offset"]),
                                 _p(out["slot_row"]), _p(disp))
    if rc != 0:
        raise ValueError("oracle_dedup_dispatch failed (%d)" % rc)
    out["n_rows"] = int(out["n_rows"][0])
    out["ddispatch"] = None if disp is None else disp[:out["n_rows"]]
    return out


QUALITY_FIELDS = ("assignments", "same_rank", "same_node", "other_node", "replica_served", "max_rank_load",
                  "min_rank_load", "replicas")


def quality(cfg: OracleCfg, plan_out: dict, l=None) -> dict:
    """Plan-quality counters of a plan (see oracle_quality), plus the imbalance max / mean."""
    l = l or lib()
    cap = cfg.E + cfg.B
    out = np.zeros(8, np.int64)
    args = [np.ascontiguousarray(plan_out[k], np.int32) for k in ("inst_expert", "inst_rank", "rank_load")]
    quota = np.ascontiguousarray(plan_out["quota"], np.int32).reshape(cfg.R, cap)
    rc = l.oracle_quality(ctypes.byref(cfg), int(np.asarray(plan_out["n_inst"]).reshape(-1)[0]), _p(args[0]),
                          _p(args[1]), _p(args[2]), _p(quota), _p(out))
    if rc != 0:
        raise ValueError("oracle_quality failed (%d)" % rc)
    res = {k: int(v) for k, v in zip(QUALITY_FIELDS, out)}
    res["imbalance"] = res["max_rank_load"] * cfg.R / res["assignments"] if res["assignments"] else 1.0
    return res


def predict(cfg: OracleCfg, topk_cur: np.ndarray, trans: np.ndarray, count_cur: np.ndarray,
            key_rank: np.ndarray | None = None, topk_next: np.ndarray | None = None, l=None) -> dict:
    """Token-shuffle prediction (see oracle_predict)."""
    l = l or lib()
    T, E, k, R = cfg.T, cfg.E, cfg.k, cfg.R
    cur = np.ascontiguousarray(topk_cur, np.int32).reshape(T, k)
    X = np.ascontiguousarray(trans, np.int32).reshape(E, E)
    cnt = np.ascontiguousarray(count_cur, np.int32).reshape(E)
    kr = None if key_rank is None else np.ascontiguousarray(key_rank, np.int32).reshape(E)
    nxt = None if topk_next is None else np.ascontiguousarray(topk_next, np.int32).reshape(T, k)
    out = dict(pred=np.zeros(T, np.int32), rank_tokens=np.zeros(R, np.int32))
    local = np.zeros(2, np.int64)
    rc = l.oracle_predict(ctypes.byref(cfg), _p(cur), _p(X), _p(cnt), _p(kr), _p(nxt), _p(out["pred"]),
                          _p(out["rank_tokens"]), _p(local))
    if rc != 0:
        raise ValueError("oracle_predict failed (%d)" % rc)
    out["local_predicted"], out["local_source"] = int(local[0]), int(local[1])
    return out


def slot_map(cfg: OracleCfg, plan_out: dict, l=None) -> dict:
    """Replica slot map of a plan (see oracle_slot_map)."""
    l = l or lib()
    ns = params(cfg, l)["n_slot"]
    R, cap = cfg.R, cfg.E + cfg.B
    out = dict(slot_expert=np.zeros((R, ns), np.int32), slot_main=np.zeros((R, ns), np.int32),
               inst_slot=np.zeros(cap, np.int32))
    ie = np.ascontiguousarray(plan_out["inst_expert"], np.int32)
    ir = np.ascontiguousarray(plan_out["inst_rank"], np.int32)
    rc = l.oracle_slot_map(ctypes.byref(cfg), int(np.asarray(plan_out["n_inst"]).reshape(-1)[0]), _p(ie), _p(ir),
                           _p(out["slot_expert"]), _p(out["slot_main"]), _p(out["inst_slot"]))
    if rc != 0:
        raise ValueError("oracle_slot_map failed (%d)" % rc)
    return out


def replica_pull(cfg: OracleCfg, slot_expert: np.ndarray, main_params: np.ndarray, replica_params: np.ndarray,
                 l=None) -> np.ndarray:
    """replica_params [R][N_slot][P] (modified in place and returned) from main_params [E][P]."""
    l = l or lib()
    P = main_params.shape[-1]
    se = np.ascontiguousarray(slot_expert, np.int32)
    mp_ = np.ascontiguousarray(main_params, np.uint16)
    assert replica_params.flags.c_contiguous and replica_params.dtype == np.uint16
    rc = l.oracle_replica_pull(ctypes.byref(cfg), _p(se), _p(mp_), int(P), _p(replica_params))
    if rc != 0:
        raise ValueError("oracle_replica_pull failed (%d)" % rc)
    return replica_params


def replica_push(cfg: OracleCfg, slot_expert: np.ndarray, replica_grads: np.ndarray, grad_accum: np.ndarray,
                 l=None) -> np.ndarray:
    """grad_accum [R][R][E/R][P] (modified in place and returned) from replica_grads [R][N_slot][P]."""
    l = l or lib()
    P = replica_grads.shape[-1]
    se = np.ascontiguousarray(slot_expert, np.int32)
    rg = np.ascontiguousarray(replica_grads, np.uint16)
    assert grad_accum.flags.c_contiguous and grad_accum.dtype == np.uint16
    rc = l.oracle_replica_push(ctypes.byref(cfg), _p(se), _p(rg), int(P), _p(grad_accum))
    if rc != 0:
        raise ValueError("oracle_replica_push failed (%d)" % rc)
    return grad_accum


def run_all(cfg: OracleCfg, logits: np.ndarray, hidden: np.ndarray | None,
            prev_topk: np.ndarray | None = None, want_cooc: bool = True, l=None) -> dict:
    """route -> plan -> dispatch for one layer; returns every output in one dict."""
    r = route(cfg, logits, prev_topk, want_cooc, l=l)
    p = plan(cfg, r["omega"], r["topk_idx"], l=l)
    d = dispatch(cfg, int(p["n_inst"][0]), p["inst_rank"], p["slot_inst"], hidden, l=l)
    out = {}
    out.update(r)
    out.update(p)
    out.update(d)
    return out
