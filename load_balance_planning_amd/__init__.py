"""MI355X-native expert-parallel dispatch planning for MoE layers.

A thin ctypes binding of the C ABI in include/moe_plan.h (library
load_balance_planning_amd/libmoe_plan.so, HIP kernels for gfx950).  The
functions named like the C entry points only marshal arguments; every step of
the path runs in the library's kernels.  `Layer` is a convenience wrapper that
allocates the caller-owned buffers as torch tensors on the current HIP device
and runs the calls on torch's current stream -- PyTorch is used for device
memory and streams only.

There is no CPU fallback: the first call loads the HIP library (building it
in-tree with hipcc when none is there yet), and when it can be neither loaded
nor built that call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

from . import build as _build

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_HIP = -3
MOE_ERR_NONFINITE = -4
MOE_ERR_INTERNAL = -5
MOE_STATUS_NAN_LOGIT = 1
MOE_STATUS_PLAN_CHECK = 2
MOE_STATUS_BAD_TOPK = 4
MOE_STATUS_BAD_PAIRS = 8
MOE_STATUS_BAD_KEY = 16
MOE_STATUS_BAD_OMEGA = 32

_ERRORS = {MOE_ERR_INVALID_ARG: "invalid argument", MOE_ERR_UNSUPPORTED: "unsupported configuration",
           MOE_ERR_HIP: "HIP runtime error", MOE_ERR_NONFINITE: "non-finite gate logit",
           MOE_ERR_INTERNAL: "internal error"}


class MoePlanError(RuntimeError):
    def __init__(self, call: str, code: int):
        super().__init__("%s failed: %s (%d)" % (call, _ERRORS.get(code, "error"), code))
        self.code = code


class moe_plan_config(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("R", ctypes.c_int32),
                ("G", ctypes.c_int32), ("H", ctypes.c_int32), ("replica_budget", ctypes.c_int32),
                ("slots_per_rank", ctypes.c_int32), ("expert_bytes", ctypes.c_int64),
                ("token_bytes", ctypes.c_int64), ("max_refine_iters", ctypes.c_int32)]


class moe_plan_sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "topk", "omega", "experts", "pair", "inst_cap", "quota", "inst_offset",
        "rank_offset", "dispatch_elems", "n_slot", "expert_bytes", "token_bytes", "max_refine_iters",
        "workspace_bytes")]


class moe_route_out(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "topk_idx", "topk_val", "expert_count", "omega", "cooc", "trans")]


class moe_plan_out(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "n_inst", "inst_expert", "inst_rank", "inst_load", "rank_load", "quota", "slot_inst", "slot_rank")]


class moe_dispatch_out(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("perm", "slot_pos", "inst_offset", "rank_offset", "dispatch")]


class moe_place_out(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("expert_rank", "rank_experts", "intra", "n_swaps")]


class moe_predict_out(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("pred", "rank_tokens", "local")]


class moe_slot_out(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("slot_expert", "slot_main", "inst_slot")]


class moe_dedup_out(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "tok_ranks", "rank_rows", "rank_slots", "n_rows", "row_token", "row_slots", "rank_row_offset", "slot_row",
        "ddispatch")]


EXPORTS = ("moe_plan_query", "moe_plan_create", "moe_plan_route", "moe_plan_hist", "moe_plan_plan",
           "moe_plan_dispatch", "moe_plan_step", "moe_plan_step_static", "moe_plan_combine", "moe_plan_place", "moe_plan_dedup_count",
           "moe_plan_dedup_dispatch", "moe_plan_quality", "moe_plan_predict", "moe_plan_slot_map",
           "moe_plan_replica_pull", "moe_plan_replica_push", "moe_plan_set_events", "moe_plan_set_gather_order",
           "moe_plan_device_info",
           "moe_plan_status", "moe_plan_destroy")

_LIB = None


def lib_path() -> str:
    return _build.LIB


def lib():
    """The loaded HIP library, built in-tree first when it is missing or was built from other
    sources than the ones in the tree (a hash of the sources is kept beside it)."""
    global _LIB
    if _LIB is None:
        if not _build.up_to_date():
            _build.build()
        l = ctypes.CDLL(_build.LIB)
        vp = ctypes.c_void_p
        l.moe_plan_query.argtypes = [vp, vp]
        l.moe_plan_create.argtypes = [vp, vp]
        l.moe_plan_route.argtypes = [vp, vp, vp, vp, vp]
        l.moe_plan_hist.argtypes = [vp, vp, vp, vp, vp]
        l.moe_plan_plan.argtypes = [vp, vp, vp, vp, vp]
        l.moe_plan_dispatch.argtypes = [vp, vp, vp, vp, vp]
        l.moe_plan_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp]
        l.moe_plan_step_static.argtypes = [vp] * 9
        l.moe_plan_combine.argtypes = [vp, vp, vp, vp, vp, vp]
        l.moe_plan_place.argtypes = [vp, vp, ctypes.c_int32, vp, vp]
        l.moe_plan_dedup_count.argtypes = [vp, vp, vp, ctypes.c_int32, vp, vp]
        l.moe_plan_dedup_dispatch.argtypes = [vp, vp, vp, ctypes.c_int32, vp, vp, vp]
        l.moe_plan_quality.argtypes = [vp, vp, vp, vp]
        l.moe_plan_predict.argtypes = [vp] * 8
        l.moe_plan_slot_map.argtypes = [vp, vp, vp, vp]
        l.moe_plan_device_info.argtypes = [ctypes.c_int, vp]
        l.moe_plan_set_events.argtypes = [vp, vp, vp]
        l.moe_plan_set_gather_order.argtypes = [vp, vp, vp]
        l.moe_plan_replica_pull.argtypes = [vp, vp, vp, ctypes.c_int64, vp, vp]
        l.moe_plan_replica_push.argtypes = [vp, vp, vp, ctypes.c_int64, vp, vp]
        l.moe_plan_status.argtypes = [vp, vp]
        l.moe_plan_destroy.argtypes = [vp]
        l.moe_plan_destroy.restype = None
        for n in EXPORTS[:-1]:
            getattr(l, n).restype = ctypes.c_int
        _LIB = l
    return _LIB


def _check(call: str, rc: int):
    if rc != MOE_OK:
        raise MoePlanError(call, rc)


# ---- entry points, same names as the C ABI ---------------------------------

def moe_plan_query(cfg: moe_plan_config) -> moe_plan_sizes:
    sz = moe_plan_sizes()
    _check("moe_plan_query", lib().moe_plan_query(ctypes.byref(cfg), ctypes.byref(sz)))
    return sz


def moe_plan_create(cfg: moe_plan_config) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check("moe_plan_create", lib().moe_plan_create(ctypes.byref(cfg), ctypes.byref(h)))
    return h


def moe_plan_route(h, logits: int, prev_topk: int | None, out: moe_route_out, stream: int):
    _check("moe_plan_route", lib().moe_plan_route(h, logits, prev_topk, ctypes.byref(out), stream))


def moe_plan_hist(h, topk_idx: int, prev_topk: int | None, out: moe_route_out, stream: int):
    _check("moe_plan_hist", lib().moe_plan_hist(h, topk_idx, prev_topk, ctypes.byref(out), stream))


def moe_plan_plan(h, omega: int, topk_idx: int | None, out: moe_plan_out, stream: int):
    _check("moe_plan_plan", lib().moe_plan_plan(h, omega, topk_idx, ctypes.byref(out), stream))


def moe_plan_dispatch(h, plan: moe_plan_out, hidden: int, out: moe_dispatch_out, stream: int):
    _check("moe_plan_dispatch", lib().moe_plan_dispatch(h, ctypes.byref(plan), hidden, ctypes.byref(out), stream))


def moe_plan_step(h, logits: int, prev_topk, hidden: int, route: moe_route_out, plan: moe_plan_out,
                  out: moe_dispatch_out, stream: int):
    _check("moe_plan_step", lib().moe_plan_step(h, logits, prev_topk, hidden, ctypes.byref(route), ctypes.byref(plan),
                                                ctypes.byref(out), stream))


def moe_plan_step_static(cfg: moe_plan_config, logits: int, prev_topk, hidden: int, route: moe_route_out,
                         plan: moe_plan_out, out: moe_dispatch_out, status: int, stream: int):
    _check("moe_plan_step_static", lib().moe_plan_step_static(ctypes.byref(cfg), logits, prev_topk, hidden,
                                                              ctypes.byref(route), ctypes.byref(plan),
                                                              ctypes.byref(out), status, stream))


def moe_plan_combine(h, topk_val: int, slot_pos: int, expert_out: int, out: int, stream: int):
    _check("moe_plan_combine", lib().moe_plan_combine(h, topk_val, slot_pos, expert_out, out, stream))


def moe_plan_place(h, cooc: int, max_swaps: int, out: moe_place_out, stream: int):
    _check("moe_plan_place", lib().moe_plan_place(h, cooc, max_swaps, ctypes.byref(out), stream))


def moe_plan_dedup_count(h, slot_key: int, key_rank, n_keys: int, out: moe_dedup_out, stream: int):
    _check("moe_plan_dedup_count", lib().moe_plan_dedup_count(h, slot_key, key_rank, n_keys, ctypes.byref(out), stream))


def moe_plan_dedup_dispatch(h, slot_key: int, key_rank, n_keys: int, hidden: int, out: moe_dedup_out, stream: int):
    _check("moe_plan_dedup_dispatch",
           lib().moe_plan_dedup_dispatch(h, slot_key, key_rank, n_keys, hidden, ctypes.byref(out), stream))


def moe_plan_quality(h, plan: moe_plan_out, out: int, stream: int):
    _check("moe_plan_quality", lib().moe_plan_quality(h, ctypes.byref(plan), out, stream))


def moe_plan_predict(h, topk_cur: int, trans: int, count_cur: int, key_rank, topk_next, out: moe_predict_out,
                     stream: int):
    _check("moe_plan_predict", lib().moe_plan_predict(h, topk_cur, trans, count_cur, key_rank, topk_next,
                                                      ctypes.byref(out), stream))


def moe_plan_slot_map(h, plan: moe_plan_out, out: moe_slot_out, stream: int):
    _check("moe_plan_slot_map", lib().moe_plan_slot_map(h, ctypes.byref(plan), ctypes.byref(out), stream))


def moe_plan_replica_pull(h, slot_expert: int, main_params: int, param_elems: int, replica_params: int, stream: int):
    _check("moe_plan_replica_pull",
           lib().moe_plan_replica_pull(h, slot_expert, main_params, param_elems, replica_params, stream))


def moe_plan_replica_push(h, slot_expert: int, replica_grads: int, param_elems: int, grad_accum: int, stream: int):
    _check("moe_plan_replica_push",
           lib().moe_plan_replica_push(h, slot_expert, replica_grads, param_elems, grad_accum, stream))


def moe_plan_set_events(h, gather_begin, gather_end):
    _check("moe_plan_set_events", lib().moe_plan_set_events(h, gather_begin, gather_end))


def moe_plan_set_gather_order(h, wait_event, done_event):
    _check("moe_plan_set_gather_order", lib().moe_plan_set_gather_order(h, wait_event, done_event))


def moe_plan_device_info(device: int = 0) -> dict:
    out = (ctypes.c_int64 * 6)()
    _check("moe_plan_device_info", lib().moe_plan_device_info(device, out))
    return dict(compute_units=out[0], clock_khz=out[1], memory_clock_khz=out[2], memory_bus_bits=out[3],
                l2_bytes=out[4], memory_bytes=out[5])


QUALITY_FIELDS = ("assignments", "same_rank", "same_node", "other_node", "replica_served", "max_rank_load",
                  "min_rank_load", "replicas")


def moe_plan_status(h) -> int:
    flags = ctypes.c_int32(0)
    _check("moe_plan_status", lib().moe_plan_status(h, ctypes.byref(flags)))
    return flags.value


def moe_plan_destroy(h):
    lib().moe_plan_destroy(h)


# ---- torch-owned buffers ----------------------------------------------------

def make_config(T, E, k, R, G, H, B, slots_per_rank=0, expert_bytes=-1, token_bytes=0,
                max_refine_iters=0) -> moe_plan_config:
    return moe_plan_config(T, E, k, R, G, H, B, slots_per_rank, expert_bytes, token_bytes, max_refine_iters)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


@dataclass
class RouteBuffers:
    topk_idx: object
    topk_val: object
    expert_count: object
    omega: object
    cooc: object
    trans: object

    def struct(self) -> moe_route_out:
        return moe_route_out(*(_ptr(getattr(self, n)) for n, _ in moe_route_out._fields_))


@dataclass
class PlanBuffers:
    n_inst: object
    inst_expert: object
    inst_rank: object
    inst_load: object
    rank_load: object
    quota: object
    slot_inst: object
    slot_rank: object

    def struct(self) -> moe_plan_out:
        return moe_plan_out(*(_ptr(getattr(self, n)) for n, _ in moe_plan_out._fields_))


@dataclass
class DispatchBuffers:
    perm: object
    slot_pos: object
    inst_offset: object
    rank_offset: object
    dispatch: object

    def struct(self) -> moe_dispatch_out:
        return moe_dispatch_out(*(_ptr(getattr(self, n)) for n, _ in moe_dispatch_out._fields_))


@dataclass
class PlaceBuffers:
    expert_rank: object
    rank_experts: object
    intra: object
    n_swaps: object

    def struct(self) -> moe_place_out:
        return moe_place_out(*(_ptr(getattr(self, n)) for n, _ in moe_place_out._fields_))


@dataclass
class DedupBuffers:
    tok_ranks: object
    rank_rows: object
    rank_slots: object
    n_rows: object = None
    row_token: object = None
    row_slots: object = None
    rank_row_offset: object = None
    slot_row: object = None
    ddispatch: object = None

    def struct(self) -> moe_dedup_out:
        return moe_dedup_out(*(_ptr(getattr(self, n)) for n, _ in moe_dedup_out._fields_))


class Layer:
    """One MoE layer's planner: a handle plus torch-allocated output buffers."""

    def __init__(self, cfg: moe_plan_config, device=None, cooc: bool = True, trans: bool = False,
                 topk_val: bool = True):
        import torch
        if not torch.cuda.is_available():
            raise RuntimeError("load_balance_planning_amd needs a HIP device")
        self.torch = torch
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        self.cfg = cfg
        self.sizes = moe_plan_query(cfg)
        with torch.cuda.device(self.device):
            self.handle = moe_plan_create(cfg)
        sz, dev, i32 = self.sizes, self.device, torch.int32
        T, E, k, R, H = cfg.T, cfg.E, cfg.k, cfg.R, cfg.H
        e = lambda n, dt=i32: torch.empty(int(n), dtype=dt, device=dev)
        self.route_out = RouteBuffers(
            topk_idx=e(sz.topk).view(T, k), topk_val=e(sz.topk, torch.float32).view(T, k) if topk_val else None,
            expert_count=e(E), omega=e(sz.omega).view(R, E),
            cooc=e(sz.pair).view(E, E) if cooc else None, trans=e(sz.pair).view(E, E) if trans else None)
        self.plan_out = PlanBuffers(
            n_inst=e(1), inst_expert=e(sz.inst_cap), inst_rank=e(sz.inst_cap), inst_load=e(sz.inst_cap),
            rank_load=e(R), quota=e(sz.quota).view(R, sz.inst_cap), slot_inst=e(sz.topk), slot_rank=e(sz.topk))
        self.dispatch_out = DispatchBuffers(
            perm=e(sz.topk), slot_pos=e(sz.topk), inst_offset=e(sz.inst_offset), rank_offset=e(sz.rank_offset),
            dispatch=e(sz.dispatch_elems, torch.int16).view(T * k, H))
        self._route_s = self.route_out.struct()
        self._plan_s = self.plan_out.struct()
        self._disp_s = self.dispatch_out.struct()
        self.place_out = None
        self.dedup_out = None

    def _stream(self, stream=None) -> int:
        s = self.torch.cuda.current_stream(self.device) if stream is None else stream
        return s.cuda_stream

    def route(self, logits, prev_topk=None, stream=None):
        self._check_tensor(logits, (self.cfg.T, self.cfg.E), self.torch.float32)
        if prev_topk is not None:
            self._check_tensor(prev_topk, (self.cfg.T, self.cfg.k), self.torch.int32)
        moe_plan_route(self.handle, _ptr(logits), _ptr(prev_topk), self._route_s, self._stream(stream))
        return self.route_out

    def hist(self, topk_idx, prev_topk=None, stream=None):
        """Histograms of a given top-k (moe_plan_hist); route_out.topk_idx is not touched."""
        self._check_tensor(topk_idx, (self.cfg.T, self.cfg.k), self.torch.int32)
        if prev_topk is not None:
            self._check_tensor(prev_topk, (self.cfg.T, self.cfg.k), self.torch.int32)
        moe_plan_hist(self.handle, _ptr(topk_idx), _ptr(prev_topk), self._route_s, self._stream(stream))
        return self.route_out

    def plan(self, omega=None, topk_idx=None, stream=None):
        """moe_plan_plan from a routing matrix [R][E] and the top-k [T][k] it counts; both default
        to this layer's route outputs."""
        omega = self.route_out.omega if omega is None else omega
        topk_idx = self.route_out.topk_idx if topk_idx is None else topk_idx
        self._check_tensor(omega, (self.cfg.R, self.cfg.E), self.torch.int32)
        self._check_tensor(topk_idx, (self.cfg.T, self.cfg.k), self.torch.int32)
        moe_plan_plan(self.handle, _ptr(omega), _ptr(topk_idx), self._plan_s, self._stream(stream))
        return self.plan_out

    def dispatch(self, hidden, stream=None):
        self._check_tensor(hidden, (self.cfg.T, self.cfg.H), None)
        if hidden.element_size() != 2:
            raise TypeError("hidden must be a 16-bit (bf16) tensor")
        moe_plan_dispatch(self.handle, self._plan_s, _ptr(hidden), self._disp_s, self._stream(stream))
        return self.dispatch_out

    def step(self, logits, hidden, prev_topk=None, stream=None):
        """route + plan + dispatch in one call (moe_plan_step)."""
        self._check_tensor(logits, (self.cfg.T, self.cfg.E), self.torch.float32)
        self._check_tensor(hidden, (self.cfg.T, self.cfg.H), None)
        if hidden.element_size() != 2:
            raise TypeError("hidden must be a 16-bit (bf16) tensor")
        if prev_topk is not None:
            self._check_tensor(prev_topk, (self.cfg.T, self.cfg.k), self.torch.int32)
        moe_plan_step(self.handle, _ptr(logits), _ptr(prev_topk), _ptr(hidden), self._route_s, self._plan_s,
                      self._disp_s, self._stream(stream))
        return self.route_out, self.plan_out, self.dispatch_out

    def combine(self, expert_out, out=None, stream=None):
        """Gate-weighted combine of expert outputs in dispatch order back to token order
        (moe_plan_combine), using this layer's topk_val and slot_pos."""
        T, k, H = self.cfg.T, self.cfg.k, self.cfg.H
        self._check_tensor(expert_out, (T * k, H), None)
        if expert_out.element_size() != 2:
            raise TypeError("expert_out must be a 16-bit (bf16) tensor")
        if self.route_out.topk_val is None:
            raise ValueError("combine needs the layer's topk_val buffer (create the Layer with topk_val=True)")
        if out is None:
            out = self.torch.empty((T, H), dtype=expert_out.dtype, device=self.device)
        self._check_tensor(out, (T, H), None)
        moe_plan_combine(self.handle, _ptr(self.route_out.topk_val), _ptr(self.dispatch_out.slot_pos),
                         _ptr(expert_out), _ptr(out), self._stream(stream))
        return out

    def place(self, cooc=None, max_swaps: int = -1, stream=None):
        """Correlated expert placement from co-selection counts (moe_plan_place);
        cooc defaults to this layer's route_out.cooc."""
        torch, E, R = self.torch, self.cfg.E, self.cfg.R
        cooc = self.route_out.cooc if cooc is None else cooc
        if cooc is None:
            raise ValueError("place needs co-selection counts (create the Layer with cooc=True or pass cooc)")
        self._check_tensor(cooc, (E, E), torch.int32)
        if self.place_out is None:
            e = lambda n, dt=torch.int32: torch.empty(int(n), dtype=dt, device=self.device)
            self.place_out = PlaceBuffers(expert_rank=e(E), rank_experts=e(E).view(R, E // R),
                                          intra=e(1, torch.int64), n_swaps=e(1))
            self._place_s = self.place_out.struct()
        moe_plan_place(self.handle, _ptr(cooc), int(max_swaps), self._place_s, self._stream(stream))
        return self.place_out

    def _dedup_buffers(self, layout: bool):
        torch, T, k, R, H = self.torch, self.cfg.T, self.cfg.k, self.cfg.R, self.cfg.H
        e = lambda n, dt=torch.int32: torch.empty(int(n), dtype=dt, device=self.device)
        if self.dedup_out is None:
            self.dedup_out = DedupBuffers(tok_ranks=e(T), rank_rows=e(R * R).view(R, R), rank_slots=e(R * R).view(R, R))
        d = self.dedup_out
        if layout and d.ddispatch is None:
            d.n_rows, d.row_token, d.row_slots = e(1), e(T * k), e(T * k)
            d.rank_row_offset, d.slot_row = e(R + 1), e(T * k)
            d.ddispatch = e(T * k * H, torch.int16).view(T * k, H)
        self._dedup_s = d.struct()
        return d

    def _keys(self, slot_key, key_rank):
        T, k = self.cfg.T, self.cfg.k
        slot_key = self.route_out.topk_idx if slot_key is None else slot_key
        if tuple(slot_key.shape) not in ((T, k), (T * k,)) or not slot_key.is_contiguous() or \
                slot_key.dtype != self.torch.int32 or slot_key.device != self.device:
            raise ValueError("slot_key must be a contiguous int32 tensor of T*k keys on %s" % self.device)
        n = 0
        if key_rank is not None:
            if key_rank.dim() != 1 or not key_rank.is_contiguous() or key_rank.dtype != self.torch.int32 or \
                    key_rank.device != self.device:
                raise ValueError("key_rank must be a contiguous 1-d int32 tensor on %s" % self.device)
            n = key_rank.numel()
        return slot_key, key_rank, n

    def dedup_count(self, slot_key=None, key_rank=None, stream=None):
        """Deduplicated row counts (moe_plan_dedup_count).  slot_key defaults to
        this layer's top-k; key_rank None means the contiguous placement."""
        slot_key, key_rank, n = self._keys(slot_key, key_rank)
        self._dedup_buffers(False)
        moe_plan_dedup_count(self.handle, _ptr(slot_key), _ptr(key_rank), n, self._dedup_s, self._stream(stream))
        return self.dedup_out

    def dedup_dispatch(self, hidden, slot_key=None, key_rank=None, stream=None):
        """Deduplicated dispatch layout and row copy (moe_plan_dedup_dispatch)."""
        self._check_tensor(hidden, (self.cfg.T, self.cfg.H), None)
        if hidden.element_size() != 2:
            raise TypeError("hidden must be a 16-bit (bf16) tensor")
        slot_key, key_rank, n = self._keys(slot_key, key_rank)
        self._dedup_buffers(True)
        moe_plan_dedup_dispatch(self.handle, _ptr(slot_key), _ptr(key_rank), n, _ptr(hidden), self._dedup_s,
                                self._stream(stream))
        return self.dedup_out

    def quality(self, stream=None):
        """Plan-quality counters of this layer's plan (moe_plan_quality): an int64 tensor of 8
        on the device, in QUALITY_FIELDS order."""
        if getattr(self, "_quality", None) is None:
            self._quality = self.torch.empty(8, dtype=self.torch.int64, device=self.device)
        moe_plan_quality(self.handle, self._plan_s, _ptr(self._quality), self._stream(stream))
        return self._quality

    def predict(self, topk_cur, trans, count_cur, key_rank=None, topk_next=None, stream=None):
        """Token-shuffle prediction (moe_plan_predict): returns (pred [T], rank_tokens [R], local [2])
        device tensors; local counts next-layer slots on the predicted / source rank when
        topk_next is given."""
        torch, T, E, k, R = self.torch, self.cfg.T, self.cfg.E, self.cfg.k, self.cfg.R
        self._check_tensor(topk_cur, (T, k), torch.int32)
        self._check_tensor(trans, (E, E), torch.int32)
        self._check_tensor(count_cur, (E,), torch.int32)
        if key_rank is not None:
            self._check_tensor(key_rank, (E,), torch.int32)
        if topk_next is not None:
            self._check_tensor(topk_next, (T, k), torch.int32)
        if getattr(self, "_pred", None) is None:
            self._pred = (torch.empty(T, dtype=torch.int32, device=self.device),
                          torch.empty(R, dtype=torch.int32, device=self.device),
                          torch.empty(2, dtype=torch.int64, device=self.device))
        out = moe_predict_out(*(_ptr(x) for x in self._pred))
        moe_plan_predict(self.handle, _ptr(topk_cur), _ptr(trans), _ptr(count_cur), _ptr(key_rank), _ptr(topk_next),
                         out, self._stream(stream))
        return self._pred

    def slot_map(self, stream=None):
        """Replica slot map of this layer's plan (moe_plan_slot_map): (slot_expert [R][N_slot],
        slot_main [R][N_slot], inst_slot [E+B]) device tensors."""
        torch, R = self.torch, self.cfg.R
        ns, cap = int(self.sizes.n_slot), int(self.sizes.inst_cap)
        if getattr(self, "_slots", None) is None:
            e = lambda n: torch.empty(n, dtype=torch.int32, device=self.device)
            self._slots = (e(R * ns).view(R, ns), e(R * ns).view(R, ns), e(cap))
        moe_plan_slot_map(self.handle, self._plan_s, moe_slot_out(*(_ptr(x) for x in self._slots)),
                          self._stream(stream))
        return self._slots

    def replica_pull(self, main_params, replica_params, stream=None):
        """moe_plan_replica_pull with this layer's slot map: main_params [E][P] -> replica_params
        [R][N_slot][P] (16-bit tensors)."""
        E, R, ns = self.cfg.E, self.cfg.R, int(self.sizes.n_slot)
        P = main_params.shape[-1]
        self._check_tensor(main_params, (E, P), None)
        self._check_tensor(replica_params, (R, ns, P), None)
        moe_plan_replica_pull(self.handle, _ptr(self._slots[0]), _ptr(main_params), int(P), _ptr(replica_params),
                              self._stream(stream))
        return replica_params

    def replica_push(self, replica_grads, grad_accum, stream=None):
        """moe_plan_replica_push with this layer's slot map: replica_grads [R][N_slot][P] ->
        grad_accum [R][R][E/R][P]."""
        E, R, ns = self.cfg.E, self.cfg.R, int(self.sizes.n_slot)
        P = replica_grads.shape[-1]
        self._check_tensor(replica_grads, (R, ns, P), None)
        self._check_tensor(grad_accum, (R, R, E // R, P), None)
        moe_plan_replica_push(self.handle, _ptr(self._slots[0]), _ptr(replica_grads), int(P), _ptr(grad_accum),
                              self._stream(stream))
        return grad_accum

    def time_gather(self, begin=None, end=None):
        """Record two torch.cuda.Events around the gather kernel of every later dispatch / step
        call of this layer (moe_plan_set_events); with no events, stop.  The events must have
        been recorded once already (torch creates the HIP event on its first record)."""
        if begin is None:
            moe_plan_set_events(self.handle, None, None)
        else:
            moe_plan_set_events(self.handle, ctypes.c_void_p(begin.cuda_event), ctypes.c_void_p(end.cuda_event))

    def order_gather(self, wait=None, done=None):
        """moe_plan_set_gather_order with torch.cuda.Events (each None for none): this layer's
        row copies wait for `wait` and record `done`.  The events must have been recorded once
        already (torch creates the HIP event on its first record)."""
        ptr = lambda ev: None if ev is None else ctypes.c_void_p(ev.cuda_event)
        moe_plan_set_gather_order(self.handle, ptr(wait), ptr(done))

    def status(self) -> int:
        return moe_plan_status(self.handle)

    def _check_tensor(self, t, shape, dtype):
        if tuple(t.shape) != tuple(shape) or not t.is_contiguous() or t.device != self.device:
            raise ValueError("expected a contiguous %s tensor of shape %s on %s" % (dtype, shape, self.device))
        if dtype is not None and t.dtype != dtype:
            raise TypeError("expected dtype %s, got %s" % (dtype, t.dtype))

    def close(self):
        if getattr(self, "handle", None) is not None:
            moe_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
