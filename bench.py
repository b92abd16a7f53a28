#!/usr/bin/env python3
"""Benchmark of the MoE dispatch-planning path on one MI355X.

A step is one pass of the whole path over every layer of the workload --
moe_plan_step, i.e. route -> plan -> dispatch in one call per layer -- with
the inputs resident in HBM.  Consecutive steps (independent batches) alternate
between two handles on two streams, so one batch's route + plan overlaps the
previous batch's gather; latency_ms_per_step gives the same steps run one at
a time on one stream.  Prints ONE JSON line:
  value       routed token-slots per second (T*k*L / step time)
  roofline    the dominant kernel (the bf16 row copy of moe_plan_step, which
              also assigns the slots): the row bytes per launch (hidden rows
              read once, dispatch rows written) / its mean duration, from HIP
              events the library records right around that kernel's launch
              (moe_plan_set_events) in a one-stream pass of the same steps
              of its own,
              against the 8 TB/s HBM peak; `traffic` is the profiler's byte
              count for the kernel, read from the committed counter summary
              named in `traffic_source` while it describes the current source
  chain       the same for the whole step (the method's bytes of every call:
              logits, top-k, histograms, quotas, permutation, rows)
  configs     the other four workloads: step time with two batches in flight
              and one at a time, the chain's and the gather's share of the
              HBM peak, and whether the layer fits the 256 MB Infinity Cache
  combine     the return path (moe_plan_combine) on the same layer, timed
              separately with the dispatch buffer as the expert outputs
  placement   correlated expert placement (moe_plan_place) from the first
              layer's co-selection counts, the oracle's time on the same
              counts beside it, and the share of rows a deduplicating
              dispatcher saves with the contiguous placement, with the
              correlated one, and with the planner's instances
  dedup_dispatch  the deduplicated dispatch (moe_plan_dedup_dispatch) with the
              correlated placement: its rows and HBM rate
  token_shuffle (workloads of several layers) moe_plan_predict from each layer
              to the next: its time and the share of the next layer's slots on
              the predicted rank, against staying on the source rank, with the
              contiguous and with the correlated placement of the next layer
  replica_pull  the replica slot map of the first layer's plan and the bf16
              parameter pull into the occupied slots (moe_plan_slot_map +
              moe_plan_replica_pull) at the modelled expert size ||W||
              (9H^2/4 bytes, capped so that all E main rows fit in 32 GB),
              event-timed, against the HBM peak
  plan_quality  the plan's rank-load imbalance (max / mean) and its shares of
              assignments on the source's rank, on another node and on replicas
              (moe_plan_quality), beside the static placement's
With --sweep quality / --sweep solver it instead prints one JSON line per point
of TopoEP's plan-quality study (router_skew 0..-4 x replica slots per rank
0..4 on the Fig. 10 shape) or solver-scaling study (Fig. 11 shapes).
  cpu_baseline  the CPU oracle on one core over a bounded sample
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "deepseek_v3_layer"
GATHER_PMC = os.path.join(ROOT, "profiles", "gather_deepseek_v3_layer_pmc.txt")


def algorithmic_bytes(w) -> dict:
    """Bytes the method itself must move per step (every layer), call by call: logits read,
    top-k written and re-read across the plan's grid-wide dependency, the routing matrix,
    expert counts, co-selection (and transition) counts, the quotas, the permutation, the
    hidden rows read once and the dispatch rows written.  Implementation traffic (the
    presence masks, tile prefixes, per-slot instances) and the dense alternatives the path
    avoids are not counted.  `gather` is the row copy alone: hidden rows read once plus the
    dispatch rows written."""
    T, E, k, R, H, B, L = w.T, w.E, w.k, w.R, w.H, w.B, w.L
    route_layer = T * E * 4 + T * k * 4 + (R * E + E + E * E) * 4
    route = route_layer * L + E * E * 4 * (L - 1)  # transition counts for every layer after the first
    plan = (T * k * 4 + R * (E + B) * 4) * L
    gather = T * H * 2 + T * k * H * 2
    dispatch = (gather + T * k * 4) * L
    combine = (T * k * H * 2             # expert output rows read
               + T * H * 2             # combined rows written
               + T * k * 4 * 2)        # selected logits and slot positions read
    return dict(route=route, plan=plan, dispatch=dispatch, gather=gather, combine=combine,
                total=route + plan + dispatch)


CACHE_BYTES = 256 * 2**20  # MI355X Infinity Cache


def working_set(w) -> int:
    """Bytes of logits, hidden rows and dispatch rows of one layer (below the 256 MB
    Infinity Cache the path is cache-resident rather than HBM-bound)."""
    return w.T * w.E * 4 + w.T * w.H * 2 + w.T * w.k * w.H * 2


def inputs_sha(w) -> dict:
    """SHA-256 (first 16 hex digits) of the generated input buffers."""
    out = {"hidden": hashlib.sha256(synth.hidden(w).tobytes()).hexdigest()[:16]}
    for l, lg in enumerate(synth.all_logits(w)):
        out["logits_layer%d" % l] = hashlib.sha256(lg.tobytes()).hexdigest()[:16]
    return out


def batch_of(w, i: int):
    """The batch of handle i of a pipeline: the workload's recipe with the i-th next seed."""
    return dataclasses.replace(w, seed=w.seed + i)


def second_batch(w):
    """The batch of the second handle."""
    return batch_of(w, 1)


def dedup_bytes(w, n_rows: int) -> int:
    """Bytes moe_plan_dedup_dispatch must move for a layer with n_rows deduplicated rows."""
    T, k, R, H = w.T, w.k, w.R, w.H
    tiles = R * ((T // R + 63) // 64)
    return (T * k * 4 * 2              # slot keys read by the mask and gather kernels
            + T * 4                    # distinct-rank counts written
            + tiles * R * (8 + 4) * 2  # per-tile rank masks and slot counts, written then read
            + tiles * R * 4 * 2        # per-tile row prefix written, read by the gather
            + T * H * 2                # hidden rows read once
            + n_rows * H * 2           # deduplicated rows written
            + n_rows * 4 * 2           # row token and slot mask
            + T * k * 4)               # row of each slot


def source_hash(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def step_copy_kernel(w) -> str:
    """The row-copy kernel moe_plan_step launches for this shape, by the library's rule: a
    part per 3584 16-byte vectors a token writes (k rows of H/8 vectors; one to four parts).
    With one part the copy assigns the slots itself; with more, assign_kernel runs first."""
    vpr = w.H // 8
    vpt = 1 if vpr <= 256 else 4
    parts = min(4, max(1, w.k * vpr // 3584))
    if parts == 1:
        return "gather_vec_kernel<%d, true> (the row copy of moe_plan_step, with the slot assignment)" % vpt
    return ("gather_vec_kernel<%d, false> (the row copy of moe_plan_step, %d parts per token, after the slot "
            "assignment's own kernel)" % (vpt, parts))


def gather_traffic(w):
    """HBM bytes per gather launch as measured by the committed rocprofv3 counter runs
    (FETCH_SIZE and WRITE_SIZE, each in a run of its own, scaled by a plain copy), if they
    still describe the current kernel source; else None.  Returns (bytes, source note)."""
    if w.name != DEFAULT_WORKLOAD or not os.path.exists(GATHER_PMC):
        return None, None
    text = open(GATHER_PMC).read()
    m = re.search(r"source_sha256_16:\s*(\w+)", text)
    src = os.path.join(ROOT, "load_balance_planning_amd", "csrc", "dispatch.hip")
    rel = os.path.relpath(GATHER_PMC, ROOT)
    if not m or m.group(1) != source_hash(src):
        return None, "%s describes another dispatch.hip (source %s, now %s): not used" % (
            rel, m.group(1) if m else "?", source_hash(src))
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not t:
        return None, None
    return float(t.group(1)), "%s (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of this bench; dispatch.hip " \
                             "sha256 %s), not measured in this run" % (rel, m.group(1))


def cpu_baseline(w, budget_s: float) -> dict:
    """The oracle, single-threaded on one core, on whole layers of the workload until the
    time budget is spent (at least one layer); then each stage of the first layer three
    times (medians)."""
    import oracle
    orig = os.sched_getaffinity(0)
    core = min(orig)
    os.sched_setaffinity(0, {core})
    stages = {"route": [], "plan": [], "dispatch": []}
    try:
        cfg = oracle.make_cfg(w.T, w.E, w.k, w.R, w.G, w.H, w.B)
        hidden = synth.hidden(w)
        layers = synth.all_logits(w)
        l = oracle.lib()
        done, t0 = 0, time.perf_counter()
        elapsed = 0.0
        while True:
            lg = layers[done % w.L]
            t1 = time.perf_counter()
            oracle.run_all(cfg, lg, hidden, l=l)
            elapsed += time.perf_counter() - t1
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        for _ in range(3):
            t1 = time.perf_counter()
            r = oracle.route(cfg, layers[0], l=l)
            t2 = time.perf_counter()
            p = oracle.plan(cfg, r["omega"], r["topk_idx"], l=l)
            t3 = time.perf_counter()
            oracle.dispatch(cfg, int(p["n_inst"][0]), p["inst_rank"], p["slot_inst"], hidden, l=l)
            t4 = time.perf_counter()
            stages["route"].append(t2 - t1)
            stages["plan"].append(t3 - t2)
            stages["dispatch"].append(t4 - t3)
    finally:
        os.sched_setaffinity(0, orig)
    slots = w.T * w.k * done
    model = "unknown CPU"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": slots / elapsed, "unit": "token-slots/s", "cores": 1, "kind": "oracle",
            "sample": "%d full layer(s) of %s (route+plan+dispatch incl. the bf16 row copy), %.1f s on 1 core of a "
                      "%d-core %s" % (done, w.name, elapsed, os.cpu_count() or 0, model),
            "stage_ms_median_of_3": {k: float(np.median(v)) * 1e3 for k, v in stages.items()}}


_STREAMS = []


def pipeline_streams(dev, n: int):
    """n streams for the batches in flight, created once per process and reused, so that every
    measurement puts its batches on the same streams (HIP maps each stream to one of a few
    hardware queues at creation; two batches on one queue run one after the other)."""
    import torch
    while len(_STREAMS) < n:
        _STREAMS.append(torch.cuda.Stream(dev))
    return _STREAMS[:n]


def time_path(w, steps: int, warmup: int, dev, keep: bool = False, flight: int = 2) -> dict:
    """time_path_on with the pipeline's streams, the first one current."""
    import torch
    streams = pipeline_streams(dev, flight)
    with torch.cuda.stream(streams[0]):
        return time_path_on(w, steps, warmup, dev, streams, keep)


def time_path_on(w, steps: int, warmup: int, dev, streams, keep: bool = False) -> dict:
    """The timed passes of one workload: `steps` steps with len(streams) batches in flight (the
    headline configuration), the same steps one at a time on one stream with the gather kernel of
    every moe_plan_step bracketed by HIP events (moe_plan_set_events), and the same steps as three
    calls per layer with events around each call and around the gather kernel of
    moe_plan_dispatch.  With keep, the first batch's layers and inputs stay open for further
    measurements (else everything is freed).  streams[0] is the current stream."""
    import torch
    import load_balance_planning_amd as mp
    flight = len(streams)
    cfg = mp.make_config(w.T, w.E, w.k, w.R, w.G, w.H, w.B)
    hidden = torch.from_numpy(synth.hidden(w).view(np.int16)).to(dev)
    logits = [torch.from_numpy(lg).to(dev) for lg in synth.all_logits(w)]
    # The other handles' batches: the same recipe with the next seeds, so that no
    # step re-reads the inputs the step before it read.
    batches = [(logits, hidden)]
    for i in range(1, flight):
        wi = batch_of(w, i)
        batches.append(([torch.from_numpy(lg).to(dev) for lg in synth.all_logits(wi)],
                        torch.from_numpy(synth.hidden(wi).view(np.int16)).to(dev)))
    # Batches in flight: consecutive steps rotate over `flight` handles (each with
    # its own buffers and batch) on as many streams, so the latency-bound route +
    # plan of one batch overlaps the HBM-bound gather of another.
    sets = [[mp.Layer(cfg, device=dev, cooc=True, trans=(l > 0)) for l in range(w.L)] for _ in range(flight)]
    layers = sets[0]
    stream = streams[0]

    # When the row copies are HBM-bound, the handles' copies take turns
    # (moe_plan_set_gather_order): each handle's copy waits for the latest copy
    # of the handle before it in the rotation, so the copies run one after the
    # other at full bandwidth while the other batches' top-k, plan and quotas
    # run beside them.  The calls are enqueued layer by layer, rotating over
    # the batches, so that every wait refers to the copy enqueued just before
    # it.  A layer whose rows stay in the Infinity Cache lets the copies overlap.
    order = working_set(w) >= CACHE_BYTES and flight > 1
    turn = [torch.cuda.Event() for _ in range(flight)]
    for ev in turn:
        ev.record(stream)  # creates the HIP events; the first copy then waits for nothing

    def pipelined(n):  # n steps, rotating over the handles
        if order:
            for i in range(flight):
                for layer in sets[i]:
                    layer.order_gather(wait=turn[(i - 1) % flight], done=turn[i])
        for s_ in range(0, n, flight):
            for l in range(w.L):
                for i in range(min(flight, n - s_)):
                    # one pass of the whole path: moe_plan_step (route + plan + dispatch in one call)
                    lgs, hid = batches[i]
                    with torch.cuda.stream(streams[i]):
                        prev = sets[i][l - 1].route_out.topk_idx if l > 0 else None
                        sets[i][l].step(lgs[l], hid, prev)
        for layer in [x for st_ in sets for x in st_]:
            layer.order_gather()

    pipelined(warmup)
    torch.cuda.synchronize()
    for layer in [x for st_ in sets for x in st_]:
        if layer.status() != 0:
            raise RuntimeError("device status word set during warm-up")
    # Timed region: exactly `steps` steps, synchronised on both sides; the end
    # event waits for every stream.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_side = [torch.cuda.Event() for _ in streams[1:]]
    torch.cuda.synchronize()
    t_start.record(stream)
    for st_ in streams[1:]:
        st_.wait_event(t_start)
    pipelined(steps)
    for ev, st_ in zip(t_side, streams[1:]):
        ev.record(st_)
        stream.wait_event(ev)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)

    def event_pairs(n):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in ev:  # torch creates the HIP event on its first record
            a.record(stream)
            b.record(stream)
        return ev

    # The same steps one at a time on one stream: the latency of a step.
    def one_stream(gev=None):
        lev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        lev[0].record(stream)
        for s_ in range(steps):
            for l, layer in enumerate(layers):
                if gev is not None:
                    layer.time_gather(*gev[s_ * w.L + l])
                prev = layers[l - 1].route_out.topk_idx if l > 0 else None
                layer.step(logits[l], hidden, prev)
            lev[s_ + 1].record(stream)
        torch.cuda.synchronize()
        return lev

    lev = one_stream()
    step_ms = [lev[i].elapsed_time(lev[i + 1]) for i in range(steps)]
    ms_serial = lev[0].elapsed_time(lev[steps])
    # Again, with the gather kernel of every moe_plan_step (the assigning gather)
    # bracketed by events the library records right around its launch.
    gev = event_pairs(steps * w.L)
    one_stream(gev)
    for layer in layers:
        layer.time_gather()
    step_gather_ms = [a.elapsed_time(b) for a, b in gev]
    for layer in [x for st_ in sets[1:] for x in st_]:
        if layer.status() != 0:
            raise RuntimeError("device status word set on another handle")
        layer.close()
    # Per-call durations from events around each call, in a third pass of the same
    # steps as three calls, and the gather kernel of moe_plan_dispatch alone.
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(w.L)] for _ in range(steps)]
    dev_ = event_pairs(steps * w.L)
    torch.cuda.synchronize()
    for s_ in range(steps):
        for l, layer in enumerate(layers):
            e = evs[s_][l]
            prev = layers[l - 1].route_out.topk_idx if l > 0 else None
            e[0].record(stream)
            layer.route(logits[l], prev)
            e[1].record(stream)
            layer.plan()
            e[2].record(stream)
            layer.time_gather(*dev_[s_ * w.L + l])
            layer.dispatch(hidden)
            e[3].record(stream)
    torch.cuda.synchronize()
    for layer in layers:
        layer.time_gather()
    per = {"route": [], "plan": [], "dispatch": []}
    for s_ in range(steps):
        for l in range(w.L):
            e = evs[s_][l]
            per["route"].append(e[0].elapsed_time(e[1]))
            per["plan"].append(e[1].elapsed_time(e[2]))
            per["dispatch"].append(e[2].elapsed_time(e[3]))
    out = dict(ms_total=ms_total, ms_serial=ms_serial, step_ms=step_ms,
               step_gather_ms=float(np.mean(step_gather_ms)), dispatch_gather_ms=float(np.mean([a.elapsed_time(b) for a, b in dev_])),
               per_call_ms={k: float(np.mean(v)) for k, v in per.items()},
               per_call_ms_median={k: float(np.median(v)) for k, v in per.items()},
               per_call_ms_min={k: float(np.min(v)) for k, v in per.items()})
    if keep:
        out.update(layers=layers, logits=logits, hidden=hidden, cfg=cfg)
    else:
        status = [layer.status() for layer in layers]
        for layer in layers:
            layer.close()
        if any(status):
            out["status_flags"] = status
        del batches, logits, hidden
        torch.cuda.empty_cache()
    return out


def config_line(w, steps: int, warmup: int, dev) -> dict:
    """The headline measurements of one more workload, for the line's `configs` object."""
    t = time_path(w, steps, warmup, dev)
    ab = algorithmic_bytes(w)
    ms = t["ms_total"] / steps
    lat = t["ms_serial"] / steps
    out = {"T": w.T, "E": w.E, "k": w.k, "R": w.R, "G": w.G, "H": w.H, "replica_budget": w.B, "layers": w.L,
           "value": w.T * w.k * w.L / (ms / 1e3), "unit": "token-slots/s", "ms_per_step": ms,
           "latency_ms_per_step": lat, "latency_us_median": float(np.median(t["step_ms"])) * 1e3,
           "chain_algorithmic_bytes": ab["total"],
           "chain_frac": ab["total"] / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
           "chain_frac_one_stream": ab["total"] / (lat / 1e3) / 1e9 / HBM_PEAK_GBS,
           "gather_us": t["step_gather_ms"] * 1e3, "gather_algorithmic_bytes": ab["gather"],
           "gather_frac": ab["gather"] / (t["step_gather_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS,
           "cache_resident": working_set(w) < CACHE_BYTES, "copies_take_turns": working_set(w) >= CACHE_BYTES}
    if "status_flags" in t:
        out["status_flags"] = t["status_flags"]
    return out


def run_gpu(w, steps: int, warmup: int) -> dict:
    import torch
    import load_balance_planning_amd as mp
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    t = time_path(w, steps, warmup, dev, keep=True)
    layers, logits, hidden, cfg = t["layers"], t["logits"], t["hidden"], t["cfg"]
    stream = torch.cuda.current_stream(dev)
    # Combine (the return path): the dispatch buffer stands in for the expert outputs.
    comb_out = [torch.empty((w.T, w.H), dtype=torch.int16, device=dev) for _ in layers]
    for l, layer in enumerate(layers):
        layer.combine(layer.dispatch_out.dispatch, out=comb_out[l])
    cev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps * w.L)]
    torch.cuda.synchronize()
    for s in range(steps):
        for l, layer in enumerate(layers):
            e = cev[s * w.L + l]
            e[0].record(stream)
            layer.combine(layer.dispatch_out.dispatch, out=comb_out[l])
            e[1].record(stream)
    torch.cuda.synchronize()
    comb_ms = [e[0].elapsed_time(e[1]) for e in cev]
    # Correlated placement from the first layer's co-selection counts, and the
    # deduplicated dispatch with it.
    lay0 = layers[0]
    lay0.place()
    pev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(5)]
    torch.cuda.synchronize()
    for e in pev:
        e[0].record(stream)
        pl = lay0.place()
        e[1].record(stream)
    torch.cuda.synchronize()
    place_ms = [e[0].elapsed_time(e[1]) for e in pev]
    expert_rank = pl.expert_rank.clone()
    place = dict(us=float(np.mean(place_ms)) * 1e3, swaps=int(pl.n_swaps.item()), intra=int(pl.intra.item()),
                 cooc=lay0.route_out.cooc.cpu().numpy())
    slots = w.T * w.k
    saved = {}
    for name, keys, table in (("contiguous", None, None), ("placed", None, expert_rank),
                              ("plan_instances", lay0.plan_out.slot_inst, lay0.plan_out.inst_rank)):
        d = lay0.dedup_count(keys, table)
        saved[name] = 1.0 - int(d.tok_ranks.sum().item()) / slots
    lay0.dedup_dispatch(hidden, key_rank=expert_rank)
    dev_ = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    for e in dev_:
        e[0].record(stream)
        dd = lay0.dedup_dispatch(hidden, key_rank=expert_rank)
        e[1].record(stream)
    torch.cuda.synchronize()
    place["rows_saved_frac"] = saved
    quality = {"plan": quality_dict(lay0.quality(), w.R)}
    # The planner on the correlated placement: renumber the experts so that expert
    # rank_experts[p] becomes p (the caller permutes its router columns once), then
    # route, plan, and count what deduplication still saves over the plan's instances.
    order = pl.rank_experts.reshape(-1).long()
    relabel = mp.Layer(cfg, device=dev, cooc=False)
    relabel.route(logits[0].index_select(1, order).contiguous())
    relabel.plan()
    quality["plan_on_correlated_placement"] = quality_dict(relabel.quality(), w.R)
    d = relabel.dedup_count(relabel.plan_out.slot_inst, relabel.plan_out.inst_rank)
    place["rows_saved_frac"]["plan_instances_on_correlated_placement"] = 1.0 - int(d.tok_ranks.sum().item()) / slots
    relabel.close()
    dedup = dict(us=float(np.mean([e[0].elapsed_time(e[1]) for e in dev_])) * 1e3, n_rows=int(dd.n_rows.item()))
    # Replica slots of the first layer's plan and the parameter pull at the modelled expert size.
    pull = None
    lay0.slot_map()
    occupied = int((lay0._slots[0] >= 0).sum().item())
    P = (9 * w.H * w.H // 4) // 2  # bf16 elements of ||W||
    P = min(P, (32 * 10**9 // (2 * w.E)) // 8 * 8)  # keep all E main rows within 32 GB
    ns = int(lay0.sizes.n_slot)
    if occupied > 0 and ns > 0:
        main_params = torch.empty((w.E, P), dtype=torch.int16, device=dev)
        main_params.random_(-32768, 32767)
        replica = torch.empty((w.R, ns, P), dtype=torch.int16, device=dev)
        lay0.replica_pull(main_params, replica)
        pev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(10)]
        torch.cuda.synchronize()
        for e in pev:
            e[0].record(stream)
            lay0.replica_pull(main_params, replica)
            e[1].record(stream)
        torch.cuda.synchronize()
        us = float(np.mean([e[0].elapsed_time(e[1]) for e in pev])) * 1e3
        nbytes = 2 * occupied * P * 2
        pull = {"kernel": "slot_copy_kernel (moe_plan_replica_pull)", "us": us, "occupied_slots": occupied,
                "slots": w.R * ns, "bytes_per_expert": P * 2, "algorithmic_bytes_per_launch": nbytes,
                "achieved": nbytes / (us / 1e6) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": nbytes / (us / 1e6) / 1e9 / HBM_PEAK_GBS}
        del main_params, replica
    shuffle = None
    if w.L > 1:
        shuffle = []
        slots = w.T * w.k
        for l in range(1, w.L):
            a, b = layers[l - 1], layers[l]
            args = (a.route_out.topk_idx, b.route_out.trans, a.route_out.expert_count)
            b.predict(*args, topk_next=b.route_out.topk_idx)
            sev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
            torch.cuda.synchronize()
            for e in sev:
                e[0].record(stream)
                _, _, loc = b.predict(*args, topk_next=b.route_out.topk_idx)
                e[1].record(stream)
            torch.cuda.synchronize()
            contiguous = loc.cpu().numpy().copy()
            placed_rank = b.place().expert_rank.clone()
            _, _, loc = b.predict(*args, key_rank=placed_rank, topk_next=b.route_out.topk_idx)
            placed = loc.cpu().numpy()
            shuffle.append({"from_layer": l - 1, "to_layer": l,
                            "us": float(np.mean([e[0].elapsed_time(e[1]) for e in sev])) * 1e3,
                            "local_frac_contiguous": {"shuffled": int(contiguous[0]) / slots,
                                                      "unshuffled": int(contiguous[1]) / slots},
                            "local_frac_correlated_placement": {"shuffled": int(placed[0]) / slots,
                                                                "unshuffled": int(placed[1]) / slots}})
    status = [layer.status() for layer in layers]
    for layer in layers:
        layer.close()
    static = mp.Layer(mp.make_config(w.T, w.E, w.k, w.R, w.G, w.H, 0), device=dev, cooc=False)
    static.route(logits[0])
    static.plan()
    quality["static_placement"] = quality_dict(static.quality(), w.R)
    static.close()
    dinfo = mp.moe_plan_device_info(0)
    copy = copy_reference(1 << 30, 10)
    out = {k: v for k, v in t.items() if k not in ("layers", "logits", "hidden", "cfg")}
    out.update(dinfo=dinfo, copy=copy, combine_ms=float(np.mean(comb_ms)), place=place, dedup=dedup,
               quality=quality, shuffle=shuffle, pull=pull, status=status, device=torch.cuda.get_device_name(dev))
    del layers, logits, hidden
    torch.cuda.empty_cache()
    return out


def quality_dict(q, R: int) -> dict:
    """moe_plan_quality's counters as the shares the pages report."""
    import load_balance_planning_amd as mp
    v = dict(zip(mp.QUALITY_FIELDS, (int(x) for x in q.cpu().numpy())))
    n = max(v["assignments"], 1)
    return {"imbalance": v["max_rank_load"] * R / n, "same_rank_frac": v["same_rank"] / n,
            "other_node_frac": v["other_node"] / n, "replica_served_frac": v["replica_served"] / n,
            "replicas": v["replicas"]}


def sweep(kind: str, warmup: int, reps: int):
    """One JSON line per point: TopoEP's plan-quality study (section 6.2 Fig. 10,
    section 6.6 Fig. 16) over its section 6.4 router_skew range, or its solver-scaling
    study (section 6.3 Fig. 11), with moe_plan_plan event-timed (warm-up, then reps)."""
    import torch
    import load_balance_planning_amd as mp
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if kind == "quality":
        points = [synth.skew_layer(sk, n) for sk in (0, -1, -2, -3, -4) for n in (0, 1, 2, 3, 4)]
    else:
        points = ([synth.skew_layer(-4, 2, E=640, R=r) for r in (8, 16, 32, 64, 128)] +
                  [synth.skew_layer(-4, 2, E=e, R=32) for e in (128, 256, 512, 1024, 2048)])
    stream = torch.cuda.current_stream(dev)
    for w in points:
        layer = mp.Layer(mp.make_config(w.T, w.E, w.k, w.R, w.G, w.H, w.B), device=dev, cooc=False)
        layer.route(torch.from_numpy(synth.logits(w)).to(dev))
        for _ in range(warmup):
            layer.plan()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        torch.cuda.synchronize()
        for e in ev:
            e[0].record(stream)
            layer.plan()
            e[1].record(stream)
        torch.cuda.synchronize()
        ms = [e[0].elapsed_time(e[1]) for e in ev]
        q = quality_dict(layer.quality(), w.R)
        st = layer.status()
        layer.close()
        line = {"sweep": kind, "workload": w.name, "router_skew": -w.zipf_s, "slots_per_rank": w.B // w.R,
                "T": w.T, "E": w.E, "k": w.k, "R": w.R, "G": w.G, "plan_us_mean": float(np.mean(ms)) * 1e3,
                "plan_us_min": float(np.min(ms)) * 1e3, "reps": reps}
        line.update(q)
        if st:
            line["status_flags"] = st
        print(json.dumps(line), flush=True)


def placement_report(w, p: dict, with_oracle: bool) -> dict:
    """The GPU placement's figures, with the oracle timed on the same counts (one core)."""
    out = {"kernel": "moe_plan_place", "us": p["us"], "swaps": p["swaps"], "intra": p["intra"],
           "rows_saved_frac": p["rows_saved_frac"]}
    if with_oracle:
        import oracle
        cfg = oracle.make_cfg(w.T, w.E, w.k, w.R, w.G, w.H, w.B)
        orig = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {min(orig)})
        try:
            t0 = time.perf_counter()
            n = 0
            while n < 3 or time.perf_counter() - t0 < 1.0:
                ref = oracle.place(cfg, p["cooc"])
                n += 1
            ms = (time.perf_counter() - t0) / n * 1e3
        finally:
            os.sched_setaffinity(0, orig)
        out["oracle_ms"] = ms
        out["oracle_cores"] = 1
        out["matches_oracle"] = ref["intra"] == p["intra"] and ref["n_swaps"] == p["swaps"]
    return out


def _timeit(fn, min_runs: int = 3, budget_s: float = 1.0):
    t0 = time.perf_counter()
    n = 0
    while n < min_runs or time.perf_counter() - t0 < budget_s:
        fn()
        n += 1
    return (time.perf_counter() - t0) / n


def oracle_beside(w, P: int, with_shuffle: bool) -> dict:
    """The oracle's time for each further call the bench measures, on one core, on the
    same layer (or a stated sample of it), to print beside the GPU's."""
    import oracle
    orig = os.sched_getaffinity(0)
    os.sched_setaffinity(0, {min(orig)})
    out = {}
    try:
        cfg = oracle.make_cfg(w.T, w.E, w.k, w.R, w.G, w.H, w.B)
        layers = synth.all_logits(w)
        hid = synth.hidden(w)
        r = oracle.route(cfg, layers[0])
        p = oracle.plan(cfg, r["omega"], r["topk_idx"])
        out["plan_quality"] = {"oracle_ms": _timeit(lambda: oracle.quality(cfg, p)) * 1e3}
        pl = oracle.place(cfg, r["cooc"])
        out["dedup_dispatch"] = {"oracle_ms": _timeit(lambda: oracle.dedup_dispatch(cfg, r["topk_idx"],
                                                                                    pl["expert_rank"], hid),
                                                      min_runs=1, budget_s=0.0) * 1e3}
        n = min(512, w.T)
        sub = oracle.make_cfg(n, w.E, w.k, 1, 1, w.H, 0)
        rows = hid[np.repeat(np.arange(n), w.k)]
        t = _timeit(lambda: oracle.combine(sub, r["topk_val"][:n], np.arange(n * w.k, dtype=np.int32), rows))
        out["combine"] = {"oracle_ms": t * w.T / n * 1e3,
                          "oracle_sample": "the first %d tokens, scaled to the layer's %d" % (n, w.T)}
        m = oracle.slot_map(cfg, p)
        ps = min(P, 1 << 20)
        main = np.zeros((w.E, ps), np.uint16)
        repl = np.zeros((w.R, m["slot_expert"].shape[1], ps), np.uint16)
        t = _timeit(lambda: oracle.replica_pull(cfg, m["slot_expert"], main, repl))
        out["replica_pull"] = {"oracle_ms": t * P / ps * 1e3,
                               "oracle_sample": "rows of %d of the %d bf16 elements, scaled" % (ps, P)}
        if with_shuffle:
            prev = r["topk_idx"]
            pred = []
            for l in range(1, w.L):
                nxt = oracle.route(cfg, layers[l], prev_topk=prev, want_cooc=False)
                cur_count = np.bincount(prev.reshape(-1), minlength=w.E).astype(np.int32)
                pred.append(_timeit(lambda: oracle.predict(cfg, prev, nxt["trans"], cur_count, None,
                                                           nxt["topk_idx"]), min_runs=1) * 1e3)
                prev = nxt["topk_idx"]
            out["token_shuffle"] = {"oracle_ms": pred}
    finally:
        os.sched_setaffinity(0, orig)
    return out


def copy_reference(nbytes: int, steps: int) -> dict:
    """A plain device-to-device copy of nbytes (torch's copy kernel), the known-size reference
    against which the HBM byte counters of the profiler are scaled."""
    import torch
    dev = torch.device("cuda", 0)
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    return {"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "ms_per_copy": ms,
            "GBps": 2 * nbytes / (ms / 1e3) / 1e9}


def ceilings(w, steps: int) -> dict:
    """Device reference rates for the gather's traffic, from torch's own kernels on the
    workload's shapes (HIP-event timed, `steps` launches each after one untimed): the k-fold
    dispatch buffer written sequentially (fill), the same rows written at the plan's positions in
    slot order (index_fill on 16-byte elements: the gather's write pattern without its reads), the
    buffer read (sum), a plain copy of it, and torch's destination-ordered equivalent of the
    gather (index_select: sequential writes, each hidden row read k times), a read of a cold
    logits-sized tensor right after a step (the memory state of the next step's top-k); beside
    them the library's own row copies."""
    import torch
    import load_balance_planning_amd as mp
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    N, H = w.T * w.k, w.H
    hidden = torch.from_numpy(synth.hidden(w).view(np.int16)).to(dev)
    layer = mp.Layer(mp.make_config(w.T, w.E, w.k, w.R, w.G, w.H, w.B), device=dev, cooc=True)
    layer.step(torch.from_numpy(synth.logits(w)).to(dev), hidden)
    torch.cuda.synchronize()
    if layer.status() != 0:
        raise RuntimeError("device status word set")
    slot_pos = layer.dispatch_out.slot_pos.to(torch.int64)         # position of slot t*k+j
    token_of_row = layer.dispatch_out.perm.to(torch.int64) // w.k  # token of each dispatch row
    disp = layer.dispatch_out.dispatch
    vecs = disp.view(torch.complex128).view(N, H // 8)  # 16-byte elements, as the gather stores them
    other = torch.empty_like(disp)
    row_bytes = H * 2

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps * 1e3

    out = {}

    def put(name, us, read, written, what):
        out[name] = {"us": us, "bytes_read": read, "bytes_written": written,
                     "GBps": (read + written) / (us / 1e6) / 1e9,
                     "frac": (read + written) / (us / 1e6) / 1e9 / HBM_PEAK_GBS, "what": what}

    put("write_sequential", timed(lambda: disp.zero_()), 0, N * row_bytes, "torch fill of the dispatch buffer")
    put("write_at_plan_positions", timed(lambda: vecs.index_fill_(0, slot_pos, 0)), N * 8, N * row_bytes,
        "torch index_fill of the rows at the plan's positions in slot order, 16-byte elements (reads the indices)")
    put("read_sequential", timed(lambda: disp.view(torch.int64).sum()), N * row_bytes, 0,
        "torch sum of the dispatch buffer")
    put("copy", timed(lambda: other.copy_(disp)), N * row_bytes, N * row_bytes, "torch copy of the dispatch buffer")
    put("gather_destination_order", timed(lambda: torch.index_select(hidden, 0, token_of_row, out=other)),
        N * row_bytes, N * row_bytes + N * 8,
        "torch index_select of the hidden rows in dispatch-row order (bytes as if every read came from HBM)")
    # The top-k's reference: a read of a logits-sized tensor that is not in any cache,
    # right after a step (whose row copy leaves the caches full of its dirty rows) -- the
    # memory state in which the next step's top-k reads its logits.
    lg = torch.from_numpy(synth.logits(w)).to(dev)
    cold = [torch.from_numpy(synth.logits(batch_of(w, i))).to(dev) for i in (1, 2, 3)]
    rd = []
    for i in range(steps + 1):
        layer.step(lg, hidden)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        cold[i % 3].sum()
        b.record()
        torch.cuda.synchronize()
        if i > 0:
            rd.append(a.elapsed_time(b) * 1e3)
    if layer.status() != 0:
        raise RuntimeError("device status word set")
    put("read_logits_after_step", float(np.median(rd)), w.T * w.E * 4, 0,
        "torch sum of a logits-sized tensor in no cache, right after a step (the next top-k's memory state; "
        "median of %d)" % steps)
    del cold
    ab = algorithmic_bytes(w)
    gev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    gev[0].record()
    gev[1].record()
    layer.time_gather(*gev)
    us = []
    for _ in range(steps):
        layer.dispatch(hidden)
        torch.cuda.synchronize()
        us.append(gev[0].elapsed_time(gev[1]) * 1e3)
    layer.time_gather()
    put("library_dispatch_gather", float(np.mean(us)), w.T * row_bytes, N * row_bytes,
        "gather_vec_kernel of moe_plan_dispatch (event-timed; algorithmic bytes %d)" % ab["gather"])
    layer.close()
    return {"workload": w.name, "rows": N, "row_bytes": row_bytes, "steps": steps, "peak_GBps": HBM_PEAK_GBS,
            "rates": out}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=synth.WORKLOAD_ORDER)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", choices=("quality", "solver"), default=None,
                    help="print TopoEP's plan-quality or solver-scaling study instead of the path benchmark")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of the path, time a plain copy of this many bytes (counter calibration)")
    ap.add_argument("--ceilings", action="store_true",
                    help="instead of the path, time torch's own fill, scattered fill, read, copy and "
                         "index_select on the workload's gather shapes (device reference rates)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the step timings of the other four workloads (the line's `configs` object)")
    ap.add_argument("--config-steps", type=int, default=20)
    ap.add_argument("--config-warmup", type=int, default=5)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the planning path runs its logical EP ranks on a single device. "
              "Run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        sweep(args.sweep, 20, 200)
        return
    if args.copy_bytes > 0:
        print(json.dumps(copy_reference(args.copy_bytes, args.steps)), flush=True)
        return
    w = synth.WORKLOADS[args.workload]
    if args.ceilings:
        print(json.dumps(ceilings(w, args.steps)), flush=True)
        return
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_budget)
    g = run_gpu(w, args.steps, args.warmup)
    ms_per_step = g["ms_total"] / args.steps
    slots = w.T * w.k * w.L
    value = slots / (ms_per_step / 1e3)
    ab = algorithmic_bytes(w)
    gather_ms = g["step_gather_ms"]
    achieved = ab["gather"] / (gather_ms / 1e3) / 1e9
    traffic, traffic_source = gather_traffic(w)
    chain_gbs = ab["total"] / (ms_per_step / 1e3) / 1e9
    chain_one = ab["total"] / (g["ms_serial"] / args.steps / 1e3) / 1e9
    configs = {}
    if not args.no_configs:
        import torch
        dev = torch.device("cuda", 0)
        for name in synth.WORKLOAD_ORDER:
            if name != w.name:
                configs[name] = config_line(synth.WORKLOADS[name], args.config_steps, args.config_warmup, dev)
    disp_gather_ms = g["dispatch_gather_ms"]
    out = {
        "metric": "routed token-slots/sec for route+plan+dispatch; gather HBM GB/s vs peak",
        "value": value, "unit": "token-slots/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "pipeline": "2 batches in flight (two handles on two streams, each with its own input batch; consecutive steps "
                    "alternate; when the layer is not cache-resident the two handles' row copies take turns "
                    "through moe_plan_set_gather_order)",
        "latency_ms_per_step": g["ms_serial"] / args.steps,
        "latency_us": {"median": float(np.median(g["step_ms"])) * 1e3, "min": float(np.min(g["step_ms"])) * 1e3,
                       "mean": float(np.mean(g["step_ms"])) * 1e3},
        "dtype": "fp32 compare (top-k), int32 plan (int64 benefits), bf16 row copy", "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "E": w.E, "k": w.k, "R": w.R, "G": w.G, "H": w.H,
                   "replica_budget": w.B, "layers": w.L, "zipf_s": w.zipf_s, "beta": w.beta,
                   "couple_p": w.couple_p, "seed": w.seed, "cache_resident": working_set(w) < CACHE_BYTES,
                   "inputs_sha256_16": inputs_sha(w), "second_batch_seed": second_batch(w).seed,
                   "second_batch_sha256_16": inputs_sha(second_batch(w))},
        "roofline": {"bound": "hbm",
                     "kernel": step_copy_kernel(w),
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "traffic_source": traffic_source,
                     "algorithmic_bytes_per_launch": ab["gather"], "launch_ms": gather_ms,
                     "timing": "HIP events the library records right before and after the kernel's launch "
                               "(moe_plan_set_events), in a one-stream pass of the same steps, mean of %d launches"
                               % (args.steps * w.L)},
        "chain": {"algorithmic_bytes_per_step": ab["total"], "achieved": chain_gbs, "peak": HBM_PEAK_GBS,
                  "unit": "GB/s", "frac": chain_gbs / HBM_PEAK_GBS, "frac_one_stream": chain_one / HBM_PEAK_GBS},
        "configs": configs,
        "combine": {"kernel": "combine (moe_plan_combine)", "us": g["combine_ms"] * 1e3,
                    "algorithmic_bytes_per_launch": ab["combine"],
                    "achieved": ab["combine"] / (g["combine_ms"] / 1e3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": ab["combine"] / (g["combine_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS},
        "placement": placement_report(w, g["place"], cpu is not None),
        "dedup_dispatch": {"kernel": "deduplicated dispatch (moe_plan_dedup_dispatch, correlated placement)",
                           "us": g["dedup"]["us"], "rows": g["dedup"]["n_rows"], "slot_rows": w.T * w.k,
                           "algorithmic_bytes_per_launch": dedup_bytes(w, g["dedup"]["n_rows"]),
                           "achieved": dedup_bytes(w, g["dedup"]["n_rows"]) / (g["dedup"]["us"] / 1e6) / 1e9,
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": dedup_bytes(w, g["dedup"]["n_rows"]) / (g["dedup"]["us"] / 1e6) / 1e9 / HBM_PEAK_GBS,
                           "vs_dispatch_us": g["per_call_ms"]["dispatch"] * 1e3},
        "replica_pull": g["pull"],
        "plan_quality": g["quality"],
        "token_shuffle": g["shuffle"],
        "stages": {name: {"us_mean": g["per_call_ms"][name] * 1e3, "us_median": g["per_call_ms_median"][name] * 1e3,
                          "us_min": g["per_call_ms_min"][name] * 1e3, "algorithmic_bytes": ab[name] / w.L,
                          "achieved_GBps": ab[name] / w.L / (g["per_call_ms"][name] / 1e3) / 1e9,
                          "frac": ab[name] / w.L / (g["per_call_ms"][name] / 1e3) / 1e9 / HBM_PEAK_GBS,
                          "bound": "hbm" if name == "dispatch" else "latency"}
                   for name in ("route", "plan", "dispatch")},
        "dispatch_gather": {"kernel": "gather_vec_kernel<4, false> (the row copy of moe_plan_dispatch)",
                            "us": disp_gather_ms * 1e3, "algorithmic_bytes_per_launch": ab["gather"],
                            "frac": ab["gather"] / (disp_gather_ms / 1e3) / 1e9 / HBM_PEAK_GBS},
        "device_info": dict(g["dinfo"], hbm_peak_GBps=HBM_PEAK_GBS, measured_copy_GBps=g["copy"]["GBps"]),
        "per_call_us": {k: v * 1e3 for k, v in g["per_call_ms"].items()},
        "per_call_us_min": {k: v * 1e3 for k, v in g["per_call_ms_min"].items()},
        "cpu_baseline": cpu,
        "device": g["device"],
    }
    if cpu is not None:
        P = g["pull"]["bytes_per_expert"] // 2 if g["pull"] else (9 * w.H * w.H // 4) // 2
        beside = oracle_beside(w, P, w.L > 1)
        for key, val in beside.items():
            if key == "token_shuffle" and out["token_shuffle"]:
                for entry, ms in zip(out["token_shuffle"], val["oracle_ms"]):
                    entry["oracle_ms"] = ms
            elif isinstance(out.get(key), dict):
                out[key].update(val)
            elif out.get(key) is None and key != "token_shuffle":
                out[key] = val
    if any(g["status"]):
        out["status_flags"] = g["status"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
