"""Seeded synthetic workloads for the MoE dispatch-planning path.

Only input generation lives here (random numbers and the logit/hidden recipe);
none of the planning arithmetic.  The CPU oracle and the HIP library both read
the arrays produced here.

The five workloads mirror the model shapes on the pages:
  * a Mixtral-shaped tiny layer (8 experts, top-2);
  * a Qwen3-30B-A3B-shaped layer (128 experts, top-8; TopoEP Table 1 and the
    Fig. 3 example use its 2,048-wide activations);
  * a DeepSeek-V3-shaped layer (256 routed experts, top-8, 7,168 hidden);
  * a Kimi-scale layer (896 experts, top-16, 7,168 hidden);
  * a 4-layer coupled-routing stack (128 experts, top-6) that exercises the
    layer-to-layer transition counts of "Expert Coupling in MoE Pretraining".
Logits follow TopoEP section 6.4 (random logits plus a fixed expert bias,
here Zipf over a seeded permutation) and the co-selection / cross-layer
structure of the coupling page (latent expert groups with a seeded group map).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field, asdict

import numpy as np

from . import build as _build

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        i32p = ctypes.POINTER(ctypes.c_int32)
        lib.synth_permutation.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int32, i32p]
        lib.synth_groups.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_double, i32p]
        lib.synth_logits.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                     ctypes.c_double, ctypes.c_double, ctypes.c_int32, i32p,
                                     ctypes.c_int32, ctypes.POINTER(ctypes.c_float)]
        lib.synth_hidden.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                     ctypes.POINTER(ctypes.c_uint16)]
        lib.synth_hidden_f32.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.POINTER(ctypes.c_float)]
        lib.synth_draws.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                    ctypes.POINTER(ctypes.c_uint64)]
        _LIB = lib
    return _LIB


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


@dataclass(frozen=True)
class Workload:
    """One MoE layer shape (or a stack of L layers) plus its logit recipe."""
    name: str
    T: int            # tokens (all logical ranks together)
    E: int            # routed experts
    k: int            # top-k
    R: int            # logical EP ranks
    G: int            # ranks per node (NVLink-domain analogue)
    H: int            # hidden size (bf16 elements per token row)
    B: int            # replica budget: extra expert instances per layer, all ranks together
    L: int = 1        # layers
    zipf_s: float = 0.0
    beta: float = 0.0
    group_size: int = 8
    couple_p: float = 0.0
    seed: int = 0

    def as_dict(self):
        return asdict(self)


WORKLOADS = {
    "mixtral_tiny": Workload("mixtral_tiny", T=4096, E=8, k=2, R=4, G=2, H=1024, B=2, zipf_s=1.0),
    "qwen3_layer": Workload("qwen3_layer", T=16384, E=128, k=8, R=8, G=4, H=2048, B=16,
                            zipf_s=1.1, beta=2.0),
    "deepseek_v3_layer": Workload("deepseek_v3_layer", T=32768, E=256, k=8, R=64, G=8, H=7168, B=32,
                                  zipf_s=1.2, beta=1.5),
    "kimi_layer": Workload("kimi_layer", T=16384, E=896, k=16, R=64, G=8, H=7168, B=64, zipf_s=1.3),
    "coupled_4layer": Workload("coupled_4layer", T=65536, E=128, k=6, R=32, G=8, H=2048, B=16, L=4,
                               beta=2.0, couple_p=0.7),
}
WORKLOAD_ORDER = ["mixtral_tiny", "qwen3_layer", "deepseek_v3_layer", "kimi_layer", "coupled_4layer"]


def skew_layer(router_skew: float, n_slot: int, E: int = 640, R: int = 32, T: int = 32768, k: int = 8, G: int = 8,
               H: int = 2048) -> Workload:
    """A layer of TopoEP section 6.4's synthetic routing: random logits plus a fixed
    expert-specific bias, router_skew 0 uniform in expectation and more negative
    values concentrating the load.  The bias is router_skew * ln(1 + rank(e)) over a
    seeded expert permutation (a Zipf law with exponent -router_skew).  Replica
    budget n_slot per rank.  Default shape: the Fig. 10 workload (32 ranks in
    nodes of 8, 640 experts, top-8)."""
    return Workload("skew%g_slots%d_E%d_R%d" % (router_skew, n_slot, E, R), T=T, E=E, k=k, R=R, G=G, H=H,
                    B=n_slot * R, zipf_s=-float(router_skew))


def permutation(seed: int, layer: int, kind: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _lib().synth_permutation(seed, layer, kind, n, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    return out


def groups(seed: int, T: int, ngroups: int, L: int, couple_p: float) -> np.ndarray:
    out = np.empty((L, T), dtype=np.int32)
    if T > 0:
        _lib().synth_groups(seed, T, ngroups, L, couple_p, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    return out


def logits(w: Workload, layer: int = 0, T: int | None = None, g: np.ndarray | None = None) -> np.ndarray:
    """Gate logits f32 [T, E] of one layer.  T defaults to w.T (a prefix of the tokens if smaller)."""
    T = w.T if T is None else T
    out = np.empty((T, w.E), dtype=np.float32)
    if T == 0:
        return out
    gp = None
    if w.beta != 0.0:
        if g is None:
            g = groups(w.seed, T, max(1, w.E // w.group_size), w.L, w.couple_p)
        g_l = np.ascontiguousarray(g[layer, :T], dtype=np.int32)
        gp = g_l.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    _lib().synth_logits(w.seed, layer, T, w.E, w.zipf_s, w.beta, w.group_size, gp, _threads(),
                        out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
    return out


def all_logits(w: Workload, T: int | None = None) -> list:
    """Logits of every layer of the workload (shared latent groups across layers)."""
    T = w.T if T is None else T
    g = None
    if w.beta != 0.0 and T > 0:
        g = groups(w.seed, T, max(1, w.E // w.group_size), w.L, w.couple_p)
    return [logits(w, l, T, g) for l in range(w.L)]


def hidden(w: Workload, T: int | None = None, H: int | None = None) -> np.ndarray:
    """bf16 hidden states as uint16 bit patterns [T, H]."""
    T = w.T if T is None else T
    H = w.H if H is None else H
    out = np.empty((T, H), dtype=np.uint16)
    if T * H > 0:
        _lib().synth_hidden(w.seed, T, H, _threads(), out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)))
    return out


def hidden_f32(w: Workload, T: int, H: int) -> np.ndarray:
    """The f32 normals that synth.hidden rounds to bf16 (tests only)."""
    out = np.empty((T, H), dtype=np.float32)
    _lib().synth_hidden_f32(w.seed, T, H, out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
    return out


def draws(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _lib().synth_draws(seed, stream, n, out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)))
    return out
