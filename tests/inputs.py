"""Seeded test inputs shared by the oracle tests and the GPU parity tests.

Random numbers and shapes only -- none of the planning arithmetic.
"""
from __future__ import annotations

import numpy as np


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def random_topk(seed: int, T: int, E: int, k: int, skew: float = 1.0) -> np.ndarray:
    """int32 [T, k]: each row k distinct experts, drawn with Zipf-like weights."""
    g = rng(seed)
    w = 1.0 / np.arange(1, E + 1) ** skew
    w = w[g.permutation(E)]
    w = w / w.sum()
    out = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        out[t] = g.choice(E, size=k, replace=False, p=w)
    return out


def random_logits(seed: int, T: int, E: int, ties: bool = False) -> np.ndarray:
    """float32 [T, E]; with ties=True values come from a small set so equal logits are common."""
    g = rng(seed)
    if ties:
        vals = np.array([-1.5, -0.0, 0.0, 0.25, 1.0, 2.0], dtype=np.float32)
        return vals[g.integers(0, len(vals), size=(T, E))]
    bias = -np.log1p(g.permutation(E)).astype(np.float64)
    return (g.standard_normal((T, E)) + bias).astype(np.float32)


def random_hidden(seed: int, T: int, H: int) -> np.ndarray:
    """uint16 bf16 bit patterns [T, H]."""
    g = rng(seed)
    return g.integers(0, 1 << 16, size=(T, H), dtype=np.uint16)


def small_configs(seed: int, n: int):
    """Random small, valid layer shapes (dicts with T, E, k, R, G, H, B, W, S, max_iters)."""
    g = rng(seed)
    out = []
    while len(out) < n:
        G = int(g.choice([1, 2, 3, 4]))
        M = int(g.choice([1, 2, 3]))
        R = G * M
        Er = int(g.integers(1, 4))
        E = R * Er
        k = int(g.integers(1, min(E, 6) + 1))
        Tr = int(g.integers(0, 70))
        T = R * Tr
        B = int(g.integers(0, 2 * R + 1))
        W = int(g.choice([0, 5, 40, -1]))
        out.append(dict(T=T, E=E, k=k, R=R, G=G, H=int(g.choice([3, 8, 16])), B=B,
                        n_slot=int(g.choice([0, 0, 1, 2])), W=W, S=int(g.choice([1, 2])),
                        max_iters=int(g.choice([0, 0, 1, 3]))))
    return out
