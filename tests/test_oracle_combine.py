"""Pins of the combine oracle (the return path of the dispatch, [TopoEP] section
2.1, Fig. 1; gate weights read as the softmax of the k selected logits).

The checks use what mathematics fixes, not the oracle's own formula:
identity experts give back the token rows (the weights sum to one), one
selected expert gives its row, equal logits give the mean, unit-vector expert
outputs expose the weights themselves (two experts: the logistic function of
the logit gap), shifting every logit leaves the result unchanged, and a
power-of-two scale of the expert outputs scales the result exactly.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from tests import inputs

BF16_ONE = 0x3F80


def bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even (values here are finite)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return r


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def finite_rows(seed: int, n: int, H: int) -> np.ndarray:
    """bf16 bit patterns [n, H] of N(0, 1) values (finite, unlike arbitrary bit patterns)."""
    g = np.random.default_rng(seed)
    return bf16(g.standard_normal((n, H)).astype(np.float32))


def routed_layer(seed, T=192, E=12, k=3, R=4, G=2, H=16, B=4, logits=None):
    """A small layer through the oracle: route, plan, dispatch (slot positions, dispatched rows)."""
    cfg = oracle.make_cfg(T, E, k, R, G, H, B)
    lg = inputs.random_logits(seed, T, E) if logits is None else logits
    hid = finite_rows(seed, T, H)
    out = oracle.run_all(cfg, lg, hid)
    return cfg, out, hid


def test_identity_experts_return_the_token_rows():
    cfg, out, hid = routed_layer(1)
    assert not np.array_equal(out["slot_pos"], np.arange(cfg.T * cfg.k))  # a real permutation
    y = oracle.combine(cfg, out["topk_val"], out["slot_pos"], out["dispatch"])
    x = bf16_to_f64(hid)
    np.testing.assert_allclose(y, x, rtol=1e-12, atol=0)


def test_one_expert_gives_its_row():
    cfg, out, hid = routed_layer(2, k=1)
    rows = finite_rows(7, cfg.T * cfg.k, cfg.H)  # arbitrary expert outputs
    y = oracle.combine(cfg, out["topk_val"], out["slot_pos"], rows)
    want = bf16_to_f64(rows)[out["slot_pos"].reshape(cfg.T)]
    np.testing.assert_array_equal(y, want)


def test_equal_logits_give_the_mean():
    cfg, out, hid = routed_layer(3, k=4)
    val = np.full((cfg.T, cfg.k), 0.75, np.float32)
    rows = finite_rows(8, cfg.T * cfg.k, cfg.H)
    y = oracle.combine(cfg, val, out["slot_pos"], rows)
    r = bf16_to_f64(rows)[out["slot_pos"].reshape(cfg.T, cfg.k)]  # [T][k][H]
    np.testing.assert_allclose(y, r.mean(axis=1), rtol=1e-13, atol=1e-15)


def unit_rows(cfg, slot_pos):
    """Expert output of slot (t, j) = the unit vector of column j."""
    rows = np.zeros((cfg.T * cfg.k, cfg.H), np.uint16)
    sp = slot_pos.reshape(cfg.T, cfg.k)
    for j in range(cfg.k):
        rows[sp[:, j], j] = BF16_ONE
    return rows


def test_unit_outputs_expose_the_weights():
    cfg, out, hid = routed_layer(4, k=2)
    y = oracle.combine(cfg, out["topk_val"], out["slot_pos"], unit_rows(cfg, out["slot_pos"]))
    v = out["topk_val"].astype(np.float64)
    # two experts: w0 = 1 / (1 + e^(v1 - v0)), the logistic function of the logit gap
    w0 = np.array([1.0 / (1.0 + math.exp(v[t, 1] - v[t, 0])) for t in range(cfg.T)])
    np.testing.assert_allclose(y[:, 0], w0, rtol=1e-14)
    np.testing.assert_allclose(y[:, 0] + y[:, 1], 1.0, rtol=1e-14)
    assert (y[:, 2:] == 0).all()
    assert (y[:, 0] >= y[:, 1]).all()  # logits come in descending order


def test_weights_for_more_experts_sum_to_one_and_follow_the_logit_order():
    cfg, out, hid = routed_layer(5, k=5, E=16)
    y = oracle.combine(cfg, out["topk_val"], out["slot_pos"], unit_rows(cfg, out["slot_pos"]))
    w = y[:, :cfg.k]
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-14)
    assert (np.diff(w, axis=1) <= 0).all()
    # ratio of two weights is e^(gap of their logits)
    v = out["topk_val"].astype(np.float64)
    np.testing.assert_allclose(w[:, 0] / w[:, 3], np.exp(v[:, 0] - v[:, 3]), rtol=1e-12)


def test_shifted_logits_change_nothing_even_when_large():
    """Logits on a 1/8 grid, so that a shift by +-1000 is exact in float32; without the
    maximum taken out first, exp(1000) would overflow."""
    cfg, out, hid = routed_layer(6, k=3)
    rows = finite_rows(9, cfg.T * cfg.k, cfg.H)
    v = np.round(out["topk_val"].astype(np.float64) * 8) / 8
    y0 = oracle.combine(cfg, v, out["slot_pos"], rows)
    for c in (1000.0, -1000.0):
        assert np.array_equal((v + c).astype(np.float32).astype(np.float64), v + c)
        y1 = oracle.combine(cfg, v + c, out["slot_pos"], rows)
        np.testing.assert_allclose(y1, y0, rtol=1e-12, atol=1e-15)


def test_power_of_two_scale_is_exact():
    cfg, out, hid = routed_layer(10, k=3)
    rows = finite_rows(11, cfg.T * cfg.k, cfg.H)
    y = oracle.combine(cfg, out["topk_val"], out["slot_pos"], rows)
    y2 = oracle.combine(cfg, out["topk_val"], out["slot_pos"], bf16(bf16_to_f64(rows).astype(np.float32) * 2))
    np.testing.assert_array_equal(y2, 2 * y)


def test_non_finite_selected_logit_is_an_error():
    cfg, out, hid = routed_layer(12, k=2)
    val = out["topk_val"].copy()
    val[5, 1] = np.inf
    with pytest.raises(ValueError):
        oracle.combine(cfg, val, out["slot_pos"], out["dispatch"])
