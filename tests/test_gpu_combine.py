"""GPU parity of the gate-weighted combine (moe_plan_combine) against the CPU oracle.

The oracle computes in float64; the kernel computes the softmax weights with
expf, accumulates in fp32 in slot order and rounds once to bf16.  Bound used
(derived from that arithmetic): with y the oracle value and S = sum_j w_j |x_j|,
  |gpu - y| <= 2^-8 |y| + 2 (2k + 30) 2^-24 S
(2^-8 |y|: the final bf16 rounding; the second term: expf within 2 ulp, the
k-term sums, the division and the fp32 FMA chain).  Identity experts (the
dispatch buffer itself) must come back bit-exact, since the weights sum to one
within a few fp32 ulps.
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


def bf16_bits(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def finite_rows(seed: int, n: int, H: int) -> np.ndarray:
    return bf16_bits(np.random.default_rng(seed).standard_normal((n, H)).astype(np.float32))


def run_layer(mp, cfg, logits, hidden):
    layer = mp.Layer(cfg, cooc=False)
    dev = layer.device
    hid = torch.from_numpy(np.ascontiguousarray(hidden).view(np.int16)).to(dev)
    layer.step(torch.from_numpy(np.ascontiguousarray(logits)).to(dev), hid)
    return layer, hid


def check_bound(cfg, got_bits, want, absum, what):
    got = bf16_to_f64(got_bits)
    bound = 2.0 ** -8 * np.abs(want) + 2 * (2 * cfg.k + 30) * 2.0 ** -24 * absum
    err = np.abs(got - want)
    bad = err > bound
    assert not bad.any(), "%s: %d elements outside the bound, worst excess %g" % (
        what, int(bad.sum()), float((err - bound).max()))


def oracle_combine_with_bound(cfg, topk_val, slot_pos, rows):
    oc = oracle.make_cfg(cfg.T, cfg.E, cfg.k, cfg.R, cfg.G, cfg.H, cfg.replica_budget)
    y = oracle.combine(oc, topk_val, slot_pos, rows)
    absum = oracle.combine(oc, topk_val, slot_pos, rows & np.uint16(0x7FFF))  # sum_j w_j |x_j|
    return y, absum


@pytest.mark.parametrize("name", ["deepseek_v3_layer", "qwen3_layer", "kimi_layer"])
def test_identity_experts_return_the_tokens_bit_exact(mp, name):
    w = synth.WORKLOADS[name]
    cfg = mp.make_config(w.T, w.E, w.k, w.R, w.G, w.H, w.B)
    print("combine identity %s T=%d k=%d H=%d" % (name, w.T, w.k, w.H), flush=True)
    hidden = synth.hidden(w)
    layer, hid = run_layer(mp, cfg, synth.logits(w), hidden)
    out = layer.combine(layer.dispatch_out.dispatch)
    torch.cuda.synchronize()
    assert layer.status() == 0
    assert torch.equal(out, hid)
    layer.close()


@pytest.mark.parametrize("shape", [(4096, 64, 8, 8, 4, 512), (1536, 128, 6, 32, 8, 264), (640, 8, 2, 4, 2, 13),
                                   (1152, 896, 16, 64, 8, 7168), (2048, 2048, 32, 256, 8, 24),
                                   # rows of 256, 257 and 1025 vectors: the edges of the store rounds
                                   (704, 64, 8, 8, 4, 2048), (704, 64, 8, 8, 4, 2056), (320, 64, 8, 8, 4, 8200)])
def test_random_expert_outputs_against_the_oracle(mp, shape):
    T, E, k, R, G, H = shape
    cfg = mp.make_config(T, E, k, R, G, H, 2 * R)
    print("combine random T=%d E=%d k=%d R=%d G=%d H=%d" % shape, flush=True)
    lg = inputs.random_logits(T + H, T, E)
    layer, _ = run_layer(mp, cfg, lg, finite_rows(1, T, H))
    rows = finite_rows(2, T * k, H)
    out = layer.combine(torch.from_numpy(rows.view(np.int16)).to(layer.device))
    torch.cuda.synchronize()
    assert layer.status() == 0
    o = oracle.run_all(oracle.make_cfg(T, E, k, R, G, H, 2 * R), lg, finite_rows(1, T, H), want_cooc=False)
    np.testing.assert_array_equal(layer.dispatch_out.slot_pos.cpu().numpy(), o["slot_pos"])
    y, absum = oracle_combine_with_bound(cfg, o["topk_val"], o["slot_pos"], rows)
    check_bound(cfg, out.cpu().numpy().view(np.uint16), y, absum, "random T=%d H=%d" % (T, H))
    layer.close()


def test_full_size_random_outputs_sampled(mp):
    """DeepSeek-V3-shaped layer at full size; 512 sampled tokens against the oracle."""
    w = synth.WORKLOADS["deepseek_v3_layer"]
    cfg = mp.make_config(w.T, w.E, w.k, w.R, w.G, w.H, w.B)
    print("combine full size sampled", flush=True)
    layer, _ = run_layer(mp, cfg, synth.logits(w), synth.hidden(w))
    g = torch.Generator(device=layer.device).manual_seed(5)
    rows = torch.randn((w.T * w.k, w.H), generator=g, device=layer.device, dtype=torch.float32).to(torch.bfloat16)
    out = layer.combine(rows.view(torch.int16))
    torch.cuda.synchronize()
    assert layer.status() == 0
    toks = np.random.default_rng(3).choice(w.T, 512, replace=False)
    val = layer.route_out.topk_val.cpu().numpy()[toks]
    sp = layer.dispatch_out.slot_pos.cpu().numpy().reshape(w.T, w.k)[toks]
    sub = rows.view(torch.int16).cpu().numpy().view(np.uint16)[sp.reshape(-1)]
    sub_cfg = mp.make_config(512, w.E, w.k, 1, 1, w.H, 0)
    y, absum = oracle_combine_with_bound(sub_cfg, val, np.arange(512 * w.k, dtype=np.int32), sub)
    check_bound(sub_cfg, out.cpu().numpy().view(np.uint16)[toks], y, absum, "full size")
    layer.close()


def test_equal_logits_and_non_finite_logits(mp):
    T, E, k, R, G, H = 512, 32, 4, 4, 2, 64
    cfg = mp.make_config(T, E, k, R, G, H, 4)
    layer, _ = run_layer(mp, cfg, inputs.random_logits(9, T, E), finite_rows(4, T, H))
    rows = finite_rows(6, T * k, H)
    rows_t = torch.from_numpy(rows.view(np.int16)).to(layer.device)
    layer.route_out.topk_val.fill_(0.5)
    out = layer.combine(rows_t)
    torch.cuda.synchronize()
    assert layer.status() == 0
    sp = layer.dispatch_out.slot_pos.cpu().numpy().reshape(T, k)
    mean = bf16_to_f64(rows)[sp].mean(axis=1)
    absum = np.abs(bf16_to_f64(rows)[sp]).mean(axis=1)
    check_bound(cfg, out.cpu().numpy().view(np.uint16), mean, absum, "equal logits")
    layer.route_out.topk_val[7, 2] = float("inf")
    layer.combine(rows_t)
    torch.cuda.synchronize()
    assert layer.status() != 0
    layer.close()
