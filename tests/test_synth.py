"""The seeded input generator: determinism, independence of streams, moments, bf16 rounding."""
import numpy as np
import torch

import synth


def test_draws_deterministic_and_streams_differ():
    a = synth.draws(0, 3, 1000)
    b = synth.draws(0, 3, 1000)
    c = synth.draws(0, 4, 1000)
    d = synth.draws(1, 3, 1000)
    assert (a == b).all()
    assert (a != c).mean() > 0.99 and (a != d).mean() > 0.99
    u = ((a >> np.uint64(11)).astype(np.float64) + 0.5) / 2.0 ** 53
    assert abs(u.mean() - 0.5) < 0.03


def test_permutation_is_a_permutation():
    p = synth.permutation(0, 0, 1, 896)
    assert sorted(p.tolist()) == list(range(896))


def test_logits_shapes_prefix_and_moments():
    w = synth.WORKLOADS["qwen3_layer"]
    lg = synth.logits(w, T=2048)
    assert lg.shape == (2048, 128) and lg.dtype == np.float32
    lg2 = synth.logits(w, T=512)
    assert (lg2 == lg[:512]).all()          # counter-based: a prefix is the same tokens
    plain = synth.Workload("plain", T=20000, E=8, k=2, R=4, G=2, H=8, B=0)
    z = synth.logits(plain).astype(np.float64)
    assert abs(z.mean()) < 0.02 and abs(z.var() - 1) < 0.03


def test_zipf_bias_makes_hot_experts():
    w = synth.WORKLOADS["kimi_layer"]
    lg = synth.logits(w, T=512)
    top1 = np.bincount(lg.argmax(1), minlength=w.E)
    assert top1.max() > 20 * max(1, np.median(top1))


def test_coupled_groups_follow_the_map():
    w = synth.WORKLOADS["coupled_4layer"]
    g = synth.groups(w.seed, 20000, w.E // w.group_size, w.L, w.couple_p)
    phi = synth.permutation(w.seed, 0, 4, w.E // w.group_size)
    kept = (g[1] == phi[g[0]]).mean()
    assert 0.70 < kept < 0.76                # 0.7 kept + 0.3/16 chance


def test_hidden_is_rne_bf16_of_normals():
    w = synth.Workload("h", T=64, E=8, k=2, R=4, G=2, H=250, B=0)
    h = synth.hidden(w)
    f = h.astype(np.uint32) << 16
    x = f.view(np.float32).astype(np.float64)
    assert abs(x.mean()) < 0.05 and abs(x.var() - 1) < 0.05
    # the bf16 bits are torch's round-to-nearest-even of the generator's f32 normals
    t = torch.from_numpy(synth.hidden_f32(w, 64, 250)).to(torch.bfloat16)
    assert (t.view(torch.int16).numpy().view(np.uint16) == h).all()
