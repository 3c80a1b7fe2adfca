"""The seeded input generator: bf16 rounding, determinism, sampled rows, planted targets."""

import json
import os

import numpy as np
import torch

from synth.configs import CONFIGS
from synth.inputs import (DrafterInputs, bf16_bits_to_f32, f32_to_bf16_bits,
                          geometric_prefix_lengths, make_rng, planted_targets, target_layer_ids)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_rounding_matches_round_to_nearest_even():
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -2.5, 3.0e-39,
                     65504.0, 1e30], dtype=np.float32)
    bits = f32_to_bf16_bits(vals)
    assert bits[0] == 0x3F80
    assert bits[1] == 0x3F80          # tie -> even
    assert bits[2] == 0x3F82          # tie -> even (odd neighbour below)
    assert bits[3] == 0x3F81          # just above the tie -> up
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * rng.choice([1e-3, 1, 1e3], size=100000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(f32_to_bf16_bits(x), ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(ref),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_target_layer_ids_golden():
    with open(os.path.join(GOLDEN, "target_layers.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        assert target_layer_ids(c["n_target_layers"]) == c["ids"]


def test_generation_is_deterministic_and_thread_independent():
    wl = CONFIGS[1]
    a = DrafterInputs(wl, threads=1)
    b = DrafterInputs(wl, threads=7)
    for n in ("embed", "fc", "l0.wq", "l0.in_norm", "lm_head"):
        np.testing.assert_array_equal(a.weight(n), b.weight(n))
    assert a.weight("l0.in_norm").min() >= 0.5 and a.weight("l0.in_norm").max() <= 1.5
    assert abs(a.weight("fc").std() - 0.02) < 0.001
    u = DrafterInputs(wl, gain_mode="unit")
    np.testing.assert_array_equal(u.weight("final_norm"), 1.0)


def test_sampled_feature_rows_equal_full_draw():
    wl = CONFIGS[3]
    inp = DrafterInputs(wl)
    lens = inp.ctx_lengths()
    assert lens.min() >= 512 and lens.max() <= 8192 and len(lens) == 32
    full = inp.ctx_feats(2, 5, n_rows=2100)
    rows = [0, 5, 1023, 1024, 2099]
    np.testing.assert_array_equal(inp.ctx_feats(2, 5, rows=rows), full[rows])
    assert full.dtype == np.uint16
    f = bf16_bits_to_f32(full)
    assert abs(f.std() - 1.0) < 0.01


def test_planted_targets_and_geometric_lengths():
    rng = make_rng(0, "t")
    d = rng.integers(0, 151935, size=(64, 15))
    k = geometric_prefix_lengths(rng, 6.5, 15, 64)
    t = planted_targets(d, k, 151936, rng)
    assert t.shape == (64, 16)
    assert t.max() <= 151934
    for b in range(64):
        kb = k[b]
        assert np.all(t[b, :kb] == d[b, :kb])
        if kb < 15:
            assert t[b, kb] != d[b, kb]
    big = geometric_prefix_lengths(make_rng(0, "g"), 6.5, 15, 200000)
    # capped geometric on {0,1,..} with mean 6.5: E[min(K,15)] = sum_{j=1..15} q^j, q = 6.5/7.5
    q = 6.5 / 7.5
    expect = sum(q ** j for j in range(1, 16))
    assert abs(big.mean() - expect) < 0.03
