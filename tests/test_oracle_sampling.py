"""Pins of the oracle's temperature sampling (Gumbel-max with Philox4x64-10
noise): the generator against its published known answers and numpy's
independent library implementation, the sampled frequencies against
softmax(logits / T), the cold limit against the greedy pick."""

import json
import os

import numpy as np
import pytest

from oracle.dflash_oracle import (OracleDrafter, gumbel_noise, lm_head_argmax, lm_head_sample,
                                  philox4x64_10)
from tests.test_oracle import MICRO, _rand_weights

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answer_vectors():
    kat = json.load(open(os.path.join(GOLDEN, "philox4x64_10_kat.json")))
    for case in kat["cases"]:
        ctr = [np.uint64(int(x, 16)) for x in case["counter"]]
        key = [np.uint64(int(x, 16)) for x in case["key"]]
        out = philox4x64_10(ctr, key)
        assert [int(x) for x in out] == [int(x, 16) for x in case["out"]]


def test_philox_matches_numpy_library_generator():
    """numpy.random.Philox is the same generator (4x64, 10 rounds); it advances
    its counter before producing a block, so counter c - 1 yields block c."""
    rng = np.random.default_rng(11)
    n = 64
    c = rng.integers(0, 2 ** 64, size=(n, 4), dtype=np.uint64)
    k = rng.integers(0, 2 ** 64, size=(n, 2), dtype=np.uint64)
    c[:4, 1:] = 0  # small counters too
    mine = philox4x64_10([c[:, j] for j in range(4)], [k[:, j] for j in range(2)])
    for i in range(n):
        cint = sum(int(c[i, j]) << (64 * j) for j in range(4))
        kint = int(k[i, 0]) | (int(k[i, 1]) << 64)
        ref = np.random.Philox(counter=(cint - 1) % (1 << 256), key=kint).random_raw(4)
        assert [int(m[i]) for m in mine] == [int(x) for x in ref], i


def test_gumbel_noise_keyed_deterministic_and_finite():
    v = np.arange(4096)
    g1 = gumbel_noise(7, 3, 2, 1000, v)
    assert np.array_equal(g1, gumbel_noise(7, 3, 2, 1000, v))
    for other in (gumbel_noise(7, 4, 2, 1000, v), gumbel_noise(8, 3, 2, 1000, v),
                  gumbel_noise(7, 3, 1, 1000, v), gumbel_noise(7, 3, 2, 1001, v)):
        assert np.mean(g1 == other) < 0.01
    assert np.all(np.isfinite(g1))
    # standard Gumbel: mean = Euler-Mascheroni constant, variance = pi^2 / 6
    g = gumbel_noise(1, 0, 0, np.arange(200)[:, None], np.arange(1000)[None, :]).ravel()
    assert abs(g.mean() - 0.5772156649) < 5 * np.sqrt(np.pi ** 2 / 6 / g.size)
    assert abs(g.var() - np.pi ** 2 / 6) < 0.02


@pytest.mark.parametrize("temperature", [0.5, 1.0, 2.0])
def test_gumbel_max_frequencies_follow_tempered_softmax(temperature):
    logits = np.array([0.0, 0.5, 1.0, 1.5, 2.0, -1.0])
    n = 120_000
    z = np.ones((n, 1))
    ids, _, _ = lm_head_sample(z, logits[:, None], temperature, seed=5, offset=9,
                               seq=np.zeros(n, dtype=np.int64), pos=np.arange(n))
    freq = np.bincount(ids, minlength=len(logits)) / n
    p = np.exp(logits / temperature)
    p /= p.sum()
    sigma = np.sqrt(p * (1 - p) / n)
    assert np.all(np.abs(freq - p) < 5 * sigma), (freq, p)


def test_cold_sampling_is_the_greedy_pick():
    rng = np.random.default_rng(3)
    z = rng.normal(size=(40, 16))
    w = rng.normal(size=(300, 16))
    g_ids, _, _ = lm_head_argmax(z, w)
    s_ids, _, _ = lm_head_sample(z, w, 1e-7, seed=1, offset=2, seq=np.zeros(40, dtype=np.int64),
                                 pos=np.arange(40))
    assert np.array_equal(g_ids, s_ids)


def test_oracle_draft_sampled_cold_equals_greedy_and_hot_differs():
    w = _rand_weights(MICRO, 21)
    rng = np.random.default_rng(4)
    outs = {}
    for name, temp in (("greedy", 0.0), ("cold", 1e-9), ("hot", 5.0)):
        o = OracleDrafter(MICRO, w, batch=2)
        for b in range(2):
            o.fuse_inject(b, [rng.normal(size=(9 + b, MICRO.feat_hidden)) for _ in range(5)])
        rng = np.random.default_rng(4)  # same features for every variant
        outs[name] = o.draft([3, 7], block=8, temperature=temp, seed=11, offset=0)["draft_ids"]
    assert np.array_equal(outs["greedy"], outs["cold"])
    assert not np.array_equal(outs["greedy"], outs["hot"])
