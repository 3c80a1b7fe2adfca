"""Pins of the oracle's temperature sampling (Gumbel-max with Philox4x32-10
noise): the generator against its published known answers and rocRAND's
independent implementation, the sampled frequencies against
softmax(logits / T), the cold limit against the greedy pick."""

import json
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle.dflash_oracle import (OracleDrafter, gumbel_noise, lm_head_argmax, lm_head_sample,
                                  philox4x32_10)
from tests.test_oracle import MICRO, _rand_weights

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ROCRAND_HEADER = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"


def test_philox_known_answer_vectors():
    kat = json.load(open(os.path.join(GOLDEN, "philox4x32_10_kat.json")))
    assert len(kat["cases"]) == 3
    for case in kat["cases"]:
        ctr = [np.uint64(int(x, 16)) for x in case["counter"]]
        key = [np.uint64(int(x, 16)) for x in case["key"]]
        out = philox4x32_10(ctr, key)
        assert [int(x) for x in out] == [int(x, 16) for x in case["out"]]


@pytest.mark.skipif(not (os.path.exists(ROCRAND_HEADER) and shutil.which("g++")),
                    reason="rocRAND headers or g++ not installed")
def test_philox_matches_rocrand_library_generator(tmp_path):
    """rocRAND's philox4x32_10 engine (header source, built here for the host)
    is an independent implementation of the same generator; its ten-round block
    function is compared on random counters and keys, small counters among them."""
    exe = str(tmp_path / "philox_block")
    src = os.path.join(os.path.dirname(__file__), "rocrand_philox_block.cpp")
    subprocess.run(["g++", "-O1", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    src, "-o", exe], check=True, capture_output=True)
    rng = np.random.default_rng(11)
    n = 256
    c = rng.integers(0, 2 ** 32, size=(n, 4), dtype=np.uint64)
    k = rng.integers(0, 2 ** 32, size=(n, 2), dtype=np.uint64)
    c[:8, 1:] = 0  # small counters, as the draft's ids, positions and sequences are
    c[8:16] = rng.integers(0, 64, size=(8, 4), dtype=np.uint64)
    lines = "".join(" ".join(f"{int(x):x}" for x in (*c[i], *k[i])) + "\n" for i in range(n))
    out = subprocess.run([exe], input=lines, check=True, capture_output=True, text=True).stdout
    ref = [[int(x, 16) for x in ln.split()] for ln in out.splitlines()]
    assert len(ref) == n
    mine = philox4x32_10([c[:, j] for j in range(4)], [k[:, j] for j in range(2)])
    for i in range(n):
        assert [int(m[i]) for m in mine] == ref[i], i


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


def test_gumbel_noise_independent_across_ids_sharing_a_block():
    """Ids v, v+16, v+32, v+48 draw from one Philox block (its four words): over
    many positions their noise, and that of every other pair among ids 0..63,
    must be uncorrelated (a word picked from the wrong id bits repeats noise)."""
    n = 4000
    g = gumbel_noise(3, 1, 0, np.arange(n)[:, None], np.arange(64)[None, :])
    corr = np.corrcoef(g.T)
    off = corr[~np.eye(64, dtype=bool)]
    assert np.max(np.abs(off)) < 6 / np.sqrt(n), np.max(np.abs(off))


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
