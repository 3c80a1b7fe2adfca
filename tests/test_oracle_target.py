"""Pins of the oracle's autoregressive parts: the synthetic target model that
verifies a drafted block and provides the features the drafter fuses, the
input-fusion variant of the injection, and the speculative loop as a whole.

- causal attention against attention over a truncated key set;
- the target and the input-fusion injection against one-token-at-a-time
  explicit-loop brute force (tests/bruteforce.py), fp64;
- chunked == one-shot (causal processing is incremental);
- a one-layer drafter with unit gains: the input-fusion cache equals the
  KV-injection cache (its only layer sees the normalised fused row either way);
- lossless: the speculative loop commits exactly the target's own greedy tokens,
  with random weights (mostly one token per round) and with a planted agreement
  that makes every draft match (full blocks accepted)."""

import numpy as np
import pytest

from oracle.dflash_oracle import (OracleDrafter, OracleTarget, autoregressive_generate,
                                  block_attention, speculative_generate)
from synth.configs import DrafterDims
from tests.bruteforce import brute_input_fusion, brute_target
from tests.test_oracle import MICRO, _rand_weights, _to_lists

TARGET = DrafterDims(n_layers=3, hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=8, inter=48,
                     vocab=64, n_feat_layers=2, feat_hidden=32, block_max=16, dtype="f32",
                     rope_theta=10000.0)
CAPTURE = [0, 2]   # the drafter fuses the states leaving target layers 0 and 2
DRAFT = DrafterDims(n_layers=2, hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=8, inter=48,
                    vocab=64, n_feat_layers=2, feat_hidden=32, block_max=16, dtype="f32",
                    rope_theta=10000.0)


def test_causal_attention_is_attention_over_the_keys_so_far():
    rng = np.random.default_rng(30)
    L, B = 5, 4
    q = rng.normal(size=(B, 4, 8))
    k = rng.normal(size=(L + B, 2, 8))
    v = rng.normal(size=(L + B, 2, 8))
    out = block_attention(q, k, v, causal_ctx=L)
    for r in range(B):
        ref = block_attention(q[r:r + 1], k[:L + r + 1], v[:L + r + 1])
        np.testing.assert_allclose(out[r], ref[0], rtol=1e-12)
    # one row: causal is the plain attention over everything
    np.testing.assert_allclose(block_attention(q[:1], k[:L + 1], v[:L + 1], causal_ctx=L),
                               block_attention(q[:1], k[:L + 1], v[:L + 1]), rtol=1e-12)


def test_target_matches_bruteforce():
    w = _rand_weights(TARGET, 31)
    rng = np.random.default_rng(32)
    ids = rng.integers(0, TARGET.vocab - 1, size=9)
    t = OracleTarget(TARGET, w, batch=1)
    nxt, top2, feats = t.forward(0, ids[:4], CAPTURE)           # a prompt ...
    nxt2, top2b, feats2 = t.forward(0, ids[4:], CAPTURE)        # ... then a block
    bf = brute_target(TARGET, _to_lists(w), list(ids), CAPTURE)
    assert list(nxt) + list(nxt2) == bf["next"]
    np.testing.assert_allclose(np.concatenate([top2, top2b]), np.array(bf["top2"]), rtol=1e-10)
    for i in range(len(CAPTURE)):
        np.testing.assert_allclose(np.concatenate([feats[i], feats2[i]]), np.array(bf["feats"][i]),
                                   rtol=1e-10, atol=1e-12)
    for l in range(TARGET.n_layers):
        np.testing.assert_allclose(t.k[l][0], np.array(bf["k"][l]), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(t.v[l][0], np.array(bf["v"][l]), rtol=1e-10, atol=1e-12)
    assert t.len[0] == 9 and t.base[0] == 4


def test_input_fusion_matches_bruteforce_and_chunks():
    d = MICRO
    w = _rand_weights(d, 33)
    rng = np.random.default_rng(34)
    feats = [rng.normal(size=(11, d.feat_hidden)) for _ in range(5)]
    one = OracleDrafter(d, w, batch=1)
    one.fuse_inject_input(0, feats)
    bf = brute_input_fusion(d, _to_lists(w), [[feats[i][t].tolist() for i in range(5)]
                                              for t in range(11)])
    for l in range(d.n_layers):
        np.testing.assert_allclose(one.k[l][0], np.array(bf["k"][l]), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(one.v[l][0], np.array(bf["v"][l]), rtol=1e-10, atol=1e-12)
    chunked = OracleDrafter(d, w, batch=1)
    for a, b in ((0, 3), (3, 4), (4, 11)):
        chunked.fuse_inject_input(0, [f[a:b] for f in feats])
    for l in range(d.n_layers):
        np.testing.assert_allclose(chunked.k[l][0], one.k[l][0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(chunked.v[l][0], one.v[l][0], rtol=1e-12, atol=1e-13)
    assert one.len[0] == chunked.len[0] == 11


def test_one_layer_input_fusion_equals_kv_injection_with_unit_gains():
    d = DrafterDims(n_layers=1, hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=8, inter=48,
                    vocab=64, n_feat_layers=5, feat_hidden=16, block_max=16, dtype="f32",
                    rope_theta=10000.0, rms_eps=0.0)
    w = _rand_weights(d, 35, gain="unit")
    rng = np.random.default_rng(36)
    feats = [rng.normal(size=(6, d.feat_hidden)) for _ in range(5)]
    a = OracleDrafter(d, w, batch=1)
    a.fuse_inject_input(0, feats)
    b = OracleDrafter(d, w, batch=1)
    b.fuse_inject(0, feats)
    np.testing.assert_allclose(a.k[0][0], b.k[0][0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(a.v[0][0], b.v[0][0], rtol=1e-12, atol=1e-13)


def _pair(seed, plant=False):
    wt = _rand_weights(TARGET, seed)
    wd = _rand_weights(DRAFT, seed + 1)
    wd["embed"], wd["lm_head"] = wt["embed"], wt["lm_head"]          # shared with the target
    if plant:
        # every embedding carries a large common direction u and lm_head row 7 points
        # along it: both models then pick id 7 everywhere, so every draft matches
        u = np.zeros(TARGET.hidden)
        u[3] = 1.0
        wt["embed"] = wt["embed"] * 0.05 + 40.0 * u
        wt["lm_head"] = wt["lm_head"].copy()
        wt["lm_head"][7] = 50.0 * u
        wd["embed"], wd["lm_head"] = wt["embed"], wt["lm_head"]
    return wt, wd


@pytest.mark.parametrize("block", [4, 16])
@pytest.mark.parametrize("input_fusion", [False, True])
def test_speculative_loop_is_lossless(block, input_fusion):
    wt, wd = _pair(40)
    prompt = list(np.random.default_rng(41).integers(0, TARGET.vocab - 1, size=6))
    ref = autoregressive_generate(OracleTarget(TARGET, wt, 1), 0, prompt, 40)
    got, acc = speculative_generate(OracleTarget(TARGET, wt, 1), OracleDrafter(DRAFT, wd, 1), 0,
                                    prompt, 40, block, CAPTURE, input_fusion=input_fusion)
    assert len(got) >= 40 and got[:40] == ref
    assert all(1 <= a <= block for a in acc)


def test_speculative_loop_with_planted_agreement_accepts_whole_blocks():
    wt, wd = _pair(42, plant=True)
    prompt = [1, 2, 3, 4, 5]
    ref = autoregressive_generate(OracleTarget(TARGET, wt, 1), 0, prompt, 50)
    got, acc = speculative_generate(OracleTarget(TARGET, wt, 1), OracleDrafter(DRAFT, wd, 1), 0,
                                    prompt, 50, 16, CAPTURE)
    assert len(got) >= 50 and got[:50] == ref
    assert set(ref) == {7}
    assert acc and all(a == 16 for a in acc[:-1]), acc


@pytest.mark.parametrize("input_fusion", [False, True])
def test_caches_after_the_loop_equal_a_fresh_pass_over_the_committed_tokens(input_fusion):
    """After the loop every cache holds exactly the committed prefix: the target's
    equals one fresh pass over prompt + committed tokens (all but the last, which
    is the next x0), and the drafter's equals one injection of that pass's
    features -- so the accept length, the trims and the re-injected rows line up."""
    for plant in (False, True):
        wt, wd = _pair(43, plant=plant)
        prompt = [3, 9, 27, 17, 51, 25]
        tgt, dft = OracleTarget(TARGET, wt, 1), OracleDrafter(DRAFT, wd, 1)
        out, acc = speculative_generate(tgt, dft, 0, prompt, 37, 8, CAPTURE,
                                        input_fusion=input_fusion)
        committed = prompt + out
        n = int(tgt.len[0])
        assert n == int(dft.len[0]) == len(prompt) + sum(acc) == len(committed) - 1
        fresh_t = OracleTarget(TARGET, wt, 1)
        _, _, feats = fresh_t.forward(0, committed[:n], CAPTURE)
        fresh_d = OracleDrafter(DRAFT, wd, 1)
        (fresh_d.fuse_inject_input if input_fusion else fresh_d.fuse_inject)(0, feats)
        for l in range(TARGET.n_layers):
            np.testing.assert_allclose(tgt.k[l][0], fresh_t.k[l][0], rtol=1e-9, atol=1e-11)
        for l in range(DRAFT.n_layers):
            np.testing.assert_allclose(dft.k[l][0], fresh_d.k[l][0], rtol=1e-9, atol=1e-11)
            np.testing.assert_allclose(dft.v[l][0], fresh_d.v[l][0], rtol=1e-9, atol=1e-11)
