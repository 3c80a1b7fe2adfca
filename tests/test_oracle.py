"""Pins of the CPU oracle against what the DFlash pages and mathematics fix.

No test here retypes the oracle's formula: each compares it with a closed form,
an invariant, a worked example, or the independent scalar-loop brute force in
``tests/bruteforce.py``.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle.dflash_oracle import (
    OracleDrafter, accept, accept_cumprod, block_attention, drafter_layer, fuse,
    lm_head_argmax, project_context_kv, rmsnorm, rope, LayerWeights,
)
from synth.configs import CONFIGS, DrafterDims, Workload
from synth.inputs import DrafterInputs, make_rng
from tests.bruteforce import brute_accept, brute_draft

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

MICRO = DrafterDims(n_layers=2, hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=8, inter=48,
                    vocab=64, n_feat_layers=5, feat_hidden=16, block_max=16, dtype="f32",
                    rope_theta=10000.0)


def _rand_weights(dims, seed, scale=0.3, gain="uniform"):
    rng = np.random.default_rng(seed)
    w = {}
    shapes = DrafterInputs(Workload(0, "x", dims, batch=1, block=4, ctx=4)).weight_shapes()
    for name, shp in shapes.items():
        if name.endswith("norm"):
            w[name] = rng.uniform(0.5, 1.5, size=shp) if gain == "uniform" else np.ones(shp)
        else:
            w[name] = rng.normal(0, scale, size=shp)
    return w


def _to_lists(w):
    return {k: v.tolist() for k, v in w.items()}


# ---------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------

def test_rmsnorm_closed_form():
    x = np.array([[3.0, 4.0]])
    out = rmsnorm(x, np.array([1.0, 2.0]), 0.0)
    # mean square = (9 + 16) / 2 = 12.5
    np.testing.assert_allclose(out, [[3 / math.sqrt(12.5), 2 * 4 / math.sqrt(12.5)]], rtol=1e-15)


def test_rmsnorm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(0)
    x = rng.normal(size=(7, 33))
    g = np.ones(33)
    y = rmsnorm(x, g, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-12)
    np.testing.assert_allclose(rmsnorm(5.5 * x, g, 0.0), y, rtol=1e-12)
    # eps enters as mean + eps under the root
    z = np.zeros((1, 4))
    z[0, 0] = 1.0
    np.testing.assert_allclose(rmsnorm(z, np.ones(4), 0.75)[0, 0], 1.0 / math.sqrt(0.25 + 0.75))


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------

def test_rope_closed_form_d2():
    # d = 2: one pair, frequency theta^0 = 1, so the pair rotates by pos radians
    for p in (0, 1, 3, 1000):
        out = rope(np.array([[[1.0, 0.0]]]), np.array([p]), 1.0e6)[0, 0]
        np.testing.assert_allclose(out, [math.cos(p), math.sin(p)], atol=1e-12)
        out = rope(np.array([[[0.0, 1.0]]]), np.array([p]), 1.0e6)[0, 0]
        np.testing.assert_allclose(out, [-math.sin(p), math.cos(p)], atol=1e-12)


def test_rope_closed_form_d4_pairs_are_half_apart():
    theta = 100.0
    x = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    p = 2
    w0, w1 = 1.0, theta ** (-0.5)
    c0, s0, c1, s1 = math.cos(p * w0), math.sin(p * w0), math.cos(p * w1), math.sin(p * w1)
    expect = [1 * c0 - 3 * s0, 2 * c1 - 4 * s1, 3 * c0 + 1 * s0, 4 * c1 + 2 * s1]
    np.testing.assert_allclose(rope(x, np.array([p]), theta)[0, 0], expect, atol=1e-12)


def test_rope_norm_identity_and_relative_position():
    rng = np.random.default_rng(1)
    q = rng.normal(size=(1, 3, 64))
    k = rng.normal(size=(1, 3, 64))
    np.testing.assert_allclose(rope(q, np.array([0]), 1e6), q, atol=0)
    for p in (5, 777, 32000):
        np.testing.assert_allclose(np.linalg.norm(rope(q, np.array([p]), 1e6), axis=-1),
                                   np.linalg.norm(q, axis=-1), rtol=1e-12)
    def dot(m, n):
        return np.sum(rope(q, np.array([m]), 1e4) * rope(k, np.array([n]), 1e4), axis=-1)
    np.testing.assert_allclose(dot(10, 3), dot(110, 103), rtol=1e-9)
    np.testing.assert_allclose(dot(7, 7), np.sum(q * k, axis=-1), rtol=1e-9)


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def test_attention_closed_form_two_keys():
    d = 4
    q = np.array([[[1.0, 0.0, 2.0, 0.0]]])            # one row, one head
    k = np.array([[[1.0, 1.0, 0.0, 0.0]], [[0.0, 0.0, 1.0, 0.0]]])
    v = np.array([[[1.0, 0.0, 0.0, 0.0]], [[0.0, 3.0, 0.0, 0.0]]])
    s0, s1 = 1.0 / math.sqrt(d), 2.0 / math.sqrt(d)   # scaled dot products
    w0 = math.exp(s0) / (math.exp(s0) + math.exp(s1))
    w1 = 1.0 - w0
    out = block_attention(q, k, v)[0, 0]
    np.testing.assert_allclose(out, [w0, 3 * w1, 0, 0], rtol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(2)
    q = rng.normal(size=(5, 4, 8))
    k1 = rng.normal(size=(1, 2, 8))
    v1 = rng.normal(size=(1, 2, 8))
    out = block_attention(q, k1, v1)                    # one key -> its value
    for j in range(4):
        np.testing.assert_allclose(out[:, j], np.broadcast_to(v1[0, j // 2], (5, 8)), rtol=1e-12)
    kk = np.repeat(k1, 6, axis=0)                        # identical keys -> mean of values
    vv = rng.normal(size=(6, 2, 8))
    out = block_attention(q, kk, vv)
    for j in range(4):
        np.testing.assert_allclose(out[:, j], np.broadcast_to(vv[:, j // 2].mean(0), (5, 8)), rtol=1e-12)
    # rows of the attention weights sum to one: constant values come back unchanged
    out = block_attention(q, rng.normal(size=(9, 2, 8)), np.full((9, 2, 8), 2.5))
    np.testing.assert_allclose(out, 2.5, rtol=1e-12)


def test_gqa_equals_mha_with_repeated_heads():
    rng = np.random.default_rng(3)
    q = rng.normal(size=(4, 6, 8))
    k = rng.normal(size=(11, 2, 8))
    v = rng.normal(size=(11, 2, 8))
    g = block_attention(q, k, v)
    kr = np.repeat(k, 3, axis=1)                         # head j reads kv head j // 3
    vr = np.repeat(v, 3, axis=1)
    np.testing.assert_allclose(g, block_attention(q, kr, vr), rtol=1e-12)


def test_layer_is_permutation_equivariant_in_block_rows():
    """Non-causal block attention: permuting the block rows together with their
    positions permutes every output row and nothing else."""
    d = MICRO
    rng = np.random.default_rng(4)
    w = _rand_weights(d, 5)
    lw = LayerWeights(*[w[f"l0.{f}"] for f in ("in_norm", "wq", "wk", "wv", "wo", "post_norm",
                                                  "w_gate", "w_up", "w_down")])
    x = rng.normal(size=(6, d.hidden))
    pos = np.arange(20, 26)
    kc = rng.normal(size=(20, d.n_kv_heads, d.head_dim))
    vc = rng.normal(size=(20, d.n_kv_heads, d.head_dim))
    args = (d.n_q_heads, d.n_kv_heads, d.head_dim, d.rope_theta, d.rms_eps)
    y, kb, vb = drafter_layer(x, lw, kc, vc, pos, *args)
    perm = np.array([3, 0, 5, 1, 4, 2])
    yp, kbp, vbp = drafter_layer(x[perm], lw, kc, vc, pos[perm], *args)
    np.testing.assert_allclose(yp, y[perm], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(kbp, kb[perm], rtol=1e-10, atol=1e-12)
    # a causal mask would break this: the first row would then see only itself
    yc = drafter_layer(x[:1], lw, kc, vc, pos[:1], *args)[0]
    assert not np.allclose(yc[0], y[0])


def test_layer_zero_output_projections_keep_residual():
    d = MICRO
    w = _rand_weights(d, 6)
    w["l0.wo"][:] = 0
    w["l0.w_down"][:] = 0
    lw = LayerWeights(*[w[f"l0.{f}"] for f in ("in_norm", "wq", "wk", "wv", "wo", "post_norm",
                                                  "w_gate", "w_up", "w_down")])
    rng = np.random.default_rng(7)
    x = rng.normal(size=(4, d.hidden))
    y = drafter_layer(x, lw, rng.normal(size=(3, 2, 8)), rng.normal(size=(3, 2, 8)),
                      np.arange(3, 7), d.n_q_heads, d.n_kv_heads, d.head_dim, d.rope_theta,
                      d.rms_eps)[0]
    np.testing.assert_array_equal(y, x)


def test_mlp_applies_silu_to_the_gate_projection():
    """SwiGLU with the attention's output projection zero and identity-like gate, up (x2)
    and down projections: each of the first `hidden` intermediate units reduces to
    silu(h) * 2h of the post-attention norm's output h, with silu(t) = t * sigmoid(t) and
    sigmoid from scipy.special.expit.  A silu on the up projection (silu(2h) * h), a
    dropped silu or a missing norm fails."""
    from scipy.special import expit
    d = MICRO
    w = _rand_weights(d, 11)
    w["l0.wo"][:] = 0
    for f in ("w_gate", "w_up", "w_down"):
        w[f"l0.{f}"][:] = 0
    for i in range(d.hidden):
        w["l0.w_gate"][i, i] = 1.0
        w["l0.w_up"][i, i] = 2.0
        w["l0.w_down"][i, i] = 1.0
    lw = LayerWeights(*[w[f"l0.{f}"] for f in ("in_norm", "wq", "wk", "wv", "wo", "post_norm",
                                                  "w_gate", "w_up", "w_down")])
    rng = np.random.default_rng(12)
    x = rng.normal(size=(4, d.hidden)) * 3.0
    y = drafter_layer(x, lw, rng.normal(size=(3, 2, 8)), rng.normal(size=(3, 2, 8)),
                      np.arange(3, 7), d.n_q_heads, d.n_kv_heads, d.head_dim, d.rope_theta,
                      d.rms_eps)[0]
    h = rmsnorm(x, w["l0.post_norm"], d.rms_eps)
    np.testing.assert_allclose(y, x + h * expit(h) * (2.0 * h), rtol=1e-12, atol=1e-12)
    assert not np.allclose(y, x + (2.0 * h) * expit(2.0 * h) * h)


def test_all_zero_layers_return_normed_embedding():
    d = MICRO
    w = _rand_weights(d, 8)
    for l in range(d.n_layers):
        for f in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
            w[f"l{l}.{f}"][:] = 0
    o = OracleDrafter(d, w, batch=1)
    rng = np.random.default_rng(9)
    o.fuse_inject(0, [rng.normal(size=(5, d.feat_hidden)) for _ in range(5)])
    r = o.draft([7], block=4)
    emb = w["embed"][[7, d.vocab - 1, d.vocab - 1, d.vocab - 1]]
    np.testing.assert_allclose(r["final_hidden"][0], rmsnorm(emb, w["final_norm"], d.rms_eps),
                               rtol=1e-12)


# ---------------------------------------------------------------------------
# Fusion
# ---------------------------------------------------------------------------

def test_fusion_concat_order_block_i_multiplies_layer_i():
    rng = np.random.default_rng(10)
    ht, h = 6, 6
    feats = [rng.normal(size=(3, ht)) for _ in range(5)]
    for i in range(5):
        w = np.zeros((h, 5 * ht))
        w[:, i * ht:(i + 1) * ht] = np.eye(ht)            # selects target layer i
        np.testing.assert_allclose(fuse(feats, w, np.ones(h), 1e-6),
                                   rmsnorm(feats[i], np.ones(h), 1e-6), rtol=1e-12)


def test_fusion_split_identity():
    rng = np.random.default_rng(11)
    feats = [rng.normal(size=(4, 8)) for _ in range(5)]
    w = rng.normal(size=(12, 40))
    y = sum(feats[i] @ w[:, 8 * i:8 * (i + 1)].T for i in range(5))
    np.testing.assert_allclose(fuse(feats, w, np.ones(12), 0.0), rmsnorm(y, np.ones(12), 0.0),
                               rtol=1e-12)


# ---------------------------------------------------------------------------
# lm_head argmax
# ---------------------------------------------------------------------------

def test_lm_head_planted_and_ties():
    rng = np.random.default_rng(12)
    z = rng.normal(size=(3, 16))
    w = rng.normal(size=(50, 16)) * 0.01
    w[37] = 5 * z[0]
    w[4] = 5 * z[1]
    w[20] = 5 * z[2]
    w[45] = 5 * z[2]                                     # exact tie: lowest id wins
    ids, top2, logits = lm_head_argmax(z, w)
    assert list(ids) == [37, 4, 20]
    assert top2[2, 0] == top2[2, 1]
    assert np.all(top2[:, 0] >= top2[:, 1])
    for r in range(3):
        assert top2[r, 0] == logits[r].max()


def test_lm_head_top2_planted_runner_up():
    """The runner-up is the second-largest logit: not the third, not the smallest,
    not the largest of another row."""
    rng = np.random.default_rng(13)
    q, _ = np.linalg.qr(rng.normal(size=(16, 16)))
    z = q[:4] * np.array([[3.0], [2.0], [2.5], [1.5]])   # orthogonal rows: planted rows of one
    w = rng.normal(size=(64, 16)) * 0.01                  # row give the others ~0
    n2 = [float(z[r] @ z[r]) for r in range(4)]
    w[37], w[11], w[3] = 5 * z[0], 4 * z[0], -6 * z[0]   # best 5|z|^2, runner-up 4|z|^2, min -6|z|^2
    w[2], w[60] = 3 * z[1], 2.5 * z[1]                    # runner-up at a higher id than the best
    w[50], w[9] = 3 * z[2], 2.9 * z[2]                    # runner-up at a lower id than the best
    w[21], w[22] = 2 * z[3], 2 * z[3]                     # exact tie: runner-up equals the best
    ids, top2, logits = lm_head_argmax(z, w)
    assert list(ids) == [37, 2, 50, 21]
    expect = [(5, 4), (3, 2.5), (3, 2.9), (2, 2)]
    for r, (a, b) in enumerate(expect):
        np.testing.assert_allclose(top2[r], [a * n2[r], b * n2[r]], rtol=1e-10)
        # the same through a plain sort of the row
        srt = sorted(logits[r].tolist())
        assert (top2[r, 0], top2[r, 1]) == (srt[-1], srt[-2])


# ---------------------------------------------------------------------------
# Acceptance
# ---------------------------------------------------------------------------

def test_accept_golden_examples():
    with open(os.path.join(GOLDEN, "accept_examples.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        a, b = accept(np.array(c["drafts"]), np.array(c["targets"]))
        assert (a, b) == (c["accept_len"], c["bonus"]), c["name"]
        assert accept_cumprod(np.array(c["drafts"]), np.array(c["targets"])) == c["accept_len"]


@pytest.mark.parametrize("block", [4, 8])
def test_accept_exhaustive_patterns(block):
    for pattern in range(2 ** (block - 1)):
        d = np.arange(block - 1) + 10
        t = np.arange(block) + 10
        for i in range(block - 1):
            if not (pattern >> i) & 1:
                t[i] = 1000 + i                           # mismatch at i
        a, b = accept(d, t)
        assert (a, b) == brute_accept(list(d), list(t))
        assert a == accept_cumprod(d, t)
        assert 1 <= a <= block
        # lossless: committed tokens after x0 are exactly the target's tokens
        committed = list(d[:a - 1]) + [b]
        assert committed == list(t[:a])


def test_accept_random_block16_planted():
    from synth.inputs import planted_targets
    rng = np.random.default_rng(13)
    for trial in range(200):
        d = rng.integers(0, 1000, size=(4, 15))
        k = rng.integers(0, 16, size=4)
        t = planted_targets(d, k, 1001, rng)
        for b in range(4):
            a, bo = accept(d[b], t[b])
            assert a == k[b] + 1
            assert (a, bo) == brute_accept(list(d[b]), list(t[b]))


def test_accept_trim_without_a_draft_keeps_the_cache_and_flags():
    """An acceptance with no preceding draft has no base to trim back to: the
    cache is left as it is, flag 4 is raised, the comparison is still reported;
    a drafted sequence in the same call is trimmed as usual."""
    d = MICRO
    w = _rand_weights(d, 18)
    rng = np.random.default_rng(19)
    o = OracleDrafter(d, w, batch=2)
    for b in range(2):
        o.fuse_inject(b, [rng.normal(size=(6, d.feat_hidden)) for _ in range(5)])
    o.base[1] = 3                                        # sequence 1 drafted at len 3
    acc, bon = o.accept_trim(np.array([[5, 6, 7], [5, 6, 7]]), np.array([[5, 6, 0, 1], [5, 9, 7, 1]]))
    assert acc.tolist() == [3, 2] and bon.tolist() == [0, 9]
    assert o.len.tolist() == [6, 5]                      # untouched; 3 + 2
    assert o.err & 4
    assert o.k[0][0].shape[0] == 6 and o.k[0][1].shape[0] == 5


# ---------------------------------------------------------------------------
# Injection state: incremental == full, trim + re-append == fresh
# ---------------------------------------------------------------------------

def _cache_of(o, seq):
    return ([k[seq].copy() for k in o.k], [v[seq].copy() for v in o.v])


def test_incremental_injection_equals_full():
    d = MICRO
    w = _rand_weights(d, 14)
    rng = np.random.default_rng(15)
    feats = [rng.normal(size=(13, d.feat_hidden)) for _ in range(5)]
    full = OracleDrafter(d, w, batch=1)
    full.fuse_inject(0, feats)
    inc = OracleDrafter(d, w, batch=1)
    for a, b in ((0, 4), (4, 5), (5, 11), (11, 13)):
        inc.fuse_inject(0, [f[a:b] for f in feats])
    for x, y in zip(_cache_of(full, 0), _cache_of(inc, 0)):
        for cx, cy in zip(x, y):
            np.testing.assert_allclose(cx, cy, rtol=1e-12, atol=1e-14)
    assert full.len[0] == inc.len[0] == 13


def test_trim_then_reappend_equals_fresh_build():
    d = MICRO
    w = _rand_weights(d, 16)
    rng = np.random.default_rng(17)
    ctx = [rng.normal(size=(9, d.feat_hidden)) for _ in range(5)]
    blk = [rng.normal(size=(4, d.feat_hidden)) for _ in range(5)]
    a = OracleDrafter(d, w, batch=1)
    a.fuse_inject(0, ctx)
    a.draft([3], block=4)
    a.fuse_inject(0, blk)                               # inject the whole verified block
    a.accept_trim(np.array([[5, 6, 7]]), np.array([[5, 9, 7, 1]]))   # accept_len = 2
    assert a.len[0] == 11
    fresh = OracleDrafter(d, w, batch=1)
    fresh.fuse_inject(0, [np.concatenate([c, b[:2]]) for c, b in zip(ctx, blk)])
    for x, y in zip(_cache_of(a, 0), _cache_of(fresh, 0)):
        for cx, cy in zip(x, y):
            np.testing.assert_allclose(cx, cy, rtol=1e-12, atol=1e-14)
    # accept before injecting gives the same cache as accept after injecting
    b = OracleDrafter(d, w, batch=1)
    b.fuse_inject(0, ctx)
    b.draft([3], block=4)
    b.accept_trim(np.array([[5, 6, 7]]), np.array([[5, 9, 7, 1]]))
    b.fuse_inject(0, [x[:2] for x in blk])
    for x, y in zip(_cache_of(a, 0), _cache_of(b, 0)):
        for cx, cy in zip(x, y):
            np.testing.assert_allclose(cx, cy, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# End to end against the scalar-loop brute force
# ---------------------------------------------------------------------------

def _bruteforce_compare(dims, w, feats_ctx, x0, block, rtol):
    o = OracleDrafter(dims, w, batch=1, dtype=np.float64)
    c = o.fuse_inject(0, feats_ctx)
    r = o.draft([x0], block=block, want_logits=True)
    L = feats_ctx[0].shape[0]
    bf = brute_draft(dims, _to_lists(w), [[feats_ctx[i][t].tolist() for i in range(5)]
                                          for t in range(L)], x0, block)
    np.testing.assert_allclose(c, np.array(bf["fused"]), rtol=rtol, atol=rtol)
    for l in range(dims.n_layers):
        np.testing.assert_allclose(o.k[l][0], np.array(bf["k_ctx"][l]), rtol=rtol, atol=rtol)
        np.testing.assert_allclose(o.v[l][0], np.array(bf["v_ctx"][l]), rtol=rtol, atol=rtol)
    np.testing.assert_allclose(r["final_hidden"][0], np.array(bf["final_hidden"]), rtol=rtol, atol=rtol)
    np.testing.assert_allclose(r["logits"][0], np.array(bf["logits"]), rtol=rtol, atol=rtol)
    assert list(r["draft_ids"][0]) == bf["draft_ids"]
    # the top-2 values behind the near-tie exclusion of draft-id parity
    np.testing.assert_allclose(r["top2"][0], np.array(bf["top2"]), rtol=rtol, atol=rtol)


@pytest.mark.parametrize("seed,block", [(20, 4), (21, 5), (22, 16)])
def test_oracle_matches_bruteforce_micro(seed, block):
    d = MICRO
    w = _rand_weights(d, seed)
    rng = np.random.default_rng(seed + 100)
    feats = [rng.normal(size=(7, d.feat_hidden)) for _ in range(5)]
    _bruteforce_compare(d, w, feats, int(rng.integers(0, d.vocab - 1)), block, 1e-10)


def test_oracle_matches_bruteforce_tiny_config():
    """The tiny fp32 workload (1 layer, hidden 256, 4/2 heads, head_dim 64,
    SwiGLU 704, vocab 1024, context 32, block 4) with its seeded inputs."""
    wl = CONFIGS[1]
    inp = DrafterInputs(wl)
    w = {n: inp.weight_f32(n).astype(np.float64) for n in inp.weight_shapes()}
    feats = [inp.ctx_feats(i, 0).astype(np.float64) for i in range(5)]
    _bruteforce_compare(wl.dims, w, feats, int(inp.x0()[0]), wl.block, 1e-9)


def test_oracle_fp32_close_to_fp64_tiny():
    wl = CONFIGS[1]
    inp = DrafterInputs(wl)
    w = {n: inp.weight_f32(n) for n in inp.weight_shapes()}
    feats = [inp.ctx_feats(i, 0) for i in range(5)]
    outs = []
    for dt in (np.float64, np.float32):
        o = OracleDrafter(wl.dims, w, batch=1, dtype=dt)
        o.fuse_inject(0, feats)
        outs.append(o.draft(inp.x0(), block=wl.block, want_logits=True))
    a, b = outs
    err = np.max(np.abs(a["final_hidden"] - b["final_hidden"])) / np.max(np.abs(a["final_hidden"]))
    assert err < 1e-5
