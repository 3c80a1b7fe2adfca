"""GPU parity: the HIP library through the C ABI against the CPU oracle on the
same seeded inputs.  Small shapes that still span several tiles and ragged
tails, plus the tiny fp32 workload; the full-size workloads are in
test_gpu_fullsize.py."""

import numpy as np
import pytest

from synth.configs import CONFIGS, DrafterDims, Workload
from tests.gpu_common import (build_pair, check_cache, draft_round, log, prefill)

pytestmark = pytest.mark.gpu

SMALL_BF16 = DrafterDims(n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
                         inter=1024, vocab=4096, n_feat_layers=5, feat_hidden=256, block_max=16,
                         dtype="bf16", rope_theta=1.0e6)
SMALL_G5_D64 = DrafterDims(n_layers=1, hidden=512, n_q_heads=20, n_kv_heads=4, head_dim=64,
                           inter=768, vocab=2048, n_feat_layers=5, feat_hidden=512, block_max=16,
                           dtype="bf16", rope_theta=1.0e6)

# An intermediate width that 192 divides: gate|up GEMMs of more than 128 rows take the
# 128 x 384 matrix-core tile with SwiGLU in its epilogue (96 intermediate indices per
# wave pair of gate and up groups).
SMALL_I768 = DrafterDims(n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
                         inter=768, vocab=4096, n_feat_layers=5, feat_hidden=256, block_max=16,
                         dtype="bf16", rope_theta=1.0e6)

# Widths at which one 16-row group takes the full-K GEMMs (output projection
# K = 2048, gate/up K = 1024, down K = 2048) with the residual, the per-row
# scaled A rows and SwiGLU in their epilogues.
MID_BF16 = DrafterDims(n_layers=2, hidden=1024, n_q_heads=16, n_kv_heads=4, head_dim=128,
                       inter=2048, vocab=4096, n_feat_layers=5, feat_hidden=512, block_max=16,
                       dtype="bf16", rope_theta=1.0e6)


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def test_accept_trim_exhaustive_block4_and_random_block16():
    torch = _torch()
    from block_diffusion_drafter_layers_amd.runtime import DeviceDrafter
    from oracle.dflash_oracle import accept
    from synth.inputs import DrafterInputs
    wl = CONFIGS[1]
    inp = DrafterInputs(wl)
    dev = DeviceDrafter(wl.dims, {n: inp.weight(n) for n in inp.weight_shapes()}, 8, 64, 64)
    rng = np.random.default_rng(5)
    for block in (4, 16):
        pats = range(2 ** (block - 1)) if block == 4 else rng.integers(0, 2 ** 15, size=64)
        pats = list(pats)
        for i0 in range(0, len(pats), 8):
            chunk = pats[i0:i0 + 8]
            n = len(chunk)
            d = rng.integers(0, 1000, size=(8, block - 1)).astype(np.int32)
            t = rng.integers(0, 1000, size=(8, block)).astype(np.int32)
            for j, pat in enumerate(chunk):
                for i in range(block - 1):
                    t[j, i] = d[j, i] if (int(pat) >> i) & 1 else 5000 + i
            base = rng.integers(0, 40, size=8).astype(np.int32)
            lens = base + rng.integers(0, block + 1, size=8).astype(np.int32)
            dev.base.copy_(torch.from_numpy(base))
            dev.len.copy_(torch.from_numpy(lens))
            acc = torch.zeros(8, dtype=torch.int32, device="cuda")
            bon = torch.zeros(8, dtype=torch.int32, device="cuda")
            dev.accept_trim(torch.from_numpy(d).cuda(), torch.from_numpy(t).cuda(), block, acc, bon)
            torch.cuda.synchronize()
            ga, gb, gl = acc.cpu().numpy(), bon.cpu().numpy(), dev.len.cpu().numpy()
            for j in range(n):
                a, bo = accept(d[j], t[j])
                assert (ga[j], gb[j]) == (a, bo), (block, chunk[j])
                assert gl[j] == min(lens[j], base[j] + a)
    # sequences without a preceding draft (base -1) next to drafted ones: the oracle
    # decides what is trimmed, what is reported and which flag is raised
    from oracle.dflash_oracle import OracleDrafter
    ora = OracleDrafter(wl.dims, {n: inp.weight_f32(n) for n in inp.weight_shapes()}, 8)
    base = np.array([-1, 3, -1, 0, 5, -1, 2, 7], dtype=np.int32)
    lens = np.array([10, 6, 10, 4, 9, 1, 5, 12], dtype=np.int32)
    ora.base[:] = base
    ora.len[:] = lens
    d = rng.integers(0, 50, size=(8, 3)).astype(np.int32)
    t = rng.integers(0, 50, size=(8, 4)).astype(np.int32)
    t[:, :3] = np.where(rng.random((8, 3)) < 0.7, d, t[:, :3])
    oacc, obon = ora.accept_trim(d, t)
    dev.base.copy_(torch.from_numpy(base))
    dev.len.copy_(torch.from_numpy(lens))
    dev.err.zero_()
    acc = torch.zeros(8, dtype=torch.int32, device="cuda")
    bon = torch.zeros(8, dtype=torch.int32, device="cuda")
    dev.accept_trim(torch.from_numpy(d).cuda(), torch.from_numpy(t).cuda(), 4, acc, bon)
    torch.cuda.synchronize()
    assert int(dev.err.item()) == ora.err == 4
    assert np.array_equal(dev.len.cpu().numpy(), ora.len.astype(np.int32))
    assert np.array_equal(acc.cpu().numpy(), oacc) and np.array_equal(bon.cpu().numpy(), obon)


@pytest.mark.parametrize("k", [0, 1, 2, 3])
def test_tiny_f32_workload(k):
    """Tiny fp32 drafter (1 layer, hidden 256, block 4, context 32) with the
    planted prefix k: fusion, injection, draft, accept, trim, re-injection."""
    _torch()
    wl = CONFIGS[1]
    log(f"[tiny f32] k={k}")
    p = build_pair(wl, max_ctx=128)
    log(f"  prefill {prefill(p)}")
    x0 = p.inp.x0()
    for rnd in range(2):
        out = draft_round(p, x0, rnd, k=np.array([k]))
        log(f"  round {rnd}: final_hidden {out['final_hidden']:.2e} logits {out['logits']:.2e}")
        assert out["accept_len"][0] == k + 1
        x0 = out["bonus"]
        check_cache(p)


@pytest.mark.parametrize("ctx,max_ctx", [(2100, 4096), (5000, 8192)])
def test_batch1_long_context_multi_tile_chunks(ctx, max_ctx):
    """A single sequence past 32 tiles of keys: the fixed-chunk attention cuts it into at
    most 32 chunks of several tiles each (2116 keys: 34 tiles in 17 chunks of two; 5016
    keys: 79 tiles in 27 chunks of three, the last one partial)."""
    _torch()
    wl = Workload(190 + ctx // 1000, f"long_b1_{ctx}", SMALL_BF16, batch=1, block=16, ctx=1,
                  accept_mean=4.0, rounds=2)
    log(f"[batch-1 long context] ctx={ctx} max_ctx={max_ctx}")
    p = build_pair(wl, max_ctx=max_ctx, ctx=np.array([ctx]))
    log(f"  prefill {prefill(p)}")
    x0 = p.inp.x0()
    for rnd in range(2):
        out = draft_round(p, x0, rnd, check_logits=rnd % 2 == 0)
        log(f"  round {rnd}: final_hidden {out['final_hidden']:.2e} ids {out['compared_ids']} "
            f"accept {out['accept_len'].tolist()}")
        x0 = out["bonus"]
    log(f"  cache {check_cache(p)}")


@pytest.mark.parametrize("batch,block,ctx,rounds", [
    (1, 16, [300], 3),            # M = 16: skinny MT=1, lm_head LDS variant
    (2, 16, [77, 190], 2),        # M = 32: MT=2, lm_head tiled (30 rows)
    (3, 16, [200, 5, 64], 2),     # M = 48: MT=4, ragged contexts
    (5, 16, [100, 260, 3, 64, 129], 2),   # M = 80: big MFMA tiles
    (1, 4, [70], 2),              # short block
    (1, 2, [50], 3),              # the smallest block: one drafted row per sequence
    (9, 2, [0, 1, 64, 65, 3, 200, 17, 128, 9], 2),   # M = 18, empty and one-row contexts
    (33, 2, [(29 * i) % 150 for i in range(33)], 2),  # M = 66: matrix-core path, block 2
    (3, 16, [0, 5, 64], 2),       # a sequence with no injected context
    (2, 8, [1000, 1500], 1),      # several attention splits
    (20, 16, [37 * i + 5 for i in range(20)], 2),   # M = 320: two padded MFMA row tiles
    # balanced attention split: more sequences than one wave scans at once, fewer
    # tiles than workgroups (long sequences cut into one-tile pieces) ...
    (70, 4, [(53 * i) % 190 + 1 for i in range(68)] + [1500, 1200], 1),
    # ... and more tiles than workgroups (pieces that cross segment boundaries)
    (66, 16, [(97 * i) % 400 + 200 for i in range(66)], 1),
])
def test_small_bf16_pipeline(batch, block, ctx, rounds):
    _torch()
    wl = Workload(100 + batch * 10 + block, f"small_b{batch}_B{block}", SMALL_BF16, batch=batch,
                  block=block, ctx=1, accept_mean=4.0, rounds=rounds)
    log(f"[small bf16] batch={batch} block={block} ctx={ctx}")
    p = build_pair(wl, max_ctx=2048, ctx=np.array(ctx))
    log(f"  prefill {prefill(p)}")
    x0 = p.inp.x0()
    for rnd in range(rounds):
        # odd rounds: no logits requested, so a batched lm_head runs its argmax-only kernel
        out = draft_round(p, x0, rnd, check_logits=rnd % 2 == 0)
        lg = f"{out['logits']:.2e}" if "logits" in out else "(not stored)"
        log(f"  round {rnd}: final_hidden {out['final_hidden']:.2e} logits {lg} "
            f"ids {out['compared_ids']} accept {out['accept_len'].tolist()}")
        x0 = out["bonus"]
    log(f"  cache {check_cache(p)}")


@pytest.mark.parametrize("batch,block,ctx", [
    (1, 16, [300]),       # M = 16
    (1, 7, [41]),         # M = 7: rows 7..15 of the group are padding
    (2, 8, [500, 3]),     # M = 16 from two sequences
])
def test_mid_bf16_full_k_group(batch, block, ctx):
    _torch()
    wl = Workload(150 + batch * 10 + block, f"mid_b{batch}_B{block}", MID_BF16, batch=batch,
                  block=block, ctx=1, accept_mean=4.0, rounds=2)
    log(f"[mid bf16] batch={batch} block={block} ctx={ctx}")
    p = build_pair(wl, max_ctx=1024, ctx=np.array(ctx))
    log(f"  prefill {prefill(p)}")
    x0 = p.inp.x0()
    for rnd in range(2):
        out = draft_round(p, x0, rnd, check_logits=rnd % 2 == 0)
        lg = f"{out['logits']:.2e}" if "logits" in out else "(not stored)"
        log(f"  round {rnd}: final_hidden {out['final_hidden']:.2e} logits {lg} "
            f"ids {out['compared_ids']} accept {out['accept_len'].tolist()}")
        x0 = out["bonus"]
    log(f"  cache {check_cache(p)}")


@pytest.mark.parametrize("batch,ctx", [(1, [700]), (3, [700, 90, 333])])
def test_sharp_scores_zero_values(batch, ctx):
    """Attention scores hundreds of nats apart with every value row zero: the softmax
    max must be the max over all of a query's keys in the tile, else a probability
    past the fp16 range of the P.V product turns into inf and 0 * inf into NaN.
    Here the exact attention output is 0 ("DFlash原理深度剖析", §二.2: block
    attention is an ordinary softmax over the keys), so any NaN is the kernel's."""
    _torch()
    from synth.inputs import bf16_bits_to_f32, f32_to_bf16_bits

    def sharpen(name, w):
        if name.endswith(".wv"):
            return np.zeros_like(w)
        if name.endswith(".wq") or name.endswith(".wk"):  # x16: exact in bf16
            return f32_to_bf16_bits(bf16_bits_to_f32(w) * np.float32(16.0))
        return w

    wl = Workload(170 + batch, f"sharp_b{batch}", SMALL_BF16, batch=batch, block=16, ctx=1,
                  accept_mean=4.0, rounds=2)
    log(f"[sharp scores] batch={batch} ctx={ctx}")
    p = build_pair(wl, max_ctx=1024, ctx=np.array(ctx), weight_map=sharpen)
    prefill(p)
    x0 = p.inp.x0()
    for rnd in range(2):
        out = draft_round(p, x0, rnd, check_logits=rnd == 0)
        log(f"  round {rnd}: final_hidden {out['final_hidden']:.2e} ids {out['compared_ids']}")
        x0 = out["bonus"]
    assert int(p.dev.err.item()) == 0, int(p.dev.err.item())


# Hidden 6144 at batch 1: the 16-row group lm_head keeps its rows in LDS only up to
# hidden 5120, so the last layer must hand the rows to the other head (a draft once
# returned an error after every layer had run).  Intermediate 1024 is not a whole
# number of the full-K down projection's k-step groups (2048), so gate/up and down
# take the split GEMMs (the full-K gate/up once ran without checking the down
# projection it feeds, and its launch failed).
WIDE_BF16 = DrafterDims(n_layers=1, hidden=6144, n_q_heads=48, n_kv_heads=8, head_dim=128,
                        inter=1024, vocab=2048, n_feat_layers=5, feat_hidden=512, block_max=16,
                        dtype="bf16", rope_theta=1.0e6)


def test_wide_hidden_batch1_lm_head_fallback():
    _torch()
    wl = Workload(161, "wide_b1", WIDE_BF16, batch=1, block=16, ctx=1, accept_mean=4.0, rounds=2)
    log("[wide bf16] hidden 6144, batch 1")
    p = build_pair(wl, max_ctx=512, ctx=np.array([200]))
    prefill(p)
    x0 = p.inp.x0()
    for rnd in range(2):  # round 1 stores no logits: the greedy head the bench times
        out = draft_round(p, x0, rnd, check_logits=rnd == 0)
        log(f"  round {rnd}: final_hidden {out['final_hidden']:.2e} ids {out['compared_ids']}")
        x0 = out["bonus"]
    check_cache(p)


@pytest.mark.parametrize("batch,block,ctx", [
    (9, 16, [40 * i + 7 for i in range(9)]),       # M = 144: the second 128-row tile ragged
    (33, 16, [(61 * i) % 300 + 1 for i in range(33)]),  # M = 528: five row tiles
])
def test_small_bf16_swiglu_wide_tile(batch, block, ctx):
    _torch()
    wl = Workload(300 + batch, f"small_i768_b{batch}", SMALL_I768, batch=batch, block=block,
                  ctx=1, accept_mean=4.0, rounds=2)
    log(f"[small bf16 I=768] batch={batch} block={block}")
    p = build_pair(wl, max_ctx=1024, ctx=np.array(ctx))
    log(f"  prefill {prefill(p)}")
    x0 = p.inp.x0()
    for rnd in range(2):
        out = draft_round(p, x0, rnd, check_logits=rnd == 0)
        log(f"  round {rnd}: final_hidden {out['final_hidden']:.2e} ids {out['compared_ids']}")
        x0 = out["bonus"]
    check_cache(p)


def test_small_bf16_group5_headdim64():
    _torch()
    wl = Workload(131, "small_g5_d64", SMALL_G5_D64, batch=2, block=16, ctx=1, accept_mean=6.0)
    log("[small bf16] G=5 d=64")
    p = build_pair(wl, max_ctx=1024, ctx=np.array([333, 90]))
    prefill(p)
    x0 = p.inp.x0()
    for rnd in range(2):
        x0 = draft_round(p, x0, rnd)["bonus"]
    check_cache(p)


def test_bulk_prefill_rows_over_chunk_and_unit_gains():
    """More rows than one fuse_inject pass (16384) in one call, unit RMSNorm
    gains (the other reading of the gain initialisation)."""
    _torch()
    wl = Workload(140, "small_bulk", SMALL_BF16, batch=2, block=16, ctx=1, accept_mean=6.0)
    log("[small bf16] bulk prefill 17000 rows")
    p = build_pair(wl, max_ctx=16384, ctx=np.array([9000, 8000]), gain_mode="unit",
                   oracle_dtype=np.float32)
    prefill(p)
    draft_round(p, p.inp.x0(), 0, check_logits=False)
