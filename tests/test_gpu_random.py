"""GPU parity over seeded random drafter shapes: widths, head layouts (GQA group 1 to 8,
head_dim 64 and 128), feature-layer counts, vocabularies, depths, batch sizes, block
sizes and context mixes drawn independently, so that the kernels' shape paths (skinny,
full-K row, matrix-core tiles, fixed and balanced attention splits, the lm_head
variants) meet combinations the hand-picked cases do not.  Each case prefills, then
runs two lockstep rounds (draft, accept + trim, re-injection) on the device and in the
oracle and compares the cache; its parameters are logged before it runs."""

import numpy as np
import pytest

from synth.configs import DrafterDims, Workload
from tests.gpu_common import build_pair, check_cache, draft_round, log, prefill

pytestmark = pytest.mark.gpu

N_CASES = 16

# (head_dim, kv heads, group) with q heads x head_dim a multiple of 256 and group x 16 <= 128
_HEADS = [(64, 1, 4), (64, 2, 2), (64, 4, 1), (64, 1, 8), (64, 2, 4), (64, 4, 5),
          (128, 1, 2), (128, 2, 1), (128, 2, 4), (128, 4, 5), (128, 1, 8), (128, 4, 2)]


def random_case(i: int):
    """Case i: (dims, batch, block, contexts), drawn from its own seed."""
    rng = np.random.default_rng(7000 + i)
    d, hkv, g = _HEADS[int(rng.integers(len(_HEADS)))]
    dims = DrafterDims(n_layers=int(rng.integers(1, 4)),
                       hidden=int(rng.choice([256, 512, 768, 1024, 1280])),
                       n_q_heads=hkv * g, n_kv_heads=hkv, head_dim=d,
                       inter=int(rng.choice([256, 512, 768, 1280, 2048])),
                       vocab=int(rng.choice([512, 1008, 2000, 4096])),
                       n_feat_layers=int(rng.integers(1, 6)),
                       feat_hidden=int(rng.choice([256, 512])), block_max=16,
                       dtype="bf16", rope_theta=float(rng.choice([1.0e4, 1.0e6])))
    batch = int(rng.choice([1, 2, 4, 9, 20, 33]))
    block = int(rng.choice([2, 3, 5, 8, 16]))
    ctx = rng.integers(0, 400, size=batch)
    ctx[rng.random(batch) < 0.15] = 0  # some sequences with no injected context
    return dims, batch, block, ctx.astype(np.int32)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_rounds(i):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dims, batch, block, ctx = random_case(i)
    log(f"[random {i}] layers {dims.n_layers} hidden {dims.hidden} heads {dims.n_q_heads}/"
        f"{dims.n_kv_heads} d {dims.head_dim} inter {dims.inter} vocab {dims.vocab} feats "
        f"{dims.n_feat_layers}x{dims.feat_hidden} batch {batch} block {block} ctx {ctx.tolist()}")
    wl = Workload(500 + i, f"random_{i}", dims, batch=batch, block=block, ctx=1,
                  accept_mean=3.0, rounds=2)
    max_ctx = int((int(ctx.max()) + block * 4 + 63) // 64 * 64)
    p = build_pair(wl, max_ctx=max_ctx, ctx=ctx)
    log(f"  prefill {prefill(p)}")
    x0 = p.inp.x0()
    for rnd in range(2):
        out = draft_round(p, x0, rnd, check_logits=rnd == 0)
        log(f"  round {rnd}: final_hidden {out['final_hidden']:.2e} ids {out['compared_ids']} "
            f"accept {out['accept_len'].tolist()}")
        x0 = out["bonus"]
    log(f"  cache {check_cache(p)}")
