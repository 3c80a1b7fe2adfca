"""GPU parity of the sampled draft (dflash_draft_block_sampled) against the
oracle's Gumbel-max sampler on the same seeded inputs: draft ids bit-exact
away from near-ties of the sampling scores, every lm_head variant (fp32, the
16-row group, the batched matrix-core head, the logits-storing head), then
the usual acceptance and trim against planted targets."""

import numpy as np
import pytest

from synth.configs import CONFIGS, Workload
from tests.gpu_common import build_pair, check_cache, draft_round, log, prefill
from tests.test_gpu_parity import MID_BF16, SMALL_BF16

pytestmark = pytest.mark.gpu


def _run(wl, ctx, rounds, temperature, max_ctx=2048, logits_rounds=(0,)):
    import torch
    assert torch.cuda.is_available()
    p = build_pair(wl, max_ctx=max_ctx, ctx=None if ctx is None else np.array(ctx))
    log(f"  prefill {prefill(p)}")
    x0 = p.inp.x0()
    compared = 0
    for rnd in range(rounds):
        out = draft_round(p, x0, rnd, check_logits=rnd in logits_rounds, temperature=temperature,
                          seed=1234 + rnd, offset=rnd)
        compared += out["compared_ids"]
        log(f"  round {rnd}: final_hidden {out['final_hidden']:.2e} ids compared "
            f"{out['compared_ids']} accept {out['accept_len'].tolist()}")
        x0 = out["bonus"]
    check_cache(p)
    return compared


@pytest.mark.parametrize("temperature", [0.7, 1.0, 1.5])
def test_tiny_f32_sampled(temperature):
    wl = CONFIGS[1]
    log(f"[sampled tiny f32] T={temperature}")
    # 3 drafted rows per round; rows within the near-tie band of their sampling
    # scores are not compared, so the floor is a third of the 12 rows
    assert _run(wl, None, 4, temperature, max_ctx=128, logits_rounds=(1,)) >= 4


@pytest.mark.parametrize("batch,block,ctx", [
    (1, 16, [300]),                     # one 16-row group: exactly normalised rows, LDS head
    (2, 16, [77, 190]),                 # 30 rows: batched matrix-core head / logits head
    (5, 16, [100, 260, 3, 64, 129]),    # 75 rows
    (3, 7, [40, 500, 1]),               # short block
    (9, 16, [120, 3, 260, 77, 1, 400, 64, 190, 33]),  # 135 rows: the 256-row matrix-core head
])
def test_small_bf16_sampled(batch, block, ctx):
    wl = Workload(300 + batch * 10 + block, f"sampled_b{batch}_B{block}", SMALL_BF16, batch=batch,
                  block=block, ctx=1, accept_mean=4.0, rounds=2)
    log(f"[sampled small bf16] batch={batch} block={block}")
    n = _run(wl, ctx, 2, 1.0)
    assert n >= batch * (block - 1)  # at least one round's worth of rows compared


def test_full_k_group_sampled():
    """The widths at which one 16-row group runs the full-K GEMMs: sampling must
    not use the per-row scaled lm_head input of the greedy path."""
    wl = Workload(391, "sampled_mid", MID_BF16, batch=1, block=16, ctx=1, accept_mean=4.0,
                  rounds=2)
    log("[sampled mid bf16] full-K group")
    assert _run(wl, [260], 2, 1.0, logits_rounds=()) >= 15


@pytest.mark.parametrize("batch", [1, 3])
def test_nonpositive_temperature_is_the_greedy_draft(batch):
    """dflash_draft_block_sampled with temperature <= 0, a temperature whose
    inverse overflows, or no sampling descriptor, drafts exactly what
    dflash_draft_block drafts."""
    import torch
    from block_diffusion_drafter_layers_amd import binding as B
    from block_diffusion_drafter_layers_amd.runtime import _stream_ptr
    assert torch.cuda.is_available()
    wl = Workload(395 + batch, f"sampled_cold_b{batch}", SMALL_BF16, batch=batch, block=16,
                  ctx=1, accept_mean=4.0)
    p = build_pair(wl, max_ctx=1024, ctx=np.array([300, 41, 170][:batch]))
    prefill(p)
    dev = p.dev
    x0 = torch.from_numpy(p.inp.x0().astype(np.int32)).cuda()
    ref = torch.zeros(batch, 15, dtype=torch.int32, device="cuda")
    dev.draft(x0, 16, ref)
    # 1e-40 is positive but its inverse overflows float: the greedy limit
    for smp in (B.dflash_sampling(0.0, 5, 6), B.dflash_sampling(-1.0, 5, 6),
                B.dflash_sampling(1e-40, 5, 6), None):
        ids = torch.full_like(ref, -1)
        rc = B.dflash_draft_block_sampled(dev.cfg, dev.wstruct, dev.kv, x0.data_ptr(), 16, smp,
                                          ids.data_ptr(), dev.ws.data_ptr(), dev.ws_bytes, None,
                                          _stream_ptr())
        assert rc == 0
        torch.cuda.synchronize()
        assert torch.equal(ids, ref)
    assert int(dev.err.item()) == 0


@pytest.mark.parametrize("batch,ctx,seed,offset", [
    (1, [300], 99, 7),
    (3, [77, 190, 5], 99, 7),
    # both key words non-zero (the seed's high half) and the largest offset
    (3, [77, 190, 5], 0xFEDCBA9876543210, 0xFFFFFFFF),
    # 135 rows: the 256-row matrix-core head that large batches run
    (9, [120, 3, 260, 77, 1, 400, 64, 190, 33], 0xFEDCBA9876543210, 0xFFFFFFFF),
])
def test_noise_alone_matches_the_oracle(batch, ctx, seed, offset):
    """With the lm_head zeroed every logit is exactly 0, so a row's sampling
    scores are its Gumbel noise alone.  The kernel's best and runner-up scores
    must equal the oracle's to fp32 rounding of the noise transform (2e-5
    absolute, about ten units in the last place at the largest of 65536 draws,
    where u is nearest 1 and -ln u smallest), and its ids the oracle's, from
    the head the benchmark runs as from the head that stores logits."""
    import dataclasses

    import torch
    assert torch.cuda.is_available()
    dims = dataclasses.replace(SMALL_BF16, vocab=65536)
    wl = Workload(410 + batch, f"noise_b{batch}", dims, batch=batch, block=16, ctx=1,
                  accept_mean=4.0)
    log(f"[sampled noise alone] batch={batch} ctx={ctx} seed={seed:#x} offset={offset:#x}")
    p = build_pair(wl, max_ctx=1024, ctx=np.array(ctx),
                   weight_map=lambda n, w: np.zeros_like(w) if n == "lm_head" else w)
    prefill(p)
    x0 = p.inp.x0()
    x0d = torch.from_numpy(np.asarray(x0, dtype=np.int32)).cuda()
    rows = (batch, 15)
    ids = torch.zeros(rows, dtype=torch.int32, device="cuda")
    ids_bench = torch.zeros(rows, dtype=torch.int32, device="cuda")
    t2 = torch.zeros(*rows, 2, dtype=torch.float32, device="cuda")
    lg = torch.full((*rows, dims.vocab), 1.0, dtype=torch.float32, device="cuda")
    p.dev.draft(x0d, 16, ids, logits=lg, top2=t2, temperature=1.0, seed=seed, offset=offset)
    p.dev.draft(x0d, 16, ids_bench, temperature=1.0, seed=seed, offset=offset)
    r = p.ora.draft(x0, 16, want_logits=True, temperature=1.0, seed=seed, offset=offset)
    torch.cuda.synchronize()
    assert not torch.any(lg != 0), "a zero lm_head gives zero logits"
    top2 = t2.cpu().numpy().astype(np.float64)
    err = np.max(np.abs(top2 - r["top2"]))
    log(f"  best {r['top2'][..., 0].min():.3f}..{r['top2'][..., 0].max():.3f}, "
        f"worst score error {err:.2e}")
    assert err < 2e-5, err
    sure = r["top2"][..., 0] - r["top2"][..., 1] > 1e-4
    assert sure.sum() >= 0.9 * sure.size
    for name, got in (("logits head", ids), ("benchmarked head", ids_bench)):
        got = got.cpu().numpy()
        assert np.array_equal(got[sure], r["draft_ids"][sure]), name
    assert int(p.dev.err.item()) == 0
