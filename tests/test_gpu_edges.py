"""Edge cases of the three calls on the GPU, against the oracle: an empty
fuse_inject, a sequence with no rows next to one with rows, an injection and a
draft that would run past the cache (the sticky overflow bit is raised, nothing
is written out of range, and the other sequences are unaffected)."""

import numpy as np
import pytest

from synth.configs import DrafterDims, Workload
from tests.gpu_common import (build_pair, check_cache, draft_ids_match, host_value, log,
                              prefill, tol_for, assert_rows_close)

pytestmark = pytest.mark.gpu

EDGE_BF16 = DrafterDims(n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
                        inter=1024, vocab=4096, n_feat_layers=5, feat_hidden=256, block_max=16,
                        dtype="bf16", rope_theta=1.0e6)


# hidden 1024: the width at which a batch-1 round takes the full-K draft GEMMs
EDGE_MID = DrafterDims(n_layers=2, hidden=1024, n_q_heads=16, n_kv_heads=4, head_dim=128,
                       inter=2048, vocab=4096, n_feat_layers=5, feat_hidden=512, block_max=16,
                       dtype="bf16", rope_theta=1.0e6)


def _wl(cfg_id, batch, dims=EDGE_BF16):
    return Workload(cfg_id, f"edge_{cfg_id}", dims, batch=batch, block=16, ctx=1,
                    accept_mean=4.0)


@pytest.mark.parametrize("dims", [EDGE_BF16, EDGE_MID], ids=["h512", "h1024"])
def test_empty_and_partial_fuse_inject(dims):
    import torch
    from block_diffusion_drafter_layers_amd.runtime import to_device
    wl = _wl(150, 3, dims)
    log(f"[edge] hidden {dims.hidden}: empty fuse_inject, then rows for sequences 0 and 2 only")
    p = build_pair(wl, max_ctx=512, ctx=np.array([40, 17, 64]))
    prefill(p)
    dims = wl.dims
    devc = p.dev.device
    nf = dims.n_feat_layers
    len0 = p.dev.len.cpu().numpy().copy()
    # total_rows = 0: nothing is launched on the rows, len unchanged, no error
    zero = torch.zeros(3, dtype=torch.int32, device=devc)
    empty = [torch.zeros(1, dims.feat_hidden, dtype=torch.bfloat16, device=devc) for _ in range(nf)]
    p.dev.fuse_inject(empty, zero, zero, 0)
    torch.cuda.synchronize()
    assert np.array_equal(p.dev.len.cpu().numpy(), len0)
    assert int(p.dev.err.item()) == 0
    # 5 rows for sequence 0, none for 1, 3 rows for 2 (packed 0..4, 5..7)
    rows = {0: 5, 2: 3}
    feats = {b: [p.inp.round_feats(i, b, 0)[:n] for i in range(nf)] for b, n in rows.items()}
    packed = [np.concatenate([feats[0][i], feats[2][i]]) for i in range(nf)]
    dfe = [to_device(x, dims.dtype, devc) for x in packed]
    rs = torch.tensor([0, 5, 5], dtype=torch.int32, device=devc)
    rc = torch.tensor([5, 0, 3], dtype=torch.int32, device=devc)
    p.dev.fuse_inject(dfe, rs, rc, 8)
    for b, n in rows.items():
        p.ora.fuse_inject(b, [host_value(feats[b][i], dims) for i in range(nf)])
    torch.cuda.synchronize()
    assert np.array_equal(p.dev.len.cpu().numpy(), len0 + np.array([5, 0, 3]))
    assert int(p.dev.err.item()) == 0
    log(f"  cache {check_cache(p)}")


def test_fuse_inject_past_the_cache_clamps_and_sets_overflow():
    """12 rows for a sequence with 8 free positions next to 4 rows for another: the
    8 that fit are written, len stops at max_ctx, the overflow bit is raised, the
    other sequence is unaffected."""
    import torch
    from block_diffusion_drafter_layers_amd.runtime import to_device
    wl = _wl(152, 2, EDGE_MID)
    log("[edge] hidden 1024: 12 rows into 8 free positions + 4 rows elsewhere")
    p = build_pair(wl, max_ctx=128, ctx=np.array([120, 30]))
    prefill(p)
    dims = wl.dims
    devc = p.dev.device
    nf = dims.n_feat_layers
    rows = {0: 12, 1: 4}
    feats = {b: [p.inp.round_feats(i, b, 0)[:n] for i in range(nf)] for b, n in rows.items()}
    packed = [np.concatenate([feats[0][i], feats[1][i]]) for i in range(nf)]
    dfe = [to_device(x, dims.dtype, devc) for x in packed]
    rs = torch.tensor([0, 12], dtype=torch.int32, device=devc)
    rc = torch.tensor([12, 4], dtype=torch.int32, device=devc)
    p.dev.fuse_inject(dfe, rs, rc, 16)
    p.ora.fuse_inject(0, [host_value(feats[0][i][:8], dims) for i in range(nf)])
    p.ora.fuse_inject(1, [host_value(feats[1][i], dims) for i in range(nf)])
    torch.cuda.synchronize()
    assert np.array_equal(p.dev.len.cpu().numpy(), np.array([128, 34]))
    assert int(p.dev.err.item()) & 1, "overflow bit not raised"
    log(f"  cache {check_cache(p)}")


def test_draft_past_the_cache_sets_overflow_and_spares_the_rest():
    import torch
    wl = _wl(151, 2)
    log("[edge] sequence 0 at 120 of 128 positions drafts a 16-row block")
    p = build_pair(wl, max_ctx=128, ctx=np.array([120, 30]))
    prefill(p)
    dims = wl.dims
    devc = p.dev.device
    B = wl.block
    x0 = p.inp.x0()
    ids = torch.zeros(2, B - 1, dtype=torch.int32, device=devc)
    fh = torch.zeros(2, B, dims.hidden, dtype=torch.float32, device=devc)
    p.dev.draft(torch.from_numpy(x0).to(devc), B, ids, final_hidden=fh)
    torch.cuda.synchronize()
    assert int(p.dev.err.item()) & 1, "overflow bit not raised"
    # sequence 1 fits: the oracle drafts it alone
    from oracle.dflash_oracle import OracleDrafter
    ora1 = OracleDrafter(dims, {n: p.inp.weight_f32(n) for n in p.inp.weight_shapes()}, 1)
    feats = [host_value(p.inp.ctx_feats(i, 1, n_rows=30), dims) for i in range(dims.n_feat_layers)]
    ora1.fuse_inject(0, feats)
    r = ora1.draft(x0[1:], B)
    e = assert_rows_close("final_hidden seq 1", fh.cpu().numpy()[1:], r["final_hidden"],
                          tol_for(dims))
    n = draft_ids_match(ids.cpu().numpy()[1:], r["draft_ids"], r["top2"])
    log(f"  seq 1: final_hidden {e:.2e}, ids compared {n}; err {int(p.dev.err.item())}")


@pytest.mark.parametrize("dims,batch,ctx", [(EDGE_BF16, 1, [70]), (EDGE_MID, 1, [130]),
                                            (EDGE_BF16, 5, [20, 300, 7, 64, 129])],
                         ids=["h512_b1", "h1024_b1", "h512_b5"])
def test_draft_ignores_stale_workspace_contents(dims, batch, ctx):
    """The workspace holds whatever earlier calls (or nothing) left: filled with
    all-ones bytes (NaN as fp32) before a draft, the draft still matches the oracle.
    (The attention merge once multiplied the weight 0 of an unused split slot by
    that slot's stale sum, and 0 x NaN is NaN.)"""
    import torch
    wl = _wl(155 + len(ctx) + dims.hidden // 512, batch, dims)
    log(f"[edge] hidden {dims.hidden} batch {batch}: draft over a NaN-filled workspace")
    p = build_pair(wl, max_ctx=512, ctx=np.array(ctx))
    prefill(p, check=False)
    p.dev.ws.fill_(255)
    torch.cuda.synchronize()
    from tests.gpu_common import draft_round
    out = draft_round(p, p.inp.x0(), 0, check_logits=False)
    assert int(p.dev.err.item()) == 0
    log(f"  final_hidden {out['final_hidden']:.2e}, ids compared {out['compared_ids']}")
