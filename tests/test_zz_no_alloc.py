"""dflash_draft_block_noalloc (the draft for callers that cannot allocate: its
workspace is the library's own scratch array) gives exactly what
dflash_draft_block gives on the same inputs, and both match the oracle, over two
calls in a row on one GPU, the second smaller than the first (a batch of three
through the split GEMMs, then one 8-row block through the full-K group path), and
for one sequence with a long cache (6016 keys: multi-tile attention chunks)."""

import numpy as np
import pytest

from synth.configs import DrafterDims, Workload
from tests.gpu_common import (assert_rows_close, build_pair, draft_ids_match, log, prefill,
                              tol_for)

pytestmark = pytest.mark.gpu

MID = DrafterDims(n_layers=2, hidden=1024, n_q_heads=16, n_kv_heads=4, head_dim=128, inter=2048,
                  vocab=4096, n_feat_layers=5, feat_hidden=512, block_max=16, dtype="bf16",
                  rope_theta=1.0e6)


@pytest.mark.parametrize("batch,block,ctx,max_ctx", [(3, 16, [300, 41, 129], 512),
                                                     (1, 8, [77], 512),
                                                     (1, 16, [6000], 8192)])
def test_noalloc_draft_equals_workspace_draft(batch, block, ctx, max_ctx):
    import torch
    from block_diffusion_drafter_layers_amd import binding as B
    wl = Workload(170 + batch, f"noalloc_b{batch}_{max_ctx}", MID, batch=batch, block=block, ctx=1,
                  accept_mean=4.0)
    log(f"[noalloc] batch {batch} block {block} ctx {ctx}")
    p = build_pair(wl, max_ctx=max_ctx, ctx=np.array(ctx))
    assert B.dflash_workspace_bytes(p.dev.cfg, batch, 0, max_ctx) <= B.DFLASH_NOALLOC_SCRATCH_BYTES
    prefill(p, check=False)
    devc = p.dev.device
    x0 = torch.from_numpy(p.inp.x0()).to(devc)
    out = {}
    for noalloc in (False, True):
        ids = torch.full((batch, block - 1), -1, dtype=torch.int32, device=devc)
        fh = torch.zeros(batch, block, MID.hidden, dtype=torch.float32, device=devc)
        p.dev.draft(x0, block, ids, final_hidden=fh, noalloc=noalloc)
        torch.cuda.synchronize()
        out[noalloc] = (ids.cpu().numpy(), fh.cpu().numpy(), p.dev.base.cpu().numpy().copy())
    assert int(p.dev.err.item()) == 0
    # the same kernels on the same inputs: identical, bit for bit
    assert np.array_equal(out[False][0], out[True][0])
    assert np.array_equal(out[False][1], out[True][1])
    assert np.array_equal(out[False][2], out[True][2])
    # and the oracle's bar
    r = p.ora.draft(p.inp.x0(), block)
    e = assert_rows_close("final_hidden", out[True][1], r["final_hidden"], tol_for(MID))
    n = draft_ids_match(out[True][0], r["draft_ids"], r["top2"])
    log(f"  identical to the workspace draft; oracle: final_hidden {e:.2e}, ids compared {n}")
