"""The three calls captured into one HIP graph and replayed give, replay after
replay, exactly what eager calls give (the library launches no memset, never
synchronises and allocates nothing, so its launches can be captured)."""

import numpy as np
import pytest

from synth.configs import Workload
from tests.gpu_common import build_pair, log, prefill
from tests.test_gpu_parity import SMALL_BF16, SMALL_I768

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dims,batch,temperature", [
    (SMALL_BF16, 1, 0.0), (SMALL_BF16, 3, 0.0), (SMALL_BF16, 3, 1.0),
    # 144 rows: the matrix-core projections (gate/up on 128 x 384 tiles), the balanced
    # attention split and the batched lm_head, as the batch-32 benchmark replays them
    (SMALL_I768, 9, 0.0),
], ids=["b1", "b3", "b3_sampled", "b9_matrix_core"])
def test_graph_replay_matches_eager(dims, batch, temperature):
    """temperature > 0: the sampled draft (its noise is keyed by position, so a replay
    at a new position draws new noise without new arguments)."""
    import torch
    from block_diffusion_drafter_layers_amd.runtime import DeviceDrafter, to_device
    assert torch.cuda.is_available()
    wl = Workload(150 + batch, f"graph_b{batch}", dims, batch=batch, block=16, ctx=1,
                  accept_mean=5.0)
    ctx = np.array([300, 41, 170, 0, 260, 7, 111, 64, 190][:batch])
    log(f"[graph] batch={batch} temperature={temperature}")
    smp = dict(temperature=temperature, seed=7, offset=3)
    p = build_pair(wl, max_ctx=1024, ctx=ctx)
    prefill(p, check=True)
    d = wl.dims
    B, bt = wl.block, wl.batch
    dev_a = p.dev
    dev_b = DeviceDrafter(d, dev_a.w, bt, dev_a.max_ctx, dev_a.max_rows, packed=True)
    for l in range(d.n_layers):
        dev_b.k[l].copy_(dev_a.k[l])
        dev_b.v[l].copy_(dev_a.v[l])
    dev_b.len.copy_(dev_a.len)
    dev_b.base.copy_(dev_a.base)
    # static buffers of the captured round
    x0_b = torch.zeros(bt, dtype=torch.int32, device="cuda")
    ids_b = torch.zeros(bt, B - 1, dtype=torch.int32, device="cuda")
    tgt_b = torch.zeros(bt, B, dtype=torch.int32, device="cuda")
    acc_b = torch.zeros(bt, dtype=torch.int32, device="cuda")
    bon_b = torch.zeros(bt, dtype=torch.int32, device="cuda")
    feats_b = [torch.zeros(bt * B, d.feat_hidden, dtype=torch.bfloat16, device="cuda")
               for _ in range(d.n_feat_layers)]
    row_start = torch.arange(0, bt * B, B, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dev_b.draft(x0_b, B, ids_b, **smp)
        dev_b.accept_trim(ids_b, tgt_b, B, acc_b, bon_b)
        dev_b.fuse_inject(feats_b, row_start, acc_b, bt * B)
    torch.cuda.synchronize()
    x0 = p.inp.x0()
    for rnd in range(4):
        # eager twin
        x0_a = torch.from_numpy(x0.astype(np.int32)).cuda()
        ids_a = torch.zeros(bt, B - 1, dtype=torch.int32, device="cuda")
        dev_a.draft(x0_a, B, ids_a, **smp)
        torch.cuda.synchronize()
        tgt = p.inp.targets_for(ids_a.cpu().numpy(), rnd)
        tgt_a = torch.from_numpy(tgt).cuda()
        acc_a = torch.zeros(bt, dtype=torch.int32, device="cuda")
        bon_a = torch.zeros(bt, dtype=torch.int32, device="cuda")
        dev_a.accept_trim(ids_a, tgt_a, B, acc_a, bon_a)
        rf = [np.concatenate([p.inp.round_feats(i, b, rnd) for b in range(bt)])
              for i in range(d.n_feat_layers)]
        fa = [to_device(x, d.dtype, dev_a.device) for x in rf]
        dev_a.fuse_inject(fa, row_start, acc_a, bt * B)
        torch.cuda.synchronize()
        # graph replay with the same inputs copied into its static buffers
        x0_b.copy_(x0_a)
        tgt_b.copy_(tgt_a)
        for i in range(d.n_feat_layers):
            feats_b[i].copy_(fa[i])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ids_b, ids_a), rnd
        assert torch.equal(acc_b, acc_a) and torch.equal(bon_b, bon_a), rnd
        assert torch.equal(dev_b.len, dev_a.len) and torch.equal(dev_b.base, dev_a.base), rnd
        for l in range(d.n_layers):
            n = int(dev_a.len.max().item())
            assert torch.equal(dev_b.k[l][:, :, :n], dev_a.k[l][:, :, :n]), (rnd, l)
            assert torch.equal(dev_b.v[l][:, :, :, :n], dev_a.v[l][:, :, :, :n]), (rnd, l)
        log(f"  replay {rnd}: identical to eager, accept {acc_a.cpu().numpy().tolist()}")
        x0 = bon_a.cpu().numpy()
    assert int(dev_a.err.item()) == 0 and int(dev_b.err.item()) == 0
