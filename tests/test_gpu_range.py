"""fp16 range safety of the bf16 storage type.  A weight that fp16 cannot hold is
counted when it is packed; a value that leaves fp16 range on the device raises
DFLASH_ERR_NONFINITE in the sticky error word instead of passing infinities on
silently (an infinite query score turns the block's attention into NaN, and the
pick of every drafted row then finds no finite score)."""

import numpy as np
import pytest

from synth.configs import DrafterDims, Workload
from synth.inputs import DrafterInputs, f32_to_bf16_bits
from tests.gpu_common import host_value, log

pytestmark = pytest.mark.gpu

RANGE_BF16 = DrafterDims(n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
                         inter=1024, vocab=4096, n_feat_layers=5, feat_hidden=256, block_max=16,
                         dtype="bf16", rope_theta=1.0e6)


def _drafter(wl, planted, ctx_rows):
    import torch
    from block_diffusion_drafter_layers_amd.runtime import DeviceDrafter, to_device
    inp = DrafterInputs(wl)
    w = {n: inp.weight(n) for n in inp.weight_shapes()}
    for (name, r, c), val in planted.items():
        m = w[name].copy()
        m[r, c] = f32_to_bf16_bits(np.array([val], np.float32))[0]
        w[name] = m
    dev = DeviceDrafter(wl.dims, w, 1, max_ctx=256, max_rows=ctx_rows)
    nf = wl.dims.n_feat_layers
    feats = [inp.ctx_feats(i, 0, n_rows=ctx_rows) for i in range(nf)]
    dev.fuse_inject([to_device(f, "bf16", dev.device) for f in feats],
                    torch.zeros(1, dtype=torch.int32, device=dev.device),
                    torch.full((1,), ctx_rows, dtype=torch.int32, device=dev.device), ctx_rows)
    torch.cuda.synchronize()
    return inp, w, dev, feats


def test_planted_weight_beyond_fp16_is_counted_and_the_draft_flags_it():
    import torch
    wl = Workload(160, "range_weight", RANGE_BF16, batch=1, block=16, ctx=1, accept_mean=4.0)
    log("[range] wq[0][3, 17] = 1e5 (bf16 99840): packed to infinity")
    inp, w, dev, _ = _drafter(wl, {("l0.wq", 3, 17): 1.0e5}, 40)
    assert int(dev.pack_overflow.item()) == 1, "the one element beyond fp16 is counted"
    assert int(dev.err.item()) == 0, "the injection does not read wq"
    ids = torch.full((1, 15), 77, dtype=torch.int32, device=dev.device)
    dev.draft(torch.from_numpy(inp.x0()).to(dev.device), 16, ids)
    torch.cuda.synchronize()
    err = int(dev.err.item())
    log(f"  err {err}, ids {ids.cpu().numpy().tolist()}")
    assert err & 8, "non-finite scores must raise DFLASH_ERR_NONFINITE"
    assert np.all(ids.cpu().numpy() == 0), "rows without a finite score draft id 0"


def test_injected_key_beyond_fp16_flags_the_cache_write():
    """wk[0][0, 5] = 65024 (finite in fp16): the injected K of a row whose fused
    feature has |c_5| around 1 or more passes 65520 and cannot be stored."""
    import torch
    from oracle.dflash_oracle import fuse, rope
    wl = Workload(161, "range_key", RANGE_BF16, batch=1, block=16, ctx=1, accept_mean=4.0)
    rows = 100
    inp, w, dev, feats = _drafter(wl, {("l0.wk", 0, 5): 65024.0}, rows)
    assert int(dev.pack_overflow.item()) == 0, "65024 is an fp16 value"
    # premise, from the oracle: some rotated key of layer 0 leaves fp16 range
    d = RANGE_BF16
    f = lambda n: host_value(w[n], d).astype(np.float64)
    c = fuse([host_value(x, d).astype(np.float64) for x in feats], f("fc"), f("fc_norm"), d.rms_eps)
    k = rope((c @ f("l0.wk").T).reshape(rows, d.n_kv_heads, d.head_dim), np.arange(rows),
             d.rope_theta)
    assert np.max(np.abs(k)) >= 65520.0, np.max(np.abs(k))
    err = int(dev.err.item())
    log(f"  oracle max |K| {np.max(np.abs(k)):.0f}, err {err}")
    assert err & 8, "an injected K/V value beyond fp16 must raise DFLASH_ERR_NONFINITE"
    assert not err & 1
