"""The speculative loop closed on one GPU: a synthetic random-weight target
(dflash_target_verify) verifies the drafted blocks and hands the drafter its
features, and the input-fusion variant of the injection
(dflash_fuse_inject_input).  Both against the oracle on the same seeded inputs:
target ids bit-exact away from near-ties, features and cache rows within the
float tolerance, and the whole loop committing exactly the oracle's tokens --
which are the target's own greedy tokens (lossless, pinned in the oracle)."""

import numpy as np
import pytest

from oracle.dflash_oracle import (OracleDrafter, OracleTarget, autoregressive_generate,
                                  speculative_generate)
from synth.configs import DrafterDims, Workload
from synth.inputs import DrafterInputs, f32_to_bf16_bits
from tests.gpu_common import (assert_rows_close, check_cache, draft_ids_match, host_value, log,
                              tol_for)

pytestmark = pytest.mark.gpu

T_DIMS = DrafterDims(n_layers=3, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, inter=1024,
                     vocab=4096, n_feat_layers=2, feat_hidden=512, block_max=16, dtype="bf16",
                     rope_theta=1.0e6)
D_DIMS = DrafterDims(n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, inter=1024,
                     vocab=4096, n_feat_layers=2, feat_hidden=512, block_max=16, dtype="bf16",
                     rope_theta=1.0e6)
T_F32 = DrafterDims(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, inter=704,
                    vocab=1024, n_feat_layers=2, feat_hidden=256, block_max=16, dtype="f32")
D_F32 = DrafterDims(n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, inter=704,
                    vocab=1024, n_feat_layers=2, feat_hidden=256, block_max=16, dtype="f32")
CAPTURE = [0, 2]


def _weights(dims, cfg_id, plant=False, shared=None):
    """Host weights (storage type) of a synthetic model; `shared`: take embed and
    lm_head from these.  plant: every embedding gets a large common direction and
    lm_head row 7 points along it, so every model picks id 7 everywhere."""
    inp = DrafterInputs(Workload(cfg_id, f"loop{cfg_id}", dims, batch=1, block=16, ctx=1))
    w = {n: inp.weight(n) for n in inp.weight_shapes()}
    if shared is not None:
        w["embed"], w["lm_head"] = shared["embed"], shared["lm_head"]
    elif plant:
        f = lambda a: host_value(a, dims).astype(np.float32)
        enc = (lambda x: f32_to_bf16_bits(x)) if dims.dtype == "bf16" else (lambda x: x)
        u = np.zeros(dims.hidden, np.float32)
        u[3] = 1.0
        w["embed"] = enc((f(w["embed"]) * 0.05 + 40.0 * u).astype(np.float32))
        lm = f(w["lm_head"]).copy()
        lm[7] = 50.0 * u
        w["lm_head"] = enc(lm)
    return w


def _f32(w, dims):
    return {n: host_value(a, dims).astype(np.float64) for n, a in w.items()}


def _models(tdims, ddims, seed, plant, max_ctx=512):
    from block_diffusion_drafter_layers_amd.runtime import DeviceDrafter
    wt = _weights(tdims, seed, plant=plant)
    wd = _weights(ddims, seed + 1, shared=wt)
    wt = {n: a for n, a in wt.items() if n not in ("fc", "fc_norm")}   # a target has no fusion
    tgt = DeviceDrafter(tdims, wt, 1, max_ctx, 64)
    dft = DeviceDrafter(ddims, wd, 1, max_ctx, 64)
    return wt, wd, tgt, dft


def _verify(tgt, ids, capture, dims, devc):
    import torch
    n = len(ids)
    bi = torch.tensor([list(ids)], dtype=torch.int32, device=devc)
    out = torch.zeros(1, n, dtype=torch.int32, device=devc)
    feats = [torch.zeros(n, dims.hidden, dtype=tgt.tdtype, device=devc) for _ in capture]
    tgt.verify(bi, n, out, capture=capture, feats_out=feats)
    return out, feats


@pytest.mark.parametrize("tdims", [T_DIMS, T_F32], ids=["bf16", "f32"])
def test_target_verify_matches_the_oracle(tdims):
    """A prompt of 40 tokens in verification passes of 16, 16 and 8, then a block of
    16: next-token ids, the captured features and the target's cache rows."""
    import torch
    from block_diffusion_drafter_layers_amd.runtime import DeviceDrafter
    cap = CAPTURE if tdims.n_layers > 2 else [0, 1]
    w = _weights(tdims, 180)
    w = {n: a for n, a in w.items() if n not in ("fc", "fc_norm")}
    tgt = DeviceDrafter(tdims, w, 1, 256, 64)
    ora = OracleTarget(tdims, _f32(w, tdims), 1)
    devc = tgt.device
    tol = tol_for(tdims)
    ids = np.random.default_rng(181).integers(0, tdims.vocab - 1, size=56)
    worst = {"feat": 0.0, "ids": 0}
    for a, b in ((0, 16), (16, 32), (32, 40), (40, 56)):
        out, feats = _verify(tgt, ids[a:b], cap, tdims, devc)
        o_ids, o_top2, o_feats = ora.forward(0, ids[a:b], cap)
        torch.cuda.synchronize()
        worst["ids"] += draft_ids_match(out.cpu().numpy()[0], o_ids, o_top2)
        for i in range(len(cap)):
            g = host_value(feats[i].view(torch.int16).cpu().numpy().view(np.uint16)
                           if tdims.dtype == "bf16" else feats[i].cpu().numpy(), tdims)
            worst["feat"] = max(worst["feat"], assert_rows_close(f"feat {i}", g, o_feats[i], tol))
        assert int(tgt.len.item()) == b and int(tgt.base.item()) == a
    assert int(tgt.err.item()) == 0
    wk = wv = 0.0
    for l in range(tdims.n_layers):
        k, v = tgt.cache_rows(l, 0, 56)
        wk = max(wk, assert_rows_close(f"K{l}", k.float().cpu().numpy(), ora.k[l][0], tol))
        wv = max(wv, assert_rows_close(f"V{l}", v.float().cpu().numpy(), ora.v[l][0], tol))
    log(f"[target] {tdims.dtype}: ids compared {worst['ids']}, features {worst['feat']:.2e}, "
        f"cache K {wk:.2e} V {wv:.2e}")
    assert worst["ids"] >= 40


def _gpu_autoregressive(wt, prompt, n_tokens):
    """The target's own greedy decoding on the GPU: the prompt in passes of 16, then
    one token per pass."""
    import torch
    from block_diffusion_drafter_layers_amd.runtime import DeviceDrafter
    tgt = DeviceDrafter(T_DIMS, wt, 1, 512, 64)
    devc = tgt.device
    out, _ = _verify(tgt, prompt[:16], CAPTURE, T_DIMS, devc)
    out, _ = _verify(tgt, prompt[16:], CAPTURE, T_DIMS, devc)
    toks = [int(out[0, -1].item())]
    while len(toks) < n_tokens:
        out, _ = _verify(tgt, [toks[-1]], CAPTURE, T_DIMS, devc)
        toks.append(int(out[0, -1].item()))
    return toks


@pytest.mark.parametrize("input_fusion", [False, True], ids=["kv_injection", "input_fusion"])
@pytest.mark.parametrize("plant", [True, False], ids=["planted", "random"])
def test_closed_loop_is_lossless(plant, input_fusion):
    """Prefill (the target's features of the prompt injected into the drafter), then
    rounds of draft -> verify -> accept + trim of both caches -> injection of the
    verified rows.  Planted weights: every draft matches, whole blocks are accepted,
    the tokens are 7 throughout, and the GPU loop reproduces the oracle's loop
    (tokens and accept lengths).  Random weights: the drafts rarely match, and the
    committed stream must equal the target's own greedy decoding on the GPU, token
    for token (a row's arithmetic does not depend on the other rows of its pass, so
    the comparison is exact; the oracle fixes the same property in fp64)."""
    import torch
    wt, wd, tgt, dft = _models(T_DIMS, D_DIMS, 190 + 2 * plant + input_fusion, plant)
    devc = tgt.device
    prompt = [int(x) for x in np.random.default_rng(191).integers(0, T_DIMS.vocab - 1, size=20)]
    n_tokens = 48
    if plant:
        ref, ref_acc = speculative_generate(OracleTarget(T_DIMS, _f32(wt, T_DIMS), 1),
                                            OracleDrafter(D_DIMS, _f32(wd, D_DIMS), 1), 0, prompt,
                                            n_tokens, 16, CAPTURE, input_fusion=input_fusion)
        ar = autoregressive_generate(OracleTarget(T_DIMS, _f32(wt, T_DIMS), 1), 0, prompt,
                                     n_tokens)
        assert ref[:n_tokens] == ar
    # the loop on the GPU
    one = torch.zeros(1, dtype=torch.int32, device=devc)

    def inject(feats, n):
        rc = torch.tensor([n], dtype=torch.int32, device=devc)
        if input_fusion:
            dft.fuse_inject_input(feats, one, rc, n, feats[0].shape[0])
        else:
            dft.fuse_inject(feats, one, rc, feats[0].shape[0])

    out, feats = _verify(tgt, prompt[:16], CAPTURE, T_DIMS, devc)
    inject(feats, 16)
    out, feats = _verify(tgt, prompt[16:], CAPTURE, T_DIMS, devc)
    inject(feats, len(prompt) - 16)
    x0 = int(out[0, -1].item())
    got, acc_lens = [x0], []
    ids = torch.zeros(1, 15, dtype=torch.int32, device=devc)
    acc = torch.zeros(1, dtype=torch.int32, device=devc)
    bonus = torch.zeros(1, dtype=torch.int32, device=devc)
    while len(got) < n_tokens:
        dft.draft(torch.tensor([x0], dtype=torch.int32, device=devc), 16, ids)
        block = torch.cat([torch.tensor([[x0]], dtype=torch.int32, device=devc), ids], dim=1)
        t_ids = torch.zeros(1, 16, dtype=torch.int32, device=devc)
        feats = [torch.zeros(16, T_DIMS.hidden, dtype=tgt.tdtype, device=devc) for _ in CAPTURE]
        tgt.verify(block, 16, t_ids, capture=CAPTURE, feats_out=feats)
        dft.accept_trim(ids, t_ids, 16, acc, bonus)
        tgt.accept_trim(ids, t_ids, 16, acc, bonus)
        a = int(acc.item())
        inject(feats, a)
        got.extend(int(v) for v in t_ids[0, :a].cpu().numpy())
        acc_lens.append(a)
        x0 = int(bonus.item())
    torch.cuda.synchronize()
    assert int(tgt.err.item()) == 0 and int(dft.err.item()) == 0
    log(f"[loop] planted={plant} input_fusion={input_fusion}: {len(got)} tokens, "
        f"accept lengths {acc_lens}")
    assert int(tgt.len.item()) == int(dft.len.item()) == len(prompt) + sum(acc_lens)
    if plant:
        assert got == ref and acc_lens == ref_acc
        assert set(got) == {7} and all(a == 16 for a in acc_lens[:-1])
    else:
        assert got[:n_tokens] == _gpu_autoregressive(wt, prompt, n_tokens)


def test_input_fusion_injection_matches_the_oracle():
    """Three sequences with ragged row counts (rows_max 40: three causal passes of
    16), then a draft from the injected caches, then the re-injection of accepted
    rows: cache rows and the draft against the oracle."""
    import torch
    from block_diffusion_drafter_layers_amd.runtime import DeviceDrafter, to_device
    dims = DrafterDims(n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
                       inter=1024, vocab=4096, n_feat_layers=5, feat_hidden=256, block_max=16,
                       dtype="bf16", rope_theta=1.0e6)
    wl = Workload(195, "input_fusion", dims, batch=3, block=16, ctx=1)
    inp = DrafterInputs(wl)
    names = list(inp.weight_shapes())
    ctx = np.array([40, 7, 23])
    dev = DeviceDrafter(dims, {n: inp.weight(n) for n in names}, 3, 256, int(ctx.sum()) + 48)
    ora = OracleDrafter(dims, {n: inp.weight_f32(n) for n in names}, 3)
    devc = dev.device
    feats = [[inp.ctx_feats(i, b, n_rows=int(ctx[b])) for i in range(5)] for b in range(3)]
    packed = [np.concatenate([feats[b][i] for b in range(3)]) for i in range(5)]
    starts = np.concatenate([[0], np.cumsum(ctx)[:-1]]).astype(np.int32)
    fused = torch.zeros(int(ctx.sum()), dims.hidden, dtype=torch.float32, device=devc)
    dev.fuse_inject_input([to_device(x, "bf16", devc) for x in packed],
                          torch.from_numpy(starts).to(devc),
                          torch.from_numpy(ctx.astype(np.int32)).to(devc), int(ctx.max()),
                          int(ctx.sum()), fused_dbg=fused)
    cs = [ora.fuse_inject_input(b, [host_value(feats[b][i], dims) for i in range(5)])
          for b in range(3)]
    torch.cuda.synchronize()
    tol = tol_for(dims)
    assert_rows_close("fused", fused.cpu().numpy(), np.concatenate(cs), tol)

    class P:  # the pieces check_cache reads
        pass
    p = P()
    p.dev, p.ora, p.wl = dev, ora, wl
    log(f"[input fusion] prefill cache {check_cache(p)}")
    # a draft from these caches, then the re-injection of 5, 16 and 1 accepted rows
    x0 = inp.x0()
    ids = torch.zeros(3, 15, dtype=torch.int32, device=devc)
    fh = torch.zeros(3, 16, dims.hidden, dtype=torch.float32, device=devc)
    dev.draft(torch.from_numpy(x0).to(devc), 16, ids, final_hidden=fh)
    r = ora.draft(x0, 16)
    torch.cuda.synchronize()
    assert_rows_close("final_hidden", fh.cpu().numpy(), r["final_hidden"], tol)
    draft_ids_match(ids.cpu().numpy(), r["draft_ids"], r["top2"])
    acc = np.array([5, 16, 1], dtype=np.int32)
    rf = [[inp.round_feats(i, b, 0) for i in range(5)] for b in range(3)]
    dev.fuse_inject_input([to_device(np.concatenate([rf[b][i] for b in range(3)]), "bf16", devc)
                           for i in range(5)],
                          torch.arange(0, 48, 16, dtype=torch.int32, device=devc),
                          torch.from_numpy(acc).to(devc), 16, 48)
    for b in range(3):
        ora.fuse_inject_input(b, [host_value(rf[b][i][:acc[b]], dims) for i in range(5)])
    torch.cuda.synchronize()
    assert int(dev.err.item()) == 0
    log(f"[input fusion] after re-injection {check_cache(p)}")
