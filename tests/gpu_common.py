"""Shared pieces of the GPU parity tests: build both sides from the same seeded
inputs, run rounds in lockstep, compare with the tolerances of the contract.

Float tolerance: per row, max |gpu - oracle| / max |oracle| <= TOL_BF16 (2e-2)
for bf16 storage, TOL_F32 (1e-4) for fp32 storage.  A row is an H-vector
(fused feature, final hidden), a head_dim-vector of one cache position and
head, or a vocab-vector of logits.  Integer outputs (acceptance, lengths, draft
ids away from near-ties) are compared bit-exactly.
"""

from __future__ import annotations

import sys
from dataclasses import dataclass
from typing import Dict, List, Optional

import numpy as np

from oracle.dflash_oracle import OracleDrafter
from synth.configs import Workload
from synth.inputs import DrafterInputs, bf16_bits_to_f32

TOL_BF16 = 2e-2
TOL_F32 = 1e-4
NEAR_TIE = 1e-2


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def tol_for(dims) -> float:
    return TOL_BF16 if dims.dtype == "bf16" else TOL_F32


def row_err(gpu: np.ndarray, ora: np.ndarray) -> np.ndarray:
    """max_j |g - o| / max_j |o| over the last axis."""
    g = np.asarray(gpu, dtype=np.float64)
    o = np.asarray(ora, dtype=np.float64)
    den = np.max(np.abs(o), axis=-1)
    den = np.where(den == 0, 1.0, den)
    return np.max(np.abs(g - o), axis=-1) / den


def assert_rows_close(name: str, gpu, ora, tol: float) -> float:
    e = row_err(gpu, ora)
    worst = float(np.max(e)) if e.size else 0.0
    assert worst <= tol, f"{name}: worst normalised row error {worst:.3e} > {tol:.1e}"
    return worst


def host_value(arr: np.ndarray, dims) -> np.ndarray:
    return bf16_bits_to_f32(arr) if dims.dtype == "bf16" else np.asarray(arr, dtype=np.float32)


def draft_ids_match(gpu_ids: np.ndarray, ora_ids: np.ndarray, top2: np.ndarray) -> int:
    """Bit-exact draft ids except rows whose oracle top-2 gap < 1e-2 * |top1|.
    Returns the number of compared ids."""
    gap = top2[..., 0] - top2[..., 1]
    tie = gap < NEAR_TIE * np.abs(top2[..., 0])
    ok = (gpu_ids == ora_ids) | tie
    bad = np.argwhere(~ok)
    assert bad.size == 0, f"draft id mismatch at {bad[:8].tolist()} (gpu {gpu_ids[~ok][:8]}, " \
                          f"oracle {ora_ids[~ok][:8]})"
    return int(np.sum(~tie))


def top2_close(gpu: np.ndarray, ora: np.ndarray, logits: np.ndarray, temperature: float,
               tol: float) -> float:
    """The GPU's (best, runner-up) scores against the oracle's, per drafted row,
    normalised like the logits row they come from (scores are logit / T plus noise,
    so the scale is max |logit| / T).  Returns the worst normalised error."""
    scale = np.max(np.abs(np.asarray(logits, dtype=np.float64)), axis=-1)
    if temperature > 0:
        scale = scale / temperature
    scale = np.where(scale == 0, 1.0, scale)
    err = np.max(np.abs(np.asarray(gpu, np.float64) - np.asarray(ora, np.float64)), axis=-1) / scale
    worst = float(np.max(err)) if err.size else 0.0
    assert worst <= tol, f"top2: worst normalised error {worst:.3e} > {tol:.1e}"
    assert np.all(gpu[..., 0] >= gpu[..., 1]), "top2: runner-up above the best"
    return worst


@dataclass
class Pair:
    """GPU drafter and oracle drafter over the same inputs."""
    wl: Workload
    inp: DrafterInputs
    dev: object
    ora: OracleDrafter
    ctx: np.ndarray


def build_pair(wl: Workload, max_ctx: int, oracle_dtype=np.float64, ctx: Optional[np.ndarray] = None,
               gain_mode: str = "uniform", device="cuda:0", weight_map=None) -> Pair:
    """weight_map(name, w) (optional): replaces a weight, in its storage type, on both
    sides before either is built."""
    import torch
    from block_diffusion_drafter_layers_amd.runtime import DeviceDrafter
    inp = DrafterInputs(wl, gain_mode=gain_mode)
    names = list(inp.weight_shapes())
    ctx = inp.ctx_lengths() if ctx is None else np.asarray(ctx, dtype=np.int32)
    max_rows = max(int(ctx.sum()), wl.batch * wl.block, 1)
    ws = {n: inp.weight(n) for n in names}
    if weight_map is not None:
        ws = {n: weight_map(n, w) for n, w in ws.items()}
    as_f32 = (lambda w: bf16_bits_to_f32(w)) if wl.dims.dtype == "bf16" else (lambda w: w)
    dev = DeviceDrafter(wl.dims, ws, wl.batch, max_ctx, max_rows, device=device)
    ora = OracleDrafter(wl.dims, {n: as_f32(w) for n, w in ws.items()}, wl.batch, dtype=oracle_dtype)
    return Pair(wl, inp, dev, ora, ctx)


def prefill(p: Pair, check: bool = True) -> Dict[str, float]:
    """Fuse + inject every context row of every sequence (one packed call)."""
    import torch
    from block_diffusion_drafter_layers_amd.runtime import to_device
    wl, dims = p.wl, p.wl.dims
    nf = dims.n_feat_layers
    feats = [[p.inp.ctx_feats(i, b, n_rows=int(p.ctx[b])) for i in range(nf)]
             for b in range(wl.batch)]
    packed = [np.concatenate([feats[b][i] for b in range(wl.batch)]) for i in range(nf)]
    total = int(p.ctx.sum())
    starts = np.concatenate([[0], np.cumsum(p.ctx)[:-1]]).astype(np.int32)
    dfe = [to_device(x, dims.dtype, p.dev.device) for x in packed]
    rs = torch.from_numpy(starts).to(p.dev.device)
    rc = torch.from_numpy(p.ctx.astype(np.int32)).to(p.dev.device)
    fused = torch.zeros(max(total, 1), dims.hidden, dtype=torch.float32, device=p.dev.device)
    p.dev.fuse_inject(dfe, rs, rc, total, fused_dbg=fused)
    res = {}
    cs = []
    for b in range(wl.batch):
        cs.append(p.ora.fuse_inject(b, [host_value(feats[b][i], dims) for i in range(nf)]))
    torch.cuda.synchronize()
    if check and total:
        res["fused"] = assert_rows_close("fused", fused.cpu().numpy()[:total], np.concatenate(cs),
                                         tol_for(dims))
        res.update(check_cache(p))
    return res


def check_cache(p: Pair, rows: Optional[Dict[int, np.ndarray]] = None) -> Dict[str, float]:
    """Compare cache rows [0, len) (or the given positions) of every layer and sequence."""
    import torch
    dims = p.wl.dims
    tol = tol_for(dims)
    lens = p.dev.len.cpu().numpy()
    assert np.array_equal(lens, p.ora.len.astype(np.int32)), (lens, p.ora.len)
    wk = wv = 0.0
    for l in range(dims.n_layers):
        for b in range(p.wl.batch):
            n = int(lens[b])
            sel = rows[b] if rows is not None else np.arange(n)
            k, v = p.dev.cache_rows(l, b, n)
            k = k.float().cpu().numpy()[sel]
            v = v.float().cpu().numpy()[sel]
            wk = max(wk, assert_rows_close(f"K l{l} b{b}", k, p.ora.k[l][b][sel], tol))
            wv = max(wv, assert_rows_close(f"V l{l} b{b}", v, p.ora.v[l][b][sel], tol))
    return {"k_cache": wk, "v_cache": wv}


def draft_round(p: Pair, x0: np.ndarray, round_idx: int, check_logits: bool = True,
                k: Optional[np.ndarray] = None, temperature: float = 0.0, seed: int = 0,
                offset: int = 0) -> Dict[str, object]:
    """One lockstep round: draft on both sides (greedy, or sampled at
    temperature > 0 with Philox seed and offset), compare; plant targets
    from the oracle's drafts; accept + trim on both sides from identical
    inputs; inject the accepted rows' features on both sides."""
    import torch
    from block_diffusion_drafter_layers_amd.runtime import to_device
    wl, dims = p.wl, p.wl.dims
    B, bt = wl.block, wl.batch
    devc = p.dev.device
    tol = tol_for(dims)
    x0d = torch.from_numpy(np.asarray(x0, dtype=np.int32)).to(devc)
    ids = torch.zeros(bt, B - 1, dtype=torch.int32, device=devc)
    fh = torch.zeros(bt, B, dims.hidden, dtype=torch.float32, device=devc)
    lg = torch.zeros(bt, B - 1, dims.vocab, dtype=torch.float32, device=devc) if check_logits else None
    # with the logits, the runner-up too (both switch the head to its parity variant;
    # rounds without them run the head the benchmark times)
    t2 = torch.zeros(bt, B - 1, 2, dtype=torch.float32, device=devc) if check_logits else None
    p.dev.draft(x0d, B, ids, final_hidden=fh, logits=lg, temperature=temperature, seed=seed,
                offset=offset, top2=t2)
    r = p.ora.draft(x0, B, want_logits=check_logits, temperature=temperature, seed=seed,
                    offset=offset)
    torch.cuda.synchronize()
    out = {}
    out["final_hidden"] = assert_rows_close("final_hidden", fh.cpu().numpy(), r["final_hidden"], tol)
    if check_logits:
        out["logits"] = assert_rows_close("logits", lg.cpu().numpy(), r["logits"], tol)
        out["top2"] = top2_close(t2.cpu().numpy(), r["top2"], r["logits"], temperature, tol)
    gids = ids.cpu().numpy()
    out["compared_ids"] = draft_ids_match(gids, r["draft_ids"], r["top2"])
    assert np.array_equal(p.dev.base.cpu().numpy(), p.ora.base.astype(np.int32))
    # targets planted against the oracle's drafts; both sides accept identical inputs
    tgt = p.inp.targets_for(r["draft_ids"], round_idx, k=k)
    dd = torch.from_numpy(r["draft_ids"].astype(np.int32)).to(devc)
    td = torch.from_numpy(tgt).to(devc)
    acc = torch.zeros(bt, dtype=torch.int32, device=devc)
    bon = torch.zeros(bt, dtype=torch.int32, device=devc)
    p.dev.accept_trim(dd, td, B, acc, bon)
    oacc, obon = p.ora.accept_trim(r["draft_ids"], tgt)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), oacc), (acc.cpu().numpy(), oacc)
    assert np.array_equal(bon.cpu().numpy(), obon)
    assert np.array_equal(p.dev.len.cpu().numpy(), p.ora.len.astype(np.int32))
    # re-inject the verified rows 0..accept_len-1 of each block
    nf = dims.n_feat_layers
    rf = [[p.inp.round_feats(i, b, round_idx) for i in range(nf)] for b in range(bt)]
    packed = [np.concatenate([rf[b][i] for b in range(bt)]) for i in range(nf)]
    dfe = [to_device(x, dims.dtype, devc) for x in packed]
    rs = torch.arange(0, bt * B, B, dtype=torch.int32, device=devc)
    p.dev.fuse_inject(dfe, rs, acc, bt * B)
    for b in range(bt):
        p.ora.fuse_inject(b, [host_value(rf[b][i][:oacc[b]], dims) for i in range(nf)])
    torch.cuda.synchronize()
    out["accept_len"] = oacc
    out["bonus"] = obon
    return out


# ---- full-size workloads, oracle on a sample of the sequences ------------------------------
@dataclass
class SampledPair:
    """GPU drafter over the full batch; oracle over the sampled sequences only.
    Sequences are independent in every call, so the sampled ones are checked
    exactly while the rest only need to be present (their features are drawn
    on the device, N(0, 1) rounded to bf16, and never compared)."""
    wl: Workload
    inp: DrafterInputs
    dev: object
    ora: OracleDrafter
    ctx: np.ndarray
    sample: List[int]


def build_sampled(wl: Workload, sample: List[int], max_ctx: int, device="cuda:0") -> SampledPair:
    from block_diffusion_drafter_layers_amd.runtime import DeviceDrafter
    inp = DrafterInputs(wl)
    names = list(inp.weight_shapes())
    ctx = inp.ctx_lengths()
    max_rows = max(int(ctx.sum()), wl.batch * wl.block)
    dev = DeviceDrafter(wl.dims, {n: inp.weight(n) for n in names}, wl.batch, max_ctx, max_rows,
                        device=device)
    ws = {}
    for n in names:  # the oracle's fp32 copies; the bf16 host copies are no longer needed
        ws[n] = inp.weight_f32(n)
        inp.drop(n)
    ora = OracleDrafter(wl.dims, ws, len(sample), dtype=np.float32)
    return SampledPair(wl, inp, dev, ora, ctx, list(sample))


def prefill_sampled(p: SampledPair) -> Dict[str, float]:
    """One packed fuse_inject of every context row; the sampled sequences' fused
    rows and K/V cache are compared with the oracle."""
    import torch
    wl, dims = p.wl, p.wl.dims
    nf, ht = dims.n_feat_layers, dims.feat_hidden
    total = int(p.ctx.sum())
    starts = np.concatenate([[0], np.cumsum(p.ctx)[:-1]]).astype(np.int64)
    gen = torch.Generator(device=p.dev.device)
    gen.manual_seed(wl.cfg_id * 7919 + 17)
    dfe = []
    host = {}
    for i in range(nf):
        t = torch.empty(total, ht, dtype=torch.bfloat16, device=p.dev.device)
        for b in range(wl.batch):
            s0, n = int(starts[b]), int(p.ctx[b])
            if b in p.sample:
                h = p.inp.ctx_feats(i, b, n_rows=n)
                host[(i, b)] = h
                t[s0:s0 + n] = torch.from_numpy(h.view(np.int16)).to(p.dev.device).view(torch.bfloat16)
            else:
                t[s0:s0 + n] = torch.randn(n, ht, generator=gen, device=p.dev.device).to(torch.bfloat16)
        dfe.append(t)
    rs = torch.from_numpy(starts.astype(np.int32)).to(p.dev.device)
    rc = torch.from_numpy(p.ctx.astype(np.int32)).to(p.dev.device)
    fused = torch.zeros(total, dims.hidden, dtype=torch.float32, device=p.dev.device)
    p.dev.fuse_inject(dfe, rs, rc, total, fused_dbg=fused)
    torch.cuda.synchronize()
    del dfe
    res = {"fused": 0.0}
    for j, b in enumerate(p.sample):
        c = p.ora.fuse_inject(j, [host_value(host[(i, b)], dims) for i in range(nf)])
        s0, n = int(starts[b]), int(p.ctx[b])
        g = fused[s0:s0 + n].cpu().numpy()
        res["fused"] = max(res["fused"], assert_rows_close(f"fused b{b}", g, c, tol_for(dims)))
    del fused
    res.update(check_cache_sampled(p))
    return res


def check_cache_sampled(p: SampledPair) -> Dict[str, float]:
    """Every cache row of the sampled sequences, every layer."""
    dims = p.wl.dims
    tol = tol_for(dims)
    lens = p.dev.len.cpu().numpy()
    wk = wv = 0.0
    for j, b in enumerate(p.sample):
        assert int(lens[b]) == int(p.ora.len[j]), (b, lens[b], p.ora.len[j])
        n = int(lens[b])
        for l in range(dims.n_layers):
            k, v = p.dev.cache_rows(l, b, n)
            wk = max(wk, assert_rows_close(f"K l{l} b{b}", k.float().cpu().numpy(), p.ora.k[l][j], tol))
            wv = max(wv, assert_rows_close(f"V l{l} b{b}", v.float().cpu().numpy(), p.ora.v[l][j], tol))
    return {"k_cache": wk, "v_cache": wv}


def draft_round_sampled(p: SampledPair, x0: np.ndarray, round_idx: int) -> Dict[str, object]:
    """One round on the full batch.  The draft is first run exactly as the
    benchmark runs it (draft ids and final hidden rows compared), then again
    with logits requested (logits compared); both sides then accept against
    targets planted on the oracle's drafts and re-inject the verified rows."""
    import torch
    from block_diffusion_drafter_layers_amd.runtime import to_device
    wl, dims = p.wl, p.wl.dims
    B, bt, devc = wl.block, wl.batch, p.dev.device
    tol = tol_for(dims)
    sm = np.asarray(p.sample)
    x0d = torch.from_numpy(np.asarray(x0, dtype=np.int32)).to(devc)
    ids = torch.zeros(bt, B - 1, dtype=torch.int32, device=devc)
    fh = torch.zeros(bt, B, dims.hidden, dtype=torch.float32, device=devc)
    p.dev.draft(x0d, B, ids, final_hidden=fh)
    gids = ids.cpu().numpy()
    ghid = fh[torch.from_numpy(sm).to(devc)].cpu().numpy()
    del fh
    lg = torch.zeros(bt, B - 1, dims.vocab, dtype=torch.float32, device=devc)
    t2 = torch.zeros(bt, B - 1, 2, dtype=torch.float32, device=devc)
    ids2 = torch.zeros_like(ids)
    p.dev.draft(x0d, B, ids2, logits=lg, top2=t2)
    glog = lg[torch.from_numpy(sm).to(devc)].cpu().numpy()
    gt2 = t2.cpu().numpy()[sm]
    del lg
    r = p.ora.draft(np.asarray(x0)[sm], B, want_logits=True)
    out = {"final_hidden": assert_rows_close("final_hidden", ghid, r["final_hidden"], tol),
           "logits": assert_rows_close("logits", glog, r["logits"], tol),
           "top2": top2_close(gt2, r["top2"], r["logits"], 0.0, tol),
           "compared_ids": draft_ids_match(gids[sm], r["draft_ids"], r["top2"])}
    assert np.array_equal(p.dev.base.cpu().numpy()[sm], p.ora.base.astype(np.int32))
    # targets: the sampled rows planted on the oracle's drafts, the rest on the GPU's
    drafts = gids.copy()
    drafts[sm] = r["draft_ids"]
    tgt = p.inp.targets_for(drafts, round_idx)
    dd = torch.from_numpy(drafts.astype(np.int32)).to(devc)
    td = torch.from_numpy(tgt).to(devc)
    acc = torch.zeros(bt, dtype=torch.int32, device=devc)
    bon = torch.zeros(bt, dtype=torch.int32, device=devc)
    p.dev.accept_trim(dd, td, B, acc, bon)
    oacc, obon = p.ora.accept_trim(r["draft_ids"], tgt[sm])
    gacc = acc.cpu().numpy()
    assert np.array_equal(gacc[sm], oacc), (gacc[sm], oacc)
    assert np.array_equal(bon.cpu().numpy()[sm], obon)
    assert np.all((gacc >= 1) & (gacc <= B))
    assert np.array_equal(p.dev.len.cpu().numpy()[sm], p.ora.len.astype(np.int32))
    nf = dims.n_feat_layers
    rf = [[p.inp.round_feats(i, b, round_idx) for i in range(nf)] for b in range(bt)]
    packed = [np.concatenate([rf[b][i] for b in range(bt)]) for i in range(nf)]
    dfe = [to_device(x, dims.dtype, devc) for x in packed]
    rs = torch.arange(0, bt * B, B, dtype=torch.int32, device=devc)
    p.dev.fuse_inject(dfe, rs, acc, bt * B)
    for j, b in enumerate(p.sample):
        p.ora.fuse_inject(j, [host_value(rf[b][i][:oacc[j]], dims) for i in range(nf)])
    torch.cuda.synchronize()
    bonus = gacc.copy()
    bonus[:] = bon.cpu().numpy()
    out["accept_len"] = oacc
    out["bonus"] = bonus
    return out
