"""Draft-step throughput of the DFlash drafter on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--block B]
                    [--temperature T]

(--block: block size 2..16 instead of the workload's; --temperature: sampled drafts,
Gumbel-max in the lm_head, instead of the greedy pick.)

A step is one speculative round on the drafter side, i.e. every step of the
hot path once over one batch: draft a block per sequence (embedding, all
drafter layers with non-causal block attention over the injected context,
final norm, lm_head + argmax), accept + trim against the target's tokens, and
fuse + inject the target features of the accepted rows.  The target model is
not part of this library: its verification is stood in for by planted target
ids built on the device from the drafts with one elementwise select per step
(prefix lengths drawn from the workload's geometric distribution).

Output: one JSON line.  The headline is the metric's batch-1 case (workload 2):
blocks/s over exactly K timed steps (HIP graphs of a divisor of K steps,
replayed), the draft alone, the whole-step, draft and dominant-kernel HBM
rooflines (kernel durations from HIP events the library records around every
launch of a class during a timed run) and the CPU oracle timed on a bounded
sample of the same workload.  The default run adds the metric's batch-32 half
(workload 3: ragged contexts 512..8192) under "batch32", with the matrix-core
roofline of all its GEMMs and its lm_head, and the attention's HBM roofline.
"measured_ceilings" holds secondary denominators measured in the same run (a
streaming read, a device copy, a large hipBLASLt GEMM through torch); every
roofline also reports its achieved rate as a fraction of the measured ceiling of
its kind ("frac_of_measured"), beside the fraction of the published peak ("frac").
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 / bf16 matrix cores
METRIC = "draft blocks/s (16-tok block) + % HBM/MFMA roofline at batch 1 and 32"


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------------------
# algorithmic work of one step
# ---------------------------------------------------------------------------------------

def gemm_launches(dims, batch: int, block: int, inject_rows: int):
    """(name, M, N, K) of every projection GEMM launch in one step, in order."""
    d = dims
    M = batch * block
    qd, kvd = d.q_dim, d.kv_dim
    out = [("fusion", inject_rows, d.hidden, d.fc_in),
           ("injection", inject_rows, d.n_layers * 2 * kvd, d.hidden)]
    for _ in range(d.n_layers):
        out += [("qkv", M, qd + 2 * kvd, d.hidden), ("o", M, d.hidden, qd),
                ("gate_up", M, 2 * d.inter, d.hidden), ("down", M, d.hidden, d.inter)]
    return out


def gemm_bytes(M, N, K, es=2):
    return N * K * es + M * K * es + M * N * es


def step_bytes(dims, batch, block, ctx_mean, accept_mean, input_fusion=False):
    """Algorithmic HBM bytes of one step: every weight the step needs once,
    the K/V the attention reads, the K/V the step writes, activations in/out.
    input_fusion: the ablation's injection instead, which streams the fusion
    Linear and every drafter layer's weights again (the last layer only its
    W_k, W_v) for its causal pass over the accepted rows."""
    d = dims
    es = 2 if d.dtype == "bf16" else 4
    rows_in = int(round(batch * accept_mean))
    b = 0
    for (name, M, N, K) in gemm_launches(d, batch, block, batch * block):
        if input_fusion and name == "injection":
            continue
        b += N * K * es                                  # weights
    if input_fusion:
        layer = (d.q_dim + 2 * d.kv_dim) * d.hidden + d.hidden * d.q_dim \
            + 3 * d.inter * d.hidden
        b += ((d.n_layers - 1) * layer + 2 * d.kv_dim * d.hidden) * es
    b += d.vocab * d.hidden * es                         # lm_head
    b += batch * block * d.hidden * es                   # embedding rows
    kv_row = d.n_layers * 2 * d.kv_dim * es
    b += batch * (ctx_mean + block) * kv_row             # attention reads
    b += batch * block * kv_row + rows_in * kv_row       # block K/V + injected K/V writes
    b += rows_in * d.fc_in * es                          # features of the accepted rows
    return b


def draft_bytes(dims, batch, block, ctx_mean):
    """Algorithmic HBM bytes of the draft alone: every layer weight and the lm_head
    once, the embedding rows, the K/V attention reads and the block's K/V written."""
    d = dims
    es = 2 if d.dtype == "bf16" else 4
    b = 0
    for (name, M, N, K) in gemm_launches(d, batch, block, batch * block):
        if name not in ("fusion", "injection"):
            b += N * K * es
    b += d.vocab * d.hidden * es
    b += batch * block * d.hidden * es
    kv_row = d.n_layers * 2 * d.kv_dim * es
    b += batch * (ctx_mean + block) * kv_row + batch * block * kv_row
    return b


# ---------------------------------------------------------------------------------------

def graph_len(steps: int, cap: int = 16) -> int:
    """Steps per captured graph: the largest divisor of `steps` up to `cap`, so that
    replays time exactly `steps` steps."""
    return max(g for g in range(1, min(cap, steps) + 1) if steps % g == 0)


def gemm_flops_per_step(d, bt, B, inject_rows):
    """2 M N K over every projection GEMM of one step (draft layers, fusion and
    injection over the rows fuse_inject computes) and the lm_head over B-1 rows."""
    f = sum(2.0 * M * N * K for (_, M, N, K) in gemm_launches(d, bt, B, inject_rows))
    return f, 2.0 * bt * (B - 1) * d.vocab * d.hidden


def run_workload(wl, args, cpu_seconds: float, with_cpu: bool) -> dict:
    """Measure one workload: K timed steps (graph replay), the draft alone, per-class
    kernel durations from library-recorded events, and the oracle on the host."""
    import torch
    from block_diffusion_drafter_layers_amd import binding as Bn
    from block_diffusion_drafter_layers_amd.runtime import DeviceDrafter, LaunchTimer, to_device
    from synth.inputs import DrafterInputs, make_rng

    d = wl.dims
    B, bt = wl.block, wl.batch
    dev_t = torch.device("cuda:0")
    t0 = time.time()
    inp = DrafterInputs(wl)
    ctx = inp.ctx_lengths()
    n_rounds = args.warmup + 8 * args.steps + 64
    max_ctx = int((ctx.max() + B * (n_rounds + 2) + 63) // 64 * 64)
    names = list(inp.weight_shapes())
    host_w = {n: inp.weight(n) for n in names}
    log(f"[bench] workload {wl.name}: weights generated in {time.time() - t0:.1f}s")
    dev = DeviceDrafter(d, host_w, bt, max_ctx, max(int(ctx.sum()), bt * B))
    if not with_cpu:
        host_w = None
        inp._cache.clear()
    log(f"[bench] uploaded; workspace {dev.ws_bytes / 1e6:.1f} MB, max_ctx {max_ctx}")

    # ---- prefill: inject the whole context ----------------------------------------------
    nf = d.n_feat_layers
    total = int(ctx.sum())
    starts = np.concatenate([[0], np.cumsum(ctx)[:-1]]).astype(np.int32)
    if total <= 16384:
        feats = [to_device(np.concatenate([inp.ctx_feats(i, b, n_rows=int(ctx[b])) for b in range(bt)]),
                           d.dtype, dev_t) for i in range(nf)]
    else:  # same distribution (N(0, 1) in the storage type), drawn on the device
        gen = torch.Generator(device=dev_t)
        gen.manual_seed(wl.cfg_id * 7919 + 3)
        feats = [torch.randn(total, d.feat_hidden, generator=gen, device=dev_t).to(dev.tdtype)
                 for _ in range(nf)]
    rs_t, rc_t = torch.from_numpy(starts).to(dev_t), torch.from_numpy(ctx.astype(np.int32)).to(dev_t)
    torch.cuda.synchronize()
    pe0, pe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pe0.record()
    if args.fusion == "input":
        dev.fuse_inject_input(feats, rs_t, rc_t, int(ctx.max()), total)
    else:
        dev.fuse_inject(feats, rs_t, rc_t, total)
    pe1.record()
    torch.cuda.synchronize()
    del feats
    pms = pe0.elapsed_time(pe1)
    pflop = 2.0 * total * (d.fc_in * d.hidden + d.hidden * d.n_layers * 2 * d.kv_dim)
    log(f"[bench] prefill of {total} rows: {pms:.2f} ms, {total / pms / 1e3:.2f} M rows/s, "
        f"{pflop / pms / 1e9:.0f} TFLOP/s in the fusion + injection GEMMs")

    # ---- per-step inputs: verified-block features and planted target ids ------------------
    rfeats = [to_device(np.concatenate([inp.round_feats(i, b, 0) for b in range(bt)]), d.dtype, dev_t)
              for i in range(nf)]
    row_start = torch.arange(0, bt * B, B, dtype=torch.int32, device=dev_t)
    rng = make_rng(wl.cfg_id, "bench_targets")
    mean = wl.accept_mean if wl.accept_mean is not None else 1.5
    p = 1.0 / (mean + 1.0)
    kk = np.minimum(rng.geometric(p, size=(n_rounds, bt)) - 1, B - 1)
    idx = np.arange(B - 1)[None, None, :]
    match = torch.from_numpy(idx < kk[:, :, None]).to(dev_t)                     # [R, bt, B-1]
    alt = torch.from_numpy(rng.integers(0, d.vocab - 1, size=(n_rounds, bt, B - 1)).astype(np.int32)).to(dev_t)
    tgt = torch.from_numpy(rng.integers(0, d.vocab - 1, size=(bt, B)).astype(np.int32)).to(dev_t)
    ids = torch.zeros(bt, B - 1, dtype=torch.int32, device=dev_t)
    acc = torch.zeros(bt, dtype=torch.int32, device=dev_t)
    x0 = torch.from_numpy(inp.x0()).to(dev_t)
    state = {"r": 0}

    def step(timer=None, itimer=None, r=None):
        if r is None:
            r = state["r"]
            state["r"] = r + 1
        dev.draft(x0, B, ids, timer=timer, temperature=args.temperature, seed=1234, offset=r)
        torch.where(match[r], ids, alt[r], out=tgt[:, :B - 1])    # stand-in for the target
        dev.accept_trim(ids, tgt, B, acc, x0)                    # bonus -> next x0
        if args.fusion == "input":  # the ablation: the drafter's own causal pass over the rows
            dev.fuse_inject_input(rfeats, row_start, acc, B, bt * B)
        else:
            dev.fuse_inject(rfeats, row_start, acc, bt * B, timer=itimer or timer)

    def draft_only(r=0):
        dev.draft(x0, B, ids, temperature=args.temperature, seed=1234, offset=r)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(dev.err.item()) == 0, f"device error bits {int(dev.err.item())}"

    def timed(n, timer=None):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            step(timer)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    G = graph_len(args.steps)

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(G):
                fn(r=n_rounds - G + i)
        torch.cuda.synchronize()
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        assert int(dev.err.item()) == 0, f"device error bits {int(dev.err.item())}"
        return g

    def timed_graph(g, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n // G):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # Every timed phase starts from the workload's contexts (each step appends the
    # accepted rows, so without a reset later phases would read longer caches); the
    # bytes a phase reads are counted at its mean context, (start + end) / 2.
    ctx0 = torch.from_numpy(ctx.astype(np.int32)).to(dev_t)

    def phase(fn):
        dev.len.copy_(ctx0)
        torch.cuda.synchronize()
        l0 = float(dev.len.float().mean())
        out = fn()
        torch.cuda.synchronize()
        return out, 0.5 * (l0 + float(dev.len.float().mean()))

    def timed_drafts(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(n):
            draft_only(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    graph = None if args.eager else capture(step)
    if graph is not None:
        ms, ctx_step = phase(lambda: timed_graph(graph, args.steps))
    else:
        ms, ctx_step = phase(lambda: timed(args.steps))
    # the draft alone (embedding, every layer, final norm, lm_head and argmax)
    if graph is not None:
        dgraph = capture(lambda r: draft_only(r))
        ms_draft, ctx_draft = phase(lambda: timed_graph(dgraph, args.steps))
    else:
        ms_draft, ctx_draft = phase(lambda: timed_drafts(args.steps))
    if args.profile_only:
        log(f"[bench] {ms:.3f} ms/step, draft {ms_draft:.3f} ms")
        if args.copy_calibration:
            a = torch.empty(1 << 30, dtype=torch.uint8, device=dev_t)
            b2 = torch.empty_like(a)
            for _ in range(3):
                b2.copy_(a)
            torch.cuda.synchronize()
        return {}

    # ---- per-kernel durations with library-recorded events over timed runs -----------------
    launches = gemm_launches(d, bt, B, bt * B)
    if args.fusion == "input":  # the ablation's injection is not event-timed: draft GEMMs only
        launches = launches[2:]
    nl = len(launches)
    ms_eager = phase(lambda: timed(args.steps))[0] if graph is not None else ms
    gt = LaunchTimer(Bn.DFLASH_TIME_GEMM, nl * args.steps)
    ms_ev = phase(lambda: timed(args.steps, gt))[0]
    gd = gt.durations_ms()
    lt = LaunchTimer(Bn.DFLASH_TIME_LMHEAD, args.steps)
    phase(lambda: timed(args.steps, lt))
    ld = lt.durations_ms()
    at = LaunchTimer(Bn.DFLASH_TIME_ATTN, d.n_layers * args.steps)
    _, ctx_attn = phase(lambda: timed(args.steps, at))
    ad = at.durations_ms()
    assert int(dev.err.item()) == 0, f"device error bits {int(dev.err.item())}"

    es = 2 if d.dtype == "bf16" else 4
    acc_mean = float(np.mean(kk[:, :] + 1))
    # GEMM launches are recorded in step order: the draft's 4 per layer, then
    # fuse_inject's fusion and injection.  One class per GEMM shape.  The re-injection
    # GEMMs run over every row slot of the batch (the accepted counts live on the
    # device), but their algorithmic work is the accepted rows only: counted at the
    # run's mean accepted rows per sequence.
    counted = gemm_launches(d, bt, B, bt * acc_mean)
    if args.fusion == "input":
        counted = counted[2:]
    order = counted if args.fusion == "input" else counted[2:] + counted[:2]
    classes = {}
    for i, dms in enumerate(gd):
        name, M, N, K = order[i % len(order)]
        c = classes.setdefault("gemm_" + name, {"ms": [], "bytes": gemm_bytes(M, N, K, es),
                                                "flops": 2.0 * M * N * K})
        c["ms"].append(dms)
    lm_bytes = d.vocab * d.hidden * es + bt * (B - 1) * d.hidden * es
    classes["lm_head_argmax"] = {"ms": ld, "bytes": lm_bytes,
                                 "flops": 2.0 * bt * (B - 1) * d.vocab * d.hidden}
    kv_row = 2 * d.kv_dim * es
    attn_bytes = bt * (ctx_attn + B) * kv_row      # per layer: the K/V read once
    classes["attention_split"] = {"ms": ad, "bytes": attn_bytes,
                                  "flops": 4.0 * bt * B * d.n_q_heads * d.head_dim * (ctx_attn + B)}
    for k, c in classes.items():
        avg = float(np.mean(c.pop("ms")))
        c["avg_launch_us"] = avg * 1e3
        c["GBps"] = c["bytes"] / (avg * 1e-3) / 1e9
        c["TFLOPs"] = c["flops"] / (avg * 1e-3) / 1e12
    for k, c in classes.items():
        per = d.n_layers if (k.startswith("gemm_") and k not in ("gemm_fusion", "gemm_injection")) \
            or k == "attention_split" else 1
        c["launches_per_step"] = per
        c["ms_per_step"] = c["avg_launch_us"] * per / 1e3
    batched = bt * B >= 256
    # the matrix cores' share of a batched step: every projection GEMM and the lm_head,
    # their flops over their summed event time per step
    gemm_f = sum(2.0 * M * N * K for (_, M, N, K) in counted)   # the event-timed GEMMs
    lm_f = 2.0 * bt * (B - 1) * d.vocab * d.hidden
    mm_ms = sum(c["ms_per_step"] for k, c in classes.items() if k.startswith("gemm_")) \
        + classes["lm_head_argmax"]["ms_per_step"]
    mm_tf = (gemm_f + lm_f) / (mm_ms * 1e-3) / 1e12
    mfma = {"bound": "mfma", "kernel": "gemm_mfma + lmhead_mfma (every projection and the lm_head)",
            "achieved": round(mm_tf, 1), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(mm_tf / MFMA_F16_PEAK_TFLOPS, 4), "ms_per_step": round(mm_ms, 4),
            "flops_per_step": gemm_f + lm_f}
    ac = classes["attention_split"]
    attn = {"bound": "hbm", "kernel": "attention_split", "achieved": round(ac["GBps"], 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ac["GBps"] / HBM_PEAK_GBS, 4),
            "ms_per_step": round(ac["ms_per_step"], 4),
            "traffic": profiled_traffic(wl.name, "attention_split")}
    if batched:
        # HBM bytes of every matrix-core GEMM and the lm_head per step
        mfma["traffic"] = profiled_traffic(wl.name, "mfma_step")
        roofline = dict(mfma)
    else:
        dom = max(classes, key=lambda k: classes[k]["ms_per_step"])
        dc = classes[dom]
        roofline = {"bound": "hbm", "kernel": dom, "achieved": round(dc["GBps"], 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dc["GBps"] / HBM_PEAK_GBS, 4),
                    "traffic": profiled_traffic(wl.name, dom)}
    sb = step_bytes(d, bt, B, ctx_step, acc_mean, input_fusion=args.fusion == "input")
    db = draft_bytes(d, bt, B, ctx_draft)
    step_gbs = sb / (ms * 1e-3) / 1e9
    draft_gbs = db / (ms_draft * 1e-3) / 1e9
    value = bt / (ms * 1e-3)
    log(f"[bench] {ms:.3f} ms/step graph ({args.steps} steps in graphs of {G}), draft alone "
        f"{ms_draft:.3f} ms, {ms_eager:.3f} eager ({ms_ev:.3f} with GEMM events); classes "
        + ", ".join(f"{k} {v['avg_launch_us']:.1f} us x {v['launches_per_step']}" for k, v in classes.items()))

    cpu = None
    if with_cpu:
        cpu = cpu_baseline(wl, inp, host_w, ctx, cpu_seconds, args.temperature,
                           input_fusion=args.fusion == "input")
    del dev
    torch.cuda.empty_cache()
    return {
        "value": round(value, 2),
        "unit": "blocks/s",
        "ms_per_step": round(ms, 4),
        "ms_per_draft": round(ms_draft, 4),
        "draft_blocks_per_s": round(bt / (ms_draft * 1e-3), 2),
        "draft_tokens_per_s": round(value * (B - 1), 1),
        "config": {"workload": wl.name, "batch": bt, "block": B, "ctx": int(np.mean(ctx)),
                   "ctx_range": [int(ctx.min()), int(ctx.max())],
                   "ctx_mean_timed": round(ctx_step, 1),
                   "layers": d.n_layers, "hidden": d.hidden, "heads": [d.n_q_heads, d.n_kv_heads],
                   "head_dim": d.head_dim, "inter": d.inter, "vocab": d.vocab,
                   "parallelism": "single GPU",
                   "draft": f"sampled, temperature {args.temperature}" if args.temperature > 0
                   else "greedy",
                   "injection": "input fusion (ablation)" if args.fusion == "input"
                   else "per-layer K/V"},
        "roofline": roofline,
        "mfma_roofline": mfma,
        "attention_roofline": attn,
        "step_roofline": {"bound": "hbm", "bytes_per_step": sb, "achieved": round(step_gbs, 1),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(step_gbs / HBM_PEAK_GBS, 4)},
        "draft_roofline": {"bound": "hbm", "bytes_per_draft": db, "achieved": round(draft_gbs, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(draft_gbs / HBM_PEAK_GBS, 4)},
        "kernels": {k: {kk2: (round(v2, 3) if isinstance(v2, float) else v2) for kk2, v2 in v.items()}
                    for k, v in sorted(classes.items(), key=lambda kv: -kv[1]["ms_per_step"])},
        "launch": "hip graph replay" if graph is not None else "eager",
        "ms_per_step_eager": round(ms_eager, 4),
        "event_overhead_pct": round(100.0 * (ms_ev - ms_eager) / ms_eager, 2),
        "mean_accept_len": round(acc_mean, 3),
        # (round, sequence) pairs of the run's planted prefixes by accepted length 1..B,
        # the draws mean_accept_len averages (the target is stood in for)
        "accept_len_hist": np.bincount((kk + 1).ravel(), minlength=B + 1)[1:].tolist(),
        "prefill": {"rows": total, "ms": round(pms, 3), "tflops": round(pflop / pms / 1e9, 1)},
        "cpu_baseline": cpu,
    }


def measured_ceilings() -> dict:
    """Secondary denominators measured on this GPU in the same run, beside the published
    peaks: a streaming read (torch row sums of 2 GiB of fp16, 4096 per row, into fp32: the
    fastest of the torch reductions tried, 6.4 TB/s against 3.6 for a 1-D sum), a device
    copy (1 GiB read + 1 GiB written), a large library GEMM (torch.matmul of two
    8192 x 8192 fp16 matrices, which ROCm's torch runs through hipBLASLt) and a library
    GEMM of the batch-1 shape (16 rows times a 4096 x 262144 fp16 matrix, 2 GiB)."""
    import torch

    def seconds(fn, reps):
        fn()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        t1.synchronize()
        return t0.elapsed_time(t1) / reps * 1e-3

    n = 1 << 30
    x = torch.full((n,), 1.0, dtype=torch.float16, device="cuda")
    rows = x.view(-1, 4096)
    read_gbs = 2 * n / seconds(lambda: rows.sum(1, dtype=torch.float32), 10) / 1e9
    z = torch.full((16, 4096), 1.0, dtype=torch.float16, device="cuda")
    wide = x.view(4096, -1)
    skinny_gbs = 2 * n / seconds(lambda: torch.matmul(z, wide), 10) / 1e9
    y = torch.empty(n // 2, dtype=torch.float16, device="cuda")
    half = x[: n // 2]
    copy_gbs = 2 * n / seconds(lambda: y.copy_(half), 10) / 1e9  # bytes read + written
    del x, y, half, rows, wide, z
    m = 8192
    a = torch.randn(m, m, dtype=torch.float16, device="cuda")
    b = torch.randn(m, m, dtype=torch.float16, device="cuda")
    gemm_tf = 2.0 * m ** 3 / seconds(lambda: torch.matmul(a, b), 10) / 1e12
    del a, b
    torch.cuda.empty_cache()
    return {"stream_read_GBps": round(read_gbs, 1), "copy_GBps": round(copy_gbs, 1),
            "library_gemm_TFLOPs": round(gemm_tf, 1),
            "library_16_row_gemm_GBps": round(skinny_gbs, 1),
            "how": "torch row sums of 2 GiB fp16 (read); copy_ of 1 GiB fp16 (read + write "
                   "bytes); torch.matmul fp16 8192^3 (hipBLASLt); torch.matmul fp16 16 x 4096 "
                   "by 4096 x 262144 (matrix bytes)"}


def frac_of_measured(roof: dict, ceil: dict):
    """The roofline's achieved rate over the measured ceiling of its kind."""
    den = ceil["stream_read_GBps"] if roof.get("unit") == "GB/s" else ceil["library_gemm_TFLOPs"]
    return round(roof["achieved"] / den, 4) if den > 0 else None


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=48)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, help="workload id (2 = the metric's batch-1 case)")
    ap.add_argument("--block", type=int, default=0,
                    help="block size override (2..16; default: the workload's)")
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="> 0: sampled drafts (Gumbel-max, dflash_draft_block_sampled)")
    ap.add_argument("--fusion", choices=("kv", "input"), default="kv",
                    help="injection of the accepted rows: per-layer K/V (the method) or the "
                         "input-fusion ablation (dflash_fuse_inject_input)")
    ap.add_argument("--no-batch32", action="store_true",
                    help="skip the metric's batch-32 record (workload 3) of the default run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--profile-only", action="store_true",
                    help="warmup + timed steps only (for rocprofv3 runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of replaying a captured HIP graph")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU (sequences shard across GPUs with no collective); run with --gpus 1",
                          "n_gpus": args.gpus}))
        return 2
    if args.steps < 1:
        print(json.dumps({"error": "--steps must be >= 1"}))
        return 2

    import torch
    from synth.configs import CONFIGS

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wl = CONFIGS[args.config]
    if args.block:
        if not 2 <= args.block <= wl.dims.block_max:
            print(json.dumps({"error": f"--block must be in [2, {wl.dims.block_max}]"}))
            return 2
        wl = wl.replace(block=args.block)
    with_cpu = not (args.no_cpu_baseline or args.profile_only)
    rec = run_workload(wl, args, args.cpu_seconds, with_cpu)
    if args.profile_only:
        if args.config == 2 and not args.no_batch32 and not args.block:
            run_workload(CONFIGS[3], args, 0.0, False)
        return 0
    # the metric's batch-32 half: the same drafter at batch 32, ragged contexts
    b32 = None
    if args.config == 2 and not args.no_batch32 and not args.block and args.fusion == "kv":
        b32 = run_workload(CONFIGS[3], args, min(8.0, args.cpu_seconds), with_cpu)
    d = wl.dims
    res = {
        "metric": METRIC,
        "value": rec["value"],
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16" if d.dtype == "bf16" else "f32",
        "arithmetic": ("bf16 storage (weights, features, embedding, gains); fp16 matrix-core "
                       "operands and K/V cache; fp32 accumulation, residual, norms and softmax")
        if d.dtype == "bf16" else "fp32 throughout",
        "data": "synthetic",
    }
    res.update({k: v for k, v in rec.items() if k not in ("value", "unit", "ms_per_step")})
    if b32 is not None:
        res["batch32"] = b32
    if d.dtype == "bf16":
        ceil = measured_ceilings()
        for r in [res] + ([b32] if b32 is not None else []):
            for k in ("roofline", "mfma_roofline", "attention_roofline"):
                if r.get(k):
                    r[k]["frac_of_measured"] = frac_of_measured(r[k], ceil)
        res["measured_ceilings"] = ceil
    print(json.dumps(res))
    return 0


_CSRC = "block_diffusion_drafter_layers_amd/csrc/"
KERNEL_SOURCES = tuple(_CSRC + f for f in ("common.h", "mfma_tile.h", "gemm.hip", "lmhead.hip",
                                           "attention.hip"))
# the sources each kernel class is built from (a traffic figure stays valid while
# they are unchanged)
CLASS_SOURCES = {
    "lm_head": ("common.h", "mfma_tile.h", "lmhead.hip"),
    "attention": ("common.h", "attention.hip"),
    "gemm": ("common.h", "mfma_tile.h", "gemm.hip"),
    # every matrix-core GEMM and the lm_head of one batched step, summed
    "mfma_step": ("common.h", "mfma_tile.h", "gemm.hip", "lmhead.hip"),
}


def class_sources(kernel_class: str):
    for prefix, files in CLASS_SOURCES.items():
        if kernel_class.startswith(prefix):
            return tuple(_CSRC + f for f in files)
    return KERNEL_SOURCES


def code_only(text: str) -> str:
    """C++ source without its comments and with runs of white space as one blank, so
    that an edit of comments alone keeps a kernel's hash."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return re.sub(r"\s+", " ", text).strip()


def kernel_source_hash(kernel_class: str = None) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in (class_sources(kernel_class) if kernel_class else KERNEL_SOURCES):
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            h.update(code_only(fh.read()).encode("utf-8"))
    return h.hexdigest()[:16]


def profiled_traffic(workload: str, kernel_class: str):
    """HBM bytes per launch of `kernel_class` measured with rocprofv3 FETCH_SIZE and
    WRITE_SIZE counters (calibrated on a plain device copy), as recorded in
    profiles/traffic_<workload>.txt; None when absent or when the class's kernel
    sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get(f"source_hash.{kernel_class}") != kernel_source_hash(kernel_class):
        return None
    v = rec.get(f"traffic_bytes.{kernel_class}")
    return float(v) if v else None


def cpu_baseline(wl, inp, host_w, ctx, seconds, temperature=0.0, input_fusion=False):
    """The oracle as it stands, timed on the host: rounds of draft + accept/trim +
    re-injection for batch 1 (sequence 0) after injecting its context."""
    import threadpoolctl
    from oracle.dflash_oracle import OracleDrafter
    from synth.inputs import bf16_bits_to_f32
    d = wl.dims
    t0 = time.time()
    conv = (lambda a: bf16_bits_to_f32(a)) if d.dtype == "bf16" else (lambda a: a)
    w = {n: conv(a) for n, a in host_w.items()}
    ora = OracleDrafter(d, w, 1, dtype=np.float32)
    del w
    L = int(ctx[0])
    inject = ora.fuse_inject_input if input_fusion else ora.fuse_inject
    inject(0, [conv(inp.ctx_feats(i, 0, n_rows=L)) for i in range(d.n_feat_layers)])
    setup = time.time() - t0
    x0 = [int(inp.x0()[0])]
    n = 0
    t1 = time.time()
    while True:
        r = ora.draft(x0, wl.block, temperature=temperature, seed=1234, offset=n)
        tg = inp.targets_for(r["draft_ids"][:1], n, k=inp.prefix_lengths(n)[:1])
        a, bo = ora.accept_trim(r["draft_ids"][:1], tg)
        rf = [conv(inp.round_feats(i, 0, n))[:a[0]] for i in range(d.n_feat_layers)]
        inject(0, rf)
        x0 = [int(bo[0])]
        n += 1
        if time.time() - t1 >= seconds:
            break
    el = time.time() - t1
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    log(f"[bench] oracle: setup {setup:.1f}s, {n} rounds in {el:.1f}s")
    return {"value": round(n / el, 4), "unit": "blocks/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} rounds (draft + accept/trim + re-injection) of sequence 0 at batch 1, "
                      f"context {L}, fp32 numpy, after injecting its context",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model(), "blas": blas_name()}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_name() -> str:
    try:
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        return f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:  # numpy builds without the dict form
        return "unknown"


if __name__ == "__main__":
    sys.exit(main())
