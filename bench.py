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

Output: one JSON line with the metric, the whole-step and dominant-kernel
rooflines (HIP events recorded by the library around every launch of the
dominant kernel class during a timed run) and the CPU oracle timed on a
bounded sample of the same workload.
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
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
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


def step_bytes(dims, batch, block, ctx_mean, accept_mean):
    """Algorithmic HBM bytes of one step: every weight the step needs once,
    the K/V the attention reads, the K/V the step writes, activations in/out."""
    d = dims
    es = 2 if d.dtype == "bf16" else 4
    rows_in = int(round(batch * accept_mean))
    b = 0
    for (_, M, N, K) in gemm_launches(d, batch, block, batch * block):
        b += N * K * es                                  # weights
    b += d.vocab * d.hidden * es                         # lm_head
    b += batch * block * d.hidden * es                   # embedding rows
    kv_row = d.n_layers * 2 * d.kv_dim * es
    b += batch * (ctx_mean + block) * kv_row             # attention reads
    b += batch * block * kv_row + rows_in * kv_row       # block K/V + injected K/V writes
    b += rows_in * d.fc_in * es                          # features of the accepted rows
    return b


# ---------------------------------------------------------------------------------------

def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, help="workload id (2 = the metric's batch-1 case)")
    ap.add_argument("--block", type=int, default=0,
                    help="block size override (2..16; default: the workload's)")
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="> 0: sampled drafts (Gumbel-max, dflash_draft_block_sampled)")
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

    import torch
    from block_diffusion_drafter_layers_amd import binding as Bn
    from block_diffusion_drafter_layers_amd.runtime import DeviceDrafter, LaunchTimer, to_device
    from synth.configs import CONFIGS
    from synth.inputs import DrafterInputs, make_rng

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wl = CONFIGS[args.config]
    if args.block:
        if not 2 <= args.block <= wl.dims.block_max:
            print(json.dumps({"error": f"--block must be in [2, {wl.dims.block_max}]"}))
            return 2
        wl = wl.replace(block=args.block)
    d = wl.dims
    B, bt = wl.block, wl.batch
    dev_t = torch.device("cuda:0")
    t0 = time.time()
    inp = DrafterInputs(wl)
    ctx = inp.ctx_lengths()
    n_rounds = args.warmup + 6 * args.steps + 64
    max_ctx = int((ctx.max() + B * (n_rounds + 2) + 63) // 64 * 64)
    names = list(inp.weight_shapes())
    host_w = {n: inp.weight(n) for n in names}
    log(f"[bench] workload {wl.name}: weights generated in {time.time() - t0:.1f}s")
    dev = DeviceDrafter(d, host_w, bt, max_ctx, max(int(ctx.sum()), bt * B))
    if args.no_cpu_baseline or args.profile_only:
        host_w = None
        inp._cache.clear()
    log(f"[bench] uploaded; workspace {dev.ws_bytes / 1e6:.1f} MB, max_ctx {max_ctx}")

    # ---- prefill: inject the whole context ----------------------------------------------
    nf = d.n_feat_layers
    total = int(ctx.sum())
    starts = np.concatenate([[0], np.cumsum(ctx)[:-1]]).astype(np.int32)
    feats = [to_device(np.concatenate([inp.ctx_feats(i, b, n_rows=int(ctx[b])) for b in range(bt)]),
                       d.dtype, dev_t) for i in range(nf)]
    rs_t, rc_t = torch.from_numpy(starts).to(dev_t), torch.from_numpy(ctx.astype(np.int32)).to(dev_t)
    torch.cuda.synchronize()
    pe0, pe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pe0.record()
    dev.fuse_inject(feats, rs_t, rc_t, total)
    pe1.record()
    torch.cuda.synchronize()
    del feats
    pms = pe0.elapsed_time(pe1)
    # fusion (fc_in -> H) and injection (H -> every layer's K and V) GEMM work of the prefill
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
        dev.fuse_inject(rfeats, row_start, acc, bt * B, timer=itimer or timer)

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

    graph = None
    GSTEPS = 8
    if not args.eager:
        # capture GSTEPS consecutive steps (distinct planted targets) into one HIP graph
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(GSTEPS):
                step(r=n_rounds - GSTEPS + i)
        torch.cuda.synchronize()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        assert int(dev.err.item()) == 0, f"device error bits {int(dev.err.item())}"

    def timed_graph(n):
        reps = max(1, n // GSTEPS)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * GSTEPS)

    ms = timed_graph(args.steps) if graph is not None else timed(args.steps)
    ms_eager = timed(args.steps) if graph is not None else ms
    if args.profile_only:
        log(f"[bench] {ms:.3f} ms/step")
        if args.copy_calibration:
            a = torch.empty(1 << 30, dtype=torch.uint8, device=dev_t)
            b2 = torch.empty_like(a)
            for _ in range(3):
                b2.copy_(a)
            torch.cuda.synchronize()
        return 0

    # ---- per-kernel durations with library-recorded events over timed runs -----------------
    launches = gemm_launches(d, bt, B, bt * B)
    nl = len(launches)
    gt = LaunchTimer(Bn.DFLASH_TIME_GEMM, nl * args.steps)
    ms_ev = timed(args.steps, gt)
    gd = gt.durations_ms()
    lt = LaunchTimer(Bn.DFLASH_TIME_LMHEAD, args.steps)
    timed(args.steps, lt)
    ld = lt.durations_ms()
    at = LaunchTimer(Bn.DFLASH_TIME_ATTN, d.n_layers * args.steps)
    timed(args.steps, at)
    ad = at.durations_ms()
    assert int(dev.err.item()) == 0, f"device error bits {int(dev.err.item())}"

    es = 2 if d.dtype == "bf16" else 4
    acc_mean = float(np.mean(kk[:, :] + 1))
    # GEMM launches are recorded in step order: the draft's 4 per layer, then
    # fuse_inject's fusion and injection.  One class per GEMM shape.
    order = launches[2:] + launches[:2]
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
    attn_bytes = bt * (float(np.mean(ctx)) + B) * kv_row      # per layer: the K/V read once
    classes["attention_split"] = {"ms": ad, "bytes": attn_bytes,
                            "flops": 4.0 * bt * B * d.n_q_heads * d.head_dim * (float(np.mean(ctx)) + B)}
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
    dom = max(classes, key=lambda k: classes[k]["ms_per_step"])
    dc = classes[dom]
    mfma_bound = bt * B >= 256 and dom.startswith("gemm_")
    if mfma_bound:
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(dc["TFLOPs"], 1),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(dc["TFLOPs"] / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None}
    else:
        roofline = {"bound": "hbm", "kernel": dom, "achieved": round(dc["GBps"], 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dc["GBps"] / HBM_PEAK_GBS, 4),
                    "traffic": profiled_traffic(wl.name, dom)}
    sb = step_bytes(d, bt, B, float(np.mean(ctx)), acc_mean)
    step_gbs = sb / (ms * 1e-3) / 1e9
    value = bt / (ms * 1e-3)
    log(f"[bench] {ms:.3f} ms/step graph, {ms_eager:.3f} eager ({ms_ev:.3f} with GEMM events); classes "
        + ", ".join(f"{k} {v['avg_launch_us']:.1f} us x {v['launches_per_step']}" for k, v in classes.items()))

    # ---- CPU oracle on a bounded sample of the same workload -------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, inp, host_w, ctx, args.cpu_seconds, args.temperature)

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if d.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": bt, "block": B, "ctx": int(np.mean(ctx)),
                   "layers": d.n_layers, "hidden": d.hidden, "heads": [d.n_q_heads, d.n_kv_heads],
                   "head_dim": d.head_dim, "inter": d.inter, "vocab": d.vocab,
                   "parallelism": "single GPU",
                   "draft": f"sampled, temperature {args.temperature}" if args.temperature > 0
                   else "greedy"},
        "draft_tokens_per_s": round(value * (B - 1), 1),
        "roofline": roofline,
        "step_roofline": {"bound": "hbm", "bytes_per_step": sb, "achieved": round(step_gbs, 1),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(step_gbs / HBM_PEAK_GBS, 4)},
        "kernels": {k: {kk2: (round(v2, 3) if isinstance(v2, float) else v2) for kk2, v2 in v.items()}
                    for k, v in sorted(classes.items(), key=lambda kv: -kv[1]["ms_per_step"])},
        "launch": "hip graph replay" if graph is not None else "eager",
        "ms_per_step_eager": round(ms_eager, 4),
        "event_overhead_pct": round(100.0 * (ms_ev - ms_eager) / ms_eager, 2),
        "mean_accept_len": round(acc_mean, 3),
        "cpu_baseline": cpu,
    }
    print(json.dumps(res))
    return 0


KERNEL_SOURCES = ("block_diffusion_drafter_layers_amd/csrc/common.h",
                  "block_diffusion_drafter_layers_amd/csrc/mfma_tile.h",
                  "block_diffusion_drafter_layers_amd/csrc/gemm.hip",
                  "block_diffusion_drafter_layers_amd/csrc/lmhead.hip",
                  "block_diffusion_drafter_layers_amd/csrc/attention.hip")


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(workload: str, kernel_class: str):
    """HBM bytes per launch of `kernel_class` measured with rocprofv3 FETCH_SIZE and
    WRITE_SIZE counters (calibrated on a plain device copy), as recorded in
    profiles/traffic_<workload>.txt; None when absent or when the kernel sources
    have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("source_hash") != kernel_source_hash():
        return None
    v = rec.get(f"traffic_bytes.{kernel_class}")
    return float(v) if v else None


def cpu_baseline(wl, inp, host_w, ctx, seconds, temperature=0.0):
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
    ora.fuse_inject(0, [conv(inp.ctx_feats(i, 0, n_rows=L)) for i in range(d.n_feat_layers)])
    setup = time.time() - t0
    x0 = [int(inp.x0()[0])]
    n = 0
    t1 = time.time()
    while True:
        r = ora.draft(x0, wl.block, temperature=temperature, seed=1234, offset=n)
        tg = inp.targets_for(r["draft_ids"][:1], n, k=inp.prefix_lengths(n)[:1])
        a, bo = ora.accept_trim(r["draft_ids"][:1], tg)
        rf = [conv(inp.round_feats(i, 0, n))[:a[0]] for i in range(d.n_feat_layers)]
        ora.fuse_inject(0, rf)
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
            "host_cpus": os.cpu_count()}


if __name__ == "__main__":
    sys.exit(main())
