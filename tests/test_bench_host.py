"""Host logic of bench.py: the algorithmic work it divides by measured time, the
HBM-traffic record lookup, and the single-GPU refusal.  No GPU is touched."""

import json
import os
import subprocess
import sys

import pytest

import bench
from synth.configs import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_projection_shapes_of_the_batch1_qwen3_8b_shape_step():
    """One step is fusion + injection, then QKV, O, gate|up and down per layer,
    with the shapes of a 4096-wide GQA layer (32 query and 8 KV heads of 128)."""
    d = CONFIGS[2].dims
    ls = bench.gemm_launches(d, batch=1, block=16, inject_rows=16)
    assert len(ls) == 2 + 4 * 5
    assert ls[0] == ("fusion", 16, 4096, 5 * 4096)
    assert ls[1] == ("injection", 16, 5 * 2 * 8 * 128, 4096)
    per_layer = ls[2:6]
    assert per_layer == [("qkv", 16, 32 * 128 + 2 * 8 * 128, 4096), ("o", 16, 4096, 32 * 128),
                         ("gate_up", 16, 2 * 12288, 4096), ("down", 16, 4096, 12288)]
    assert ls[2:6] * 5 == ls[2:]


def test_weight_bytes_per_kernel_class():
    """bf16 weights read once per launch: 50.3 MB QKV, 33.6 MB O, 201.3 MB gate|up,
    100.7 MB down, plus the 16 input and output rows."""
    es = 2
    assert bench.gemm_bytes(16, 6144, 4096, es) == 6144 * 4096 * 2 + 16 * (4096 + 6144) * 2
    assert bench.gemm_bytes(16, 4096, 4096, es) - 16 * 8192 * 2 == 33_554_432
    assert bench.gemm_bytes(16, 24576, 4096, es) - 16 * (4096 + 24576) * 2 == 201_326_592
    assert bench.gemm_bytes(16, 4096, 12288, es) - 16 * (12288 + 4096) * 2 == 100_663_296


def test_step_bytes_batch1_qwen3_8b_shape():
    """Every weight once (5 layers, fusion, injection, the 151 936 x 4096 lm_head), the
    embedding rows, the context's K/V read by attention, the block's and the accepted
    rows' K/V written and the accepted rows' target features read."""
    d = CONFIGS[2].dims
    es, H, kv = 2, 4096, 8 * 128
    layer_w = (H * (4096 + 2 * kv) + 4096 * H + H * 2 * 12288 + 12288 * H) * es
    fuse_w = 5 * H * H * es + H * 5 * 2 * kv * es
    lm = 151936 * H * es
    kv_row = 5 * 2 * kv * es
    acc = 6                                       # 1 sequence x 6.4 accepted rows
    want = (5 * layer_w + fuse_w + lm + 16 * H * es + (1024 + 16) * kv_row
            + 16 * kv_row + acc * kv_row + acc * 5 * H * es)
    assert bench.step_bytes(d, 1, 16, 1024.0, 6.4) == want
    assert 3.40e9 < want < 3.50e9


def test_traffic_record_needs_matching_sources(tmp_path, monkeypatch):
    """A traffic figure is reported only while its class's kernel sources hash as recorded."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    for f in bench.KERNEL_SOURCES:
        dst = tmp_path / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_bytes(open(os.path.join(ROOT, f), "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    hl = bench.kernel_source_hash("lm_head_argmax")
    ha = bench.kernel_source_hash("attention_split")
    assert hl != ha
    (prof / "traffic_w.txt").write_text(
        f"# test\nsource_hash.lm_head_argmax: {hl}\ntraffic_bytes.lm_head_argmax: 1234.5\n"
        f"source_hash.attention_split: {ha}\ntraffic_bytes.attention_split: 99.0\n"
        f"source_hash.gemm_o: {hl}\ntraffic_bytes.gemm_o: 7.0\n")
    assert bench.profiled_traffic("w", "lm_head_argmax") == 1234.5
    assert bench.profiled_traffic("w", "attention_split") == 99.0
    assert bench.profiled_traffic("w", "gemm_o") is None          # recorded for other sources
    assert bench.profiled_traffic("w", "gemm_down") is None       # not recorded
    assert bench.profiled_traffic("absent", "lm_head_argmax") is None
    # comments and white space do not count
    src = tmp_path / (bench._CSRC + "attention.hip")
    src.write_bytes(src.read_bytes() + b"\n// a note\n/* and\n another */\n\n")
    assert bench.profiled_traffic("w", "attention_split") == 99.0
    # an attention change voids the attention figure only; a shared header voids both
    src.write_bytes(src.read_bytes() + b"\nstatic int probe_value = 1;\n")
    assert bench.profiled_traffic("w", "attention_split") is None
    assert bench.profiled_traffic("w", "lm_head_argmax") == 1234.5
    src = tmp_path / (bench._CSRC + "common.h")
    src.write_bytes(src.read_bytes() + b"\nstatic int probe_value = 1;\n")
    assert bench.profiled_traffic("w", "lm_head_argmax") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_graph_length_divides_the_timed_steps():
    """Replays time exactly K steps: graphs hold a divisor of K (at most 16)."""
    for k in (1, 7, 13, 16, 20, 48, 50, 97, 1000):
        g = bench.graph_len(k)
        assert 1 <= g <= 16 and k % g == 0
    assert bench.graph_len(20) == 10 and bench.graph_len(48) == 16 and bench.graph_len(17) == 1


def test_draft_bytes_leave_out_the_injection():
    """The draft alone reads every layer weight and the lm_head once, the context and
    block K/V, and writes the block's K/V; no fusion or injection weights."""
    d = CONFIGS[2].dims
    es, H, kv = 2, 4096, 8 * 128
    fuse_w = 5 * H * H * es + H * 5 * 2 * kv * es
    sb = bench.step_bytes(d, 1, 16, 1024.0, 6.4)
    acc = 6
    kv_row = 5 * 2 * kv * es
    assert bench.draft_bytes(d, 1, 16, 1024.0) == sb - fuse_w - acc * kv_row - acc * 5 * H * es
    assert 3.19e9 < bench.draft_bytes(d, 1, 16, 1024.0) < 3.21e9


def test_batched_flops_count_every_projection_and_the_head():
    d = CONFIGS[3].dims
    g, lm = bench.gemm_flops_per_step(d, 32, 16, 512)
    per_layer = 2 * 512 * 4096 * (6144 + 4096 + 2 * 12288 + 4096)   # K = 4096 except down
    per_layer += 2 * 512 * 4096 * 12288 - 2 * 512 * 4096 * 4096      # down: K = 12288, N = 4096
    inject = 2 * 512 * (20480 * 4096 + 4096 * 10240)
    assert g == 5 * per_layer + inject
    assert lm == 2 * 32 * 15 * 151936 * 4096


def test_frac_of_measured_picks_the_ceiling_of_the_roofline_kind():
    ceil = {"stream_read_GBps": 6000.0, "copy_GBps": 5000.0, "library_gemm_TFLOPs": 1250.0}
    assert bench.frac_of_measured({"unit": "GB/s", "achieved": 4500.0}, ceil) == 0.75
    assert bench.frac_of_measured({"unit": "TFLOP/s", "achieved": 1000.0}, ceil) == 0.8
    assert bench.frac_of_measured({"unit": "GB/s", "achieved": 1.0},
                                  dict(ceil, stream_read_GBps=0.0)) is None


def test_host_description_for_the_cpu_baseline():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()
    assert isinstance(bench.blas_name(), str) and bench.blas_name()
