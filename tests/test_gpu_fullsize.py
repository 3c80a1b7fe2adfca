"""GPU parity at the workloads' full sizes, in the launch configuration bench.py
times.  The oracle runs in fp32 here (host memory); where a full oracle pass is
too slow for a test, outputs are sampled (sequences, cache positions) and the
oracle computes just those."""

import numpy as np
import pytest

from synth.configs import CONFIGS
from tests.gpu_common import build_pair, check_cache, draft_round, log, prefill

pytestmark = pytest.mark.gpu


def test_qwen3_8b_shape_batch1_full():
    """5 layers, hidden 4096, 32/8 heads, head_dim 128, SwiGLU 12288, vocab 151936,
    fusion 20480 -> 4096; context 1024; block 16; three lockstep rounds."""
    import torch
    assert torch.cuda.is_available()
    wl = CONFIGS[2]
    log("[full] cfg batch-1 Qwen3-8B shape: building inputs")
    p = build_pair(wl, max_ctx=1024 + 4 * 16 + 64, oracle_dtype=np.float32)
    log(f"  prefill {prefill(p)}")
    x0 = p.inp.x0()
    for rnd in range(3):
        out = draft_round(p, x0, rnd)
        log(f"  round {rnd}: final_hidden {out['final_hidden']:.2e} logits {out['logits']:.2e} "
            f"ids compared {out['compared_ids']} accept {out['accept_len'].tolist()}")
        x0 = out["bonus"]
    log(f"  cache {check_cache(p)}")
