"""The five draft-step workloads, as plain shape descriptions.

Dimensions follow the drafter described on the DFlash pages: a few
Transformer layers with grouped-query attention and a SwiGLU MLP, a fusion
Linear over the concatenated hidden states of five target layers, and an
embedding / lm_head shared with the target ("DFlash：drafter 的答案…",
section 设计; "DFlash原理深度剖析", §二.3).  The sizes themselves are workload
choices: a tiny fp32 drafter, a Qwen3-8B-shaped drafter at batch 1 and 32, a
32K-context injection stress and a deeper, wider 8-layer drafter.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class DrafterDims:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    inter: int
    vocab: int
    n_feat_layers: int
    feat_hidden: int
    block_max: int = 16
    rope_theta: float = 1.0e6
    rms_eps: float = 1.0e-6
    dtype: str = "bf16"          # "f32" or "bf16": storage type of weights, activations and cache
    target_layers: int = 36      # depth of the (synthetic) target, metadata only

    @property
    def mask_token_id(self) -> int:
        # A reserved id looked up in the shared embedding marks the masked
        # block positions (reading R7); ordinary ids are drawn below it.
        return self.vocab - 1

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def fc_in(self) -> int:
        return self.n_feat_layers * self.feat_hidden


@dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    dims: DrafterDims
    batch: int
    block: int
    # context lengths: fixed value, or inclusive uniform range (lo, hi)
    ctx: Optional[int] = None
    ctx_range: Optional[Tuple[int, int]] = None
    # planted acceptance: "fixed" (tiny: one case per k), or geometric mean
    accept_mean: Optional[float] = None
    rounds: int = 1
    bulk: bool = False           # config 4: bulk fusion + injection of the whole context
    notes: str = field(default="", compare=False)

    def replace(self, **kw) -> "Workload":
        return replace(self, **kw)


_TINY = DrafterDims(n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                    inter=704, vocab=1024, n_feat_layers=5, feat_hidden=256,
                    block_max=16, dtype="f32", target_layers=36)
_QWEN8B = DrafterDims(n_layers=5, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
                      inter=12288, vocab=151936, n_feat_layers=5, feat_hidden=4096,
                      block_max=16, dtype="bf16", target_layers=36)
_WIDE = DrafterDims(n_layers=8, hidden=5120, n_q_heads=40, n_kv_heads=8, head_dim=128,
                    inter=17408, vocab=151936, n_feat_layers=5, feat_hidden=5120,
                    block_max=16, dtype="bf16", target_layers=64)

CONFIGS = {
    1: Workload(1, "tiny_f32_b4_ctx32", _TINY, batch=1, block=4, ctx=32,
                notes="1 layer, hidden 256, 4/2 heads, head_dim 64, inter 704, vocab 1024; "
                      "planted prefix k in {0..3}"),
    2: Workload(2, "qwen3_8b_shape_bs1_ctx1024", _QWEN8B, batch=1, block=16, ctx=1024,
                accept_mean=6.5, rounds=1),
    3: Workload(3, "qwen3_8b_shape_bs32_ragged512_8192", _QWEN8B, batch=32, block=16,
                ctx_range=(512, 8192), accept_mean=6.5, rounds=8),
    4: Workload(4, "qwen3_8b_shape_bs8_ctx32768_bulk", _QWEN8B, batch=8, block=16,
                ctx=32768, bulk=True, accept_mean=6.5, rounds=1),
    5: Workload(5, "wide_8l_5120_bs64_ctx4096", _WIDE, batch=64, block=16, ctx=4096,
                accept_mean=7.0, rounds=1),
}


def get_workload(cfg_id: int) -> Workload:
    return CONFIGS[int(cfg_id)]
