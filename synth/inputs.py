"""Seeded synthetic inputs: weights, target-layer features, token ids, planted targets.

Every tensor is drawn from its own numpy PCG64 stream keyed by
``[SEED, cfg_id, crc32(name), chunk...]`` so that any slice of a large tensor
can be regenerated on its own, independent of thread count.  bf16 workloads
are rounded to bf16 on the host (round-to-nearest-even) and the *bits* are
kept, so the oracle and the HIP library see bit-identical values.

Value recipe (the workload descriptions fix it):
  * weight matrices (Linear layers, embedding, lm_head): N(0, 0.02)
  * RMSNorm gains: U(0.5, 1.5) by default, or all ones (``gain_mode="unit"``)
  * target-layer features: N(0, 1)
  * token ids: uniform over the ordinary ids [0, vocab-2] (vocab-1 is the mask id)
"""

from __future__ import annotations

import os
import zlib
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence

import numpy as np

from .configs import Workload

SEED = 1234
_CHUNK_ELEMS = 1 << 22


def make_rng(cfg_id: int, name: str, *extra: int) -> np.random.Generator:
    key = [SEED, int(cfg_id), zlib.crc32(name.encode("utf-8"))] + [int(e) for e in extra]
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _workers() -> int:
    env = os.environ.get("DFLASH_SYNTH_THREADS")
    if env:
        return max(1, int(env))
    return max(1, min(16, os.cpu_count() or 1))


def target_layer_ids(n_target_layers: int, n_feat: int = 5) -> List[int]:
    """Target layers whose hidden states are fused: evenly spread, shallow to deep,
    from layer 2 to the third-from-last layer (0-based), floor rounding (reading R1).
    Metadata only: the features themselves are synthetic."""
    lo, hi = 2, n_target_layers - 3
    if n_feat == 1:
        return [lo]
    return [lo + (i * (hi - lo)) // (n_feat - 1) for i in range(n_feat)]


def geometric_prefix_lengths(rng: np.random.Generator, mean: float, cap: int, size: int) -> np.ndarray:
    """Planted matching-prefix lengths k >= 0 with the given mean before capping
    (geometric on {0, 1, ...}, p = 1/(mean+1)), then capped at ``cap`` (reading R16)."""
    p = 1.0 / (mean + 1.0)
    k = rng.geometric(p, size=size) - 1
    return np.minimum(k, cap).astype(np.int32)


def planted_targets(drafts: np.ndarray, k: np.ndarray, vocab: int, rng: np.random.Generator) -> np.ndarray:
    """Synthetic target ids that agree with ``drafts`` on exactly the first k[b]
    positions (reading R15).

    drafts: [batch, B-1] int; k: [batch] in [0, B-1].  Returns [batch, B] int32:
    t[i] = d[i] for i < k; t[k] != d[k] when k < B-1; the rest uniform over the
    ordinary ids [0, vocab-2]."""
    drafts = np.asarray(drafts, dtype=np.int64)
    batch, bm1 = drafts.shape
    t = rng.integers(0, vocab - 1, size=(batch, bm1 + 1), dtype=np.int64)
    for b in range(batch):
        kb = int(k[b])
        assert 0 <= kb <= bm1
        t[b, :kb] = drafts[b, :kb]
        if kb < bm1:
            d = int(drafts[b, kb])
            if 0 <= d <= vocab - 2:
                u = int(rng.integers(0, vocab - 2))
                t[b, kb] = (d + 1 + u) % (vocab - 1)
            # a draft equal to the mask id never matches an ordinary id
    return t.astype(np.int32)


class DrafterInputs:
    """Lazily generated, cached synthetic tensors for one workload.

    ``weight(name)`` returns bf16 bits (uint16) for bf16 workloads and float32
    for the fp32 workload; ``weight_f32(name)`` always returns float32 values.
    Weight names: embed, fc, fc_norm, final_norm, lm_head and, per layer l,
    ``l{l}.in_norm, l{l}.wq, l{l}.wk, l{l}.wv, l{l}.wo, l{l}.post_norm,
    l{l}.w_gate, l{l}.w_up, l{l}.w_down``.  Linear weights are [out, in]."""

    def __init__(self, wl: Workload, gain_mode: str = "uniform", threads: Optional[int] = None):
        assert gain_mode in ("uniform", "unit")
        self.wl = wl
        self.dims = wl.dims
        self.gain_mode = gain_mode
        self.threads = threads or _workers()
        self._cache: Dict[str, np.ndarray] = {}

    # ---- shapes -------------------------------------------------------------
    def weight_shapes(self) -> Dict[str, tuple]:
        d = self.dims
        s = {
            "embed": (d.vocab, d.hidden),
            "fc": (d.hidden, d.fc_in),
            "fc_norm": (d.hidden,),
            "final_norm": (d.hidden,),
            "lm_head": (d.vocab, d.hidden),
        }
        for l in range(d.n_layers):
            s[f"l{l}.in_norm"] = (d.hidden,)
            s[f"l{l}.wq"] = (d.q_dim, d.hidden)
            s[f"l{l}.wk"] = (d.kv_dim, d.hidden)
            s[f"l{l}.wv"] = (d.kv_dim, d.hidden)
            s[f"l{l}.wo"] = (d.hidden, d.q_dim)
            s[f"l{l}.post_norm"] = (d.hidden,)
            s[f"l{l}.w_gate"] = (d.inter, d.hidden)
            s[f"l{l}.w_up"] = (d.inter, d.hidden)
            s[f"l{l}.w_down"] = (d.hidden, d.inter)
        return s

    @staticmethod
    def is_gain(name: str) -> bool:
        return name.endswith("norm")

    # ---- generation ---------------------------------------------------------
    def _store(self, x32: np.ndarray) -> np.ndarray:
        if self.dims.dtype == "bf16":
            return f32_to_bf16_bits(x32)
        return np.ascontiguousarray(x32, dtype=np.float32)

    def _gen_matrix(self, name: str, shape: tuple, std: float, key: str) -> np.ndarray:
        rows, cols = shape
        rpc = max(1, _CHUNK_ELEMS // cols)
        nchunks = (rows + rpc - 1) // rpc
        out = np.empty(shape, dtype=np.uint16 if self.dims.dtype == "bf16" else np.float32)

        def work(c):
            r0 = c * rpc
            r1 = min(rows, r0 + rpc)
            g = make_rng(self.wl.cfg_id, key, c)
            z = g.standard_normal((r1 - r0, cols), dtype=np.float32)
            z *= np.float32(std)
            out[r0:r1] = self._store(z)

        if nchunks == 1:
            work(0)
        else:
            with ThreadPoolExecutor(self.threads) as ex:
                list(ex.map(work, range(nchunks)))
        return out

    def weight(self, name: str) -> np.ndarray:
        if name in self._cache:
            return self._cache[name]
        shape = self.weight_shapes()[name]
        if self.is_gain(name):
            if self.gain_mode == "unit":
                x = np.ones(shape, dtype=np.float32)
            else:
                x = make_rng(self.wl.cfg_id, name).uniform(0.5, 1.5, size=shape).astype(np.float32)
            w = self._store(x)
        else:
            w = self._gen_matrix(name, shape, 0.02, name)
        self._cache[name] = w
        return w

    def weight_f32(self, name: str) -> np.ndarray:
        w = self.weight(name)
        return bf16_bits_to_f32(w) if self.dims.dtype == "bf16" else w

    def drop(self, name: str) -> None:
        self._cache.pop(name, None)

    # ---- per-sequence data --------------------------------------------------
    def ctx_lengths(self) -> np.ndarray:
        wl = self.wl
        if wl.ctx_range is not None:
            lo, hi = wl.ctx_range
            return make_rng(wl.cfg_id, "ctx").integers(lo, hi + 1, size=wl.batch).astype(np.int32)
        return np.full(wl.batch, wl.ctx, dtype=np.int32)

    def x0(self, round_idx: int = 0) -> np.ndarray:
        v = self.dims.vocab
        return make_rng(self.wl.cfg_id, "x0", round_idx).integers(0, v - 1, size=self.wl.batch).astype(np.int32)

    FEAT_ROWBLOCK = 1024

    def ctx_feats(self, layer_i: int, seq: int, rows: Sequence[int] | None = None,
                  n_rows: Optional[int] = None) -> np.ndarray:
        """Target-layer features for committed context positions of one
        sequence, [n, feat_hidden] (bf16 bits or float32).  Rows are drawn in
        blocks of FEAT_ROWBLOCK so that a sample of rows regenerates cheaply."""
        ht = self.dims.feat_hidden
        if n_rows is None:
            n_rows = int(self.ctx_lengths()[seq])
        if rows is None:
            rows = range(n_rows)
        rows = np.asarray(list(rows), dtype=np.int64)
        out = np.empty((len(rows), ht), dtype=np.uint16 if self.dims.dtype == "bf16" else np.float32)
        blocks = np.unique(rows // self.FEAT_ROWBLOCK)
        for blk in blocks:
            g = make_rng(self.wl.cfg_id, "feat", layer_i, seq, int(blk))
            z = g.standard_normal((self.FEAT_ROWBLOCK, ht), dtype=np.float32)
            zb = self._store(z)
            sel = np.nonzero(rows // self.FEAT_ROWBLOCK == blk)[0]
            out[sel] = zb[rows[sel] - blk * self.FEAT_ROWBLOCK]
        return out

    def round_feats(self, layer_i: int, seq: int, round_idx: int) -> np.ndarray:
        """Target-layer features the target would produce at the B rows of a
        verified block in round ``round_idx`` ([block, feat_hidden])."""
        g = make_rng(self.wl.cfg_id, "feat_round", layer_i, seq, round_idx)
        z = g.standard_normal((self.wl.block, self.dims.feat_hidden), dtype=np.float32)
        return self._store(z)

    def prefix_lengths(self, round_idx: int) -> np.ndarray:
        wl = self.wl
        cap = wl.block - 1
        g = make_rng(wl.cfg_id, "accept_k", round_idx)
        if wl.accept_mean is None:
            return g.integers(0, cap + 1, size=wl.batch).astype(np.int32)
        return geometric_prefix_lengths(g, wl.accept_mean, cap, wl.batch)

    def targets_for(self, drafts: np.ndarray, round_idx: int, k: Optional[np.ndarray] = None) -> np.ndarray:
        if k is None:
            k = self.prefix_lengths(round_idx)
        g = make_rng(self.wl.cfg_id, "targets", round_idx)
        return planted_targets(drafts, k, self.dims.vocab, g)
