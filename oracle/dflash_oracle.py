"""CPU oracle for the DFlash draft step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and imports nothing from it.

It is a plain, slow, obviously correct numpy implementation of what the draft
step computes, in the order the DFlash pages describe it.  Floating point is
carried in ``dtype`` (float64 unless the caller asks for float32, which the
large workloads use to fit host memory); matrix products are plain ``@``.

Sources (web pages about DFlash: Block Diffusion for Flash Speculative Decoding):
  [P3] "DFlash：drafter 的答案，早写在 target model 的隐层里" — section 设计
       (Feature Fusion / KV Injection / Parallel Drafting), section 训练 paragraph.
  [P4] "DFlash原理深度剖析：块扩散如何用一次前向并行起草整块token" — §二.1 (the
       mask block), §二.2 (non-causal attention inside the block), §二.3 (what is
       reused from the target), §三 steps 1-3 (draft, verify, accept + trim).
  [P1] "DFlash：块扩散草稿模型实现最高15倍吞吐量提升" — section
       "“目标模型最懂”的洞见" (features injected into every layer's K/V).

Readings where the pages leave a step open (numbered R1-R24; each is listed with
its justification in the design notes of this repository):
  R2 concat order = ascending target layer; R3 no fusion bias; R4 RMSNorm
  x * (mean(x^2) + eps)^-1/2 * g; R5 injected K/V use each layer's own W_k/W_v,
  the fused feature is not re-normalised; R6 rotate-half RoPE with
  inv_freq_i = theta^(-2i/d) at absolute 0-based positions, V not rotated;
  R7 mask token = reserved id vocab-1 in the shared embedding; R8 pre-norm
  residual layer (attention, then SwiGLU MLP), no biases, scale 1/sqrt(d),
  q-head j reads kv-head j // G; R9 final RMSNorm before the shared lm_head;
  R10 block rows 1..B-1 are drafted, row r predicts the token at position L+r;
  R11 target_ids[i] is the target's token for position base+1+i; R12 accept
  the longest matching prefix n, accept_len = n+1, bonus = target_ids[n];
  R13 trim to base + accept_len; R14 sequences are independent; R18 argmax
  ties go to the lowest id; R21 x0 sits at position L (first uncached);
  R24 a sampled draft row takes argmax(logit / T + Gumbel noise), each row on
  its own, with Philox4x32-10 uniforms at counter (id, position, sequence);
  R26 the feature of target layer l is the residual stream leaving layer l;
  R27 in the input-fusion variant the fused feature is the first layer's
  input of its context row, and every layer's context K/V come from the
  drafter's own causal pass over those rows.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


# ----------------------------------------------------------------------------
# Elementary operations
# ----------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis (R4): x / sqrt(mean(x^2) + eps) * g.
    [P4] §二.3 and [P3] 设计/Feature Fusion name an RMSNorm after the fusion Linear."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope_cos_sin(pos: np.ndarray, head_dim: int, theta: float) -> Tuple[np.ndarray, np.ndarray]:
    """Rotation angles for rotary position embedding (R6), in float64:
    angle[t, i] = pos[t] * theta^(-2i/d) for i < d/2."""
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = np.power(np.float64(theta), -2.0 * i / head_dim)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang), np.sin(ang)


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half RoPE (R6) on x [T, heads, d] at absolute positions pos [T]:
    (x1, x2) -> (x1 cos - x2 sin, x2 cos + x1 sin), pairs (i, i + d/2)."""
    d = x.shape[-1]
    half = d // 2
    cos, sin = rope_cos_sin(pos, d, theta)
    cos = cos[:, None, :].astype(x.dtype)
    sin = sin[:, None, :].astype(x.dtype)
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def softmax_rows(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


# ----------------------------------------------------------------------------
# Method steps
# ----------------------------------------------------------------------------

def fuse(feats: Sequence[np.ndarray], w_fc: np.ndarray, g_fc: np.ndarray, eps: float) -> np.ndarray:
    """Feature fusion ([P3] 设计/Feature Fusion; [P4] §二.3): concatenate the
    hidden states of the chosen target layers (shallow to deep, R2), apply one
    Linear without bias (R3), then RMSNorm.  feats: list of [T, Ht] -> [T, H]."""
    cat = np.concatenate(list(feats), axis=-1)
    y = cat @ w_fc.T
    return rmsnorm(y, g_fc, eps)


def project_context_kv(c: np.ndarray, wk: np.ndarray, wv: np.ndarray, pos: np.ndarray,
                       n_kv: int, d: int, theta: float) -> Tuple[np.ndarray, np.ndarray]:
    """KV injection for one drafter layer ([P3] 设计/KV Injection; [P1] “目标模型最懂”):
    the fused context feature is projected with the layer's own K and V weights
    (R5); K gets RoPE at the context positions, V does not (R6).
    c [T, H] -> K, V [T, Hkv, d]."""
    t = c.shape[0]
    k = (c @ wk.T).reshape(t, n_kv, d)
    v = (c @ wv.T).reshape(t, n_kv, d)
    return rope(k, pos, theta), v


def block_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                    causal_ctx: Optional[int] = None) -> np.ndarray:
    """Non-causal attention of the block ([P4] §二.2): every block row attends
    to every key — all context positions and all block positions — with no mask.
    q [B, Hq, d], k/v [Lk, Hkv, d] -> [B, Hq, d].  q-head j uses kv-head j // G (R8).

    causal_ctx = L (the keys are L context positions followed by the block's own):
    the causal form of an autoregressive model instead, where block row r sees
    keys 0 .. L + r only (used by the target model and the input-fusion variant)."""
    b, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    out = np.empty_like(q)
    scale = 1.0 / np.sqrt(np.float64(d))
    if causal_ctx is not None:
        hidden = np.arange(k.shape[0])[None, :] > (causal_ctx + np.arange(b))[:, None]
    for j in range(hq):
        kh = k[:, j // g, :]
        vh = v[:, j // g, :]
        s = (q[:, j, :] @ kh.T) * q.dtype.type(scale)
        if causal_ctx is not None:
            s = np.where(hidden, -np.inf, s)
        p = softmax_rows(s)
        out[:, j, :] = p @ vh
    return out


@dataclass
class LayerWeights:
    in_norm: np.ndarray
    wq: np.ndarray
    wk: np.ndarray
    wv: np.ndarray
    wo: np.ndarray
    post_norm: np.ndarray
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray


def drafter_layer(x: np.ndarray, w: LayerWeights, k_ctx: np.ndarray, v_ctx: np.ndarray,
                  pos: np.ndarray, n_q: int, n_kv: int, d: int, theta: float,
                  eps: float, causal: bool = False) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One drafter Transformer layer over the block of one sequence (R8).

    x [B, H] residual stream of the block rows at positions pos [B];
    k_ctx / v_ctx [L, Hkv, d] the injected context K/V of this layer.
    causal: block row r sees only the context and block rows 0..r (the layer of
    an autoregressive model: the target, the input-fusion variant's context rows).
    Returns (x_out, K_blk, V_blk)."""
    b = x.shape[0]
    h = rmsnorm(x, w.in_norm, eps)
    q = rope((h @ w.wq.T).reshape(b, n_q, d), pos, theta)
    kb = rope((h @ w.wk.T).reshape(b, n_kv, d), pos, theta)
    vb = (h @ w.wv.T).reshape(b, n_kv, d)
    keys = np.concatenate([k_ctx, kb], axis=0)
    vals = np.concatenate([v_ctx, vb], axis=0)
    o = block_attention(q, keys, vals, k_ctx.shape[0] if causal else None).reshape(b, n_q * d)
    x = x + o @ w.wo.T
    h2 = rmsnorm(x, w.post_norm, eps)
    x = x + (silu(h2 @ w.w_gate.T) * (h2 @ w.w_up.T)) @ w.w_down.T
    return x, kb, vb


def lm_head_argmax(z: np.ndarray, w_lm: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Shared lm_head ([P4] §二.3) and greedy pick per row, lowest id on ties (R18).
    z [R, H] -> (ids [R], top2 values [R, 2], logits [R, V])."""
    logits = z @ w_lm.T
    ids = np.argmax(logits, axis=-1)            # first maximum = lowest index
    part = np.partition(logits, -2, axis=-1)[:, -2:]
    top2 = np.stack([part[:, 1], part[:, 0]], axis=-1)
    top2 = np.sort(top2, axis=-1)[:, ::-1]
    return ids.astype(np.int32), top2, logits


# ----------------------------------------------------------------------------
# Temperature sampling of the draft: Gumbel-max with counter-based noise
# ----------------------------------------------------------------------------
# The pages report drafting under sampling (temperature 1) and verify against
# the target's sampled tokens ([P3] results; [P4] §三 step 3).  A draft row
# samples from softmax(logits / T); here in the Gumbel-max form
# argmax_v(logit_v / T + g_v) with g_v = -log(-log u_v), u_v uniform in (0, 1).
# The uniforms come from Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
# "Parallel random numbers: as easy as 1, 2, 3", SC 2011): counter
# (v with bits 4 and 5 cleared, position, sequence, offset), key (seed mod 2^32,
# seed div 2^32), word x = (v / 16) mod 4 of the block (so one block serves ids
# v, v+16, v+32, v+48), u = (2 floor(x / 2^9) + 1) / 2^24.
# The pages fix none of this: which generator, counter and word feed which
# (id, position, sequence) is a free convention of this library (any one-to-one
# assignment of blocks and words gives independent uniforms, so a valid
# sampler).  The 32-bit member of the Philox family is taken because its round
# needs two 32 x 32 -> 64-bit products, which the chip's integer units form in
# one instruction each, where the 64-bit member needs a dozen; the assignment
# lets one block serve the four ids that one lane of the batched head holds.
# It is part of the sampling contract, not of the method's arithmetic, and both
# sides implement it from this definition.

_M32 = np.uint64(0xFFFFFFFF)
PHILOX4x32_M = (0xD2511F53, 0xCD9E8D57)  # round multipliers
PHILOX4x32_W = (0x9E3779B9, 0xBB67AE85)  # key increments


def philox4x32_10(ctr: Sequence[np.ndarray], key: Sequence[np.ndarray]) -> List[np.ndarray]:
    """The 4-word Philox4x32-10 block of counter words ctr[0..3] and key words
    key[0..1] (32-bit values in uint64 arrays, broadcast together): ten rounds,
    each (c0, c1, c2, c3) -> (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1,
    lo(M0 c0)) with hi / lo the upper / lower 32 bits of the 64-bit product, and
    the key advanced by the Weyl increments (modulo 2^32) between rounds."""
    c = [np.asarray(x, dtype=np.uint64) for x in np.broadcast_arrays(*ctr, *key)]
    assert all(np.all(x <= _M32) for x in c), "Philox4x32 words are 32-bit"
    c0, c1, c2, c3, k0, k1 = [x.copy() for x in c]
    for _ in range(10):
        p0 = np.uint64(PHILOX4x32_M[0]) * c0  # exact: both factors < 2^32
        p1 = np.uint64(PHILOX4x32_M[1]) * c2
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & _M32,
                          (p0 >> np.uint64(32)) ^ c3 ^ k1, p0 & _M32)
        k0 = (k0 + np.uint64(PHILOX4x32_W[0])) & _M32
        k1 = (k1 + np.uint64(PHILOX4x32_W[1])) & _M32
    return [c0, c1, c2, c3]


def gumbel_noise(seed: int, offset: int, seq, pos, v) -> np.ndarray:
    """Standard Gumbel noise of (vocabulary id v, position pos, sequence seq)
    under seed (64-bit) and offset (32-bit), float64, broadcast over the three
    index arrays."""
    assert 0 <= seed < 1 << 64 and 0 <= offset < 1 << 32
    u64 = lambda x: np.asarray(x, dtype=np.int64).astype(np.uint64)
    v = np.asarray(v, dtype=np.int64)
    words = philox4x32_10([u64(v & ~0x30), u64(pos), u64(seq), np.uint64(offset)],
                          [np.uint64(seed & 0xFFFFFFFF), np.uint64(seed >> 32)])
    sel = np.broadcast_to((v >> 4) & 3, np.broadcast(words[0], v).shape)
    x = np.choose(sel, words)
    u = (2.0 * (x >> np.uint64(9)).astype(np.float64) + 1.0) / float(1 << 24)
    return -np.log(-np.log(u))


def lm_head_sample(z: np.ndarray, w_lm: np.ndarray, temperature: float, seed: int, offset: int,
                   seq: np.ndarray, pos: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Shared lm_head and the sampled pick of every row: row i (sequence seq[i],
    drafting position pos[i]) takes argmax_v(logit_v / T + g_v), lowest id on
    ties.  Returns (ids [R], top-2 scores [R, 2], logits [R, V])."""
    logits = z @ w_lm.T
    g = gumbel_noise(seed, offset, np.asarray(seq)[:, None], np.asarray(pos)[:, None],
                     np.arange(logits.shape[1])[None, :])
    scores = logits.astype(np.float64) / float(temperature) + g
    ids = np.argmax(scores, axis=-1)
    top2 = -np.sort(-np.partition(scores, -2, axis=-1)[:, -2:], axis=-1)
    return ids.astype(np.int32), top2, logits


def accept(drafts: np.ndarray, targets: np.ndarray) -> Tuple[int, int]:
    """Longest-matching-prefix acceptance with the bonus token ([P4] §三 step 3,
    直观理解): compare the B-1 drafts with the target's tokens position by
    position, keep the run of matches from the start (n of them), and take the
    target's own token at the first mismatch (or after the last draft) as the
    bonus.  Returns (accept_len = n + 1, bonus = targets[n]) (R11, R12)."""
    n = 0
    while n < len(drafts) and int(drafts[n]) == int(targets[n]):
        n += 1
    return n + 1, int(targets[n])


def accept_cumprod(drafts: np.ndarray, targets: np.ndarray) -> int:
    """The same count written as the pages phrase it: the sum of the cumulative
    product of the per-position match indicators ([P4] §三 step 3)."""
    m = (np.asarray(drafts) == np.asarray(targets)[: len(drafts)]).astype(np.int64)
    return int(np.sum(np.cumprod(m))) + 1


# ----------------------------------------------------------------------------
# Stateful drafter: per-sequence, per-layer injected KV cache
# ----------------------------------------------------------------------------

WEIGHT_LAYER_FIELDS = ("in_norm", "wq", "wk", "wv", "wo", "post_norm", "w_gate", "w_up", "w_down")


class OracleDrafter:
    """The whole draft step for a batch of independent sequences (R14).

    ``weights`` maps names (embed, fc, fc_norm, final_norm, lm_head and
    ``l{l}.<field>``) to float arrays; Linear weights are [out, in]."""

    def __init__(self, dims, weights: Dict[str, np.ndarray], batch: int, dtype=np.float64):
        self.dims = dims
        self.dtype = np.dtype(dtype)
        cv = lambda a: np.asarray(a, dtype=self.dtype)
        self.embed = cv(weights["embed"])
        self.fc = cv(weights["fc"])
        self.fc_norm = cv(weights["fc_norm"])
        self.final_norm = cv(weights["final_norm"])
        self.lm_head = cv(weights["lm_head"])
        self.layers = [LayerWeights(*[cv(weights[f"l{l}.{f}"]) for f in WEIGHT_LAYER_FIELDS])
                       for l in range(dims.n_layers)]
        self.batch = batch
        d = dims
        empty = lambda: np.zeros((0, d.n_kv_heads, d.head_dim), dtype=self.dtype)
        self.k = [[empty() for _ in range(batch)] for _ in range(d.n_layers)]
        self.v = [[empty() for _ in range(batch)] for _ in range(d.n_layers)]
        self.len = np.zeros(batch, dtype=np.int64)
        self.base = np.full(batch, -1, dtype=np.int64)
        # sticky flags of the calls, with the bit values of the library's err word:
        # 4 = an acceptance for a sequence that has no draft (no base) to trim back to
        self.err = 0

    # -- fusion + injection ---------------------------------------------------
    def fuse(self, feats: Sequence[np.ndarray]) -> np.ndarray:
        return fuse([np.asarray(f, dtype=self.dtype) for f in feats], self.fc, self.fc_norm,
                    self.dims.rms_eps)

    def fuse_inject(self, seq: int, feats: Sequence[np.ndarray]) -> np.ndarray:
        """Fuse ``T`` rows of target features of sequence ``seq`` and append
        their K/V to every layer's cache at positions len .. len+T-1."""
        d = self.dims
        c = self.fuse(feats)
        t = c.shape[0]
        pos = np.arange(self.len[seq], self.len[seq] + t)
        for l, w in enumerate(self.layers):
            k, v = project_context_kv(c, w.wk, w.wv, pos, d.n_kv_heads, d.head_dim, d.rope_theta)
            self.k[l][seq] = np.concatenate([self.k[l][seq], k], axis=0)
            self.v[l][seq] = np.concatenate([self.v[l][seq], v], axis=0)
        self.len[seq] += t
        return c

    def fuse_inject_input(self, seq: int, feats: Sequence[np.ndarray]) -> np.ndarray:
        """The input-fusion variant of the injection (the ablation of [P3] Results:
        the target feature enters only the drafter's first-layer input, as in
        EAGLE-3, instead of every layer's K/V; [P3] 设计/KV Injection contrasts the
        two).  The fused rows c are the first layer's input at positions
        len .. len+T-1; every layer runs causally over the drafter's own cache
        (each row sees the cached context and the rows before it) and appends
        the K/V it computes; the last layer's K/V are all that is needed of it.
        len += T.  Returns c."""
        d = self.dims
        c = self.fuse(feats)
        t = c.shape[0]
        pos = np.arange(self.len[seq], self.len[seq] + t)
        x = c
        for l, w in enumerate(self.layers):
            if l + 1 == len(self.layers):
                h = rmsnorm(x, w.in_norm, d.rms_eps)
                kb = rope((h @ w.wk.T).reshape(t, d.n_kv_heads, d.head_dim), pos, d.rope_theta)
                vb = (h @ w.wv.T).reshape(t, d.n_kv_heads, d.head_dim)
            else:
                x, kb, vb = drafter_layer(x, w, self.k[l][seq], self.v[l][seq], pos, d.n_q_heads,
                                          d.n_kv_heads, d.head_dim, d.rope_theta, d.rms_eps,
                                          causal=True)
            self.k[l][seq] = np.concatenate([self.k[l][seq], kb], axis=0)
            self.v[l][seq] = np.concatenate([self.v[l][seq], vb], axis=0)
        self.len[seq] += t
        return c

    # -- draft ------------------------------------------------------------------
    def draft(self, x0: Sequence[int], block: int, want_logits: bool = False,
              temperature: float = 0.0, seed: int = 0, offset: int = 0) -> Dict[str, np.ndarray]:
        """One draft step for every sequence ([P4] §二.1, §三 step 1; [P3] 设计/
        Parallel Drafting): the block is the last verified token followed by
        block-1 mask tokens (R7), at positions len .. len+block-1 (R21); one
        forward pass through all layers; the final hidden rows 1..block-1 go
        through the final norm and the shared lm_head (R9, R10).  Records
        base = len.  Returns draft ids [batch, block-1], top-2 logits, final
        hidden rows [batch, block, H] and, on request, logits.  With
        temperature > 0 each row is sampled (lm_head_sample) instead, and top2
        holds the top-2 sampling scores."""
        d = self.dims
        mask_id = d.vocab - 1
        out_ids = np.zeros((self.batch, block - 1), dtype=np.int32)
        top2 = np.zeros((self.batch, block - 1, 2), dtype=self.dtype)
        hid = np.zeros((self.batch, block, d.hidden), dtype=self.dtype)
        logits_all = [] if want_logits else None
        for b in range(self.batch):
            ids = np.array([int(x0[b])] + [mask_id] * (block - 1))
            x = self.embed[ids].copy()
            pos = np.arange(self.len[b], self.len[b] + block)
            for l, w in enumerate(self.layers):
                x, _, _ = drafter_layer(x, w, self.k[l][b], self.v[l][b], pos, d.n_q_heads,
                                        d.n_kv_heads, d.head_dim, d.rope_theta, d.rms_eps)
            z = rmsnorm(x, self.final_norm, d.rms_eps)
            hid[b] = z
            if temperature > 0:
                rpos = np.arange(self.len[b] + 1, self.len[b] + block)
                ids_b, t2, lg = lm_head_sample(z[1:], self.lm_head, temperature, seed, offset,
                                               np.full(block - 1, b), rpos)
            else:
                ids_b, t2, lg = lm_head_argmax(z[1:], self.lm_head)
            out_ids[b] = ids_b
            top2[b] = t2
            if want_logits:
                logits_all.append(lg)
            self.base[b] = self.len[b]
        res = {"draft_ids": out_ids, "top2": top2, "final_hidden": hid}
        if want_logits:
            res["logits"] = np.stack(logits_all)
        return res

    # -- accept + trim ------------------------------------------------------------
    def accept_trim(self, drafts: np.ndarray, targets: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        """Per sequence: longest-prefix acceptance plus bonus, then trim the
        drafter cache to the committed length base + accept_len ([P4] §三 step 3:
        the caches are cut back to the confirmed length right after acceptance).
        A sequence that was never drafted has no base (-1): the committed length
        is undefined, so its cache is left as it is and flag 4 is raised; its
        acceptance and bonus are still the comparison's."""
        acc = np.zeros(self.batch, dtype=np.int32)
        bonus = np.zeros(self.batch, dtype=np.int32)
        for b in range(self.batch):
            a, bo = accept(drafts[b], targets[b])
            acc[b], bonus[b] = a, bo
            if self.base[b] < 0:
                self.err |= 4
                continue
            self.trim(b, int(self.base[b]) + a)
        return acc, bonus

    def trim(self, seq: int, new_len: int) -> None:
        new_len = min(int(self.len[seq]), int(new_len))
        for l in range(self.dims.n_layers):
            self.k[l][seq] = self.k[l][seq][:new_len]
            self.v[l][seq] = self.v[l][seq][:new_len]
        self.len[seq] = new_len


# ----------------------------------------------------------------------------
# A synthetic target model: verification and the features the drafter fuses
# ----------------------------------------------------------------------------

class OracleTarget:
    """An autoregressive target of the drafter's layer form (R8, causal), with
    random weights: embed and lm_head (shared with the drafter, [P4] §二.3),
    n_layers pre-norm layers, a final norm, and its own per-sequence cache.

    forward(seq, ids) runs rows of tokens at positions len .. len+T-1 through
    every layer causally over the cache, appends their K/V (len += T), and
    returns the greedy next token after each row (its lm_head argmax; the
    target's token for position len+1+i, R11), the top-2 logits, and the hidden
    states after each captured layer (R26: the feature of target layer l is the
    residual stream leaving layer l).  Verification of a block ([P4] §三 step 2)
    is forward() over [x0, drafts]; prefill is forward() over the prompt."""

    def __init__(self, dims, weights: Dict[str, np.ndarray], batch: int, dtype=np.float64):
        self.dims = dims
        self.dtype = np.dtype(dtype)
        cv = lambda a: np.asarray(a, dtype=self.dtype)
        self.embed = cv(weights["embed"])
        self.final_norm = cv(weights["final_norm"])
        self.lm_head = cv(weights["lm_head"])
        self.layers = [LayerWeights(*[cv(weights[f"l{l}.{f}"]) for f in WEIGHT_LAYER_FIELDS])
                       for l in range(dims.n_layers)]
        self.batch = batch
        d = dims
        empty = lambda: np.zeros((0, d.n_kv_heads, d.head_dim), dtype=self.dtype)
        self.k = [[empty() for _ in range(batch)] for _ in range(d.n_layers)]
        self.v = [[empty() for _ in range(batch)] for _ in range(d.n_layers)]
        self.len = np.zeros(batch, dtype=np.int64)
        self.base = np.full(batch, -1, dtype=np.int64)

    def forward(self, seq: int, ids: Sequence[int], capture: Sequence[int]):
        d = self.dims
        ids = np.asarray(ids, dtype=np.int64)
        t = ids.shape[0]
        pos = np.arange(self.len[seq], self.len[seq] + t)
        x = self.embed[ids].copy()
        feats = {}
        for l, w in enumerate(self.layers):
            x, kb, vb = drafter_layer(x, w, self.k[l][seq], self.v[l][seq], pos, d.n_q_heads,
                                      d.n_kv_heads, d.head_dim, d.rope_theta, d.rms_eps,
                                      causal=True)
            self.k[l][seq] = np.concatenate([self.k[l][seq], kb], axis=0)
            self.v[l][seq] = np.concatenate([self.v[l][seq], vb], axis=0)
            if l in capture:
                feats[l] = x.copy()
        self.base[seq] = self.len[seq]
        self.len[seq] += t
        ids_next, top2, logits = lm_head_argmax(rmsnorm(x, self.final_norm, d.rms_eps), self.lm_head)
        return ids_next, top2, [feats[l] for l in capture]

    def trim(self, seq: int, new_len: int) -> None:
        new_len = min(int(self.len[seq]), int(new_len))
        for l in range(self.dims.n_layers):
            self.k[l][seq] = self.k[l][seq][:new_len]
            self.v[l][seq] = self.v[l][seq][:new_len]
        self.len[seq] = new_len


def speculative_generate(target: OracleTarget, drafter: OracleDrafter, seq: int,
                         prompt: Sequence[int], n_tokens: int, block: int,
                         capture: Sequence[int], input_fusion: bool = False):
    """The whole speculative loop of one sequence ([P4] §三 steps 1-3): prefill
    the target with the prompt and inject the features of its rows into the
    drafter; then per round draft a block from the last verified token x0,
    verify [x0, drafts] with one target pass, accept the longest matching prefix
    plus the bonus token, trim both caches to the committed length and inject
    the target features of the verified rows 0..n, until at least n_tokens are
    generated.  Returns every generated token (the first is the target's own
    token after the prompt; the last is the next round's x0, not yet in either
    cache) and the accept lengths of the rounds."""
    assert drafter.batch == 1 and target.batch == 1 and seq == 0, "one sequence"
    ids, _, feats = target.forward(seq, prompt, capture)
    inject = drafter.fuse_inject_input if input_fusion else drafter.fuse_inject
    inject(seq, feats)
    x0 = int(ids[-1])
    out = [x0]
    acc_lens = []
    while len(out) < n_tokens:
        drafts = drafter.draft([x0], block)["draft_ids"][0]
        t_ids, _, tf = target.forward(seq, [x0] + [int(v) for v in drafts], capture)
        a, bonus = accept(drafts, t_ids)
        acc_lens.append(a)
        target.trim(seq, int(target.base[seq]) + a)
        drafter.trim(seq, int(drafter.base[seq]) + a)
        inject(seq, [f[:a] for f in tf])
        out.extend(int(v) for v in t_ids[:a])
        x0 = int(bonus)
    return out, acc_lens


def autoregressive_generate(target: OracleTarget, seq: int, prompt: Sequence[int],
                            n_tokens: int) -> List[int]:
    """The target's own greedy decoding, one token per pass: the reference the
    speculative loop must reproduce exactly (lossless, [P4] §三 step 3)."""
    ids, _, _ = target.forward(seq, prompt, [])
    out = [int(ids[-1])]
    while len(out) < n_tokens:
        ids, _, _ = target.forward(seq, [out[-1]], [])
        out.append(int(ids[-1]))
    return out
