"""Brute-force fp64 draft step in explicit scalar loops, used only to pin the oracle.

Written independently of ``oracle/``: every product is an explicit loop over
indices (inner products via ``math.fsum`` over Python floats), RoPE is a
complex rotation z * exp(i * pos * w) of the pair (x_i, x_{i+d/2}), softmax is
computed per query with ``math.exp``.  Only usable on very small shapes.
"""

from __future__ import annotations

import cmath
import math
from typing import Dict, List, Sequence


def _matvec(w, x) -> List[float]:
    """y[o] = sum_i w[o][i] * x[i] for a weight given as [out][in]."""
    return [math.fsum(w_row[i] * x[i] for i in range(len(x))) for w_row in w]


def _rms(x: Sequence[float], g: Sequence[float], eps: float) -> List[float]:
    ms = math.fsum(v * v for v in x) / len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [x[i] * r * g[i] for i in range(len(x))]


def _rope_head(vec: Sequence[float], pos: int, theta: float) -> List[float]:
    d = len(vec)
    half = d // 2
    out = [0.0] * d
    for i in range(half):
        w = theta ** (-(2.0 * i) / d)
        z = complex(vec[i], vec[i + half]) * cmath.exp(1j * pos * w)
        out[i] = z.real
        out[i + half] = z.imag
    return out


def _heads(flat: Sequence[float], n: int, d: int) -> List[List[float]]:
    return [list(flat[h * d:(h + 1) * d]) for h in range(n)]


def _silu(v: float) -> float:
    return v / (1.0 + math.exp(-v))


def brute_fuse_row(feat_rows: Sequence[Sequence[float]], w_fc, g_fc, eps) -> List[float]:
    cat: List[float] = []
    for f in feat_rows:
        cat.extend(f)
    return _rms(_matvec(w_fc, cat), g_fc, eps)


def brute_draft(dims, w: Dict[str, list], ctx_feats: List[List[List[float]]], x0: int,
                block: int) -> Dict[str, object]:
    """Full pipeline for one sequence: fuse + inject the context rows at
    positions 0..L-1, then draft one block at positions L..L+block-1.

    w: weights as nested Python lists ([out][in]); ctx_feats[t][i] is the
    feature row of target layer i at context position t."""
    H, nq, nkv, d = dims.hidden, dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    theta, eps = dims.rope_theta, dims.rms_eps
    G = nq // nkv
    L = len(ctx_feats)
    # context K/V per layer: [layer][pos][head] -> vector
    kc = []
    vc = []
    fused = []
    for t in range(L):
        fused.append(brute_fuse_row(ctx_feats[t], w["fc"], w["fc_norm"], eps))
    for l in range(dims.n_layers):
        kl, vl = [], []
        for t in range(L):
            k = _heads(_matvec(w[f"l{l}.wk"], fused[t]), nkv, d)
            v = _heads(_matvec(w[f"l{l}.wv"], fused[t]), nkv, d)
            kl.append([_rope_head(k[h], t, theta) for h in range(nkv)])
            vl.append(v)
        kc.append(kl)
        vc.append(vl)
    mask = dims.vocab - 1
    ids = [x0] + [mask] * (block - 1)
    x = [list(w["embed"][i]) for i in ids]
    for l in range(dims.n_layers):
        hs = [_rms(x[r], w[f"l{l}.in_norm"], eps) for r in range(block)]
        q = [[_rope_head(hh, L + r, theta) for hh in _heads(_matvec(w[f"l{l}.wq"], hs[r]), nq, d)]
             for r in range(block)]
        kb = [[_rope_head(hh, L + r, theta) for hh in _heads(_matvec(w[f"l{l}.wk"], hs[r]), nkv, d)]
              for r in range(block)]
        vb = [_heads(_matvec(w[f"l{l}.wv"], hs[r]), nkv, d) for r in range(block)]
        keys = kc[l] + kb
        vals = vc[l] + vb
        scale = 1.0 / math.sqrt(d)
        new_x = []
        for r in range(block):
            o_flat: List[float] = []
            for j in range(nq):
                hk = j // G
                sc = [math.fsum(q[r][j][e] * keys[p][hk][e] for e in range(d)) * scale
                      for p in range(len(keys))]
                mx = max(sc)
                ex = [math.exp(s - mx) for s in sc]
                den = math.fsum(ex)
                o = [math.fsum(ex[p] * vals[p][hk][e] for p in range(len(keys))) / den
                     for e in range(d)]
                o_flat.extend(o)
            proj = _matvec(w[f"l{l}.wo"], o_flat)
            new_x.append([x[r][i] + proj[i] for i in range(H)])
        x = new_x
        for r in range(block):
            h2 = _rms(x[r], w[f"l{l}.post_norm"], eps)
            gt = _matvec(w[f"l{l}.w_gate"], h2)
            up = _matvec(w[f"l{l}.w_up"], h2)
            a = [_silu(gt[i]) * up[i] for i in range(len(gt))]
            dn = _matvec(w[f"l{l}.w_down"], a)
            x[r] = [x[r][i] + dn[i] for i in range(H)]
    z = [_rms(x[r], w["final_norm"], eps) for r in range(block)]
    drafts = []
    logits = []
    top2 = []
    for r in range(1, block):
        lg = _matvec(w["lm_head"], z[r])
        best = 0
        for vtok in range(1, len(lg)):
            if lg[vtok] > lg[best]:
                best = vtok
        # runner-up: the largest logit of any other id (equal to the best on a tie)
        second = None
        for vtok in range(len(lg)):
            if vtok != best and (second is None or lg[vtok] > second):
                second = lg[vtok]
        drafts.append(best)
        logits.append(lg)
        top2.append([lg[best], second])
    return {"draft_ids": drafts, "final_hidden": z, "logits": logits, "top2": top2,
            "fused": fused, "k_ctx": kc, "v_ctx": vc}


def brute_accept(drafts: Sequence[int], targets: Sequence[int]):
    """Acceptance by enumeration of candidate prefix lengths: the largest n such
    that all of drafts[:n] equal targets[:n]."""
    best = 0
    for n in range(len(drafts) + 1):
        if all(drafts[i] == targets[i] for i in range(n)):
            best = n
    return best + 1, targets[best]


def _attend_row(q_heads, keys, vals, G, d):
    """Attention of one query row over the given cached keys/values (lists over
    positions of per-kv-head vectors), explicit loops."""
    out: List[float] = []
    scale = 1.0 / math.sqrt(d)
    for j, qj in enumerate(q_heads):
        hk = j // G
        sc = [math.fsum(qj[e] * keys[p][hk][e] for e in range(d)) * scale for p in range(len(keys))]
        mx = max(sc)
        ex = [math.exp(s - mx) for s in sc]
        den = math.fsum(ex)
        out.extend(math.fsum(ex[p] * vals[p][hk][e] for p in range(len(keys))) / den
                   for e in range(d))
    return out


def _row_through_layers(dims, w, x, pos, kc, vc, last_kv_only=False, capture=(), feats=None):
    """One row at position pos through every layer, one token at a time: its K/V
    are appended to each layer's cache before it attends, so it sees exactly the
    rows before it and itself.  kc/vc: per layer lists of cached positions."""
    H, nq, nkv, d = dims.hidden, dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    theta, eps = dims.rope_theta, dims.rms_eps
    G = nq // nkv
    for l in range(dims.n_layers):
        h = _rms(x, w[f"l{l}.in_norm"], eps)
        kc[l].append([_rope_head(hh, pos, theta) for hh in _heads(_matvec(w[f"l{l}.wk"], h), nkv, d)])
        vc[l].append(_heads(_matvec(w[f"l{l}.wv"], h), nkv, d))
        if last_kv_only and l == dims.n_layers - 1:
            break
        q = [_rope_head(hh, pos, theta) for hh in _heads(_matvec(w[f"l{l}.wq"], h), nq, d)]
        o = _attend_row(q, kc[l], vc[l], G, d)
        proj = _matvec(w[f"l{l}.wo"], o)
        x = [x[i] + proj[i] for i in range(H)]
        h2 = _rms(x, w[f"l{l}.post_norm"], eps)
        gt = _matvec(w[f"l{l}.w_gate"], h2)
        up = _matvec(w[f"l{l}.w_up"], h2)
        dn = _matvec(w[f"l{l}.w_down"], [_silu(gt[i]) * up[i] for i in range(len(gt))])
        x = [x[i] + dn[i] for i in range(H)]
        if feats is not None and l in capture:
            feats[l].append(list(x))
    return x


def brute_target(dims, w, ids: Sequence[int], capture: Sequence[int]):
    """An autoregressive target from an empty cache, one token after another:
    per row the greedy next token (first maximum), the two largest logits, and
    the hidden state leaving each captured layer."""
    kc = [[] for _ in range(dims.n_layers)]
    vc = [[] for _ in range(dims.n_layers)]
    feats = {l: [] for l in capture}
    nxt, top2 = [], []
    for t, tok in enumerate(ids):
        x = _row_through_layers(dims, w, list(w["embed"][tok]), t, kc, vc, capture=capture,
                                feats=feats)
        lg = _matvec(w["lm_head"], _rms(x, w["final_norm"], dims.rms_eps))
        best = 0
        for v in range(1, len(lg)):
            if lg[v] > lg[best]:
                best = v
        second = max(lg[v] for v in range(len(lg)) if v != best)
        nxt.append(best)
        top2.append([lg[best], second])
    return {"next": nxt, "top2": top2, "feats": [feats[l] for l in capture], "k": kc, "v": vc}


def brute_input_fusion(dims, w, feat_rows) -> Dict[str, object]:
    """The input-fusion variant's injection into an empty drafter cache, one row
    at a time: the fused row is the first layer's input; the last layer only
    contributes its K/V."""
    kc = [[] for _ in range(dims.n_layers)]
    vc = [[] for _ in range(dims.n_layers)]
    for t, fr in enumerate(feat_rows):
        c = brute_fuse_row(fr, w["fc"], w["fc_norm"], dims.rms_eps)
        _row_through_layers(dims, w, c, t, kc, vc, last_kv_only=True)
    return {"k": kc, "v": vc}
