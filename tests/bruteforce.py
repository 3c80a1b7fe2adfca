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
