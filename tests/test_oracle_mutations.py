"""The oracle's pins, tested against plausible slips: each slip below (a dropped term, a
wrong sign, index, operand or order) is planted in a copy of the oracle, alone, and the
oracle's pin suites (test_oracle, test_oracle_target, test_oracle_sampling) must fail on
it.  The copy lives in a temporary directory with the suites and their helpers; the
oracle in the repository is never modified."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["tests/test_oracle.py", "tests/test_oracle_target.py", "tests/test_oracle_sampling.py"]

# (what the slip is, the oracle's text, the slipped text)
SLIPS = [
    ("RMSNorm without eps", "return x / np.sqrt(ms + eps) * g", "return x / np.sqrt(ms) * g"),
    ("RMSNorm by the sum of squares", "ms = np.mean(x * x, axis=-1, keepdims=True)",
     "ms = np.sum(x * x, axis=-1, keepdims=True)"),
    ("RMSNorm without its gain", "return x / np.sqrt(ms + eps) * g", "return x / np.sqrt(ms + eps)"),
    ("RoPE frequency exponent", "-2.0 * i / head_dim", "-1.0 * i / head_dim"),
    ("RoPE rotation sign", "x1 * cos - x2 * sin, x2 * cos + x1 * sin",
     "x1 * cos + x2 * sin, x2 * cos - x1 * sin"),
    ("RoPE on adjacent pairs", "x1 = x[..., :half]\n    x2 = x[..., half:]",
     "x1 = x[..., 0::2]\n    x2 = x[..., 1::2]"),
    ("attention without 1/sqrt(d)", " * q.dtype.type(scale)", ""),
    ("GQA head mapping", "kh = k[:, j // g, :]\n        vh = v[:, j // g, :]",
     "kh = k[:, j % hkv, :]\n        vh = v[:, j % hkv, :]"),
    ("softmax shift over the wrong axis", "m = np.max(s, axis=-1, keepdims=True)",
     "m = np.max(s, axis=0, keepdims=True)"),
    ("attention residual dropped", "x = x + o @ w.wo.T", "x = o @ w.wo.T"),
    ("MLP residual dropped", "x = x + (silu(h2 @ w.w_gate.T)", "x = (silu(h2 @ w.w_gate.T)"),
    ("post-attention norm with the input norm's gain", "h2 = rmsnorm(x, w.post_norm, eps)",
     "h2 = rmsnorm(x, w.in_norm, eps)"),
    ("silu on the up projection", "silu(h2 @ w.w_gate.T) * (h2 @ w.w_up.T)",
     "(h2 @ w.w_gate.T) * silu(h2 @ w.w_up.T)"),
    ("RoPE on the block's V", "vb = (h @ w.wv.T).reshape(b, n_kv, d)",
     "vb = rope((h @ w.wv.T).reshape(b, n_kv, d), pos, theta)"),
    ("RoPE on the injected V", "return rope(k, pos, theta), v",
     "return rope(k, pos, theta), rope(v, pos, theta)"),
    ("fusion concat order reversed", "cat = np.concatenate(list(feats), axis=-1)",
     "cat = np.concatenate(list(feats)[::-1], axis=-1)"),
    ("fusion without its RMSNorm", "    return rmsnorm(y, g_fc, eps)", "    return y"),
    ("mask token id", "mask_id = d.vocab - 1", "mask_id = 0"),
    ("block positions off by one", "pos = np.arange(self.len[b], self.len[b] + block)",
     "pos = np.arange(self.len[b] + 1, self.len[b] + block + 1)"),
    ("lm_head on rows 0..B-2", "ids_b, t2, lg = lm_head_argmax(z[1:], self.lm_head)",
     "ids_b, t2, lg = lm_head_argmax(z[:-1], self.lm_head)"),
    ("final norm dropped", "z = rmsnorm(x, self.final_norm, d.rms_eps)", "z = x"),
    ("argmax ties to the highest id", "ids = np.argmax(logits, axis=-1)",
     "ids = logits.shape[-1] - 1 - np.argmax(logits[:, ::-1], axis=-1)"),
    ("accept length without the bonus", "return n + 1, int(targets[n])",
     "return n, int(targets[n])"),
    ("bonus token from the wrong position", "return n + 1, int(targets[n])",
     "return n + 1, int(targets[max(n - 1, 0)])"),
    ("injected positions off by one",
     "pos = np.arange(self.len[seq], self.len[seq] + t)\n        for l, w in enumerate(self.layers):\n            k, v",
     "pos = np.arange(self.len[seq] + 1, self.len[seq] + t + 1)\n        for l, w in enumerate(self.layers):\n            k, v"),
    ("runner-up taken as the minimum", "top2 = np.stack([part[:, 1], part[:, 0]], axis=-1)",
     "top2 = np.stack([part[:, 1], logits.min(axis=-1)], axis=-1)"),
    ("causal mask hides the diagonal", "np.arange(k.shape[0])[None, :] > (causal_ctx",
     "np.arange(k.shape[0])[None, :] >= (causal_ctx"),
    # sampling
    ("logits times the temperature", "scores = logits.astype(np.float64) / float(temperature) + g",
     "scores = logits.astype(np.float64) * float(temperature) + g"),
    ("exponential instead of Gumbel noise", "return -np.log(-np.log(u))", "return -np.log(u)"),
    ("Philox with nine rounds", "for _ in range(10):", "for _ in range(9):"),
    ("Philox key increments swapped", "k0 = (k0 + np.uint64(PHILOX4x32_W[0])) & _M32\n        k1 = (k1 + np.uint64(PHILOX4x32_W[1])) & _M32",
     "k0 = (k0 + np.uint64(PHILOX4x32_W[1])) & _M32\n        k1 = (k1 + np.uint64(PHILOX4x32_W[0])) & _M32"),
    ("Philox multipliers swapped", "p0 = np.uint64(PHILOX4x32_M[0]) * c0", "p0 = np.uint64(PHILOX4x32_M[1]) * c0"),
    ("Philox product halves swapped", "(p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & _M32,",
     "(p1 & _M32) ^ c1 ^ k0, p1 >> np.uint64(32),"),
    ("Philox key not wrapped to 32 bits", "k1 = (k1 + np.uint64(PHILOX4x32_W[1])) & _M32",
     "k1 = k1 + np.uint64(PHILOX4x32_W[1])"),
    # (ids of one counter block sharing a word: equal noise for different ids)
    ("noise word from the wrong bits", "sel = np.broadcast_to((v >> 4) & 3,", "sel = np.broadcast_to((v >> 2) & 3,"),
]
# Not listed: which bits of a Philox word form the uniform, or which position number
# keys a row's noise.  Any one-to-one choice is a valid sampler, so no pin of the
# oracle fixes it; the library's sampled drafts against the oracle's (GPU parity) do.


@pytest.fixture(scope="module")
def pin_tree(tmp_path_factory):
    """The oracle, the pin suites and what they import, copied once."""
    d = tmp_path_factory.mktemp("pins")
    shutil.copytree(os.path.join(ROOT, "oracle"), d / "oracle",
                    ignore=shutil.ignore_patterns("__pycache__", "*.so", "*.o"))
    shutil.copytree(os.path.join(ROOT, "synth"), d / "synth",
                    ignore=shutil.ignore_patterns("__pycache__"))
    (d / "tests").mkdir()
    for f in (["__init__.py", "conftest.py", "bruteforce.py", "rocrand_philox_block.cpp"]
              + [os.path.basename(s) for s in SUITES]):
        shutil.copy(os.path.join(ROOT, "tests", f), d / "tests" / f)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), d / "tests" / "golden")
    return d


def _run_pins(tree):
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           *SUITES], cwd=str(tree), capture_output=True, text=True, timeout=600)


def test_unslipped_copy_passes_its_pins(pin_tree):
    r = _run_pins(pin_tree)
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name,text,slipped", SLIPS, ids=[s[0] for s in SLIPS])
def test_pins_fail_on_a_planted_slip(pin_tree, name, text, slipped):
    path = pin_tree / "oracle" / "dflash_oracle.py"
    src = open(os.path.join(ROOT, "oracle", "dflash_oracle.py")).read()
    assert src.count(text) == 1, f"{name}: the oracle's text is not found once"
    try:
        path.write_text(src.replace(text, slipped))
        r = _run_pins(pin_tree)
    finally:
        path.write_text(src)
    assert r.returncode != 0, f"{name}: no pin fails\n{r.stdout[-1500:]}"
