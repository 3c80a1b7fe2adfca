"""dflash_pack_weight performs exactly the conversion and permutation that
include/dflash.h documents, bit for bit: bf16 -> fp16 rounded to nearest even
(subnormal results and overflow to infinity included), then the fragment order."""

import numpy as np
import pytest

from synth.inputs import bf16_bits_to_f32
from tests.gpu_common import log

pytestmark = pytest.mark.gpu


def _bf16_patterns(rng, n, k):
    """Random bf16 bit patterns over every exponent (NaN payloads excluded: their
    fp16 payload is not part of the contract), plus some exact edge values."""
    bits = rng.integers(0, 1 << 16, size=(n, k), dtype=np.uint16)
    nan = ((bits & 0x7F80) == 0x7F80) & ((bits & 0x007F) != 0)
    bits[nan] &= 0xFF80                                   # -> +-inf
    edge = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x477F, 0x4780, 0x3880, 0x3800, 0x3300,
                     0x0001, 0x7F80, 0xFF80], dtype=np.uint16)
    bits.reshape(-1)[:edge.size] = edge
    return bits


@pytest.mark.parametrize("n,k", [(16, 32), (48, 96), (4096, 256), (80, 20480)])
def test_pack_is_documented_conversion_and_permutation(n, k):
    import torch
    from block_diffusion_drafter_layers_amd import binding as B
    log(f"[pack] n={n} k={k}")
    bits = _bf16_patterns(np.random.default_rng(n * 7919 + k), n, k)
    src = torch.from_numpy(bits.view(np.int16)).cuda()
    dst = torch.full_like(src, -1)
    count = torch.full((1,), 5, dtype=torch.int32, device="cuda")    # the call adds to it
    B.check("dflash_pack_weight", B.dflash_pack_weight(
        src.data_ptr(), n, k, dst.data_ptr(), n_overflow=count.data_ptr(),
        stream=torch.cuda.current_stream().cuda_stream))
    got = dst.cpu().numpy().view(np.uint16).reshape(-1)
    with np.errstate(over="ignore"):
        hf = bf16_bits_to_f32(bits).reshape(n, k).astype(np.float16)
        h = hf.view(np.uint16)
    # the overflow count: every element whose fp16 is not finite (the edge values
    # and the random patterns above 65504 or already infinite)
    assert int(count.item()) == 5 + int(np.sum(~np.isfinite(hf)))
    # W[16c + r][32t + 8g + j] -> position (((c * k/32 + t) * 64 + (r + 16 g)) * 8 + j)
    want = np.empty(n * k, dtype=np.uint16)
    c, r, t, g, j = np.meshgrid(np.arange(n // 16), np.arange(16), np.arange(k // 32),
                                np.arange(4), np.arange(8), indexing="ij")
    pos = ((c * (k // 32) + t) * 64 + (r + 16 * g)) * 8 + j
    want[pos.reshape(-1)] = h[(16 * c + r).reshape(-1), (32 * t + 8 * g + j).reshape(-1)]
    assert np.array_equal(got, want)
