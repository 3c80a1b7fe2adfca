"""dflash_pack_bf16 performs exactly the permutation include/dflash.h documents,
bit for bit, on raw 16-bit patterns (NaN and denormal patterns included)."""

import numpy as np
import pytest

from tests.gpu_common import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,k", [(16, 32), (48, 96), (4096, 256), (80, 20480)])
def test_pack_is_documented_permutation(n, k):
    import torch
    from block_diffusion_drafter_layers_amd import binding as B
    log(f"[pack] n={n} k={k}")
    bits = np.random.default_rng(n * 7919 + k).integers(0, 1 << 16, size=(n, k), dtype=np.uint16)
    src = torch.from_numpy(bits.view(np.int16)).cuda()
    dst = torch.full_like(src, -1)
    B.check("dflash_pack_bf16", B.dflash_pack_bf16(src.data_ptr(), n, k, dst.data_ptr(),
                                                   torch.cuda.current_stream().cuda_stream))
    got = dst.cpu().numpy().view(np.uint16).reshape(-1)
    # W[16c + r][32t + 8g + j] -> position (((c * k/32 + t) * 64 + (r + 16 g)) * 8 + j)
    want = np.empty(n * k, dtype=np.uint16)
    c, r, t, g, j = np.meshgrid(np.arange(n // 16), np.arange(16), np.arange(k // 32),
                                np.arange(4), np.arange(8), indexing="ij")
    pos = ((c * (k // 32) + t) * 64 + (r + 16 * g)) * 8 + j
    want[pos.reshape(-1)] = bits[(16 * c + r).reshape(-1), (32 * t + 8 * g + j).reshape(-1)]
    assert np.array_equal(got, want)
