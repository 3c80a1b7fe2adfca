"""The C ABI on the host: the library loads, exports every function that
include/dflash.h declares, sizes workspaces, and rejects bad arguments before
any launch.  Calls here either fail validation or are pure host functions, so
they never touch a GPU (none is needed)."""

import ctypes
import os
import re

import pytest

from block_diffusion_drafter_layers_amd import binding as B
from block_diffusion_drafter_layers_amd.runtime import make_config
from synth.configs import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "dflash.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = B.load_library()
    names = _declared_functions()
    assert set(names) >= {"dflash_fuse_inject", "dflash_draft_block", "dflash_accept_trim",
                          "dflash_workspace_bytes", "dflash_strerror"}
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layouts_match_header():
    # 11 int32 + 2 float + 1 int32
    assert ctypes.sizeof(B.dflash_config) == 14 * 4
    assert ctypes.sizeof(B.dflash_weights) == 14 * 8 + 8  # + int32 layout, padded
    assert ctypes.sizeof(B.dflash_kv) == 5 * 8 + 2 * 4
    assert ctypes.sizeof(B.dflash_debug) == 4 * 8 + 3 * 4 + 4 + 8  # padded to 8, then top2
    assert B.dflash_debug.top2.offset == 48
    assert ctypes.sizeof(B.dflash_sampling) == 4 + 4 + 2 * 8  # float, padding, two uint64
    assert B.dflash_sampling.seed.offset == 8


def test_strerror():
    assert B.dflash_strerror(0) == "ok"
    assert "workspace" in B.dflash_strerror(B.DFLASH_ENOSPC)
    assert B.dflash_strerror(-99) == "unknown error"


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4, 5])
def test_workspace_bytes_positive_and_monotone(cfg_id):
    wl = CONFIGS[cfg_id]
    c = make_config(wl.dims)
    a = B.dflash_workspace_bytes(c, wl.batch, 16 * wl.batch, 4096)
    b = B.dflash_workspace_bytes(c, wl.batch, 16 * wl.batch, 8192)
    assert 0 < a <= b
    assert B.dflash_workspace_bytes(c, wl.batch, 100000, 4096) >= a


@pytest.mark.parametrize("cfg_id,batch", [(2, 1), (2, 3), (5, 1), (1, 1)])
def test_workspace_bytes_never_shrinks_as_rows_grow(cfg_id, batch):
    """The size for max_rows must cover every call of fewer rows: split partials
    do not grow monotonically with a pass's row count (758..768 rows once needed
    more than 1024), so the size is non-decreasing over a scan of row counts,
    across the 16384-row pass boundary too."""
    c = make_config(CONFIGS[cfg_id].dims)
    rows = list(range(0, 1300)) + list(range(16000, 16500, 7)) + [32768 + 5, 40000]
    prev = 0
    for r in rows:
        b = B.dflash_workspace_bytes(c, batch, r, 4096)
        assert b >= prev, (r, b, prev)
        prev = b


def test_workspace_bytes_never_shrinks_as_blocks_or_context_grow():
    c = make_config(CONFIGS[2].dims)
    prev = 0
    for bmax in range(2, 17):
        c.block_max = bmax
        b = B.dflash_workspace_bytes(c, 2, 16, 2048)
        assert b >= prev, (bmax, b, prev)
        prev = b
    c = make_config(CONFIGS[2].dims)
    prev = 0
    for ctx in range(64, 40000, 832):
        b = B.dflash_workspace_bytes(c, 1, 16, ctx)
        assert b >= prev, (ctx, b, prev)
        prev = b


def test_workspace_bytes_rejects_bad_config():
    c = make_config(CONFIGS[2].dims)
    c.head_dim = 96
    assert B.dflash_workspace_bytes(c, 1, 16, 1024) == 0
    c = make_config(CONFIGS[2].dims)
    assert B.dflash_workspace_bytes(c, 0, 16, 1024) == 0


def _fake_structs(dims, n_layers=None):
    """Structs whose device addresses are never dereferenced: every call made
    with them is rejected on the host."""
    n = n_layers or dims.n_layers
    fake = 0x1000
    w = B.dflash_weights()
    w.layout = B.DFLASH_LAYOUT_PACKED if dims.dtype == "bf16" else B.DFLASH_LAYOUT_ROWMAJOR
    for f in ("embed", "fc", "fc_norm", "final_norm", "lm_head"):
        setattr(w, f, fake)
    keep = []
    for f in ("in_norm", "wq", "wk", "wv", "wo", "post_norm", "w_gate", "w_up", "w_down"):
        arr = B.ptr_array([fake] * n)
        keep.append(arr)
        setattr(w, f, B.as_pvp(arr))
    kv = B.dflash_kv()
    ka = B.ptr_array([fake] * n)
    keep.append(ka)
    kv.k = kv.v = B.as_pvp(ka)
    kv.len = kv.base = kv.err = fake
    kv.batch, kv.max_ctx = 1, 1024
    return w, kv, keep


def test_host_validation_errors():
    dims = CONFIGS[2].dims
    c = make_config(dims)
    w, kv, keep = _fake_structs(dims)
    fake = 0x2000
    lib = B.load_library()
    # block outside [2, block_max]
    assert B.dflash_draft_block(c, w, kv, fake, 17, fake, fake, 1 << 40) == B.DFLASH_ERANGE
    assert B.dflash_draft_block(c, w, kv, fake, 1, fake, fake, 1 << 40) == B.DFLASH_ERANGE
    # workspace too small
    assert B.dflash_draft_block(c, w, kv, fake, 16, fake, fake, 1024) == B.DFLASH_ENOSPC
    # null token pointer
    assert B.dflash_draft_block(c, w, kv, None, 16, fake, fake, 1 << 40) == B.DFLASH_EINVAL
    # null weight entry
    w2, _, keep2 = _fake_structs(dims)
    arr = B.ptr_array([0x1000] * (dims.n_layers - 1) + [0])
    w2.w_down = B.as_pvp(arr)
    assert B.dflash_draft_block(c, w2, kv, fake, 16, fake, fake, 1 << 40) == B.DFLASH_EINVAL
    # max_ctx not a multiple of 64
    kv.max_ctx = 1000
    assert B.dflash_draft_block(c, w, kv, fake, 16, fake, fake, 1 << 40) == B.DFLASH_ERANGE
    kv.max_ctx = 1024
    # unsupported head_dim / dtype
    c.head_dim = 96
    assert B.dflash_draft_block(c, w, kv, fake, 16, fake, fake, 1 << 40) == B.DFLASH_ERANGE
    c = make_config(dims)
    c.dtype = 7
    assert B.dflash_accept_trim(c, fake, fake, 16, fake, fake, kv) == B.DFLASH_ERANGE
    c = make_config(dims)
    # heads not divisible
    c.n_q_heads = 30
    assert B.dflash_fuse_inject(c, w, None, fake, fake, 0, kv, fake, 1 << 40) == B.DFLASH_EINVAL
    c = make_config(dims)
    # fuse_inject: rows but no feature pointers; negative rows; small workspace
    assert B.dflash_fuse_inject(c, w, None, fake, fake, 16, kv, fake, 1 << 40) == B.DFLASH_EINVAL
    assert B.dflash_fuse_inject(c, w, None, fake, fake, -1, kv, fake, 1 << 40) == B.DFLASH_EINVAL
    fa = B.ptr_array([0x3000] * 5)
    assert B.dflash_fuse_inject(c, w, B.as_pvp(fa), fake, fake, 16, kv, fake, 16) == B.DFLASH_ENOSPC
    # accept_trim argument checks
    assert B.dflash_accept_trim(c, None, fake, 16, fake, fake, kv) == B.DFLASH_EINVAL
    assert B.dflash_accept_trim(c, fake, fake, 40, fake, fake, kv) == B.DFLASH_ERANGE
    kv.batch = 0
    assert B.dflash_accept_trim(c, fake, fake, 16, fake, fake, kv) == B.DFLASH_EINVAL
    # bf16 weights must be declared fragment-packed
    w.layout = B.DFLASH_LAYOUT_ROWMAJOR
    assert B.dflash_draft_block(c, w, kv, fake, 16, fake, fake, 1 << 40) == B.DFLASH_EINVAL
    assert B.dflash_fuse_inject(c, w, None, fake, fake, 0, kv, fake, 1 << 40) == B.DFLASH_EINVAL
    w.layout = B.DFLASH_LAYOUT_PACKED
    # sampled draft: the same checks, a NaN temperature and an offset past 32 bits
    kv.batch = 1
    smp = B.dflash_sampling(1.0, 1, 2)
    assert B.dflash_draft_block_sampled(c, w, kv, fake, 17, smp, fake, fake, 1 << 40) == B.DFLASH_ERANGE
    assert B.dflash_draft_block_sampled(c, w, kv, fake, 16, smp, fake, fake, 1024) == B.DFLASH_ENOSPC
    assert B.dflash_draft_block_sampled(c, w, kv, None, 16, smp, fake, fake, 1 << 40) == B.DFLASH_EINVAL
    for bad in (float("nan"), float("inf"), float("-inf")):
        smp.temperature = bad
        assert B.dflash_draft_block_sampled(c, w, kv, fake, 16, smp, fake, fake, 1 << 40) == B.DFLASH_EINVAL
    # the offset is a 32-bit Philox counter word
    smp.temperature = 1.0
    for bad in (1 << 32, (1 << 64) - 1):
        smp.offset = bad
        assert B.dflash_draft_block_sampled(c, w, kv, fake, 16, smp, fake, fake, 1 << 40) == B.DFLASH_EINVAL
    del keep, keep2, lib


def test_noalloc_draft_rejects_before_touching_the_device():
    """The allocation-free draft validates like dflash_draft_block and refuses a
    draft whose workspace would not fit its scratch, all before any HIP call."""
    fake = 0x2000
    dims = CONFIGS[5].dims
    c = make_config(dims)
    w, kv, keep = _fake_structs(dims)
    kv.batch, kv.max_ctx = 64, 8192           # the wide drafter at batch 64: far above the scratch
    assert B.dflash_workspace_bytes(c, 64, 0, 8192) > B.DFLASH_NOALLOC_SCRATCH_BYTES
    assert B.dflash_draft_block_noalloc(c, w, kv, fake, 16, fake) == B.DFLASH_ENOSPC
    assert B.dflash_draft_block_noalloc(c, w, kv, fake, 17, fake) == B.DFLASH_ERANGE
    assert B.dflash_draft_block_noalloc(c, w, kv, None, 16, fake) == B.DFLASH_EINVAL
    w.layout = B.DFLASH_LAYOUT_ROWMAJOR
    assert B.dflash_draft_block_noalloc(c, w, kv, fake, 16, fake) == B.DFLASH_EINVAL
    del keep


def test_pack_weights_argument_checks():
    """dflash_pack_weights rejects, before any launch: fp32 configs, wrong layouts,
    a missing matrix, a destination that is its source."""
    dims = CONFIGS[2].dims
    c = make_config(dims)
    src, _, k1 = _fake_structs(dims)
    dst, _, k2 = _fake_structs(dims)
    src.layout = B.DFLASH_LAYOUT_ROWMAJOR
    dst.layout = B.DFLASH_LAYOUT_PACKED
    # every destination equal to its source (the fake structs share one address)
    assert B.dflash_pack_weights(c, src, dst) == B.DFLASH_EINVAL
    dst.layout = B.DFLASH_LAYOUT_ROWMAJOR
    assert B.dflash_pack_weights(c, src, dst) == B.DFLASH_EINVAL
    dst.layout = B.DFLASH_LAYOUT_PACKED
    src.layout = B.DFLASH_LAYOUT_PACKED
    assert B.dflash_pack_weights(c, src, dst) == B.DFLASH_EINVAL
    src.layout = B.DFLASH_LAYOUT_ROWMAJOR
    arr = B.ptr_array([0x1000] * (dims.n_layers - 1) + [0])
    src.wv = B.as_pvp(arr)
    assert B.dflash_pack_weights(c, src, dst) == B.DFLASH_EINVAL
    c32 = make_config(CONFIGS[1].dims)
    assert B.dflash_pack_weights(c32, src, dst) == B.DFLASH_ERANGE
    del k1, k2, arr


def test_pack_weight_argument_checks():
    fake = 0x2000
    assert B.dflash_pack_weight(None, 16, 32, fake) == B.DFLASH_EINVAL
    assert B.dflash_pack_weight(fake, 16, 32, None) == B.DFLASH_EINVAL
    assert B.dflash_pack_weight(fake, 0, 32, fake) == B.DFLASH_EINVAL
    assert B.dflash_pack_weight(fake, 16, -32, fake) == B.DFLASH_EINVAL
    assert B.dflash_pack_weight(fake, 24, 32, fake) == B.DFLASH_ERANGE
    assert B.dflash_pack_weight(fake, 16, 48, fake) == B.DFLASH_ERANGE


@pytest.mark.parametrize("cfg_id", [2, 5])
def test_batch1_draft_workspace_fits_the_noalloc_scratch_at_any_cache_size(cfg_id):
    """The batch-1 attention cuts a sequence into at most 32 chunks, so the draft's
    workspace stops growing with the cache and the allocation-free entry point covers
    batch-1 drafting at any capacity."""
    c = make_config(CONFIGS[cfg_id].dims)
    sizes = [B.dflash_workspace_bytes(c, 1, 0, mc) for mc in (2048, 8192, 32768, 131072)]
    assert sizes[1] == sizes[2] == sizes[3]
    assert max(sizes) <= 64 << 20


def test_random_parity_shapes_are_configs_the_library_takes():
    """The seeded random shapes of the GPU parity sweep pass the library's own
    configuration checks (a workspace size comes back for each)."""
    from tests.test_gpu_random import N_CASES, random_case
    for i in range(N_CASES):
        dims, batch, block, ctx = random_case(i)
        assert 2 <= block <= dims.block_max and len(ctx) == batch
        max_ctx = int((int(ctx.max()) + block * 4 + 63) // 64 * 64)
        rows = max(int(ctx.sum()), batch * block, 1)
        assert B.dflash_workspace_bytes(make_config(dims), batch, rows, max_ctx) > 0, i
