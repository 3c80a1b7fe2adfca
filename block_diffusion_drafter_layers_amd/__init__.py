"""DFlash draft step on AMD Instinct MI355X (gfx950): hand-written HIP kernels
behind the C ABI of ``include/dflash.h``.

``binding`` mirrors the C calls one to one; ``runtime.DeviceDrafter`` holds the
device memory (allocated with torch) and forwards to them.
"""

from .binding import (  # noqa: F401
    DFLASH_BF16, DFLASH_F32, DFLASH_OK, DFlashError, dflash_accept_trim, dflash_draft_block,
    dflash_fuse_inject, dflash_strerror, dflash_workspace_bytes, load_library,
)
