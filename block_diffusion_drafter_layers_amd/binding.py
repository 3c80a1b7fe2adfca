"""ctypes binding of ``include/dflash.h``: the same names, argument marshalling only.

Every step of the draft path runs inside ``libdflash.so``; this module only
declares the C structs and forwards calls.  Loading fails loudly when the
library has not been built: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

DFLASH_F32 = 0
DFLASH_BF16 = 1

DFLASH_OK = 0
DFLASH_EINVAL = -1
DFLASH_ERANGE = -2
DFLASH_ENOSPC = -3
DFLASH_EHIP = -4

DFLASH_ERR_CTX_OVERFLOW = 1
DFLASH_ERR_TOKEN_RANGE = 2
DFLASH_ERR_NO_BASE = 4
DFLASH_ERR_NONFINITE = 8

DFLASH_NOALLOC_SCRATCH_BYTES = 64 << 20

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdflash.so")

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_pvp = ctypes.POINTER(ctypes.c_void_p)
_pi32 = ctypes.c_void_p  # device int32 pointers travel as raw addresses


class dflash_config(ctypes.Structure):
    _fields_ = [(n, _i32) for n in ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim",
                                    "inter", "vocab", "n_feat_layers", "feat_hidden", "block_max",
                                    "mask_token_id")] + [
        ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float), ("dtype", _i32)]


DFLASH_LAYOUT_ROWMAJOR = 0
DFLASH_LAYOUT_PACKED = 1


class dflash_weights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("embed", "fc", "fc_norm", "final_norm", "lm_head")] + [
        (n, _pvp) for n in ("in_norm", "wq", "wk", "wv", "wo", "post_norm", "w_gate", "w_up",
                            "w_down")] + [("layout", _i32)]


class dflash_kv(ctypes.Structure):
    _fields_ = [("k", _pvp), ("v", _pvp), ("len", _pi32), ("base", _pi32), ("err", _pi32),
                ("batch", _i32), ("max_ctx", _i32)]


DFLASH_TIME_NONE = 0
DFLASH_TIME_GEMM = 1
DFLASH_TIME_LMHEAD = 2
DFLASH_TIME_ATTN = 3


class dflash_debug(ctypes.Structure):
    _fields_ = [("fused", _vp), ("final_hidden", _vp), ("logits", _vp), ("events", _pvp),
                ("n_events", _i32), ("n_used", _i32), ("timed", _i32), ("top2", _vp)]


class dflash_sampling(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("seed", ctypes.c_uint64),
                ("offset", ctypes.c_uint64)]


_lib: Optional[ctypes.CDLL] = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libdflash.so (built by ``block_diffusion_drafter_layers_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"libdflash.so not built at {p}: run "
                          "`python -m block_diffusion_drafter_layers_amd.build` first")
    lib = ctypes.CDLL(p)
    P = ctypes.POINTER
    lib.dflash_workspace_bytes.restype = ctypes.c_size_t
    lib.dflash_workspace_bytes.argtypes = [P(dflash_config), _i32, _i32, _i32]
    lib.dflash_fuse_inject.restype = ctypes.c_int
    lib.dflash_fuse_inject.argtypes = [P(dflash_config), P(dflash_weights), _pvp, _pi32, _pi32,
                                       _i32, P(dflash_kv), _vp, ctypes.c_size_t,
                                       P(dflash_debug), _vp]
    lib.dflash_draft_block.restype = ctypes.c_int
    lib.dflash_draft_block.argtypes = [P(dflash_config), P(dflash_weights), P(dflash_kv), _pi32,
                                       _i32, _pi32, _vp, ctypes.c_size_t, P(dflash_debug), _vp]
    lib.dflash_draft_block_sampled.restype = ctypes.c_int
    lib.dflash_draft_block_sampled.argtypes = [P(dflash_config), P(dflash_weights), P(dflash_kv),
                                               _pi32, _i32, P(dflash_sampling), _pi32, _vp,
                                               ctypes.c_size_t, P(dflash_debug), _vp]
    lib.dflash_accept_trim.restype = ctypes.c_int
    lib.dflash_accept_trim.argtypes = [P(dflash_config), _pi32, _pi32, _i32, _pi32, _pi32,
                                       P(dflash_kv), _vp]
    lib.dflash_draft_block_noalloc.restype = ctypes.c_int
    lib.dflash_draft_block_noalloc.argtypes = [P(dflash_config), P(dflash_weights), P(dflash_kv),
                                               _pi32, _i32, _pi32, P(dflash_debug), _vp]
    lib.dflash_target_verify.restype = ctypes.c_int
    lib.dflash_target_verify.argtypes = [P(dflash_config), P(dflash_weights), P(dflash_kv), _pi32,
                                         _i32, _vp, _pvp, _pi32, _vp, ctypes.c_size_t, _vp]
    lib.dflash_fuse_inject_input_workspace_bytes.restype = ctypes.c_size_t
    lib.dflash_fuse_inject_input_workspace_bytes.argtypes = [P(dflash_config), _i32, _i32, _i32]
    lib.dflash_fuse_inject_input.restype = ctypes.c_int
    lib.dflash_fuse_inject_input.argtypes = [P(dflash_config), P(dflash_weights), _pvp, _pi32,
                                             _pi32, _i32, _i32, P(dflash_kv), _vp,
                                             ctypes.c_size_t, P(dflash_debug), _vp]
    lib.dflash_pack_weight.restype = ctypes.c_int
    lib.dflash_pack_weight.argtypes = [_vp, _i32, _i32, _vp, _pi32, _vp]
    lib.dflash_pack_weights.restype = ctypes.c_int
    lib.dflash_pack_weights.argtypes = [P(dflash_config), P(dflash_weights), P(dflash_weights),
                                        _pi32, _vp]
    lib.dflash_strerror.restype = ctypes.c_char_p
    lib.dflash_strerror.argtypes = [ctypes.c_int]
    if path is None:
        _lib = lib
    return lib


def _ref(x):
    return None if x is None else ctypes.byref(x)


def dflash_workspace_bytes(cfg: dflash_config, batch: int, max_rows: int, max_ctx: int) -> int:
    return int(load_library().dflash_workspace_bytes(ctypes.byref(cfg), batch, max_rows, max_ctx))


def dflash_fuse_inject(cfg, w, feats, row_start, row_count, total_rows, kv, ws, ws_bytes,
                       dbg=None, stream=None) -> int:
    return int(load_library().dflash_fuse_inject(ctypes.byref(cfg), ctypes.byref(w), feats,
                                                 row_start, row_count, total_rows,
                                                 ctypes.byref(kv), ws, ws_bytes, _ref(dbg),
                                                 stream))


def dflash_draft_block(cfg, w, kv, last_tok, block, draft_ids, ws, ws_bytes, dbg=None,
                       stream=None) -> int:
    return int(load_library().dflash_draft_block(ctypes.byref(cfg), ctypes.byref(w),
                                                 ctypes.byref(kv), last_tok, block, draft_ids,
                                                 ws, ws_bytes, _ref(dbg), stream))


def dflash_draft_block_sampled(cfg, w, kv, last_tok, block, smp, draft_ids, ws, ws_bytes,
                               dbg=None, stream=None) -> int:
    return int(load_library().dflash_draft_block_sampled(ctypes.byref(cfg), ctypes.byref(w),
                                                         ctypes.byref(kv), last_tok, block,
                                                         _ref(smp), draft_ids, ws, ws_bytes,
                                                         _ref(dbg), stream))


def dflash_draft_block_noalloc(cfg, w, kv, last_tok, block, draft_ids, dbg=None,
                               stream=None) -> int:
    return int(load_library().dflash_draft_block_noalloc(ctypes.byref(cfg), ctypes.byref(w),
                                                         ctypes.byref(kv), last_tok, block,
                                                         draft_ids, _ref(dbg), stream))


def dflash_target_verify(cfg, w, kv, block_ids, block, capture, feats_out, target_ids, ws,
                         ws_bytes, stream=None) -> int:
    return int(load_library().dflash_target_verify(ctypes.byref(cfg), ctypes.byref(w),
                                                   ctypes.byref(kv), block_ids, block, capture,
                                                   feats_out, target_ids, ws, ws_bytes, stream))


def dflash_fuse_inject_input_workspace_bytes(cfg, batch: int, max_rows: int, max_ctx: int) -> int:
    return int(load_library().dflash_fuse_inject_input_workspace_bytes(ctypes.byref(cfg), batch,
                                                                       max_rows, max_ctx))


def dflash_fuse_inject_input(cfg, w, feats, row_start, row_count, rows_max, total_rows, kv, ws,
                             ws_bytes, dbg=None, stream=None) -> int:
    return int(load_library().dflash_fuse_inject_input(ctypes.byref(cfg), ctypes.byref(w), feats,
                                                       row_start, row_count, rows_max, total_rows,
                                                       ctypes.byref(kv), ws, ws_bytes, _ref(dbg),
                                                       stream))


def dflash_accept_trim(cfg, draft_ids, target_ids, block, accept_len, bonus, kv,
                       stream=None) -> int:
    return int(load_library().dflash_accept_trim(ctypes.byref(cfg), draft_ids, target_ids, block,
                                                 accept_len, bonus, ctypes.byref(kv), stream))


def dflash_pack_weight(src, n, k, dst, n_overflow=None, stream=None) -> int:
    return int(load_library().dflash_pack_weight(src, n, k, dst, n_overflow, stream))


def dflash_pack_weights(cfg, src, dst, n_overflow=None, stream=None) -> int:
    return int(load_library().dflash_pack_weights(ctypes.byref(cfg), ctypes.byref(src),
                                                  ctypes.byref(dst), n_overflow, stream))


def dflash_strerror(code: int) -> str:
    return load_library().dflash_strerror(int(code)).decode()


class DFlashError(RuntimeError):
    def __init__(self, call: str, code: int):
        super().__init__(f"{call} failed: {code} ({dflash_strerror(code)})")
        self.code = code


def check(call: str, code: int) -> None:
    if code != DFLASH_OK:
        raise DFlashError(call, code)


def ptr_array(ptrs) -> ctypes.Array:
    """A host array of device pointers (kept alive by the caller)."""
    arr = (ctypes.c_void_p * len(ptrs))(*[int(p) for p in ptrs])
    return arr


def as_pvp(arr) -> ctypes.POINTER(ctypes.c_void_p):
    return ctypes.cast(arr, _pvp)
