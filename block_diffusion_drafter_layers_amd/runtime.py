"""Device-side state of a drafter: torch allocates the memory, the library computes.

``DeviceDrafter`` uploads the weights, allocates the per-layer K/V cache, the
len/base/err words and the workspace with torch, fills the C structs of
``include/dflash.h`` with their addresses and forwards the three calls.  No
step of the method runs here.
"""

from __future__ import annotations

import ctypes
from typing import Dict, Optional, Sequence

import numpy as np
import torch

from . import binding as B

LAYER_FIELDS = ("in_norm", "wq", "wk", "wv", "wo", "post_norm", "w_gate", "w_up", "w_down")
# matrices the bf16-storage kernels stream as fp16 in the fragment-packed layout
PACKED_FIELDS = ("lm_head", "fc", "wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


def is_packed_name(name: str) -> bool:
    return name.split(".")[-1] in PACKED_FIELDS


def pack_weight(t: torch.Tensor, n_overflow: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Row-major bf16 [n, k] device tensor -> a new fp16 tensor in the fragment-packed layout
    (n_overflow: a device int32 counter the call adds the non-fp16 elements to)."""
    assert t.dtype == torch.bfloat16 and t.dim() == 2 and t.is_contiguous()
    out = torch.empty(t.shape, dtype=torch.float16, device=t.device)
    B.check("dflash_pack_weight", B.dflash_pack_weight(
        t.data_ptr(), t.shape[0], t.shape[1], out.data_ptr(),
        n_overflow=None if n_overflow is None else n_overflow.data_ptr(), stream=_stream_ptr()))
    return out


def _stream_ptr() -> int:
    return torch.cuda.current_stream().cuda_stream


def make_config(dims) -> B.dflash_config:
    """dims: any object with the DrafterDims attribute names."""
    c = B.dflash_config()
    for n in ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "inter", "vocab",
              "n_feat_layers", "feat_hidden", "block_max"):
        setattr(c, n, int(getattr(dims, n)))
    c.mask_token_id = int(getattr(dims, "mask_token_id", dims.vocab - 1))
    c.rope_theta = float(dims.rope_theta)
    c.rms_eps = float(dims.rms_eps)
    c.dtype = B.DFLASH_BF16 if dims.dtype == "bf16" else B.DFLASH_F32
    return c


def to_device(arr: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Host array (bf16 bits as uint16, or float32) -> device tensor of the storage type."""
    if dtype == "bf16":
        assert arr.dtype == np.uint16
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device)
        return t.view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


class LaunchTimer:
    """HIP events the library records around every launch of one class
    (DFLASH_TIME_GEMM / _LMHEAD / _ATTN), for up to ``max_launches`` launches.

    The events are created without the system-scope fence (hipEventDisableSystemFence):
    they only time, and a fenced event would add a cache write-back to every
    bracketed kernel.  They live as long as the process (a few dozen handles)."""

    _FLAGS = 0x20000000  # hipEventDisableSystemFence (timing stays enabled)

    def __init__(self, timed: int, max_launches: int):
        lib = B.load_library()  # resolves the HIP runtime the library itself uses
        self._create = lib.hipEventCreateWithFlags
        self._create.restype = ctypes.c_int
        self._create.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self._elapsed = lib.hipEventElapsedTime
        self._elapsed.restype = ctypes.c_int
        self._elapsed.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.events = []
        for _ in range(2 * max_launches):
            ev = ctypes.c_void_p()
            if self._create(ctypes.byref(ev), self._FLAGS) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.events.append(ev.value)
        self.arr = B.ptr_array(self.events)
        self.dbg = B.dflash_debug()
        self.dbg.events = B.as_pvp(self.arr)
        self.dbg.n_events = len(self.events)
        self.dbg.n_used = 0
        self.dbg.timed = timed

    def reset(self) -> None:
        self.dbg.n_used = 0

    def durations_ms(self):
        torch.cuda.synchronize()
        out = []
        for i in range(self.dbg.n_used):
            ms = ctypes.c_float()
            if self._elapsed(ctypes.byref(ms), self.events[2 * i], self.events[2 * i + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append(ms.value)
        return out


class DeviceDrafter:
    """``weights``: name -> row-major host array or device tensor (bf16 matrices
    are packed on upload), or, with ``packed=True``, the ``.w`` dict of another
    DeviceDrafter of the same dims (shared as is)."""

    def __init__(self, dims, weights: Dict[str, object], batch: int, max_ctx: int,
                 max_rows: int, device="cuda:0", packed: bool = False):
        B.load_library()
        self.dims = dims
        self.device = torch.device(device)
        self.batch = int(batch)
        self.max_ctx = int(max_ctx)
        self.max_rows = int(max_rows)
        self.cfg = make_config(dims)
        self.tdtype = torch.bfloat16 if dims.dtype == "bf16" else torch.float32
        self.w: Dict[str, torch.Tensor] = {}
        bf16 = dims.dtype == "bf16"
        self._keep = []
        # elements of the bf16 matrices that did not fit fp16 when packed (device int32)
        self.pack_overflow = torch.zeros(1, dtype=torch.int32, device=self.device)
        for name, arr in weights.items():
            t = arr if isinstance(arr, torch.Tensor) else to_device(arr, dims.dtype, self.device)
            self.w[name] = t
        if bf16 and not packed:
            # the one-time preparation of a bf16 checkpoint: every matrix packed by the
            # library into fp16 buffers allocated here (dflash_pack_weights)
            src = self._struct(self.w, B.DFLASH_LAYOUT_ROWMAJOR)
            out = {n: (torch.empty(t.shape, dtype=torch.float16, device=self.device)
                       if is_packed_name(n) else t) for n, t in self.w.items()}
            dst = self._struct(out, B.DFLASH_LAYOUT_PACKED)
            B.check("dflash_pack_weights", B.dflash_pack_weights(
                self.cfg, src, dst, self.pack_overflow.data_ptr(), _stream_ptr()))
            torch.cuda.current_stream().synchronize()  # before the row-major copies go
            self._keep = []
            self.w = out
        self.wstruct = self._struct(self.w, B.DFLASH_LAYOUT_PACKED if bf16
                                    else B.DFLASH_LAYOUT_ROWMAJOR)
        d = dims
        # the K/V cache is fp16 for the bf16 storage type, fp32 for fp32
        self.cache_dtype = torch.float16 if bf16 else torch.float32
        self.k = [torch.zeros(batch, d.n_kv_heads, max_ctx, d.head_dim, dtype=self.cache_dtype,
                              device=self.device) for _ in range(d.n_layers)]
        self.v = [torch.zeros(batch, d.n_kv_heads, d.head_dim, max_ctx, dtype=self.cache_dtype,
                              device=self.device) for _ in range(d.n_layers)]
        self.len = torch.zeros(batch, dtype=torch.int32, device=self.device)
        self.base = torch.full((batch,), -1, dtype=torch.int32, device=self.device)
        self.err = torch.zeros(1, dtype=torch.int32, device=self.device)
        kv = B.dflash_kv()
        ka = B.ptr_array([t.data_ptr() for t in self.k])
        va = B.ptr_array([t.data_ptr() for t in self.v])
        self._keep += [ka, va]
        kv.k, kv.v = B.as_pvp(ka), B.as_pvp(va)
        kv.len, kv.base, kv.err = self.len.data_ptr(), self.base.data_ptr(), self.err.data_ptr()
        kv.batch, kv.max_ctx = batch, max_ctx
        self.kv = kv
        self.ws_bytes = B.dflash_workspace_bytes(self.cfg, batch, max_rows, max_ctx)
        if self.ws_bytes == 0:
            raise B.DFlashError("dflash_workspace_bytes", B.DFLASH_EINVAL)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)

    def _struct(self, w: Dict[str, torch.Tensor], layout: int) -> B.dflash_weights:
        """dflash_weights with the addresses of ``w`` (host pointer arrays kept alive)."""
        ws = B.dflash_weights()
        ws.layout = layout
        for n in ("embed", "fc", "fc_norm", "final_norm", "lm_head"):
            setattr(ws, n, w[n].data_ptr() if n in w else None)  # a target model has no fusion
        for f in LAYER_FIELDS:
            arr = B.ptr_array([w[f"l{l}.{f}"].data_ptr() for l in range(self.dims.n_layers)])
            self._keep.append(arr)
            setattr(ws, f, B.as_pvp(arr))
        return ws

    # ---- the three calls ------------------------------------------------------------------
    def fuse_inject(self, feats: Sequence[torch.Tensor], row_start: torch.Tensor,
                    row_count: torch.Tensor, total_rows: int,
                    fused_dbg: Optional[torch.Tensor] = None,
                    timer: Optional[LaunchTimer] = None) -> None:
        fa = B.ptr_array([f.data_ptr() for f in feats])
        dbg = timer.dbg if timer is not None else None
        if fused_dbg is not None:
            dbg = B.dflash_debug()
            dbg.fused = fused_dbg.data_ptr()
        rc = B.dflash_fuse_inject(self.cfg, self.wstruct, B.as_pvp(fa), row_start.data_ptr(),
                                  row_count.data_ptr(), int(total_rows), self.kv,
                                  self.ws.data_ptr(), self.ws_bytes, dbg, _stream_ptr())
        B.check("dflash_fuse_inject", rc)

    def draft(self, last_tok: torch.Tensor, block: int, draft_ids: torch.Tensor,
              final_hidden: Optional[torch.Tensor] = None,
              logits: Optional[torch.Tensor] = None,
              timer: Optional[LaunchTimer] = None,
              temperature: float = 0.0, seed: int = 0, offset: int = 0,
              top2: Optional[torch.Tensor] = None, noalloc: bool = False) -> None:
        """Greedy draft (dflash_draft_block), or with temperature > 0 the sampled
        draft (dflash_draft_block_sampled, Philox key seed, counter word offset); noalloc:
        the greedy draft on the library's own scratch (dflash_draft_block_noalloc)."""
        dbg = timer.dbg if timer is not None else None
        if final_hidden is not None or logits is not None or top2 is not None:
            dbg = B.dflash_debug()
            dbg.final_hidden = None if final_hidden is None else final_hidden.data_ptr()
            dbg.logits = None if logits is None else logits.data_ptr()
            dbg.top2 = None if top2 is None else top2.data_ptr()
        if noalloc:
            assert temperature <= 0, "the allocation-free entry point drafts greedily"
            rc = B.dflash_draft_block_noalloc(self.cfg, self.wstruct, self.kv, last_tok.data_ptr(),
                                              int(block), draft_ids.data_ptr(), dbg, _stream_ptr())
            B.check("dflash_draft_block_noalloc", rc)
            return
        if temperature > 0:
            smp = B.dflash_sampling(float(temperature), int(seed), int(offset))
            rc = B.dflash_draft_block_sampled(self.cfg, self.wstruct, self.kv, last_tok.data_ptr(),
                                              int(block), smp, draft_ids.data_ptr(),
                                              self.ws.data_ptr(), self.ws_bytes, dbg,
                                              _stream_ptr())
            B.check("dflash_draft_block_sampled", rc)
            return
        rc = B.dflash_draft_block(self.cfg, self.wstruct, self.kv, last_tok.data_ptr(), int(block),
                                  draft_ids.data_ptr(), self.ws.data_ptr(), self.ws_bytes, dbg,
                                  _stream_ptr())
        B.check("dflash_draft_block", rc)

    def verify(self, block_ids: torch.Tensor, block: int, target_ids: torch.Tensor,
               capture=None, feats_out=None) -> None:
        """dflash_target_verify: this object holding a (target) model, one causal pass
        over block_ids [batch, block]; the next token of every row into target_ids and,
        with capture (layer ids), the states leaving those layers into feats_out."""
        cap = None
        fo = None
        if capture is not None:
            cap = (ctypes.c_int32 * len(capture))(*[int(c) for c in capture])
            fo = B.ptr_array([t.data_ptr() for t in feats_out])
        rc = B.dflash_target_verify(self.cfg, self.wstruct, self.kv, block_ids.data_ptr(),
                                    int(block), cap, None if fo is None else B.as_pvp(fo),
                                    target_ids.data_ptr(), self.ws.data_ptr(), self.ws_bytes,
                                    _stream_ptr())
        B.check("dflash_target_verify", rc)

    def fuse_inject_input(self, feats: Sequence[torch.Tensor], row_start: torch.Tensor,
                          row_count: torch.Tensor, rows_max: int, total_rows: int,
                          fused_dbg: Optional[torch.Tensor] = None) -> None:
        """dflash_fuse_inject_input: the input-fusion variant of the injection (its
        workspace is allocated on first use)."""
        need = B.dflash_fuse_inject_input_workspace_bytes(self.cfg, self.batch, self.max_rows,
                                                          self.max_ctx)
        if getattr(self, "ws_input", None) is None or self.ws_input.numel() < need:
            self.ws_input = torch.empty(need, dtype=torch.uint8, device=self.device)
        fa = B.ptr_array([f.data_ptr() for f in feats])
        dbg = None
        if fused_dbg is not None:
            dbg = B.dflash_debug()
            dbg.fused = fused_dbg.data_ptr()
        rc = B.dflash_fuse_inject_input(self.cfg, self.wstruct, B.as_pvp(fa), row_start.data_ptr(),
                                        row_count.data_ptr(), int(rows_max), int(total_rows),
                                        self.kv, self.ws_input.data_ptr(), self.ws_input.numel(),
                                        dbg, _stream_ptr())
        B.check("dflash_fuse_inject_input", rc)

    def accept_trim(self, draft_ids: torch.Tensor, target_ids: torch.Tensor, block: int,
                    accept_len: torch.Tensor, bonus: torch.Tensor) -> None:
        rc = B.dflash_accept_trim(self.cfg, draft_ids.data_ptr(), target_ids.data_ptr(), int(block),
                                  accept_len.data_ptr(), bonus.data_ptr(), self.kv, _stream_ptr())
        B.check("dflash_accept_trim", rc)

    # ---- the cache as [len, Hkv, d] fp32 rows, for inspection -----------------------------
    def cache_rows(self, layer: int, seq: int, n: int):
        """fp32: K is [Hkv][max_ctx][d], V [Hkv][d][max_ctx].  fp16 (bf16 storage):
        both are fragment-packed per (sequence, kv head) as include/dflash.h describes."""
        d, L = self.dims.head_dim, self.max_ctx
        if self.cache_dtype == torch.float32:
            k = self.k[layer][seq, :, :n, :].permute(1, 0, 2)
            v = self.v[layer][seq, :, :, :n].permute(2, 0, 1)
            return k, v
        hk = self.k[layer].shape[1]
        # K fragment (g, c): lane (lq, lr), slot j = K[16g + lr][32c + 8 lq + j]
        k = self.k[layer][seq].reshape(hk, L // 16, d // 32, 4, 16, 8)
        k = k.permute(0, 1, 4, 2, 3, 5).reshape(hk, L, d)[:, :n].permute(1, 0, 2)
        # V fragment (h, e): lane (g, dr), slot j = V[32h + key(g, j)][16e + dr]
        v = self.v[layer][seq].reshape(hk, L // 32, d // 16, 4, 16, 8)
        v = v.permute(0, 1, 2, 4, 3, 5).reshape(hk, L // 32, d // 16, 16, 32)   # [..., g*8 + j]
        idx = torch.tensor([(kk // 4) * 8 + kk % 4 if kk < 16 else ((kk - 16) // 4) * 8 + 4 + (kk - 16) % 4
                            for kk in range(32)], device=v.device)
        v = v.index_select(4, idx)                                              # [..., key]
        v = v.permute(0, 1, 4, 2, 3).reshape(hk, L, d)[:, :n].permute(1, 0, 2)
        return k.float(), v.float()
