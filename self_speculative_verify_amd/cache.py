"""A RIPE cache on the GPU: PyTorch-owned storage bound to a libripe handle.

Thin convenience layer over the C ABI (argument marshalling only).
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import torch

from . import ripe as _r

# Launch choices applied to every cache created while it is set (a dict of
# RipeTuning fields), for test fixtures that run every kernel variant.
DEFAULT_TUNING: Optional[dict] = None


class RipeCache:
    """Storage tensor + handle for one configuration.

    Tensors passed in are bfloat16 on the cache's device:
      append: deep_k/deep_v [B][Hkv][T][d]; win_k/win_v [B][R-1][Hkv][U][d]
      verify: q [B][n_rows][Hq][d]; blk_k/blk_v [B][R][Hkv][Dmax][d]
    """

    def __init__(self, n_layers: int, n_loops: int, n_heads_q: int, n_heads_kv: int,
                 head_dim: int, window: int, batch: int, capacity: int, max_block: int,
                 anchor: int = _r.RIPE_ANCHOR_QUERY, device="cuda", stream=None,
                 tuning: Optional[dict] = None, image: Optional[torch.Tensor] = None):
        """image: a copy of another cache's storage (same configuration) to
        resume from, e.g. a checkpoint on the host; None starts empty."""
        self.cfg = _r.config(n_layers, n_loops, n_heads_q, n_heads_kv, head_dim, window, batch,
                             capacity, max_block, anchor)
        nbytes = _r.ripe_cache_bytes(self.cfg)
        if nbytes == 0:
            raise ValueError("invalid RIPE configuration")
        self.storage = torch.empty(nbytes, dtype=torch.uint8, device=device)
        if self.storage.data_ptr() % 256:
            raise RuntimeError("storage allocation is not 256-byte aligned")
        if image is None:
            self.handle = _r.ripe_cache_create(self.cfg, self.storage, stream)
        else:
            if image.dtype != torch.uint8 or image.numel() != nbytes:
                raise ValueError("image must be %d bytes of uint8" % nbytes)
            self.storage.copy_(image.reshape(-1))
            if stream is not None:          # the copy ran on the current stream
                torch.cuda.current_stream(self.storage.device).synchronize()
            self.handle = _r.ripe_cache_open(self.cfg, self.storage, stream)
        self._ws = None
        tuning = DEFAULT_TUNING if tuning is None else tuning
        if tuning:
            _r.ripe_set_tuning(self.handle, tuning)

    # ------------------------------------------------------------------
    @property
    def batch(self) -> int:
        return self.cfg.batch

    def close(self) -> None:
        if getattr(self, "handle", None) is not None:
            _r.ripe_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def lengths(self, layer: int):
        return _r.ripe_get_lengths(self.handle, layer, self.cfg.batch)

    def section(self, which: int) -> torch.Tensor:
        """The bytes of one storage section (a view of the storage tensor)."""
        lo = _r.ripe_section_offset(self.cfg, which)
        ends = [_r.ripe_section_offset(self.cfg, s) for s in range(which + 1, _r.RIPE_SECTION_END + 1)]
        return self.storage[lo:min(ends)]

    # ------------------------------------------------------------------
    def append(self, layer: int, n_new: Sequence[int], deep_k: torch.Tensor,
               deep_v: torch.Tensor, win_k: Optional[torch.Tensor] = None,
               win_v: Optional[torch.Tensor] = None, stream=None) -> None:
        dk, dv = _r.kv_view(deep_k, "bhtd"), _r.kv_view(deep_v, "bhtd")
        if win_k is not None and win_k.numel() > 0:
            wk, wv = _r.kv_view(win_k, "bphtd"), _r.kv_view(win_v, "bphtd")
        else:
            wk = wv = _r.null_view()
        _r.ripe_append(self.handle, layer, list(n_new), dk, dv, wk, wv, stream)

    def workspace(self, n_rows: int) -> Optional[torch.Tensor]:
        n = _r.ripe_workspace_bytes(self.handle, n_rows)
        if n == 0:
            return None
        if self._ws is None or self._ws.numel() < n:
            self._ws = torch.empty(n, dtype=torch.uint8, device=self.storage.device)
        return self._ws

    def verify(self, layer: int, rows: Sequence[Tuple[int, int]], q: torch.Tensor,
               blk_k: torch.Tensor, blk_v: torch.Tensor, n_blk: int,
               out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
               stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
        B, Hq, d = self.cfg.batch, self.cfg.n_heads_q, self.cfg.head_dim
        n = len(rows)
        if out is None:
            out = torch.empty((B, n, Hq, d), dtype=torch.float32, device=q.device)
        if lse is None:
            lse = torch.empty((B, n, Hq), dtype=torch.float32, device=q.device)
        ws = self.workspace(n)
        _r.ripe_verify_attn(self.handle, layer, [i for i, _ in rows], [r for _, r in rows], q,
                            _r.kv_view(blk_k, "bphtd"), _r.kv_view(blk_v, "bphtd"), n_blk,
                            out, lse, ws, stream)
        return out, lse

    def draft(self, layer: int, rows: Sequence[Tuple[int, int]], q: torch.Tensor,
              blk_k: torch.Tensor, blk_v: torch.Tensor, n_blk: int, n_sink: int, w_draft: int,
              out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
              stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
        """Windowed draft attention: committed keys are the first n_sink
        positions and the w_draft positions before each query."""
        B, Hq, d = self.cfg.batch, self.cfg.n_heads_q, self.cfg.head_dim
        n = len(rows)
        if out is None:
            out = torch.empty((B, n, Hq, d), dtype=torch.float32, device=q.device)
        if lse is None:
            lse = torch.empty((B, n, Hq), dtype=torch.float32, device=q.device)
        _r.ripe_draft_attn(self.handle, layer, [i for i, _ in rows], [r for _, r in rows], q,
                           _r.kv_view(blk_k, "bphtd"), _r.kv_view(blk_v, "bphtd"), n_blk,
                           n_sink, w_draft, out, lse, stream)
        return out, lse
