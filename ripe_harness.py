"""Load seeded synthetic workloads into a GPU RIPE cache through the C ABI.

Used by the GPU tests, the smoke check and the benchmark.  Data comes from
``synth`` (the shared seeded generator); every write into the cache goes
through ``ripe_append``.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from self_speculative_verify_amd import RipeCache
from synth import Workload


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bfloat16 bits -> bfloat16 device tensor (bit copy)."""
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def make_cache(wl: Workload, device="cuda", window: Optional[int] = None,
               anchor: Optional[int] = None) -> RipeCache:
    return RipeCache(wl.n_layers, wl.n_loops, wl.n_heads_q, wl.n_heads_kv, wl.head_dim,
                     wl.window if window is None else window, wl.batch, wl.capacity,
                     wl.max_block, wl.anchor if anchor is None else anchor, device=device)


def ring_slots(cache: RipeCache) -> int:
    c = cache.cfg
    return 0 if c.n_loops == 1 else min(c.window, c.capacity)


def load_prefix(cache: RipeCache, wl: Workload, layers: Optional[Sequence[int]] = None,
                device="cuda") -> None:
    """Append every sequence's committed prefix (L_b tokens), one sequence per
    call: loop R of all L_b tokens and loops 1..R-1 of the last min(L_b, WR)."""
    B = wl.batch
    wr = ring_slots(cache)
    for layer in (range(wl.n_layers) if layers is None else layers):
        for b in range(B):
            L = wl.lens[b]
            if L == 0:
                continue
            nw = min(L, wr)
            dk, dv, wk, wv = wl.prefix(layer, b, n_win=nw)
            n_new = [0] * B
            n_new[b] = L
            H, d = wl.n_heads_kv, wl.head_dim
            tk = to_dev(dk, device).view(1, H, L, d).expand(B, H, L, d)
            tv = to_dev(dv, device).view(1, H, L, d).expand(B, H, L, d)
            if nw > 0:
                R1 = wl.n_loops - 1
                twk = to_dev(wk, device).view(1, R1, H, nw, d).expand(B, R1, H, nw, d)
                twv = to_dev(wv, device).view(1, R1, H, nw, d).expand(B, R1, H, nw, d)
            else:
                twk = twv = None
            cache.append(layer, n_new, tk, tv, twk, twv)


def verify_inputs(wl: Workload, layer: int, device="cuda"):
    """(q, blk_k, blk_v) device tensors of one layer's verify call."""
    q = to_dev(wl.queries(layer), device)
    bk, bv = wl.block(layer)
    return q, to_dev(bk, device), to_dev(bv, device)
