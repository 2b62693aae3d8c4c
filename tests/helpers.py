"""Shared test helpers: building append steps from the seeded generator."""
from __future__ import annotations

from typing import List, Sequence

import numpy as np
import torch

from synth import Workload


def ring_slots(wl: Workload) -> int:
    return 0 if wl.n_loops == 1 else min(wl.window, wl.capacity)


def step_arrays(wl: Workload, layer: int, L0: Sequence[int], n_new: Sequence[int]):
    """Arrays for one append of n_new[b] tokens after L0[b] committed ones.

    Returns deep_k, deep_v [B][Hkv][T][d] and win_k, win_v [B][R-1][Hkv][U][d]
    (the last min(n_new[b], ring slots) tokens, oldest first), T = max n_new.
    """
    B, R, H, d = wl.batch, wl.n_loops, wl.n_heads_kv, wl.head_dim
    wr = ring_slots(wl)
    T = max(max(n_new), 1)
    U = max(min(max(n_new), wr), 1)
    dk = np.zeros((B, H, T, d), np.uint16)
    dv = np.zeros_like(dk)
    wk = np.zeros((B, max(R - 1, 1), H, U, d), np.uint16)
    wv = np.zeros_like(wk)
    for b in range(B):
        n = n_new[b]
        if n == 0:
            continue
        a, c = wl.deep_planes(layer, b, L0[b], L0[b] + n)
        dk[b, :, :n] = a
        dv[b, :, :n] = c
        nw = min(n, wr)
        if nw > 0:
            x, y = wl.planes(layer, b, L0[b] + n - nw, L0[b] + n, range(1, R))
            wk[b, :, :, :nw] = x
            wv[b, :, :, :nw] = y
    return dk, dv, wk, wv


def split_steps(lens: Sequence[int], n_steps: int, rng: np.random.Generator) -> List[List[int]]:
    """Split each committed length into n_steps random appends."""
    out = [[0] * len(lens) for _ in range(n_steps)]
    for b, L in enumerate(lens):
        cuts = sorted(rng.integers(0, L + 1, size=n_steps - 1).tolist()) if n_steps > 1 else []
        edges = [0] + cuts + [L]
        for s in range(n_steps):
            out[s][b] = edges[s + 1] - edges[s]
    return out


# Named launch choices for fixtures that run every kernel variant on the same
# inputs (fields of the C ABI's ripe_tuning; absent fields are the planner's).
TUNINGS = {
    "auto": {"items_target": 1},
    "planner": None,
    "keys": {"kernel": 1, "items_target": 1},
    "keys-4waves": {"kernel": 1, "keys_waves": 4},
    "keys-8waves": {"kernel": 1, "keys_waves": 8, "items_target": 1},
    "rows": {"kernel": 2, "items_target": 1},
    "rows-2tiles": {"kernel": 2, "row_tiles": 2, "items_target": 1},
    "rows-private": {"kernel": 2, "private_waves": 2, "items_target": 1},
    "rows-noprivate": {"kernel": 2, "private_waves": 1, "items_target": 1},
    "keys-chunked": {"kernel": 1, "items_target": 100000, "min_chunk": 32},
    "keys-8waves-chunked": {"kernel": 1, "keys_waves": 8, "items_target": 100000, "min_chunk": 32},
    "rows-chunked": {"kernel": 2, "items_target": 100000, "min_chunk": 32},
    "rows-planner": {"kernel": 2},
    "keys-8waves-planner": {"kernel": 1, "keys_waves": 8},
}


def use_tuning(monkeypatch, name: str) -> None:
    """Make every RipeCache created from now on use the named launch choices."""
    from self_speculative_verify_amd import cache as cache_mod
    monkeypatch.setattr(cache_mod, "DEFAULT_TUNING", TUNINGS[name])


# Guard bands: a buffer handed to the library as the middle of a larger
# allocation whose edges hold a fixed byte pattern.
GUARD = 4096          # bytes on each side (keeps the middle 256-byte aligned)
PATTERN = 0xA5        # every guard byte; a float of four such bytes is -2.9e-16


def guarded(nbytes: int, device="cuda"):
    """(whole allocation, middle nbytes) with the pattern everywhere."""
    full = torch.full((2 * GUARD + nbytes,), PATTERN, dtype=torch.uint8, device=device)
    return full, full[GUARD:GUARD + nbytes]


def edges_intact(full: torch.Tensor, nbytes: int) -> bool:
    head = full[:GUARD]
    tail = full[GUARD + nbytes:]
    return (tail.numel() == GUARD and bool(torch.all(head == PATTERN).item())
            and bool(torch.all(tail == PATTERN).item()))


def all_written(middle: torch.Tensor) -> bool:
    """No 4-byte word of the middle still holds the pattern."""
    words = middle.view(torch.int32)
    pat = int(np.array([PATTERN] * 4, np.uint8).view(np.int32)[0])
    return not bool(torch.any(words == pat).item())
