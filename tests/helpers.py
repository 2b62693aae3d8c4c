"""Shared test helpers: building append steps from the seeded generator."""
from __future__ import annotations

from typing import List, Sequence

import numpy as np

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
