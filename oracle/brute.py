"""Brute-force RIPE cache simulation -- TEST INFRASTRUCTURE ONLY (tiny inputs).

An independent second implementation of the method, written without the byte
layout: the cache is a dictionary from (sequence, KV head, position, loop) to
the stored key and value vectors.

* append (RIPE abstract, fourth sentence: the deepest plane is kept for every
  position, all planes only inside a window of recent positions): every new
  position stores its loop-R plane; the last min(n_new, W) new positions also
  store loops 1..R-1; afterwards every entry (p, r < R) with p older than the
  W most recent committed positions is deleted ("collapsed" to loop R).
* verify: for each (row, head) it walks keys 0..L+i, picks the plane with the
  anchor rule, ASSERTS that the entry is still stored (so the rule is
  implementable from RIPE storage), and evaluates a naive softmax in Python
  floats.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

from synth import bf16_to_f32


class BruteCache:
    def __init__(self, n_loops: int, n_heads_q: int, n_heads_kv: int, head_dim: int,
                 window: int, batch: int, capacity: int, anchor: int = 0):
        self.R, self.Hq, self.H, self.d = n_loops, n_heads_q, n_heads_kv, head_dim
        self.W, self.B, self.cap, self.anchor = window, batch, capacity, anchor
        self.slots = min(window, capacity) if n_loops > 1 else 0
        self.lens: List[int] = [0] * batch
        self.store: Dict[Tuple[int, int, int, int], Tuple[np.ndarray, np.ndarray]] = {}

    def append(self, b: int, deep_k, deep_v, win_k, win_v) -> None:
        """deep_*: uint16 [H][n][d] (loop R); win_*: uint16 [R-1][H][nw][d],
        the last nw = min(n, slots) tokens at loops 1..R-1."""
        n = deep_k.shape[1]
        L0 = self.lens[b]
        assert L0 + n <= self.cap
        for t in range(n):
            for g in range(self.H):
                self.store[(b, g, L0 + t, self.R)] = (deep_k[g, t].copy(), deep_v[g, t].copy())
        nw = min(n, self.slots)
        for u in range(nw):
            p = L0 + n - nw + u
            for r in range(1, self.R):
                for g in range(self.H):
                    self.store[(b, g, p, r)] = (win_k[r - 1, g, u].copy(), win_v[r - 1, g, u].copy())
        self.lens[b] = L0 + n
        oldest_kept = self.lens[b] - self.slots
        for key in [k for k in self.store if k[0] == b and k[3] < self.R and k[2] < oldest_kept]:
            del self.store[key]

    def entries(self, b: int, g: int) -> int:
        return sum(1 for k in self.store if k[0] == b and k[1] == g)

    def verify_one(self, b: int, i: int, r: int, h: int, q, blk_k, blk_v,
                   sink_window=None) -> Tuple[np.ndarray, float]:
        """q: uint16 [d]; blk_*: uint16 [R][H][Dmax][d] of sequence b.
        sink_window = (n_sink, w): a windowed draft row keeps only the committed
        positions s < n_sink or s >= L + i - w (page "Windowed-MTP", abstract:
        sliding window plus attention sink on the draft's attention)."""
        L = self.lens[b]
        t = L + i
        beta = t - self.W if self.anchor == 0 else L - self.W
        g = h // (self.Hq // self.H)
        qf = [float(x) for x in bf16_to_f32(q)]
        keys, vals = [], []
        for s in range(t + 1):
            if s < L and sink_window is not None and not (s < sink_window[0] or s >= t - sink_window[1]):
                continue
            if s >= L:
                k, v = blk_k[r - 1, g, s - L], blk_v[r - 1, g, s - L]
            else:
                plane = r if s >= beta else self.R
                assert (b, g, s, plane) in self.store, f"entry {(s, plane)} is not stored"
                k, v = self.store[(b, g, s, plane)]
            keys.append([float(x) for x in bf16_to_f32(k)])
            vals.append([float(x) for x in bf16_to_f32(v)])
        scale = 1.0 / math.sqrt(self.d)
        scores = [sum(a * c for a, c in zip(qf, kk)) * scale for kk in keys]
        m = max(scores)
        z = sum(math.exp(s - m) for s in scores)
        out = np.zeros(self.d)
        for s, vv in zip(scores, vals):
            w = math.exp(s - m) / z
            for e in range(self.d):
                out[e] += w * vv[e]
        return out, m + math.log(z)

    def verify(self, rows: Sequence[Tuple[int, int]], q, blk_k, blk_v, sink_window=None):
        """q: uint16 [B][n_rows][Hq][d]; blk_*: uint16 [B][R][H][Dmax][d]."""
        out = np.zeros((self.B, len(rows), self.Hq, self.d))
        lse = np.zeros((self.B, len(rows), self.Hq))
        for b in range(self.B):
            for k, (i, r) in enumerate(rows):
                for h in range(self.Hq):
                    out[b, k, h], lse[b, k, h] = self.verify_one(b, i, r, h, q[b, k, h],
                                                                 blk_k[b], blk_v[b], sink_window)
        return out, lse
