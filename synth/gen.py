"""Seeded synthetic RIPE workloads (inputs only).

Every random number comes from a NumPy ``default_rng`` stream keyed by a
``SeedSequence`` of small integers, so any piece of a workload (one layer, one
sequence, one block of 64 positions) can be regenerated on its own.  Values are
drawn in float32 and rounded once to bfloat16 (round to nearest even); arrays
of bfloat16 are carried as ``uint16`` bit patterns.

Data recipe (the pages fix only the per-loop decay rates and the heavy-tail
statistic; shapes come from the named workloads):

* plane R (the deepest loop) of K and V: N(0, 1);
* plane r < R: ``K_r = K_R + rho**(R - r) * N(0, 1)`` (same for V), so the
  planes approach the last one geometrically as r grows (RIPE abstract, second
  sentence: 0.88 and 0.81 per loop);
* heavy tails: 1% of the tail positions, ``round(0.01 * (L - W))`` per
  (layer, sequence) with W the workload's own window, drawn without
  replacement from the tail [0, L - W), get their r < R offsets scaled by 30
  (RIPE abstract, third sentence: 1% of positions carry most of the
  deepest-plane error).  A RIPE cache with that window stores only the
  deepest plane of those positions; the full per-loop cache (or a wider
  window) reads their scaled planes;
* queries: N(0, 1).

The module holds no cache-layout or attention arithmetic.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "WINDOW_FULL", "ANCHOR_QUERY", "ANCHOR_CACHE", "POS_BLOCK",
    "f32_to_bf16", "bf16_to_f32", "Workload", "grid_rows", "wave_rows",
    "named_workload", "WORKLOAD_NAMES", "ragged_lengths",
]

WINDOW_FULL = 2**31 - 1          # "keep every position at full depth"
ANCHOR_QUERY = 0
ANCHOR_CACHE = 1
POS_BLOCK = 64                   # positions per random stream

# stream kinds (last-but-one seed word)
_K_BASE, _V_BASE, _K_OFF, _V_OFF, _Q, _HEAVY, _LENS = range(7)

_POOL = ThreadPoolExecutor(max_workers=8)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits (uint16) to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _normals(words: Sequence[int], n: int) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence([int(w) for w in words]))
    return rng.standard_normal(n, dtype=np.float32)


def grid_rows(n_blk: int, n_loops: int) -> List[Tuple[int, int]]:
    """The D x R verification grid: every block offset i at every loop r."""
    return [(i, r) for i in range(n_blk) for r in range(1, n_loops + 1)]


def wave_rows(width: int, n_loops: int, stride: int) -> List[Tuple[int, int]]:
    """A WaveFront diagonal: block offset j at loop R - stride*j (oldest deepest)."""
    rows = [(j, n_loops - stride * j) for j in range(width)]
    assert all(r >= 1 for _, r in rows)
    return rows


def ragged_lengths(seed: int, batch: int, lo: int, hi: int) -> List[int]:
    rng = np.random.default_rng(np.random.SeedSequence([seed, _LENS]))
    return [int(x) for x in rng.integers(lo, hi + 1, size=batch)]


@dataclasses.dataclass
class Workload:
    """Shape and data recipe of one synthetic verification workload."""
    name: str
    seed: int
    n_layers: int
    n_loops: int                 # R
    n_heads_q: int
    n_heads_kv: int
    head_dim: int
    window: int                  # W (WINDOW_FULL for the full R-plane cache)
    n_blk: int                   # D, draft block length
    lens: List[int]              # committed length per sequence
    rho: float
    rows: List[Tuple[int, int]]  # verified (block offset i, loop r) pairs
    heavy_frac: float = 0.0
    heavy_scale: float = 30.0
    anchor: int = ANCHOR_QUERY
    capacity: Optional[int] = None
    max_block: Optional[int] = None

    def __post_init__(self):
        if self.capacity is None:
            self.capacity = max(self.lens) + self.n_blk
        if self.max_block is None:
            self.max_block = self.n_blk

    # -- shapes ---------------------------------------------------------
    @property
    def batch(self) -> int:
        return len(self.lens)

    @property
    def n_rows(self) -> int:
        return len(self.rows)

    @property
    def ring_slots(self) -> int:
        return min(self.window, self.capacity)

    def replace(self, **kw) -> "Workload":
        d = dataclasses.asdict(self)
        d.update(kw)
        if ("lens" in kw or "n_blk" in kw) and "capacity" not in kw:
            d["capacity"] = None      # recomputed from the new shape
        if "n_blk" in kw and "max_block" not in kw:
            d["max_block"] = None
        return Workload(**d)

    # -- random pieces --------------------------------------------------
    def _block_base(self, layer: int, b: int, kind: int, pb: int) -> np.ndarray:
        n = POS_BLOCK * self.n_heads_kv * self.head_dim
        x = _normals([self.seed, layer, b, kind, pb], n)
        return x.reshape(POS_BLOCK, self.n_heads_kv, self.head_dim)

    def _block_off(self, layer: int, b: int, kind: int, pb: int) -> np.ndarray:
        nr = self.n_loops - 1
        n = POS_BLOCK * nr * self.n_heads_kv * self.head_dim
        x = _normals([self.seed, layer, b, kind, pb], n)
        return x.reshape(POS_BLOCK, nr, self.n_heads_kv, self.head_dim)

    def heavy_positions(self, layer: int, b: int) -> np.ndarray:
        """Heavy-tail positions of a sequence: drawn from its tail [0, L - W)
        (W: the workload's window)."""
        tail = max(self.lens[b] - min(self.window, self.lens[b]), 0)
        n = int(round(self.heavy_frac * tail))
        if n == 0:
            return np.zeros(0, dtype=np.int64)
        rng = np.random.default_rng(np.random.SeedSequence([self.seed, layer, b, _HEAVY]))
        return np.sort(rng.choice(tail, size=n, replace=False)).astype(np.int64)

    def planes(self, layer: int, b: int, p0: int, p1: int,
               loops: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
        """K and V of positions [p0, p1) at the given loops (1-based).

        Returns two uint16 arrays of shape [len(loops)][Hkv][p1 - p0][d].
        """
        loops = list(loops)
        n = p1 - p0
        H, dd, R = self.n_heads_kv, self.head_dim, self.n_loops
        outk = np.zeros((len(loops), H, n, dd), dtype=np.uint16)
        outv = np.zeros_like(outk)
        if n <= 0:
            return outk, outv
        heavy = set(self.heavy_positions(layer, b).tolist())
        need_off = any(r < R for r in loops)
        blocks = list(range(p0 // POS_BLOCK, (p1 - 1) // POS_BLOCK + 1))

        def work(pb):
            lo = max(p0, pb * POS_BLOCK)
            hi = min(p1, (pb + 1) * POS_BLOCK)
            s = slice(lo - pb * POS_BLOCK, hi - pb * POS_BLOCK)
            kb = self._block_base(layer, b, _K_BASE, pb)[s]
            vb = self._block_base(layer, b, _V_BASE, pb)[s]
            if need_off:
                ko = self._block_off(layer, b, _K_OFF, pb)[s]
                vo = self._block_off(layer, b, _V_OFF, pb)[s]
                scale = np.ones(hi - lo, dtype=np.float32)
                for p in range(lo, hi):
                    if p in heavy:
                        scale[p - lo] = self.heavy_scale
            for a, r in enumerate(loops):
                if r == R:
                    kr, vr = kb, vb
                else:
                    c = (np.float32(self.rho) ** np.float32(R - r)) * scale
                    kr = kb + c[:, None, None] * ko[:, r - 1]
                    vr = vb + c[:, None, None] * vo[:, r - 1]
                outk[a, :, lo - p0:hi - p0] = f32_to_bf16(kr).transpose(1, 0, 2)
                outv[a, :, lo - p0:hi - p0] = f32_to_bf16(vr).transpose(1, 0, 2)

        list(_POOL.map(work, blocks))
        return outk, outv

    def deep_planes(self, layer: int, b: int, p0: int, p1: int):
        """Plane R of positions [p0, p1): two uint16 arrays [Hkv][n][d]."""
        k, v = self.planes(layer, b, p0, p1, [self.n_loops])
        return k[0], v[0]

    def queries(self, layer: int) -> np.ndarray:
        """bf16 queries [B][n_rows][Hq][d] for one layer's verify call."""
        shape = (self.batch, self.n_rows, self.n_heads_q, self.head_dim)
        x = _normals([self.seed, layer, _Q], int(np.prod(shape)))
        return f32_to_bf16(x).reshape(shape)

    def block(self, layer: int) -> Tuple[np.ndarray, np.ndarray]:
        """Draft-block planes: uint16 [B][R][Hkv][max_block][d] (zero past D)."""
        B, R, H, dd = self.batch, self.n_loops, self.n_heads_kv, self.head_dim
        k = np.zeros((B, R, H, self.max_block, dd), dtype=np.uint16)
        v = np.zeros_like(k)
        for b in range(B):
            L = self.lens[b]
            kk, vv = self.planes(layer, b, L, L + self.n_blk, range(1, R + 1))
            k[b, :, :, :self.n_blk] = kk
            v[b, :, :, :self.n_blk] = vv
        return k, v

    def prefix(self, layer: int, b: int, n_win: Optional[int] = None):
        """What an append of the committed prefix of sequence b carries.

        Returns (deep_k, deep_v, win_k, win_v): plane R of all L positions
        ([Hkv][L][d]) and planes 1..R-1 of the last ``n_win`` positions
        ([R-1][Hkv][n_win][d]); ``n_win`` defaults to min(L, ring slots).
        """
        L = self.lens[b]
        if n_win is None:
            n_win = min(L, self.ring_slots) if self.n_loops > 1 else 0
        dk, dv = self.deep_planes(layer, b, 0, L)
        if n_win > 0:
            wk, wv = self.planes(layer, b, L - n_win, L, range(1, self.n_loops))
        else:
            shp = (max(self.n_loops - 1, 0), self.n_heads_kv, 0, self.head_dim)
            wk = np.zeros(shp, dtype=np.uint16)
            wv = np.zeros(shp, dtype=np.uint16)
        return dk, dv, wk, wv


WORKLOAD_NAMES = ("tiny", "huginn", "gqa", "ragged", "wave")


def named_workload(name: str, **overrides) -> Workload:
    """The five workloads the verification path is measured on.

    tiny:   1 layer, R=8, 2 heads, d=64, L=128, W=16, D=4, batch 1.
    huginn: 4 layers, R=32, 55 heads (MHA), d=96, L=1024, W=64, D=8, batch 1,
            rho=0.88, heavy tails (1% of positions, offsets x30).
    gqa:    4 layers, R=32, 32 query / 8 KV heads, d=128, L=4096, W=0, D=8,
            batch 4, rho=0.81.
    ragged: 4 layers, R=32, 32/8 heads, d=128, W=64, D=8, batch 8,
            lengths uniform in [1024, 32768], rho=0.88.
    wave:   4 layers, R=32, 55 heads, d=96, L=8192, W=64, batch 1; one
            position per depth, block offset j at loop 32 - 4j, j = 0..7.
    """
    if name == "tiny":
        wl = Workload(name, 1001, 1, 8, 2, 2, 64, 16, 4, [128], 0.88, grid_rows(4, 8))
    elif name == "huginn":
        wl = Workload(name, 1002, 4, 32, 55, 55, 96, 64, 8, [1024], 0.88,
                      grid_rows(8, 32), heavy_frac=0.01)
    elif name == "gqa":
        wl = Workload(name, 1003, 4, 32, 32, 8, 128, 0, 8, [4096] * 4, 0.81,
                      grid_rows(8, 32))
    elif name == "ragged":
        lens = ragged_lengths(1004, 8, 1024, 32768)
        wl = Workload(name, 1004, 4, 32, 32, 8, 128, 64, 8, lens, 0.88,
                      grid_rows(8, 32))
    elif name == "wave":
        wl = Workload(name, 1005, 4, 32, 55, 55, 96, 64, 8, [8192], 0.88,
                      wave_rows(8, 32, 4))
    else:
        raise KeyError(name)
    if overrides:
        wl = wl.replace(**overrides)
    return wl
