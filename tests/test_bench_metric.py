"""The bench's metric arithmetic (host only, no GPU).

unique_kv_bytes counts the distinct (position, loop) key and value vectors one
verification call reads with closed-form ranges per sequence.  Here the same
quantity is counted by walking the brute-force cache (oracle/brute.py) with
every row and head of the call and recording each stored entry and each block
vector it reads; the two counts must be equal for both anchors, windows from
0 to past the length, the D x R grid, the mixed-depth wave, per-loop row sets
and the windowed draft's sink-and-window key sets.  Also checked: the flop
count against a per-row sum, the roofline's choice of bound, and the
percentile summary.
"""
import itertools

import numpy as np
import pytest

import bench
from oracle.brute import BruteCache
from synth import Workload, grid_rows, wave_rows


class _Recorder(dict):
    """The brute-force store, recording every key that verify reads."""

    def __init__(self, *a, **kw):
        super().__init__(*a, **kw)
        self.read = set()

    def __getitem__(self, key):
        self.read.add(key)
        return super().__getitem__(key)


class _Block:
    """Stands in for blk_k / blk_v of one sequence: records (loop, head, j)."""

    def __init__(self, b, d, seen):
        self.b, self.d, self.seen = b, d, seen

    def __getitem__(self, idx):
        r1, g, j = idx
        self.seen.add((self.b, g, j, r1 + 1))
        return np.zeros(self.d, np.uint16)


def _walked_bytes(R, Hq, H, d, W, lens, rows, anchor, sink_window=None):
    cap = max(lens) + 8
    bc = BruteCache(R, Hq, H, d, W, len(lens), cap, anchor)
    z = np.zeros
    for b, L in enumerate(lens):
        if L == 0:
            continue
        nw = min(L, bc.slots)
        bc.append(b, z((H, L, d), np.uint16), z((H, L, d), np.uint16),
                  z((R - 1, H, nw, d), np.uint16), z((R - 1, H, nw, d), np.uint16))
    store = _Recorder(bc.store)
    bc.store = store
    blocks = set()
    q = z(d, np.uint16)
    for b in range(len(lens)):
        blk = _Block(b, d, blocks)
        for i, r in rows:
            for h in range(Hq):
                bc.verify_one(b, i, r, h, q, blk, blk, sink_window)
    # each stored entry and each block position is one key and one value of
    # d bf16 each
    return (len(store.read) + len(blocks)) * 2 * d * 2


def _wl(R, Hq, H, d, W, lens, rows, n_blk):
    return Workload("t", 0, 1, R, Hq, H, d, W, n_blk, list(lens), 0.88, list(rows))


ROW_SETS = {
    "grid": lambda D, R: grid_rows(D, R),
    "per-loop": lambda D, R: [(i, 2) for i in range(D)],
    "deep-only": lambda D, R: [(i, R) for i in range(D)],
    "wave": lambda D, R: wave_rows(min(D, 3), R, 1),
    "one-row": lambda D, R: [(D - 1, 1)],
}


@pytest.mark.parametrize("rows_name", sorted(ROW_SETS))
@pytest.mark.parametrize("anchor", [0, 1])
@pytest.mark.parametrize("W", [0, 1, 3, 8, 40])
def test_unique_bytes_equal_the_brute_force_walk(rows_name, anchor, W):
    R, Hq, H, d, D = 4, 4, 2, 8, 3
    lens = [0, 5, 17, 30]
    rows = ROW_SETS[rows_name](D, R)
    wl = _wl(R, Hq, H, d, W, lens, rows, D)
    want = _walked_bytes(R, Hq, H, d, W, lens, rows, anchor)
    assert bench.unique_kv_bytes(wl, W, anchor, rows, lens) == want


@pytest.mark.parametrize("n_sink,w", [(0, 0), (2, 3), (4, 10), (1, 40)])
@pytest.mark.parametrize("W", [0, 4, 40])
def test_windowed_draft_bytes_equal_the_brute_force_walk(n_sink, w, W):
    R, Hq, H, d, D = 4, 2, 1, 8, 3
    lens = [6, 23]
    rows = [(i, r) for i in range(D) for r in (1, 2)]
    wl = _wl(R, Hq, H, d, W, lens, rows, D)
    want = _walked_bytes(R, Hq, H, d, W, lens, rows, 0, (n_sink, w))
    assert bench.unique_kv_bytes(wl, W, 0, rows, lens, (n_sink, w)) == want


def test_flops_count_every_attended_key():
    R, Hq, H, d, D = 3, 6, 2, 16, 4
    lens = [0, 9, 31]
    rows = grid_rows(D, R)
    wl = _wl(R, Hq, H, d, 8, lens, rows, D)
    keys = sum(1 for L in lens for i, _ in rows for _s in range(L + i + 1))
    assert bench.flops(wl, rows, lens) == 4 * d * Hq * keys


def test_roofline_picks_the_binding_roof():
    # equal times on both roofs at U/8e12 == F/2.5e15
    u = 8e12 * 1e-4
    hbm = bench.roofline_of(u, 2.5e15 * 1e-4 * 0.5, 2e-4)
    assert hbm["bound"] == "hbm" and abs(hbm["frac"] - 0.5) < 1e-4
    mm = bench.roofline_of(u * 0.5, 2.5e15 * 1e-4, 4e-4)
    assert mm["bound"] == "mfma" and abs(mm["frac"] - 0.25) < 1e-4


def test_spread_is_a_percentile_summary():
    xs = list(range(101))
    for perm in itertools.islice(itertools.permutations([3, 1, 2]), 3):
        assert bench.spread(list(perm)) == {"median": 2, "p10": 1, "p90": 3}
    s = bench.spread([float(x) for x in xs])
    assert s == {"median": 50.0, "p10": 10.0, "p90": 90.0}
    assert bench.spread([]) is None
