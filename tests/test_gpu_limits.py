"""GPU parity at the edges of the launch configuration: calls with more rows
than one launch takes (256), batches larger than one append launch takes (64),
draft blocks longer than one 32-key tile up to the largest (256 positions),
the most loops a configuration allows (255), and windows longer than the
capacity.  Same bar as the other parity tests (bit-exact layout, max |dO| <=
2e-3, relative LSE error <= 1e-5), against the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import WINDOW_FULL, Workload, grid_rows, ragged_lengths

from helpers import use_tuning

pytestmark = pytest.mark.gpu

TOL_O = 2e-3
TOL_LSE = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import self_speculative_verify_amd.ripe as r
    r.load()
    yield


@pytest.fixture(params=["planner", "keys-4waves", "keys-8waves-planner", "rows-planner", "keys-chunked",
                        "rows-chunked"],
                autouse=True)
def kernel_choice(request, monkeypatch):
    use_tuning(monkeypatch, request.param)
    yield request.param


def run(wl, rows=None):
    import ripe_harness as H
    cache = H.make_cache(wl)
    H.load_prefix(cache, wl)
    oc = oracle.prefix_cache(wl, layers=[0])
    torch.cuda.synchronize()
    assert np.array_equal(cache.storage.cpu().numpy(), oc.image), "layout differs from the oracle"
    rows = wl.rows if rows is None else rows
    q, bk, bv = H.verify_inputs(wl, 0)
    out, lse = cache.verify(0, rows, q, bk, bv, wl.n_blk)
    torch.cuda.synchronize()
    ref_o, ref_l = oc.verify(0, rows, wl.queries(0), *wl.block(0), wl.n_blk)
    o = out.cpu().double().numpy()
    l = lse.cpu().double().numpy()
    err_o = float(np.max(np.abs(o - ref_o)))
    err_l = float(np.max(np.abs(l - ref_l) / np.maximum(1.0, np.abs(ref_l))))
    print(f"{wl.name}: {len(rows)} rows, batch {wl.batch}: max|dO|={err_o:.3e} rel dLSE={err_l:.3e}",
          flush=True)
    assert err_o <= TOL_O and err_l <= TOL_LSE


def test_more_rows_than_one_launch():
    """12 x 24 = 288 rows: two launches of one call."""
    run(Workload("rows288", 91, 1, 24, 4, 2, 64, 16, 12, [150, 61], 0.88, grid_rows(12, 24),
                 heavy_frac=0.05))


def test_batch_larger_than_one_append_launch():
    """70 sequences of ragged lengths (two append launches per layer)."""
    lens = ragged_lengths(92, 70, 0, 90)
    run(Workload("b70", 92, 1, 4, 2, 1, 64, 12, 3, lens, 0.88, grid_rows(3, 4)))


@pytest.mark.parametrize("D", [33, 40])
def test_draft_block_longer_than_a_tile(D):
    run(Workload(f"blk{D}", 93, 1, 3, 4, 4, 96, 48, D, [200, 7], 0.88, grid_rows(D, 3)))


def test_largest_draft_block():
    """max_block = 256, the largest the row words hold: block offsets 0..255
    (eight 32-key block tiles per loop), 512 rows in two launches."""
    run(Workload("blk256", 98, 1, 2, 2, 1, 64, 300, 256, [40, 300], 0.88, grid_rows(256, 2),
                 heavy_frac=0.05))


@pytest.mark.parametrize("D", [1, 2])
def test_most_loops(D):
    """R = 255 loops, the most the row words hold: with one block position a
    rows workgroup's 128 rows are 128 different loops (both halves of its
    loop list full), with two the call takes two launches."""
    run(Workload(f"r255d{D}", 99, 1, 255, 1, 1, 64, 8, D, [50], 0.88, grid_rows(D, 255)))


@pytest.mark.parametrize("W", [500, WINDOW_FULL])
def test_window_longer_than_the_capacity(W):
    run(Workload("wcap", 94, 1, 6, 4, 2, 128, W, 4, [120, 300, 33], 0.81, grid_rows(4, 6)))


@pytest.mark.parametrize("d,lens", [(64, [1999, 1501]), (96, [2047, 700]), (128, [1500, 333])])
def test_long_streams_every_head_size(d, lens):
    """Deep streams of 20-64 tiles per key half at each head size, so the rows
    kernel's stage pipeline runs through its steady state (barriers every
    third step at head_dim 64 and 96, every step at 128), with tile counts
    that end on every phase of the barrier period; 128 or more row-heads per
    KV head with two heads per group."""
    rows = grid_rows(8, 8)                       # 64 rows x 2 query heads per KV head
    run(Workload(f"long{d}", 95 + d, 1, 8, 4, 2, d, 64, 8, lens, 0.88, rows, heavy_frac=0.01))


def test_long_sequence_split_for_balance(kernel_choice):
    """Four sequences whose row blocks alone fill the chip (8 KV heads x 8 row
    blocks x 4 sequences = 256 workgroups), one of them ten times longer than
    the others: the planner splits it into chunks no longer than the mean load
    of a workgroup slot and lists the (sequence, chunk) items longest first.
    Outputs are compared on a seeded sample of (sequence, row, head), every
    row of one head of the long sequence included."""
    import ripe_harness as H
    wl = Workload("balance", 97, 1, 32, 32, 8, 128, 64, 8, [3000, 200, 310, 150], 0.88, grid_rows(8, 32))
    cache = H.make_cache(wl)
    H.load_prefix(cache, wl)
    if kernel_choice in ("planner", "rows-planner"):
        assert cache.workspace(wl.n_rows) is not None, "the rows kernel's call may split its keys"
    q, bk, bv = H.verify_inputs(wl, 0)
    out, lse = cache.verify(0, wl.rows, q, bk, bv, wl.n_blk)
    torch.cuda.synchronize()
    want = np.zeros((wl.batch, wl.n_rows, wl.n_heads_q), dtype=np.uint8)
    rng = np.random.default_rng(97)
    want.reshape(-1)[rng.integers(0, want.size, size=200)] = 1
    want[0, :, 3] = 1
    want[:, -1, :] = 1
    oc = oracle.prefix_cache(wl, layers=[0])
    ref_o, ref_l = oc.verify(0, wl.rows, wl.queries(0), *wl.block(0), wl.n_blk, want=want)
    sel = want.astype(bool)
    o = out.cpu().double().numpy()[sel]
    l = lse.cpu().double().numpy()[sel]
    err_o = float(np.max(np.abs(o - ref_o[sel])))
    err_l = float(np.max(np.abs(l - ref_l[sel]) / np.maximum(1.0, np.abs(ref_l[sel]))))
    print(f"balance split: {int(sel.sum())} outputs, max|dO|={err_o:.3e} rel dLSE={err_l:.3e}", flush=True)
    assert err_o <= TOL_O and err_l <= TOL_LSE
