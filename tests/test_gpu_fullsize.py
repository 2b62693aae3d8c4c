"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (planner defaults, one layer's call; every layer's call has
the same shape).

The cache layout is compared byte for byte with the oracle's image of the
whole storage; attention outputs are compared on a seeded sample of
(sequence, row, query head) outputs, which the oracle computes one by one:
max |O - O_ref| <= 2e-3, |LSE - LSE_ref| / max(1, |LSE_ref|) <= 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import WINDOW_FULL, grid_rows, named_workload

pytestmark = pytest.mark.gpu

TOL_O = 2e-3
TOL_LSE = 1e-5
N_SAMPLE = 96


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import self_speculative_verify_amd.ripe as r
    r.load()
    yield


def _sample_mask(wl, seed):
    """A seeded set of outputs: every row of one query head of sequence 0,
    the last row of every sequence at every head, and N_SAMPLE random picks."""
    B, n, Hq = wl.batch, wl.n_rows, wl.n_heads_q
    want = np.zeros((B, n, Hq), dtype=np.uint8)
    rng = np.random.default_rng(seed)
    want[0, :, int(rng.integers(Hq))] = 1
    want[:, n - 1, :] = 1
    idx = rng.integers(0, B * n * Hq, size=N_SAMPLE)
    want.reshape(-1)[idx] = 1
    return want


def _run_full(wl, window=None, seed=4242, want=None):
    """Prefix append and one verify call of layer 0 at full size (planner
    defaults); layout compared whole, outputs on a seeded sample."""
    import ripe_harness as H
    window = wl.window if window is None else window
    print(f"full-size {wl.name}: batch {wl.batch}, lens {wl.lens if wl.batch <= 8 else '...'}, "
          f"rows {wl.n_rows}, heads {wl.n_heads_q}/{wl.n_heads_kv}, d {wl.head_dim}, W {window}",
          flush=True)
    cache = H.make_cache(wl, window=window)
    H.load_prefix(cache, wl)
    q, bk, bv = H.verify_inputs(wl, 0)
    out, lse = cache.verify(0, wl.rows, q, bk, bv, wl.n_blk)
    torch.cuda.synchronize()
    oc = oracle.prefix_cache(wl, layers=[0], window=window)
    assert np.array_equal(cache.storage.cpu().numpy(), oc.image), "layout differs from the oracle"
    del cache
    if want is None:
        want = _sample_mask(wl, seed)
    ref_o, ref_l = oc.verify(0, wl.rows, wl.queries(0), *wl.block(0), wl.n_blk, want=want)
    sel = want.astype(bool)
    o = out.cpu().double().numpy()[sel]
    l = lse.cpu().double().numpy()[sel]
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    err_o = float(np.max(np.abs(o - ref_o[sel])))
    err_l = float(np.max(np.abs(l - ref_l[sel]) / np.maximum(1.0, np.abs(ref_l[sel]))))
    print(f"full-size {wl.name} W={window}: {int(sel.sum())} outputs, max|dO|={err_o:.3e} "
          f"max rel dLSE={err_l:.3e}", flush=True)
    assert err_o <= TOL_O
    assert err_l <= TOL_LSE


@pytest.mark.parametrize("name", ["tiny", "huginn", "gqa", "ragged", "wave"])
def test_full_size_sampled(name):
    _run_full(named_workload(name).replace(n_layers=1))


# the windows the Huginn-scale workload is compared at besides its own (64),
# and the GQA workload's full per-loop cache (every position at all 32 loops)
@pytest.mark.parametrize("name,window", [("huginn", 0), ("huginn", 8), ("huginn", 1024),
                                         ("gqa", WINDOW_FULL)])
@pytest.mark.timeout(600)
def test_full_size_other_windows(name, window):
    _run_full(named_workload(name).replace(n_layers=1), window=window, seed=4400 + (window % 4099))


def test_full_size_gqa_288_rows():
    """The GQA shape with a 9-token block: 9 x 32 = 288 rows, so the call runs
    a launch of 256 rows and one of the 32 left; the short one splits the
    committed positions into chunks and needs the workspace (its size must
    cover that launch too).  Sampled outputs include every row of the second
    launch (loops 29..32) at one head."""
    wl = named_workload("gqa", n_layers=1, n_blk=9, rows=grid_rows(9, 32))
    want = _sample_mask(wl, 4545)
    late = [k for k, (i, r) in enumerate(wl.rows) if r >= 29]
    want[:, late, 5] = 1
    _run_full(wl, want=want)


def test_full_size_ragged_append_then_verify():
    """The ragged workload's full step: append the D accepted tokens of every
    sequence (ring slots of the oldest window positions are overwritten), then
    verify the next block at the new lengths."""
    import ripe_harness as H
    wl = named_workload("ragged").replace(n_layers=1)
    wl = wl.replace(capacity=max(wl.lens) + 2 * wl.n_blk)
    cache = H.make_cache(wl)
    H.load_prefix(cache, wl)
    oc = oracle.prefix_cache(wl, layers=[0])
    bk, bv = wl.block(0)
    D, R = wl.n_blk, wl.n_loops
    tbk, tbv = H.to_dev(bk), H.to_dev(bv)
    cache.append(0, [D] * wl.batch, tbk[:, R - 1, :, :D], tbv[:, R - 1, :, :D],
                 tbk[:, :R - 1, :, :D], tbv[:, :R - 1, :, :D])
    assert oc.append(0, [D] * wl.batch, np.ascontiguousarray(bk[:, R - 1, :, :D]),
                     np.ascontiguousarray(bv[:, R - 1, :, :D]), bk[:, :R - 1, :, :D],
                     bv[:, :R - 1, :, :D]) == oracle.ORA_OK
    torch.cuda.synchronize()
    assert np.array_equal(cache.storage.cpu().numpy(), oc.image), "layout after the block append"
    assert cache.lengths(0) == [L + D for L in wl.lens]
    wl2 = wl.replace(lens=[L + D for L in wl.lens], capacity=wl.capacity)
    q, bk2, bv2 = H.verify_inputs(wl2, 0)
    out, lse = cache.verify(0, wl2.rows, q, bk2, bv2, D)
    torch.cuda.synchronize()
    want = _sample_mask(wl2, 4343)
    ref_o, ref_l = oc.verify(0, wl2.rows, wl2.queries(0), *wl2.block(0), D, want=want)
    sel = want.astype(bool)
    err_o = float(np.max(np.abs(out.cpu().double().numpy()[sel] - ref_o[sel])))
    l = lse.cpu().double().numpy()[sel]
    err_l = float(np.max(np.abs(l - ref_l[sel]) / np.maximum(1.0, np.abs(ref_l[sel]))))
    print(f"full-size ragged after append: max|dO|={err_o:.3e} max rel dLSE={err_l:.3e}", flush=True)
    assert err_o <= TOL_O
    assert err_l <= TOL_LSE
