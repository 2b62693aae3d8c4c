"""Batch capacity at fixed memory on a real allocation (GPU).

RIPE's memory saving (RIPE abstract, fourth and fifth sentences) read as
sequences per budget: for a budget of device memory, ripe_max_batch names the
largest batch whose storage fits.  Here the budget holds several hundred
short sequences (more than one append or verify launch takes for its
per-sequence arguments, 64), the cache is created at exactly that batch on a
buffer of exactly the budget, and one more sequence is refused on the same
buffer.  Every sequence's committed prefix goes in with one ripe_append; the
whole storage is compared byte for byte with the oracle's image, and one
verify call of the D x R grid over every sequence is compared with the fp64
oracle (max |dO| <= 2e-3, relative LSE error <= 1e-5).
"""
import numpy as np
import pytest
import torch

import oracle
from self_speculative_verify_amd import RipeCache, ripe
from synth import Workload, grid_rows, ragged_lengths

from helpers import step_arrays, use_tuning

pytestmark = pytest.mark.gpu

TOL_O = 2e-3
TOL_LSE = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ripe.load()
    yield


@pytest.fixture(params=["planner", "keys-chunked", "rows-planner"], autouse=True)
def kernel_choice(request, monkeypatch):
    use_tuning(monkeypatch, request.param)
    yield request.param


@pytest.mark.parametrize("window", [16, 0])
def test_verify_at_the_batch_a_budget_holds(window):
    R, Hq, Hkv, d, D, cap = 8, 4, 2, 64, 4, 132
    target = 300
    cfg = ripe.config(1, R, Hq, Hkv, d, window, target, cap, D)
    one_more = ripe.config(1, R, Hq, Hkv, d, window, target + 1, cap, D)
    budget = ripe.ripe_cache_bytes(cfg) + (ripe.ripe_cache_bytes(one_more) - ripe.ripe_cache_bytes(cfg)) // 2
    B = ripe.ripe_max_batch(cfg, budget)
    assert B == target > 64
    # exactly the budget: B sequences fit, B + 1 do not
    storage = torch.empty(budget, dtype=torch.uint8, device="cuda")
    with pytest.raises(ripe.RipeError) as e:
        ripe.ripe_cache_create(one_more, storage)
    assert e.value.status == ripe.RIPE_EINVAL
    lens = ragged_lengths(71, B, 1, cap - D)
    wl = Workload("capacity", 71, 1, R, Hq, Hkv, d, window, D, lens, 0.88, grid_rows(D, R),
                  heavy_frac=0.02, capacity=cap)
    c = RipeCache(1, R, Hq, Hkv, d, window, B, cap, D, device="cuda")
    # the binding allocates its own storage; bind a second handle to the budget buffer too
    h2 = ripe.ripe_cache_create(c.cfg, storage)
    ripe.load().ripe_destroy(h2)
    dk, dv, wk, wv = step_arrays(wl, 0, [0] * B, lens)
    import ripe_harness as H
    c.append(0, lens, H.to_dev(dk), H.to_dev(dv), H.to_dev(wk) if window else None,
             H.to_dev(wv) if window else None)
    oc = oracle.OracleCache(oracle.config_of(wl))
    assert oc.append(0, lens, dk, dv, wk, wv) == oracle.ORA_OK
    torch.cuda.synchronize()
    assert c.lengths(0) == lens
    assert np.array_equal(c.storage.cpu().numpy(), oc.image), "layout differs from the oracle"
    q, bk, bv = H.verify_inputs(wl, 0)
    out, lse = c.verify(0, wl.rows, q, bk, bv, D)
    torch.cuda.synchronize()
    ref_o, ref_l = oc.verify(0, wl.rows, wl.queries(0), *wl.block(0), D)
    o = out.cpu().double().numpy()
    l = lse.cpu().double().numpy()
    err_o = float(np.max(np.abs(o - ref_o)))
    err_l = float(np.max(np.abs(l - ref_l) / np.maximum(1.0, np.abs(ref_l))))
    print(f"capacity W={window}: batch {B} in {budget} bytes: max|dO|={err_o:.3e} rel dLSE={err_l:.3e}",
          flush=True)
    assert err_o <= TOL_O and err_l <= TOL_LSE
