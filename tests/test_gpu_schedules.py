"""GPU parity of the other call schedules of a decoding step: verification
loop by loop (R calls of D rows) and the draft pass (D x r_draft calls of one
row each, block keys 0..j only).

Every call goes through the C ABI and is compared with the fp64 oracle on the
same rows (max |O - O_ref| <= 2e-3, |LSE - LSE_ref| / max(1, |LSE_ref|) <=
1e-5).  A row's result does not depend on the rest of its call, so the
schedules are also compared, row by row, with the batched D x R call.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import Workload, grid_rows, named_workload
from self_speculative_verify_amd.schedule import batched_verify, draft_pass, per_loop_verify

from helpers import use_tuning

pytestmark = pytest.mark.gpu

TOL_O = 2e-3
TOL_LSE = 1e-5
BF16_NAN = 0x7FC0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import self_speculative_verify_amd.ripe as r
    r.load()
    yield


@pytest.fixture(params=["planner", "keys-chunked", "rows-planner"], autouse=True)
def kernel_choice(request, monkeypatch):
    use_tuning(monkeypatch, request.param)
    yield request.param


def _check(o, l, ref_o, ref_l, what):
    o = o.detach().cpu().double().numpy()
    l = l.detach().cpu().double().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), what
    err_o = float(np.max(np.abs(o - ref_o)))
    err_l = float(np.max(np.abs(l - ref_l) / np.maximum(1.0, np.abs(ref_l))))
    assert err_o <= TOL_O, f"{what}: max |dO| = {err_o}"
    assert err_l <= TOL_LSE, f"{what}: max rel dLSE = {err_l}"
    return err_o, err_l


WORKLOADS = {
    "huginn": lambda: named_workload("huginn", n_layers=1, n_heads_q=11, n_heads_kv=11, lens=[700]),
    "gqa": lambda: named_workload("gqa", n_layers=1, lens=[1024, 333], window=64),
    "ragged": lambda: named_workload("ragged", n_layers=1, lens=[1500, 33, 700, 2100]),
    "edge": lambda: Workload("edge", 81, 1, 5, 4, 2, 64, 3, 6, [0, 2, 37], 0.88, grid_rows(6, 5),
                             heavy_frac=0.05),
}


def _setup(name):
    import ripe_harness as H
    wl = WORKLOADS[name]()
    assert wl.rows == batched_verify(wl.n_blk, wl.n_loops)[0].rows
    cache = H.make_cache(wl)
    H.load_prefix(cache, wl)
    q, bk, bv = H.verify_inputs(wl, 0)
    oc = oracle.prefix_cache(wl, layers=[0])
    ref_o, ref_l = oc.verify(0, wl.rows, wl.queries(0), *wl.block(0), wl.n_blk)
    bo, bl = cache.verify(0, wl.rows, q, bk, bv, wl.n_blk)
    torch.cuda.synchronize()
    _check(bo, bl, ref_o, ref_l, f"{name} batched")
    return wl, cache, q, bk, bv, ref_o, ref_l, bo.clone(), bl.clone()


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_per_loop_verify(name):
    """R calls of the D rows of one loop each (the queries of the batched call
    split by loop) give the batched call's rows."""
    wl, cache, q, bk, bv, ref_o, ref_l, bo, bl = _setup(name)
    calls = per_loop_verify(wl.n_blk, wl.n_loops)
    assert len(calls) == wl.n_loops
    worst = 0.0
    for c in calls:
        idx = [wl.rows.index(x) for x in c.rows]
        o, l = cache.verify(0, c.rows, q[:, idx].contiguous(), bk, bv, c.n_blk)
        torch.cuda.synchronize()
        _check(o, l, ref_o[:, idx], ref_l[:, idx], f"{name} loop {c.rows[0][1]}")
        worst = max(worst, float((o - bo[:, idx]).abs().max()), float((l - bl[:, idx]).abs().max()))
    print(f"{name}: per-loop vs batched max diff {worst:.3e}", flush=True)
    assert worst <= 2 * TOL_O


@pytest.mark.parametrize("name", list(WORKLOADS))
@pytest.mark.parametrize("r_draft", [1, 4])
def test_draft_pass(name, r_draft):
    """Draft calls of the single row (j, r) with block keys 0..j; the block
    tokens after j hold NaN, so a read past n_blk would show in the output."""
    wl, cache, q, bk, bv, ref_o, ref_l, bo, bl = _setup(name)
    r_draft = min(r_draft, wl.n_loops)
    calls = draft_pass(wl.n_blk, r_draft)
    assert len(calls) == wl.n_blk * r_draft
    worst = 0.0
    for c in calls:
        (j, r), = c.rows
        assert c.n_blk == j + 1
        k = wl.rows.index((j, r))
        pk, pv = bk.clone(), bv.clone()
        pk.view(torch.int16)[:, :, :, j + 1:] = BF16_NAN
        pv.view(torch.int16)[:, :, :, j + 1:] = BF16_NAN
        o, l = cache.verify(0, c.rows, q[:, [k]].contiguous(), pk, pv, c.n_blk)
        torch.cuda.synchronize()
        _check(o, l, ref_o[:, [k]], ref_l[:, [k]], f"{name} draft ({j}, {r})")
        worst = max(worst, float((o - bo[:, [k]]).abs().max()), float((l - bl[:, [k]]).abs().max()))
    print(f"{name}: draft (r_draft={r_draft}) vs batched max diff {worst:.3e}", flush=True)
    assert worst <= 2 * TOL_O
