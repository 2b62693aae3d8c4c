"""GPU parity of windowed draft attention (ripe_draft_attn) against the fp64
oracle: the draft pass's single-row calls (block keys 0..j, later block
tokens poisoned with NaN) and whole-grid calls, for several sink counts and
window lengths, including a window of zero (block keys only) and one past
the context (the full-context draft, compared with verification too).
Bar: max |O - O_ref| <= 2e-3, |LSE - LSE_ref| / max(1, |LSE_ref|) <= 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import Workload, grid_rows, named_workload
from self_speculative_verify_amd.schedule import draft_pass

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


def _check(o, l, ref_o, ref_l, what):
    o = o.detach().cpu().double().numpy()
    l = l.detach().cpu().double().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), what
    err_o = float(np.max(np.abs(o - ref_o)))
    err_l = float(np.max(np.abs(l - ref_l) / np.maximum(1.0, np.abs(ref_l))))
    assert err_o <= TOL_O, f"{what}: max |dO| = {err_o}"
    assert err_l <= TOL_LSE, f"{what}: max rel dLSE = {err_l}"


WORKLOADS = {
    "huginn": lambda: named_workload("huginn", n_layers=1, n_heads_q=11, n_heads_kv=11, lens=[700]),
    "gqa": lambda: named_workload("gqa", n_layers=1, lens=[1024, 333], window=64),
    "ragged": lambda: named_workload("ragged", n_layers=1, lens=[1500, 33, 700, 2100]),
    "edge": lambda: Workload("edge", 82, 1, 5, 4, 2, 64, 3, 6, [0, 2, 37], 0.88, grid_rows(6, 5),
                             heavy_frac=0.05),
}
WINDOWS = [(4, 16), (0, 0), (1, 64), (32, 100), (3, 5000), (40, 33)]


@pytest.fixture(scope="module")
def loaded():
    import ripe_harness as H
    cache = {}

    def get(name):
        if name not in cache:
            wl = WORKLOADS[name]()
            c = H.make_cache(wl)
            H.load_prefix(c, wl)
            q, bk, bv = H.verify_inputs(wl, 0)
            oc = oracle.prefix_cache(wl, layers=[0])
            cache[name] = (wl, c, q, bk, bv, oc)
        return cache[name]
    return get


@pytest.mark.parametrize("name", list(WORKLOADS))
@pytest.mark.parametrize("n_sink,w", WINDOWS)
def test_windowed_draft_pass(loaded, name, n_sink, w):
    wl, cache, q, bk, bv, oc = loaded(name)
    qn = wl.queries(0)
    bkn, bvn = wl.block(0)
    for c in draft_pass(wl.n_blk, min(2, wl.n_loops)):
        (j, r), = c.rows
        k = wl.rows.index((j, r))
        pk, pv = bk.clone(), bv.clone()
        pk.view(torch.int16)[:, :, :, j + 1:] = BF16_NAN
        pv.view(torch.int16)[:, :, :, j + 1:] = BF16_NAN
        o, l = cache.draft(0, c.rows, q[:, [k]].contiguous(), pk, pv, c.n_blk, n_sink, w)
        torch.cuda.synchronize()
        ref_o, ref_l = oc.draft(0, c.rows, np.ascontiguousarray(qn[:, [k]]), bkn, bvn, c.n_blk, n_sink, w)
        _check(o, l, ref_o, ref_l, f"{name} sinks {n_sink} window {w} row ({j}, {r})")


@pytest.mark.parametrize("name", list(WORKLOADS))
@pytest.mark.parametrize("n_sink,w", WINDOWS)
def test_windowed_draft_whole_grid(loaded, name, n_sink, w):
    """Every (i, r) in one call: row blocks mix loops and offsets, so the
    skipped stretch of deep tiles is bounded by the lowest window start."""
    wl, cache, q, bk, bv, oc = loaded(name)
    o, l = cache.draft(0, wl.rows, q, bk, bv, wl.n_blk, n_sink, w)
    torch.cuda.synchronize()
    ref_o, ref_l = oc.draft(0, wl.rows, wl.queries(0), *wl.block(0), wl.n_blk, n_sink, w)
    _check(o, l, ref_o, ref_l, f"{name} grid sinks {n_sink} window {w}")


def test_window_past_the_context_is_verification(loaded):
    wl, cache, q, bk, bv, oc = loaded("ragged")
    o, l = cache.draft(0, wl.rows, q, bk, bv, wl.n_blk, 0, max(wl.lens) + wl.n_blk)
    vo, vl = cache.verify(0, wl.rows, q, bk, bv, wl.n_blk)
    torch.cuda.synchronize()
    assert float((o - vo).abs().max()) <= 2 * TOL_O
    assert float(((l - vl).abs() / vl.abs().clamp(min=1)).max()) <= 2 * TOL_LSE
