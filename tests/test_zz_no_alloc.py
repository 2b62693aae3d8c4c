"""ripe_verify_attn_noalloc (the library's fixed scratch instead of a caller
workspace) against ripe_verify_attn on the same inputs, through the C ABI.

Two calls in a row on one device, the second with a smaller input (fewer
rows, shorter contexts), each split into chunks so the partial states go
through the scratch; outputs must equal the workspace call's exactly (same
plan, same kernels) and match the fp64 oracle to max |dO| <= 2e-3 and
relative LSE error <= 1e-5.  A call whose partial states would pass the
scratch's size is refused with RIPE_ESCRATCH and writes nothing.
"""
import numpy as np
import pytest
import torch

import oracle
from self_speculative_verify_amd import RipeCache, ripe
from synth import Workload, grid_rows, named_workload

pytestmark = pytest.mark.gpu

TOL_O = 2e-3
TOL_LSE = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ripe.load()
    yield


def _case(wl, rows, tuning):
    import ripe_harness as H
    cache = H.make_cache(wl)
    if tuning:
        ripe.ripe_set_tuning(cache.handle, tuning)
    H.load_prefix(cache, wl)
    wl_r = wl.replace(rows=list(rows))
    q, bk, bv = H.verify_inputs(wl_r, 0)
    n = len(rows)
    B, Hq, d = wl.batch, wl.n_heads_q, wl.head_dim
    assert ripe.ripe_workspace_bytes(cache.handle, n) > 0, "the case must split its keys"
    ref = cache.verify(0, rows, q, bk, bv, wl.n_blk)
    out = torch.full((B, n, Hq, d), float("nan"), device="cuda")
    lse = torch.full((B, n, Hq), float("nan"), device="cuda")
    ripe.ripe_verify_attn_noalloc(cache.handle, 0, [i for i, _ in rows], [r for _, r in rows], q,
                                  ripe.kv_view(bk, "bphtd"), ripe.kv_view(bv, "bphtd"), wl.n_blk,
                                  out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), "differs from ripe_verify_attn"
    oc = oracle.prefix_cache(wl, layers=[0])
    ref_o, ref_l = oc.verify(0, rows, wl_r.queries(0), *wl_r.block(0), wl.n_blk)
    o = out.cpu().double().numpy()
    l = lse.cpu().double().numpy()
    err_o = float(np.max(np.abs(o - ref_o)))
    err_l = float(np.max(np.abs(l - ref_l) / np.maximum(1.0, np.abs(ref_l))))
    print(f"noalloc {wl.name}: {n} rows: max|dO|={err_o:.3e} rel dLSE={err_l:.3e}", flush=True)
    assert err_o <= TOL_O and err_l <= TOL_LSE


def test_two_calls_in_a_row_second_smaller():
    # the planner's own split: a per-loop row set of the Huginn-scale shape
    # (11 heads) at L = 2000, then a forced split of a smaller call
    big = named_workload("huginn", n_layers=1, n_heads_q=11, n_heads_kv=11, lens=[2000])
    _case(big, [(i, 7) for i in range(8)], None)
    small = Workload("noalloc-small", 61, 1, 4, 4, 2, 64, 8, 3, [300, 77], 0.88, grid_rows(3, 4))
    _case(small, [(0, 1), (2, 4)], {"kernel": 1, "items_target": 100000, "min_chunk": 32})


def test_over_the_scratch_is_refused():
    R, Hq, Hkv, d, B, L = 32, 32, 8, 128, 8, 4096
    c = RipeCache(1, R, Hq, Hkv, d, 0, B, L + 8, 8, device="cuda")
    ripe.ripe_set_tuning(c.handle, {"kernel": 2, "items_target": 100000, "min_chunk": 32})
    dk = torch.randn((B, Hkv, L, d), device="cuda").to(torch.bfloat16)
    c.append(0, [L] * B, dk, dk)
    rows = grid_rows(8, R)
    assert ripe.ripe_workspace_bytes(c.handle, len(rows)) > ripe.RIPE_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, len(rows), Hq, d), dtype=torch.bfloat16, device="cuda")
    blk = torch.zeros((B, R, Hkv, 8, d), dtype=torch.bfloat16, device="cuda")
    out = torch.full((B, len(rows), Hq, d), 7.0, device="cuda")
    lse = torch.full((B, len(rows), Hq), 7.0, device="cuda")
    with pytest.raises(ripe.RipeError) as e:
        ripe.ripe_verify_attn_noalloc(c.handle, 0, [i for i, _ in rows], [r for _, r in rows], q,
                                      ripe.kv_view(blk, "bphtd"), ripe.kv_view(blk, "bphtd"), 8,
                                      out, lse)
    torch.cuda.synchronize()
    assert e.value.status == ripe.RIPE_ESCRATCH
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all())
