"""Call schedules of a decoding step (host logic) and, on the oracle, the fact
the GPU schedule tests rely on: a row's result does not depend on the other
rows of its call, and a draft row (j, r) needs only the block tokens 0..j.
"""
import numpy as np
import pytest

import oracle
from synth import Workload, grid_rows
from self_speculative_verify_amd.schedule import batched_verify, draft_pass, per_loop_verify


@pytest.mark.parametrize("D,R", [(1, 1), (8, 32), (3, 5)])
def test_per_loop_covers_the_grid_once(D, R):
    (grid,) = batched_verify(D, R)
    calls = per_loop_verify(D, R)
    assert len(calls) == R
    seen = [row for c in calls for row in c.rows]
    assert sorted(seen) == sorted(grid.rows) and len(seen) == len(set(seen)) == D * R
    for r, c in enumerate(calls, start=1):
        assert c.n_blk == D and {x[1] for x in c.rows} == {r}


@pytest.mark.parametrize("D,rd", [(1, 1), (8, 4), (5, 5)])
def test_draft_pass_order(D, rd):
    calls = draft_pass(D, rd)
    assert [c.rows[0] for c in calls] == [(j, r) for j in range(D) for r in range(1, rd + 1)]
    assert all(len(c.rows) == 1 and c.n_blk == c.rows[0][0] + 1 for c in calls)
    with pytest.raises(ValueError):
        draft_pass(D, 0)


@pytest.mark.parametrize("W,anchor", [(3, 0), (2, 1), (40, 0)])
def test_oracle_rows_do_not_depend_on_their_call(W, anchor):
    wl = Workload("s", 11, 1, 4, 4, 2, 32, W, 5, [0, 9, 30], 0.88, grid_rows(5, 4),
                  heavy_frac=0.1, anchor=anchor)
    oc = oracle.prefix_cache(wl, layers=[0])
    q = wl.queries(0)
    bk, bv = wl.block(0)
    ref_o, ref_l = oc.verify(0, wl.rows, q, bk, bv, wl.n_blk)
    for c in per_loop_verify(wl.n_blk, wl.n_loops):
        idx = [wl.rows.index(x) for x in c.rows]
        o, l = oc.verify(0, c.rows, np.ascontiguousarray(q[:, idx]), bk, bv, c.n_blk)
        assert np.array_equal(o, ref_o[:, idx]) and np.array_equal(l, ref_l[:, idx])
    for c in draft_pass(wl.n_blk, wl.n_loops):
        (j, r), = c.rows
        k = wl.rows.index((j, r))
        # block tokens past j are never read: poison them
        pk, pv = bk.copy(), bv.copy()
        pk[:, :, :, j + 1:] = 0x7FC0
        pv[:, :, :, j + 1:] = 0x7FC0
        o, l = oc.verify(0, c.rows, np.ascontiguousarray(q[:, [k]]), pk, pv, c.n_blk)
        assert np.array_equal(o, ref_o[:, [k]]) and np.array_equal(l, ref_l[:, [k]])
