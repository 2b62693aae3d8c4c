"""Pins of the oracle's windowed draft attention (page "Windowed-MTP:
Removing the Full-Context Draft-KV Tax at Million-Token Context", abstract: a
sliding window plus an attention sink on the draft's attention only).

A draft row (i, r) keeps, among its committed positions, the first n_sink and
those at or after L + i - w; every draft-block key 0..i stays; planes follow
the verification rule.  Pinned against: the brute-force dictionary cache
(which also asserts every plane it reads is stored), ordinary attention over
the row's key set built from the generator's planes (SDPA, fp64), the full
verification when the window covers everything, and attention over the block
keys alone when it covers nothing.
"""
import numpy as np
import pytest

import oracle
from synth import WINDOW_FULL

from test_oracle import _keys_for, build_both, sdpa_row, tiny


def _cases():
    out = []
    for L, W, anchor in [(11, 3, 0), (11, 5, 1), (6, 0, 0), (9, WINDOW_FULL, 0), (0, 2, 0), (13, 7, 0)]:
        for n_sink, w in [(0, 0), (1, 2), (3, 4), (2, 100), (0, 6), (20, 1)]:
            out.append((L, W, anchor, n_sink, w))
    return out


@pytest.mark.parametrize("L,W,anchor,n_sink,w", _cases())
def test_draft_against_brute_force(L, W, anchor, n_sink, w):
    wl = tiny([L, max(L - 3, 0)], 3, 2, 1, 4, W, anchor=anchor, seed=31 * L + n_sink, heavy=0.2)
    oc, brutes = build_both(wl, n_steps=3, seed=L + w)
    for layer, bc in enumerate(brutes):
        q = wl.queries(layer)
        bk, bv = wl.block(layer)
        out, lse = oc.draft(layer, wl.rows, q, bk, bv, wl.n_blk, n_sink, w)
        bout, blse = bc.verify(wl.rows, q, bk, bv, sink_window=(n_sink, w))
        np.testing.assert_allclose(out, bout, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, blse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n_sink,w,W", [(2, 5, 6), (0, 3, 3), (4, 9, 2), (1, 0, 4)])
def test_draft_is_attention_over_its_key_set(n_sink, w, W):
    """Ordinary attention (SDPA) over exactly the row's kept keys, each at the
    plane the rule names, built from the generator's planes."""
    wl = tiny([23, 10], 3, 2, 2, 4, W, rho=0.9, heavy=0.1)
    oc, _ = build_both(wl, n_steps=2)
    R = wl.n_loops
    grp = wl.n_heads_q // wl.n_heads_kv
    q = wl.queries(0)
    bk, bv = wl.block(0)
    out, lse = oc.draft(0, wl.rows, q, bk, bv, wl.n_blk, n_sink, w)
    for b in range(wl.batch):
        L = wl.lens[b]
        for kk, (i, r) in enumerate(wl.rows):
            t = L + i
            beta = t - W
            K, V = _keys_for(wl, 0, b, i, r, lambda s: r if s >= beta else R)
            keep = [s for s in range(t + 1) if s >= L or s < n_sink or s >= t - w]
            for h in range(wl.n_heads_q):
                o, l = sdpa_row(q[b, kk, h], K[h // grp][keep], V[h // grp][keep])
                np.testing.assert_allclose(out[b, kk, h], o, rtol=0, atol=1e-10)
                assert abs(lse[b, kk, h] - l) < 1e-10


@pytest.mark.parametrize("n_sink", [0, 3])
def test_draft_with_a_window_over_everything_is_verification(n_sink):
    wl = tiny([17, 40], 4, 4, 2, 4, 6, heavy=0.1)
    oc, _ = build_both(wl, n_steps=2)
    q = wl.queries(1)
    bk, bv = wl.block(1)
    v_out, v_lse = oc.verify(1, wl.rows, q, bk, bv, wl.n_blk)
    d_out, d_lse = oc.draft(1, wl.rows, q, bk, bv, wl.n_blk, n_sink, max(wl.lens) + wl.n_blk)
    assert np.array_equal(v_out, d_out) and np.array_equal(v_lse, d_lse)


def test_draft_without_sinks_or_window_sees_the_block_only():
    wl = tiny([17, 5], 4, 2, 2, 4, 6)
    oc, _ = build_both(wl, n_steps=1)
    q = wl.queries(0)
    bk, bv = wl.block(0)
    out, lse = oc.draft(0, wl.rows, q, bk, bv, wl.n_blk, 0, 0)
    for b in range(wl.batch):
        for kk, (i, r) in enumerate(wl.rows):
            for h in range(wl.n_heads_q):
                g = h // (wl.n_heads_q // wl.n_heads_kv)
                o, l = sdpa_row(q[b, kk, h], bk[b, r - 1, g, :i + 1], bv[b, r - 1, g, :i + 1])
                np.testing.assert_allclose(out[b, kk, h], o, rtol=0, atol=1e-10)
                assert abs(lse[b, kk, h] - l) < 1e-10


def test_draft_rejects_negative_window():
    wl = tiny([5], 2, 1, 1, 2, 3)
    oc, _ = build_both(wl, n_steps=1)
    q = wl.queries(0)
    bk, bv = wl.block(0)
    with pytest.raises(RuntimeError):
        oc.draft(0, wl.rows, q, bk, bv, wl.n_blk, -1, 3)
    with pytest.raises(RuntimeError):
        oc.draft(0, wl.rows, q, bk, bv, wl.n_blk, 0, -2)
