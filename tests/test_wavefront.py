"""WaveFront scheduling (host logic): the diagonal wave, commits, rollbacks
and the calls it takes per committed token.

Pins: the steady wave's rows are the wave workload's diagonal (block offset j
at loop R - r_draft*j, the oldest deepest); a rejection clears at most the
wave's width; every committed position ran loops 1..R in order; calls per
token are exactly r_draft when every draft is accepted and R when none is,
and match alpha*r_draft + (1 - alpha)*R for seeded Bernoulli acceptance.
"""
import math

import numpy as np
import pytest

from self_speculative_verify_amd.wavefront import (WaveScheduler, expected_calls_per_token,
                                                   kernel_rows)
from synth import wave_rows


def run(R, rd, n_calls, accept, L0=100):
    s = WaveScheduler(R, rd, L0)
    loops_done = {}            # version -> loops run, in order
    pos_of = {}
    commits = []
    for _ in range(n_calls):
        rows = s.rows()
        assert [i for i, _ in rows] == list(range(len(rows)))
        depths = [r for _, r in rows]
        assert all(1 <= r <= R for r in depths)
        assert all(a > b for a, b in zip(depths, depths[1:])), "older positions are deeper"
        assert len(rows) <= math.ceil(R / rd)
        for x, (_, r) in zip(s.wave, rows):
            loops_done.setdefault(x.version, []).append(r)
            pos_of[x.version] = x.pos
        committed_version = s.wave[0].version
        ev = s.after_call(accept)
        if ev.committed is not None:
            assert loops_done[committed_version] == list(range(1, R + 1))
            assert pos_of[committed_version] == ev.committed
            commits.append((s.calls, ev.committed))
        if ev.rejected:
            assert 1 <= ev.dropped <= math.ceil(R / rd) - 1
    return s, commits


@pytest.mark.parametrize("R,rd", [(32, 4), (8, 2), (8, 3), (5, 4)])
def test_all_accepted_steady_wave(R, rd):
    s, commits = run(R, rd, 40 * R, lambda: True)
    pos = [p for _, p in commits]
    assert pos == list(range(100, 100 + len(pos))), "commits are consecutive positions"
    gaps = np.diff([c for c, _ in commits])
    assert commits[0][0] == R and np.all(gaps == rd)
    assert s.rejections == 0 and s.dropped_loops == 0


def test_steady_rows_are_the_wave_diagonal():
    R, rd = 32, 4
    s = WaveScheduler(R, rd, 0)
    seen = False
    for _ in range(200):
        rows = s.rows()
        if rows[0][1] == R:
            assert rows == wave_rows(8, R, rd)
            seen = True
        s.after_call(lambda: True)
    assert seen


@pytest.mark.parametrize("R,rd", [(32, 4), (8, 2)])
def test_all_rejected_restarts_every_token(R, rd):
    s, commits = run(R, rd, 30 * R, lambda: False)
    gaps = np.diff([c for c, _ in commits])
    assert commits[0][0] == R and np.all(gaps == R)
    assert s.rejections == len(commits)     # the wave is full whenever a position commits


@pytest.mark.parametrize("alpha", [0.5, 0.8, 0.95])
def test_calls_per_token_matches_closed_form(alpha):
    R, rd = 32, 4
    rng = np.random.default_rng(np.random.SeedSequence([77, int(alpha * 100)]))
    s, commits = run(R, rd, 60000, lambda: bool(rng.random() < alpha))
    n = len(commits) - 1
    per_token = (commits[-1][0] - commits[0][0]) / n
    want = expected_calls_per_token(R, rd, alpha)
    sd = (R - rd) * math.sqrt(alpha * (1 - alpha) / n)
    assert abs(per_token - want) <= 4 * sd + 1e-9, (per_token, want, sd)


def test_rejection_clears_later_positions():
    """R = 8, r_draft = 2 from position 10: positions commit at calls 8, 10,
    12; the third check fails, so the three positions behind position 12
    (at depths 6, 4, 2) are cleared and the corrected token for position 13
    is alone in the wave at depth 0."""
    R, rd = 8, 2
    answers = iter([True, True, False] + [True] * 100)
    s = WaveScheduler(R, rd, 10)
    for call in range(1, 13):
        ev = s.after_call(lambda: next(answers))
        if call in (8, 10):
            assert ev.committed == 10 + (call - 8) // 2 and not ev.rejected
    assert ev.committed == 12 and ev.rejected
    assert ev.dropped == 3 and ev.dropped_loops == 6 + 4 + 2
    assert [(x.pos, x.depth) for x in s.wave] == [(13, 0)]
    assert s.rows() == [(0, 1)]


def test_shared_kv_rows():
    rows = [(0, 32), (1, 28), (2, 24)]
    assert kernel_rows(rows, True) == [(0, 1), (1, 1), (2, 1)]
    assert kernel_rows(rows, False) == rows


def test_bad_parameters():
    for R, rd in [(1, 1), (8, 0), (8, 8)]:
        with pytest.raises(ValueError):
            WaveScheduler(R, rd, 0)
