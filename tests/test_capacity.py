"""Batch capacity at fixed memory (full cache, RIPE, deepest plane alone).

The oracle's closed form (oracle/memory.py) is pinned by the page's 11.9%
figure and by the brute-force dictionary's vector count (test_oracle.py); here
it is also checked against what it must reduce to (the full cache holds R
times the deepest plane's vectors, RIPE sits between the two), and the
library's storage size and ripe_max_batch are checked against it: with the
capacity and the window multiples of 32 the library's sections hold exactly
the closed form's bytes per sequence, next to a 256-byte-aligned lengths
section.  Host functions of the library only (no device).
"""
import pytest

from oracle.memory import max_batch, ripe_fraction, sequence_bytes, vector_bytes
from self_speculative_verify_amd import ripe

FULL = ripe.RIPE_WINDOW_FULL


def cfg(L, W, R, Hq, Hkv, d, NL, B=1, D=8):
    return ripe.config(NL, R, Hq, Hkv, d, W, B, L, D, 0)


def up(x, a):
    return (x + a - 1) // a * a


@pytest.mark.parametrize("L,R,Hkv,d", [(1024, 32, 55, 96), (4096, 32, 8, 128), (256, 4, 2, 64)])
def test_closed_form_end_points(L, R, Hkv, d):
    full = sequence_bytes(L, L, R, Hkv, d, 4)
    deep = sequence_bytes(L, 0, R, Hkv, d, 4)
    assert full == R * deep == 4 * R * L * vector_bytes(Hkv, d)
    for W in (1, 64, L - 1):
        mid = sequence_bytes(L, W, R, Hkv, d, 4)
        assert deep < mid < full
        assert mid / full == pytest.approx(ripe_fraction(L, W, R, 4))
    assert sequence_bytes(L, 10 * L, R, Hkv, d, 4) == full      # a window past L stores all


@pytest.mark.parametrize("L,W,R,Hq,Hkv,d,NL", [
    (1024, 64, 32, 55, 55, 96, 4),       # Huginn-sized recurrent block, 64-position window
    (1024, 0, 32, 55, 55, 96, 4),        # deepest plane alone
    (1024, FULL, 32, 55, 55, 96, 4),     # full per-loop cache
    (4096, 64, 32, 32, 8, 128, 4),
    (4096, 0, 32, 32, 8, 128, 4),
    (128, 32, 8, 2, 2, 64, 1),
])
@pytest.mark.parametrize("B", [1, 3, 17])
def test_library_storage_matches_closed_form(L, W, R, Hq, Hkv, d, NL, B):
    c = cfg(L, W, R, Hq, Hkv, d, NL, B=B)
    lens_section = up(4 * NL * B, 256)
    per_seq = sequence_bytes(L, min(W, L), R, Hkv, d, NL)
    assert ripe.ripe_cache_bytes(c) == lens_section + B * per_seq


@pytest.mark.parametrize("L,W,R,Hq,Hkv,d,NL", [
    (1024, 64, 32, 55, 55, 96, 4), (1024, 0, 32, 55, 55, 96, 4), (1024, FULL, 32, 55, 55, 96, 4),
    (4096, 64, 32, 32, 8, 128, 4), (128, 32, 8, 2, 2, 64, 1)])
@pytest.mark.parametrize("gib", [1, 8, 32, 96])
def test_max_batch_at_fixed_memory(L, W, R, Hq, Hkv, d, NL, gib):
    budget = gib << 30
    per_seq = sequence_bytes(L, min(W, L), R, Hkv, d, NL)
    want = min(4096, max_batch(budget, per_seq))
    got = ripe.ripe_max_batch(cfg(L, W, R, Hq, Hkv, d, NL), budget)
    # the lengths section (256-byte aligned) may cost the last sequence
    assert got in (want, want - 1)
    if got > 0:
        assert ripe.ripe_cache_bytes(cfg(L, W, R, Hq, Hkv, d, NL, B=got)) <= budget
    if 0 < got < 4096:
        assert ripe.ripe_cache_bytes(cfg(L, W, R, Hq, Hkv, d, NL, B=got + 1)) > budget


def test_max_batch_edges():
    c = cfg(1024, 64, 32, 55, 55, 96, 4)
    one = ripe.ripe_cache_bytes(c)
    assert ripe.ripe_max_batch(c, one) == 1
    assert ripe.ripe_max_batch(c, one - 1) == 0
    assert ripe.ripe_max_batch(c, 1 << 62) == 4096
    bad = cfg(1024, 64, 32, 55, 55, 80, 4)          # head_dim 80 is not supported
    assert ripe.ripe_max_batch(bad, 1 << 40) == -1


def test_capacity_ratios_huginn_shape():
    """Sequences per budget: the full cache holds R times fewer than the
    deepest plane alone, RIPE (W = 64 at 1024 positions) 1/fraction times
    more than the full cache."""
    L, R, H, d = 1024, 32, 55, 96
    budget = 64 << 30
    full = max_batch(budget, sequence_bytes(L, L, R, H, d, 4))
    ripe_b = max_batch(budget, sequence_bytes(L, 64, R, H, d, 4))
    deep = max_batch(budget, sequence_bytes(L, 0, R, H, d, 4))
    assert deep // full in (R - 1, R, R + 1)
    assert ripe_b / full == pytest.approx(1 / ripe_fraction(L, 64, R, 4), rel=0.1)
