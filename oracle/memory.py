"""Closed forms of the RIPE cache's memory -- TEST INFRASTRUCTURE ONLY.

RIPE (page "Prefix Keys and Values Matter Late", abstract, fourth and fifth
sentences) keeps the deepest plane of every position plus all R planes of the
W most recent positions, against R planes of every position for the full
per-loop cache.  Counting stored (position, plane) vectors per layer:

  full cache, recurrent layer  : R * L
  RIPE,       recurrent layer  : L + min(W, L) * (R - 1)
  any non-recurrent layer      : L (one plane)
"""
from __future__ import annotations


def full_vectors(L: int, R: int, n_recurrent: int, n_plain: int = 0) -> int:
    return n_plain * L + n_recurrent * R * L


def ripe_vectors(L: int, W: int, R: int, n_recurrent: int, n_plain: int = 0) -> int:
    return n_plain * L + n_recurrent * (L + min(W, L) * (R - 1))


def ripe_fraction(L: int, W: int, R: int, n_recurrent: int, n_plain: int = 0) -> float:
    """RIPE memory as a fraction of the full per-loop cache."""
    return ripe_vectors(L, W, R, n_recurrent, n_plain) / full_vectors(L, R, n_recurrent, n_plain)
