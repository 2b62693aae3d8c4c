"""Closed forms of the RIPE cache's memory -- TEST INFRASTRUCTURE ONLY.

RIPE (page "Prefix Keys and Values Matter Late", abstract, fourth and fifth
sentences) keeps the deepest plane of every position plus all R planes of the
W most recent positions, against R planes of every position for the full
per-loop cache.  Counting stored (position, plane) vectors per layer:

  full cache, recurrent layer  : R * L
  RIPE,       recurrent layer  : L + min(W, L) * (R - 1)
  any non-recurrent layer      : L (one plane)

A vector is a key and a value of all KV heads in bf16 (4 * Hkv * d bytes), so
a sequence's bytes are the vector count times that, and a memory budget holds
floor(budget / bytes per sequence) sequences: the batch capacity at fixed
memory, for the full cache (W >= L), RIPE (window W) and the deepest plane
alone (W = 0).
"""
from __future__ import annotations


def full_vectors(L: int, R: int, n_recurrent: int, n_plain: int = 0) -> int:
    return n_plain * L + n_recurrent * R * L


def ripe_vectors(L: int, W: int, R: int, n_recurrent: int, n_plain: int = 0) -> int:
    return n_plain * L + n_recurrent * (L + min(W, L) * (R - 1))


def ripe_fraction(L: int, W: int, R: int, n_recurrent: int, n_plain: int = 0) -> float:
    """RIPE memory as a fraction of the full per-loop cache."""
    return ripe_vectors(L, W, R, n_recurrent, n_plain) / full_vectors(L, R, n_recurrent, n_plain)


def vector_bytes(n_heads_kv: int, head_dim: int) -> int:
    """Key and value of one (position, loop) for all KV heads, bf16."""
    return 2 * n_heads_kv * head_dim * 2


def sequence_bytes(L: int, W: int, R: int, n_heads_kv: int, head_dim: int,
                   n_recurrent: int, n_plain: int = 0) -> int:
    """Cache bytes of one sequence holding L positions (W >= L: full cache)."""
    return ripe_vectors(L, W, R, n_recurrent, n_plain) * vector_bytes(n_heads_kv, head_dim)


def max_batch(budget_bytes: int, per_sequence_bytes: int) -> int:
    """Sequences a memory budget holds."""
    return budget_bytes // per_sequence_bytes
