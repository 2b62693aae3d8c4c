"""WaveFront decoding of a looped model over a RIPE cache (host side).

WaveFront page ("Draft and verification go through the model at the same
time"): one batched call of the shared block processes positions at different
depths -- the newest reaches the draft depth, earlier ones continue, the
oldest reaches full depth and is checked -- so the (position, depth) states
form a diagonal wave.  On a mismatch the scheduler keeps the full-depth
token, clears the later states and grows the wave again; the discarded work is
bounded by the wave's width.

Readings taken here (the page gives no algorithm):

* A call runs one loop of the block for every position in flight: position
  p at depth d (loops done) is the row (p - L, d + 1) of the attention call,
  L the committed length.
* The newest position drafts the next token when it reaches depth r_draft;
  the new position enters the next call at depth 0.  In steady state the
  positions sit r_draft loops apart and the wave is ceil(R / r_draft) wide.
* A position that reaches depth R is committed: all its planes go to the
  cache (ripe_append of one token).  Its full-depth prediction then checks
  the next position's token: if it differs, every later position is dropped
  and the corrected token re-enters at depth 0.  Nothing but committed
  positions ever reaches the cache, so a rollback leaves the ring and the
  deep rows untouched; the planes of positions in flight live in the wave
  buffer, which the caller owns.
* Shared KV across loops (the page's faster, approximate variant): one plane
  per position; a position in flight exposes the plane of its latest loop
  and a committed one its last.  As a plane map this is a one-plane cache
  (n_loops = 1) and every row at loop 1; the scheduling is unchanged.

Calls per committed token: r_draft when every draft is accepted, R when none
is, and in expectation alpha * r_draft + (1 - alpha) * R for an acceptance
probability alpha (after the first token, which needs R calls).
"""
from __future__ import annotations

import dataclasses
from typing import Callable, List, Optional, Tuple

import torch


@dataclasses.dataclass
class InFlight:
    pos: int        # absolute position
    depth: int      # loops done
    version: int    # distinct for every token that ever occupied a position


@dataclasses.dataclass
class StepEvent:
    committed: Optional[int] = None     # position committed after this call
    rejected: bool = False              # the next position's draft was replaced
    dropped: int = 0                    # positions cleared by the rejection
    dropped_loops: int = 0              # loops of work they had done
    drafted: Optional[int] = None       # position that entered the wave


class WaveScheduler:
    """The wave's state for one sequence; decides the rows of every call."""

    def __init__(self, n_loops: int, r_draft: int, committed: int):
        if n_loops < 2 or not 1 <= r_draft < n_loops:
            raise ValueError("WaveFront needs R >= 2 loops and 1 <= r_draft < R")
        self.R, self.r_draft = n_loops, r_draft
        self.L = committed
        self._versions = 0
        self.wave: List[InFlight] = [self._new(committed)]
        self.calls = self.commits = self.rejections = 0
        self.dropped_loops = 0

    def _new(self, pos: int) -> InFlight:
        self._versions += 1
        return InFlight(pos, 0, self._versions)

    @property
    def width(self) -> int:
        return len(self.wave)

    def rows(self) -> List[Tuple[int, int]]:
        """(block offset, loop) of every position in flight, oldest first."""
        return [(x.pos - self.L, x.depth + 1) for x in self.wave]

    def after_call(self, accept: Callable[[], bool]) -> StepEvent:
        """Advance the state past one call.  ``accept()`` is asked once per
        commit that has a successor in flight: does the successor's draft
        token equal the committed position's full-depth prediction?"""
        ev = StepEvent()
        for x in self.wave:
            x.depth += 1
        self.calls += 1
        if self.wave[0].depth == self.R:
            done = self.wave.pop(0)
            ev.committed = done.pos
            self.L = done.pos + 1
            self.commits += 1
            if not self.wave:
                self.wave.append(self._new(self.L))        # next token is certain
            elif not accept():
                ev.rejected = True
                ev.dropped = len(self.wave)
                ev.dropped_loops = sum(x.depth for x in self.wave)
                self.dropped_loops += ev.dropped_loops
                self.rejections += 1
                self.wave = [self._new(self.L)]             # corrected token
        if self.wave[-1].depth == self.r_draft:
            nxt = self._new(self.wave[-1].pos + 1)
            self.wave.append(nxt)
            ev.drafted = nxt.pos
        return ev


def expected_calls_per_token(n_loops: int, r_draft: int, alpha: float) -> float:
    """Steady-state calls per committed token for acceptance probability alpha."""
    return alpha * r_draft + (1.0 - alpha) * n_loops


class WaveBuffer:
    """Device planes of the positions in flight, laid out so the verify call's
    draft-block view is a plain strided view: bf16 [B][P][Hkv][slots][d] with
    P = n_loops planes (1 for shared KV).  Positions occupy consecutive slots
    from `start`; when the end is reached the live slots move to the front."""

    def __init__(self, batch: int, planes: int, n_heads_kv: int, head_dim: int,
                 slots: int = 64, device="cuda"):
        self.k = torch.zeros((batch, planes, n_heads_kv, slots, head_dim), dtype=torch.bfloat16,
                             device=device)
        self.v = torch.zeros_like(self.k)
        self.slots, self.start, self.count = slots, 0, 0

    def reset(self, keep: int = 0) -> None:
        """Keep the first `keep` positions in flight (drop the rest)."""
        self.count = keep

    def push(self) -> int:
        """Slot for a new newest position."""
        if self.start + self.count == self.slots:
            n = self.count
            self.k[:, :, :, :n] = self.k[:, :, :, self.start:self.start + n].clone()
            self.v[:, :, :, :n] = self.v[:, :, :, self.start:self.start + n].clone()
            self.start = 0
        self.count += 1
        return self.start + self.count - 1

    def pop_oldest(self) -> None:
        self.start += 1
        self.count -= 1
        if self.count == 0:
            self.start = 0

    def slot(self, j: int) -> int:
        return self.start + j

    def block(self) -> Tuple[torch.Tensor, torch.Tensor]:
        """Views [B][P][Hkv][count..][d] starting at the oldest position."""
        return self.k[:, :, :, self.start:], self.v[:, :, :, self.start:]

    def oldest_planes(self):
        """(deep_k, deep_v, win_k, win_v) of the oldest position for
        ripe_append: its last plane and, with more than one plane, the others."""
        s = self.start
        dk, dv = self.k[:, -1, :, s:s + 1], self.v[:, -1, :, s:s + 1]
        if self.k.shape[1] > 1:
            return dk, dv, self.k[:, :-1, :, s:s + 1], self.v[:, :-1, :, s:s + 1]
        return dk, dv, None, None


def kernel_rows(rows: List[Tuple[int, int]], shared_kv: bool) -> List[Tuple[int, int]]:
    """Rows as the verify call takes them: with shared KV every loop reads the
    one stored plane, so every row is at loop 1 of a one-plane cache."""
    return [(i, 1) for i, _ in rows] if shared_kv else list(rows)


__all__ = ["InFlight", "StepEvent", "WaveScheduler", "expected_calls_per_token", "WaveBuffer",
           "kernel_rows"]
