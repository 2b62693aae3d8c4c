"""Row sets of the attention calls that one decoding step of a looped model makes.

A verify call attends rows (block offset i, loop r) of the draft block; which
rows go into one call is a scheduling choice, and the kernels take any set.
Three schedules (page "Prefix Keys and Values Matter Late", abstract, first
sentence: a draft runs a few loops, the verification runs all R of them; the
WaveFront page, "Draft and verification go through the model at the same
time", for the order a forward pass runs in):

* ``batched_verify``: the whole D x R grid in one call.  Every loop's rows see
  the deepest plane of the shared prefix once.
* ``per_loop_verify``: loop by loop, as a forward pass runs them: R calls of D
  rows (loop r's queries only exist once loop r - 1 is done).  Each call reads
  the shared prefix again.
* ``draft_pass``: drafting token j runs loops 1..r_draft on position L + j one
  after the other, each a call of the single row (j, r) over the committed
  cache and the draft tokens 0..j; D * r_draft calls per block.

A row's result does not depend on which other rows share its call, so every
schedule gives, row by row, the result of the batched call (the block keys a
row (j, r) reads are the tokens 0..j, so a draft call needs only n_blk = j + 1).
"""
from __future__ import annotations

from typing import List, NamedTuple, Tuple

Row = Tuple[int, int]


class Call(NamedTuple):
    rows: List[Row]      # (block offset i, loop r), 0 <= i < n_blk, 1 <= r <= R
    n_blk: int           # draft-block tokens the call reads (block keys 0..n_blk-1)


def batched_verify(n_blk: int, n_loops: int) -> List[Call]:
    return [Call([(i, r) for i in range(n_blk) for r in range(1, n_loops + 1)], n_blk)]


def per_loop_verify(n_blk: int, n_loops: int) -> List[Call]:
    return [Call([(i, r) for i in range(n_blk)], n_blk) for r in range(1, n_loops + 1)]


def draft_pass(n_blk: int, r_draft: int) -> List[Call]:
    if r_draft < 1:
        raise ValueError("a draft runs at least one loop")
    return [Call([(j, r)], j + 1) for j in range(n_blk) for r in range(1, r_draft + 1)]
