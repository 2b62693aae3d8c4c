"""Guard bands around every buffer the library writes (GPU).

Each buffer a call writes (output rows, LSE, workspace, cache storage) is
handed to the library as the middle of a larger allocation whose edges hold
a fixed byte pattern: a kernel that writes past either end of its buffer, or
a launch whose grid covers more than its outputs, changes an edge.  Inputs a
call only reads (queries, draft-block planes, and the storage while it
verifies) must come back bit-identical, and every output element must be
written (no pattern left inside).  The guarded calls must also give the same
bits as the same calls on ordinarily allocated buffers.

Covered: every launch choice of the parity tests (both kernels, four and
eight waves, one and two row tiles, with and without private waves, split
key ranges with their workspace and combine launch) at each head size, a
call of more rows than one launch takes, appends that evict window
positions and a batch larger than one append launch, windowed draft
attention, and the allocation-free entry point.
"""
import pytest
import torch

from self_speculative_verify_amd import RipeCache, ripe
from synth import Workload, grid_rows, ragged_lengths

from helpers import TUNINGS, all_written, edges_intact, guarded, step_arrays

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ripe.load()
    yield


class GuardedCache(RipeCache):
    """A RipeCache whose storage is the middle of a guarded allocation."""

    def __init__(self, wl: Workload, tuning=None):
        self.cfg = ripe.config(wl.n_layers, wl.n_loops, wl.n_heads_q, wl.n_heads_kv, wl.head_dim,
                               wl.window, wl.batch, wl.capacity, wl.max_block, wl.anchor)
        self.nbytes = ripe.ripe_cache_bytes(self.cfg)
        assert self.nbytes > 0
        self.full, self.storage = guarded(self.nbytes)
        self.handle = ripe.ripe_cache_create(self.cfg, self.storage)
        self._ws = None
        if tuning:
            ripe.ripe_set_tuning(self.handle, tuning)


def guarded_verify(cache: RipeCache, wl: Workload, q, bk, bv, noalloc=False):
    """One verify call of wl.rows with guarded out / LSE / workspace; checks the
    guards and that every output was written; returns (out, lse) copies."""
    B, n, Hq, d = wl.batch, wl.n_rows, wl.n_heads_q, wl.head_dim
    o_bytes, l_bytes = B * n * Hq * d * 4, B * n * Hq * 4
    o_full, o_mid = guarded(o_bytes)
    l_full, l_mid = guarded(l_bytes)
    ws_bytes = 0 if noalloc else ripe.ripe_workspace_bytes(cache.handle, n)
    ws_full, ws_mid = guarded(ws_bytes) if ws_bytes else (None, None)
    out = o_mid.view(torch.float32).view(B, n, Hq, d)
    lse = l_mid.view(torch.float32).view(B, n, Hq)
    rb, rl = [i for i, _ in wl.rows], [r for _, r in wl.rows]
    kv = ripe.kv_view(bk, "bphtd"), ripe.kv_view(bv, "bphtd")
    if noalloc:
        ripe.ripe_verify_attn_noalloc(cache.handle, 0, rb, rl, q, *kv, wl.n_blk, out, lse)
    else:
        ripe.ripe_verify_attn(cache.handle, 0, rb, rl, q, *kv, wl.n_blk, out, lse, ws_mid)
    torch.cuda.synchronize()
    assert edges_intact(o_full, o_bytes), "write outside the output rows"
    assert edges_intact(l_full, l_bytes), "write outside the LSE array"
    if ws_full is not None:
        assert edges_intact(ws_full, ws_bytes), "write outside the workspace"
    assert all_written(o_mid), "output element left unwritten"
    assert all_written(l_mid), "LSE element left unwritten"
    return out.clone(), lse.clone()


def check_case(wl: Workload, tuning_name: str):
    import ripe_harness as H
    tuning = TUNINGS[tuning_name]
    cache = GuardedCache(wl, tuning)
    H.load_prefix(cache, wl, [0])
    torch.cuda.synchronize()
    assert edges_intact(cache.full, cache.nbytes), "append wrote outside the storage"
    q, bk, bv = H.verify_inputs(wl, 0)
    before = [t.clone() for t in (cache.storage, q, bk, bv)]
    out, lse = guarded_verify(cache, wl, q, bk, bv)
    for a, b, what in zip((cache.storage, q, bk, bv), before, ("storage", "queries", "block K", "block V")):
        assert torch.equal(a, b), f"verify changed its input ({what})"
    assert edges_intact(cache.full, cache.nbytes), "verify wrote outside the storage"
    # the same call on ordinary buffers gives the same bits
    plain = H.make_cache(wl)
    if tuning:
        ripe.ripe_set_tuning(plain.handle, tuning)
    H.load_prefix(plain, wl, [0])
    o2, l2 = plain.verify(0, wl.rows, q, bk, bv, wl.n_blk)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, l2), "guarded and plain calls differ"
    print(f"{wl.name} [{tuning_name}]: guards intact, {out.numel()} outputs written", flush=True)
    return cache


SHAPES = {
    # head size, query / KV heads, loops, window, lengths, rows
    "d64": Workload("g64", 71, 1, 4, 4, 2, 64, 8, 4, [150, 61, 7], 0.88, grid_rows(4, 4)),
    "d96": Workload("g96", 72, 1, 6, 4, 4, 96, 16, 8, [230, 40], 0.88, grid_rows(8, 6),
                    heavy_frac=0.02),
    "d128": Workload("g128", 73, 1, 8, 8, 2, 128, 16, 8, [300, 41], 0.81, grid_rows(8, 8)),
}


@pytest.mark.parametrize("shape", list(SHAPES))
@pytest.mark.parametrize("tuning_name", ["planner", "keys", "keys-8waves", "rows", "rows-2tiles",
                                         "rows-private", "rows-noprivate", "keys-chunked",
                                         "keys-8waves-chunked", "rows-chunked"])
def test_verify_guard_bands(shape, tuning_name):
    check_case(SHAPES[shape], tuning_name)


def test_more_rows_than_one_launch_guard_bands():
    """288 rows: a launch of 256 rows and one of 32, the second split into
    chunks (its workspace share is the larger one)."""
    wl = Workload("g288", 74, 1, 24, 4, 2, 64, 16, 12, [150, 61], 0.88, grid_rows(12, 24))
    check_case(wl, "planner")
    check_case(wl, "rows-chunked")


def test_append_guard_bands_with_eviction_and_two_launches():
    """70 sequences (two append launches per layer), a prefix and then a
    block of accepted tokens that evicts window positions: storage edges
    intact after each append, and the bytes equal those of an ordinary
    cache that took the same appends."""
    import ripe_harness as H
    lens = ragged_lengths(75, 70, 0, 40)
    wl = Workload("gapp", 75, 1, 3, 2, 1, 64, 6, 5, lens, 0.88, grid_rows(5, 3))
    g = GuardedCache(wl)
    p = H.make_cache(wl)
    for c in (g, p):
        H.load_prefix(c, wl, [0])
    n_new = [(b % 5) + 1 for b in range(wl.batch)]
    arrs = [H.to_dev(a) for a in step_arrays(wl, 0, lens, n_new)]
    for c in (g, p):
        c.append(0, n_new, *arrs)
    torch.cuda.synchronize()
    assert edges_intact(g.full, g.nbytes), "append wrote outside the storage"
    assert torch.equal(g.storage, p.storage), "guarded and plain storage differ"
    assert g.lengths(0) == [L + k for L, k in zip(lens, n_new)]


def test_draft_attn_guard_bands():
    """Windowed draft attention (sinks plus a window, single-row calls and a
    whole grid): output and LSE edges intact, every element written."""
    import ripe_harness as H
    wl = SHAPES["d96"]
    cache = GuardedCache(wl)
    H.load_prefix(cache, wl, [0])
    q, bk, bv = H.verify_inputs(wl, 0)
    kv = ripe.kv_view(bk, "bphtd"), ripe.kv_view(bv, "bphtd")
    for rows in (wl.rows, [(3, 2)]):
        B, n, Hq, d = wl.batch, len(rows), wl.n_heads_q, wl.head_dim
        qq = q[:, :n].contiguous() if n < wl.n_rows else q
        o_bytes, l_bytes = B * n * Hq * d * 4, B * n * Hq * 4
        o_full, o_mid = guarded(o_bytes)
        l_full, l_mid = guarded(l_bytes)
        out = o_mid.view(torch.float32).view(B, n, Hq, d)
        lse = l_mid.view(torch.float32).view(B, n, Hq)
        ripe.ripe_draft_attn(cache.handle, 0, [i for i, _ in rows], [r for _, r in rows], qq, *kv,
                             wl.n_blk, 2, 24, out, lse)
        torch.cuda.synchronize()
        assert edges_intact(o_full, o_bytes) and edges_intact(l_full, l_bytes)
        assert all_written(o_mid) and all_written(l_mid)
    assert edges_intact(cache.full, cache.nbytes)


def test_noalloc_guard_bands():
    """The allocation-free entry point (its partial states in the library's
    own scratch): output edges intact, every element written, same bits as
    ripe_verify_attn with a workspace."""
    import ripe_harness as H
    wl = SHAPES["d128"]
    cache = GuardedCache(wl, TUNINGS["rows-chunked"])
    H.load_prefix(cache, wl, [0])
    q, bk, bv = H.verify_inputs(wl, 0)
    o1, l1 = guarded_verify(cache, wl, q, bk, bv, noalloc=True)
    o2, l2 = guarded_verify(cache, wl, q, bk, bv)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
