"""Calls run asynchronously on the stream they are given (GPU).

Every launch of a call (verify and combine, append) must be ordered after the
work queued before it on the caller's stream, and the call must return to the
host without waiting for that work.  Queued on stream A behind a long spin
and a copy that fills the call's inputs (which hold zeros until then), a call
on A returns while A is still busy and, once A is done, gives exactly the
result of the same call on the real inputs: a launch on any other stream would
have read the zeros.  (Observing the outputs from a third stream instead
proves nothing: with a few hardware queues per process, two streams may share
one and run in order.)  Two handles driven from two streams at once give the
same bits as the same calls made one after the other.  All streams have the
default priority.
"""
import pytest
import torch

from synth import Workload, grid_rows

from helpers import TUNINGS, step_arrays

pytestmark = pytest.mark.gpu

SPIN = 200_000_000          # spin cycles queued ahead of the call


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import self_speculative_verify_amd.ripe as r
    r.load()
    yield


def _cache(wl, tuning):
    import ripe_harness as H
    from self_speculative_verify_amd import ripe
    c = H.make_cache(wl)
    if tuning:
        ripe.ripe_set_tuning(c.handle, tuning)
    H.load_prefix(c, wl)
    return c


@pytest.mark.parametrize("tuning_name", ["planner", "keys-chunked", "rows-chunked", "keys-8waves"])
def test_verify_is_ordered_on_the_given_stream(tuning_name):
    import ripe_harness as H
    wl = Workload("stream", 85, 1, 4, 4, 2, 96, 8, 4, [300, 70], 0.88, grid_rows(4, 4))
    cache = _cache(wl, TUNINGS[tuning_name])
    q, bk, bv = H.verify_inputs(wl, 0)
    ref_o, ref_l = cache.verify(0, wl.rows, q, bk, bv, wl.n_blk)     # also sizes the workspace
    qz, bkz, bvz = torch.zeros_like(q), torch.zeros_like(bk), torch.zeros_like(bv)
    out, lse = torch.zeros_like(ref_o), torch.zeros_like(ref_l)
    torch.cuda.synchronize()
    a = torch.cuda.Stream()
    with torch.cuda.stream(a):
        torch.cuda._sleep(SPIN)
        qz.copy_(q)
        bkz.copy_(bk)
        bvz.copy_(bv)
        cache.verify(0, wl.rows, qz, bkz, bvz, wl.n_blk, out=out, lse=lse, stream=a)
    assert not a.query(), "the call waited for the stream's earlier work"
    a.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), "a launch did not follow the stream's order"


def test_append_is_ordered_on_the_given_stream():
    import ripe_harness as H
    wl = Workload("stream_app", 86, 1, 4, 4, 2, 64, 8, 4, [40, 10], 0.88, grid_rows(4, 4), capacity=64)
    ref = _cache(wl, None)
    cache = _cache(wl, None)
    arrs = [H.to_dev(x) for x in step_arrays(wl, 0, wl.lens, [6, 3])]
    ref.append(0, [6, 3], *arrs)
    zs = [torch.zeros_like(x) for x in arrs]
    torch.cuda.synchronize()
    a = torch.cuda.Stream()
    with torch.cuda.stream(a):
        torch.cuda._sleep(SPIN)
        for z, x in zip(zs, arrs):
            z.copy_(x)
        cache.append(0, [6, 3], *zs, stream=a)
    assert not a.query(), "the append waited for the stream's earlier work"
    a.synchronize()
    assert torch.equal(cache.storage, ref.storage), "the append did not follow the stream's order"
    assert cache.lengths(0) == [46, 13]


def test_two_handles_on_two_streams():
    """Interleaved calls of two caches on two streams equal the same calls
    made one after the other on one stream."""
    import ripe_harness as H
    wls = [Workload("s1", 87, 1, 4, 4, 2, 128, 8, 4, [400, 90], 0.81, grid_rows(4, 4)),
           Workload("s2", 88, 1, 3, 4, 4, 96, 16, 4, [250], 0.88, grid_rows(4, 3))]
    caches = [_cache(w, TUNINGS["keys-chunked"]) for w in wls]
    ins = [H.verify_inputs(w, 0) for w in wls]
    torch.cuda.synchronize()
    ref = []
    for c, w, (q, bk, bv) in zip(caches, wls, ins):
        ref.append([t.clone() for t in c.verify(0, w.rows, q, bk, bv, w.n_blk)])
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.empty_like(t) for t in r] for r in ref]
    for rep in range(4):
        for k in (0, 1):
            with torch.cuda.stream(streams[k]):
                q, bk, bv = ins[k]
                caches[k].verify(0, wls[k].rows, q, bk, bv, wls[k].n_blk, out=outs[k][0], lse=outs[k][1],
                                 stream=streams[k])
    for s in streams:
        s.synchronize()
    for r, o in zip(ref, outs):
        assert torch.equal(r[0], o[0]) and torch.equal(r[1], o[1])
