"""Calls captured in a HIP graph (GPU).

A step's calls can be captured once and replayed (the bench times such
replays).  Every replay must give the bits of the same calls made eagerly:
each case captures one verify call and one windowed draft call on two layers
(split key ranges, with their workspace and combine launch, in the chunked
choices), then replays the graph several times with the program's own eager
work between replays (outputs cleared, a call on another row set that
reuses the workspace, synchronizations) and compares every replay with the
eager results.  The library records no memset or allocation in a call.
"""
import pytest
import torch

from synth import Workload, grid_rows

from helpers import TUNINGS

pytestmark = pytest.mark.gpu

N_SINK, W_DRAFT = 2, 24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from self_speculative_verify_amd import ripe
    ripe.load()
    yield


def _calls(cache, wl, ins, outs):
    q0, bk0, bv0 = ins[0]
    q1, bk1, bv1 = ins[1]
    cache.verify(0, wl.rows, q0, bk0, bv0, wl.n_blk, out=outs[0][0], lse=outs[0][1])
    cache.draft(1, wl.rows, q1, bk1, bv1, wl.n_blk, N_SINK, W_DRAFT, out=outs[1][0], lse=outs[1][1])


@pytest.mark.parametrize("d", [96, 128])
@pytest.mark.parametrize("tuning_name", ["planner", "keys-chunked", "rows-chunked", "keys-8waves"])
def test_graph_replays_equal_eager_calls(tuning_name, d):
    import ripe_harness as H
    from self_speculative_verify_amd import ripe
    wl = Workload("graph", 89, 2, 4, 4, 2, d, 8, 4, [300, 90], 0.81, grid_rows(4, 4))
    cache = H.make_cache(wl)
    if TUNINGS[tuning_name]:
        ripe.ripe_set_tuning(cache.handle, TUNINGS[tuning_name])
    H.load_prefix(cache, wl)
    ins = [H.verify_inputs(wl, layer) for layer in (0, 1)]
    B, n, Hq = wl.batch, wl.n_rows, wl.n_heads_q
    ref = [(torch.empty(B, n, Hq, d, device="cuda"), torch.empty(B, n, Hq, device="cuda")) for _ in (0, 1)]
    sub = wl.rows[:3]
    q_sub = ins[0][0][:, :3].contiguous()
    # eager calls first: they size the handle's workspace for both row sets,
    # so the call between replays does not replace the buffer the graph holds
    cache.verify(0, sub, q_sub, ins[0][1], ins[0][2], wl.n_blk)
    _calls(cache, wl, ins, ref)
    torch.cuda.synchronize()
    outs = [(torch.empty_like(o), torch.empty_like(l)) for o, l in ref]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _calls(cache, wl, ins, outs)
    torch.cuda.synchronize()
    ws_captured = cache._ws                      # kept alive while the graph is replayed
    for rep in range(4):
        for o, l in outs:
            o.fill_(float("nan"))
            l.fill_(float("nan"))
        cache.verify(0, sub, q_sub, ins[0][1], ins[0][2], wl.n_blk)      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (o, l), (ro, rl) in zip(outs, ref):
            assert torch.equal(o, ro) and torch.equal(l, rl), f"replay {rep} differs from the eager calls"
    assert cache._ws is ws_captured
    print(f"graph [{tuning_name}] d={d}: 4 replays equal the eager calls", flush=True)
