"""Error paths of the real library on a live handle (GPU).

Every refused call must return its status before anything is enqueued: the
storage bytes, the committed lengths (host copy and storage) and the output
buffers stay exactly as they were.  Covered: an append past the capacity
(RIPE_ECAPACITY), rows with a block offset or loop out of range, n_blk past
max_block, a workspace one byte short, a null workspace when one is needed
(RIPE_EINVAL), and calls on a destroyed handle (refused; a second destroy is
harmless).
"""
import ctypes

import numpy as np
import pytest
import torch

from self_speculative_verify_amd import RipeCache, ripe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ripe.load()
    yield


R, HQ, HKV, D_HEAD, W, B, CAP, DMAX = 4, 4, 2, 64, 8, 3, 100, 4


def _filled_cache():
    torch.manual_seed(5)
    c = RipeCache(1, R, HQ, HKV, D_HEAD, W, B, CAP, DMAX, device="cuda")
    n = [60, 17, 99]
    T, U = max(n), min(max(n), W)
    dk = torch.randn(B, HKV, T, D_HEAD, device="cuda").to(torch.bfloat16)
    dv = torch.randn_like(dk)
    wk = torch.randn(B, R - 1, HKV, U, D_HEAD, device="cuda").to(torch.bfloat16)
    wv = torch.randn_like(wk)
    c.append(0, n, dk, dv, wk, wv)
    torch.cuda.synchronize()
    return c, n


def _snapshot(c):
    torch.cuda.synchronize()
    return c.storage.cpu().numpy().copy(), list(c.lengths(0))


def _verify_raw(c, rows_blk, rows_loop, n_blk, out, lse, ws=None, ws_bytes=None):
    q = torch.zeros((B, len(rows_blk), HQ, D_HEAD), dtype=torch.bfloat16, device="cuda")
    blk = torch.zeros((B, R, HKV, DMAX, D_HEAD), dtype=torch.bfloat16, device="cuda")
    v = ripe.kv_view(blk, "bphtd")
    L = ripe.load()
    n = len(rows_blk)
    rb = (ctypes.c_int32 * n)(*rows_blk)
    rl = (ctypes.c_int32 * n)(*rows_loop)
    ws_ptr = ctypes.c_void_p(ws.data_ptr()) if ws is not None else ctypes.c_void_p()
    if ws_bytes is None:
        ws_bytes = ws.numel() if ws is not None else 0
    st = L.ripe_verify_attn(c.handle, 0, n, rb, rl, ctypes.c_void_p(q.data_ptr()), v, v, n_blk,
                            ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
                            ws_ptr, ws_bytes, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return st


def test_append_past_capacity_changes_nothing():
    c, n = _filled_cache()
    img, lens = _snapshot(c)
    assert lens == n
    T = 2
    dk = torch.randn(B, HKV, T, D_HEAD, device="cuda").to(torch.bfloat16)
    wk = torch.randn(B, R - 1, HKV, T, D_HEAD, device="cuda").to(torch.bfloat16)
    with pytest.raises(ripe.RipeError) as e:
        c.append(0, [1, 1, 2], dk, dk, wk, wk)      # the last sequence would reach 101 > 100
    assert e.value.status == ripe.RIPE_ECAPACITY
    img2, lens2 = _snapshot(c)
    assert lens2 == lens
    assert np.array_equal(img, img2), "a refused append wrote to the storage"
    # the capacity itself is reachable
    c.append(0, [0, 0, 1], dk, dk, wk, wk)
    assert c.lengths(0) == [60, 17, 100]
    lens_dev = c.section(ripe.RIPE_SECTION_LENS)[:4 * B].cpu().numpy().view(np.int32).tolist()
    assert lens_dev == [60, 17, 100]


@pytest.mark.parametrize("case", ["offset>=n_blk", "negative-offset", "loop0", "loopR+1",
                                  "n_blk>max_block", "n_blk0"])
def test_bad_rows_refused_without_side_effect(case):
    c, _ = _filled_cache()
    img, lens = _snapshot(c)
    rows_blk, rows_loop, n_blk = [0, 1, 2], [1, 2, R], 3
    if case == "offset>=n_blk":
        rows_blk = [0, 3, 1]
    elif case == "negative-offset":
        rows_blk = [0, -1, 1]
    elif case == "loop0":
        rows_loop = [0, 1, 1]
    elif case == "loopR+1":
        rows_loop = [1, R + 1, 1]
    elif case == "n_blk>max_block":
        n_blk = DMAX + 1
    elif case == "n_blk0":
        n_blk = 0
    out = torch.full((B, 3, HQ, D_HEAD), 7.0, device="cuda")
    lse = torch.full((B, 3, HQ), 7.0, device="cuda")
    assert _verify_raw(c, rows_blk, rows_loop, n_blk, out, lse) == ripe.RIPE_EINVAL
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all()), "a refused call wrote outputs"
    img2, lens2 = _snapshot(c)
    assert lens2 == lens and np.array_equal(img, img2)


def test_undersized_and_missing_workspace_refused():
    c, _ = _filled_cache()
    ripe.ripe_set_tuning(c.handle, {"kernel": 1, "items_target": 100000, "min_chunk": 32})
    rows_blk, rows_loop = [0, 1, 2, 3], [1, 2, 3, 4]
    need = ripe.ripe_workspace_bytes(c.handle, len(rows_blk))
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = torch.full((B, 4, HQ, D_HEAD), 7.0, device="cuda")
    lse = torch.full((B, 4, HQ), 7.0, device="cuda")
    assert _verify_raw(c, rows_blk, rows_loop, DMAX, out, lse, ws, need - 1) == ripe.RIPE_EINVAL
    assert _verify_raw(c, rows_blk, rows_loop, DMAX, out, lse, None, need) == ripe.RIPE_EINVAL
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all())
    # the exact size is accepted and gives the same result as the unsplit call
    assert _verify_raw(c, rows_blk, rows_loop, DMAX, out, lse, ws, need) == ripe.RIPE_OK
    ripe.ripe_set_tuning(c.handle, None)
    out2, lse2 = torch.empty_like(out), torch.empty_like(lse)
    need2 = ripe.ripe_workspace_bytes(c.handle, len(rows_blk))
    ws2 = torch.empty(max(need2, 1), dtype=torch.uint8, device="cuda")
    assert _verify_raw(c, rows_blk, rows_loop, DMAX, out2, lse2, ws2, need2) == ripe.RIPE_OK
    assert float((out - out2).abs().max()) <= 1e-5
    assert float(((lse - lse2).abs() / lse2.abs().clamp(min=1)).max()) <= 1e-6


def test_destroyed_handle_refused_and_second_destroy_harmless():
    c, _ = _filled_cache()
    h = c.handle
    L = ripe.load()
    L.ripe_destroy(h)
    L.ripe_destroy(h)                       # already destroyed: ignored
    arr = (ctypes.c_int32 * B)()
    assert L.ripe_get_lengths(h, 0, arr) == ripe.RIPE_EINVAL
    assert L.ripe_workspace_bytes(h, 4) == 0
    out = torch.full((B, 1, HQ, D_HEAD), 7.0, device="cuda")
    lse = torch.full((B, 1, HQ), 7.0, device="cuda")
    c.handle = h
    assert _verify_raw(c, [0], [1], 1, out, lse) == ripe.RIPE_EINVAL
    c.handle = None                          # the binding's close() must not destroy it again
