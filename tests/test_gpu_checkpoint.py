"""Checkpoint and resume of a RIPE cache (GPU).

A cache's storage is its whole state: the lengths section and the planes.  The
test copies one cache's storage to the host part-way through a stream of
appends, binds a fresh handle to a device copy of that image with
ripe_cache_open, applies the same later appends (ring wrap-around, windows
that evict, a sequence filled to capacity) to both caches, and requires after
every append byte-equal storage and equal lengths, and at the end bit-equal
verify outputs (the same kernels over the same bytes).  An image with a
length past the capacity is refused and binds no handle.
"""
import ctypes

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


NL, R, HQ, HKV, D_HEAD, W, B, CAP, DMAX = 2, 4, 4, 2, 64, 40, 3, 300, 8


def _cache(image=None):
    return RipeCache(NL, R, HQ, HKV, D_HEAD, W, B, CAP, DMAX, device="cuda", image=image)


def _append(caches, gen, layer, n):
    T, U = max(max(n), 1), max(min(max(n), 64), 1)
    dk = torch.randn(B, HKV, T, D_HEAD, generator=gen, device="cuda").to(torch.bfloat16)
    dv = torch.randn(B, HKV, T, D_HEAD, generator=gen, device="cuda").to(torch.bfloat16)
    wk = torch.randn(B, R - 1, HKV, U, D_HEAD, generator=gen, device="cuda").to(torch.bfloat16)
    wv = torch.randn(B, R - 1, HKV, U, D_HEAD, generator=gen, device="cuda").to(torch.bfloat16)
    for c in caches:
        c.append(layer, n, dk, dv, wk, wv)
    torch.cuda.synchronize()


def _same(a, b):
    torch.cuda.synchronize()
    assert torch.equal(a.storage, b.storage)
    for layer in range(NL):
        assert list(a.lengths(layer)) == list(b.lengths(layer))


def test_resume_from_a_host_image_matches_the_uninterrupted_cache():
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    a = _cache()
    # before the checkpoint: prefixes of different lengths on both layers
    _append([a], gen, 0, [150, 37, 0])
    _append([a], gen, 1, [5, 260, 61])
    _append([a], gen, 0, [8, 8, 8])
    torch.cuda.synchronize()
    image = a.storage.cpu()                      # the checkpoint, on the host
    b = _cache(image=image)
    _same(a, b)
    # after it: the same appends on both
    for layer, n in [(0, [40, 1, 64]), (1, [0, 39, 100]), (0, [102, 0, 7]), (1, [35, 1, 0]),
                     (0, [0, 254, 1])]:
        _append([a, b], gen, layer, n)
        _same(a, b)
    assert list(a.lengths(0)) == [300, 300, 80]
    # both refuse the same append past the capacity, and stay equal
    for c in (a, b):
        with pytest.raises(ripe.RipeError):
            _append([c], torch.Generator(device="cuda").manual_seed(1), 0, [1, 0, 0])
    _same(a, b)
    # verification over the two images gives the same bits
    rows = [(i, r) for i in range(DMAX) for r in range(1, R + 1)]
    q = torch.randn(B, len(rows), HQ, D_HEAD, generator=gen, device="cuda").to(torch.bfloat16)
    blk_k = torch.randn(B, R, HKV, DMAX, D_HEAD, generator=gen, device="cuda").to(torch.bfloat16)
    blk_v = torch.randn(B, R, HKV, DMAX, D_HEAD, generator=gen, device="cuda").to(torch.bfloat16)
    for layer in range(NL):
        oa, la = a.verify(layer, rows, q, blk_k, blk_v, DMAX)
        ob, lb = b.verify(layer, rows, q, blk_k, blk_v, DMAX)
        torch.cuda.synchronize()
        assert torch.isfinite(oa).all()
        assert torch.equal(oa, ob) and torch.equal(la, lb)
    a.close()
    b.close()


def test_image_with_a_length_past_capacity_is_refused():
    gen = torch.Generator(device="cuda")
    gen.manual_seed(12)
    a = _cache()
    _append([a], gen, 0, [10, 20, 30])
    torch.cuda.synchronize()
    image = a.storage.cpu().clone()
    lens_at = ripe.ripe_section_offset(a.cfg, ripe.RIPE_SECTION_LENS)
    lens = image[lens_at:lens_at + 4 * NL * B].view(torch.int32)
    lens[B + 2] = CAP + 1                         # layer 1, sequence 2
    storage = torch.empty_like(a.storage)
    storage.copy_(image)
    torch.cuda.synchronize()
    h = ctypes.c_void_p()
    st = ripe.load().ripe_cache_open(ctypes.byref(a.cfg), ctypes.c_void_p(storage.data_ptr()),
                                     storage.numel(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream),
                                     ctypes.byref(h))
    assert st == ripe.RIPE_EINVAL and not h.value
    lens[B + 2] = 0                               # the untouched image opens
    b = _cache(image=image)
    assert list(b.lengths(0)) == [10, 20, 30] and list(b.lengths(1)) == [0, 0, 0]
    a.close()
    b.close()
