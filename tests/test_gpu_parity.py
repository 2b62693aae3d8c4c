"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Layout: storage bytes bit-exact against the oracle's image after prefix
appends and after block appends that evict positions from the window.
Attention: max |O - O_ref| <= 2e-3 and |LSE - LSE_ref| / max(1, |LSE_ref|)
<= 1e-5 on every output, for reduced versions of the five workloads (sizes
the oracle finishes in seconds) and edge cases; the tagged-value probe checks
the exact key set of every row.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import WINDOW_FULL, Workload, f32_to_bf16, grid_rows, named_workload, wave_rows

from helpers import step_arrays, use_tuning

pytestmark = pytest.mark.gpu

TOL_O = 2e-3
TOL_LSE = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import self_speculative_verify_amd.ripe as r
    r.load()   # raises if the HIP library is not built
    yield


# Every case runs through both matrix-core kernels: the planner's choice, and
# the other one forced (keys: waves split keys; rows: waves own rows), each
# with one chunk and with several chunks per sequence (combine kernel), the
# keys kernel with four and with eight waves, the rows kernel with two row
# tiles per wave where the head size allows, and the rows kernel with and
# without its private waves (where the head size allows them).
@pytest.fixture(params=["auto", "keys", "keys-8waves", "rows", "rows-2tiles", "rows-private",
                        "rows-noprivate", "keys-chunked", "keys-8waves-chunked", "rows-chunked"],
                autouse=True)
def kernel_choice(request, monkeypatch):
    use_tuning(monkeypatch, request.param)
    yield request.param


def _h():
    import ripe_harness
    return ripe_harness


def assert_close(out, lse, ref_out, ref_lse, what=""):
    o = out.detach().cpu().double().numpy()
    l = lse.detach().cpu().double().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), what
    err_o = float(np.max(np.abs(o - ref_out))) if o.size else 0.0
    err_l = float(np.max(np.abs(l - ref_lse) / np.maximum(1.0, np.abs(ref_lse)))) if l.size else 0.0
    print(f"{what}: max|dO|={err_o:.3e} max rel dLSE={err_l:.3e}", flush=True)
    assert err_o <= TOL_O, f"{what}: max |dO| = {err_o}"
    assert err_l <= TOL_LSE, f"{what}: max rel dLSE = {err_l}"


def run_case(wl: Workload, window=None, anchor=None, layers=(0,), rows=None):
    H = _h()
    window = wl.window if window is None else window
    anchor = wl.anchor if anchor is None else anchor
    cache = H.make_cache(wl, window=window, anchor=anchor)
    H.load_prefix(cache, wl, layers)
    oc = oracle.prefix_cache(wl, layers=layers, anchor=anchor, window=window)
    torch.cuda.synchronize()
    assert np.array_equal(cache.storage.cpu().numpy(), oc.image), "layout differs from the oracle"
    rows = wl.rows if rows is None else rows
    wl_r = wl.replace(rows=list(rows))
    for layer in layers:
        q, bk, bv = H.verify_inputs(wl_r, layer)
        out, lse = cache.verify(layer, rows, q, bk, bv, wl.n_blk)
        torch.cuda.synchronize()
        ref_o, ref_l = oc.verify(layer, rows, wl_r.queries(layer), *wl_r.block(layer), wl.n_blk)
        assert_close(out, lse, ref_o, ref_l, f"{wl.name} W={window} anchor={anchor} layer={layer}")
    return cache, oc


# ---------------------------------------------------------------- workloads

@pytest.mark.parametrize("window", [16, WINDOW_FULL])
@pytest.mark.parametrize("anchor", [0, 1])
def test_tiny_both_layouts(window, anchor):
    run_case(named_workload("tiny"), window=window, anchor=anchor)


@pytest.mark.parametrize("window", [0, 8, 64, 1024])
def test_huginn_one_layer(window):
    wl = named_workload("huginn", n_layers=1, n_heads_q=11, n_heads_kv=11)
    run_case(wl, window=window)


@pytest.mark.parametrize("window,anchor", [(0, 0), (WINDOW_FULL, 0), (1024, 0), (1024, 1)])
def test_gqa_reduced(window, anchor):
    wl = named_workload("gqa", n_layers=1, lens=[1024, 1024])
    run_case(wl, window=window, anchor=anchor)


def test_ragged_reduced_with_block_append():
    wl = named_workload("ragged", n_layers=1, lens=[1500, 33, 700, 2100])
    cache, oc = run_case(wl)
    # accept the whole draft block: append its D tokens (loop R to the deep rows,
    # loops 1..R-1 to the ring, evicting the oldest window positions)
    H = _h()
    bk, bv = wl.block(0)
    D = wl.n_blk
    R = wl.n_loops
    tbk, tbv = H.to_dev(bk), H.to_dev(bv)
    cache.append(0, [D] * wl.batch, tbk[:, R - 1, :, :D], tbv[:, R - 1, :, :D],
                 tbk[:, :R - 1, :, :D], tbv[:, :R - 1, :, :D])
    deep_k = np.ascontiguousarray(bk[:, R - 1, :, :D])
    deep_v = np.ascontiguousarray(bv[:, R - 1, :, :D])
    assert oc.append(0, [D] * wl.batch, deep_k, deep_v, bk[:, :R - 1, :, :D],
                     bv[:, :R - 1, :, :D]) == oracle.ORA_OK
    torch.cuda.synchronize()
    assert np.array_equal(cache.storage.cpu().numpy(), oc.image), "layout after block append"
    assert cache.lengths(0) == [L + D for L in wl.lens]
    # verify the next block at the new lengths
    wl2 = wl.replace(lens=[L + D for L in wl.lens], capacity=wl.capacity)
    q, bk2, bv2 = H.verify_inputs(wl2, 0)
    out, lse = cache.verify(0, wl2.rows, q, bk2, bv2, D)
    torch.cuda.synchronize()
    ref_o, ref_l = oc.verify(0, wl2.rows, wl2.queries(0), *wl2.block(0), D)
    assert_close(out, lse, ref_o, ref_l, "ragged after append")


def test_wave_reduced():
    wl = named_workload("wave", n_layers=1, lens=[2048], n_heads_q=11, n_heads_kv=11)
    run_case(wl)


# ---------------------------------------------------------------- edge cases

@pytest.mark.parametrize("lens,window,anchor", [
    ([0, 5, 37], 4, 0),          # empty and short sequences
    ([31, 32, 33], 40, 0),       # window longer than the context
    ([64, 3, 100], 7, 1),
    ([90, 90, 1], WINDOW_FULL, 1),
])
def test_edge_lengths(lens, window, anchor):
    wl = Workload("edge", 77, 1, 5, 4, 2, 64, window, 3, lens, 0.88, grid_rows(3, 5),
                  heavy_frac=0.05, max_block=5)
    run_case(wl, window=window, anchor=anchor)


def test_row_subset_any_order_with_repeats():
    wl = Workload("rows", 78, 1, 6, 4, 1, 128, 9, 5, [200, 50], 0.81, grid_rows(5, 6))
    rows = [(4, 2), (0, 6), (4, 2), (2, 1), (3, 6), (1, 3), (0, 1)]
    run_case(wl, rows=rows)


def test_single_loop_model():
    wl = Workload("r1", 79, 1, 1, 2, 2, 96, 8, 4, [70, 129], 0.88, grid_rows(4, 1))
    run_case(wl)


def test_tagged_probe_exact_key_sets():
    """Zero keys and tagged values: O is the mean plane index / position of
    the attended keys, LSE = ln(#keys) (closed form, not the oracle)."""
    R, D, L, W, d = 6, 4, 45, 9, 64
    H = _h()
    from self_speculative_verify_amd import RipeCache
    for anchor in (0, 1):
        cache = RipeCache(1, R, 1, 1, d, W, 1, L + D, D, anchor)
        zero = np.zeros((1, 1, L, d), np.float32)

        def tag(p, r):
            v = np.zeros(d, np.float32)
            v[0], v[1], v[2] = r, p, 1.0
            return v
        dv = np.stack([tag(p, R) for p in range(L)])[None, None]
        wv = np.stack([np.stack([tag(p, r) for p in range(L - W, L)]) for r in range(1, R)])[None, :, None]
        dev = lambda a: H.to_dev(f32_to_bf16(a).reshape(a.shape))
        cache.append(0, [L], dev(zero), dev(dv), dev(np.zeros_like(wv)), dev(wv))
        bv = np.stack([np.stack([tag(L + j, r) for j in range(D)]) for r in range(1, R + 1)])[None, :, None]
        rows = grid_rows(D, R)
        q = dev(np.random.default_rng(5).standard_normal((1, len(rows), 1, d)).astype(np.float32))
        out, lse = cache.verify(0, rows, q, dev(np.zeros_like(bv)), dev(bv), D)
        out, lse = out.cpu().double().numpy(), lse.cpu().double().numpy()
        for k, (i, r) in enumerate(rows):
            t = L + i
            n = t + 1
            beta = t - W if anchor == 0 else L - W
            n_deep = min(max(beta, 0), L) if r < R else L
            assert abs(lse[0, k, 0] - math.log(n)) < 1e-5
            assert abs(out[0, k, 0, 0] - (R * n_deep + r * (n - n_deep)) / n) < 1e-5, (i, r)
            assert abs(out[0, k, 0, 1] - t / 2) < 1e-4, (i, r)
            assert abs(out[0, k, 0, 2] - 1.0) < 1e-6


def test_block_independence_on_gpu():
    """Query anchor with W >= D - 1: one D-row call equals two calls with the
    first part of the block appended in between."""
    H = _h()
    wl = Workload("bi", 80, 1, 4, 4, 2, 64, 5, 6, [300, 41], 0.88, grid_rows(6, 4))
    cache = H.make_cache(wl)
    H.load_prefix(cache, wl)
    q, bk, bv = H.verify_inputs(wl, 0)
    full_o, full_l = cache.verify(0, wl.rows, q, bk, bv, 6)
    k = 3
    first = [(i, r) for (i, r) in wl.rows if i < k]
    idx1 = [wl.rows.index(x) for x in first]
    o1, l1 = cache.verify(0, first, q[:, idx1].contiguous(), bk, bv, 6)
    R = wl.n_loops
    cache.append(0, [k, k], bk[:, R - 1, :, :k], bv[:, R - 1, :, :k], bk[:, :R - 1, :, :k],
                 bv[:, :R - 1, :, :k])
    second = [(i - k, r) for (i, r) in wl.rows if i >= k]
    idx2 = [wl.rows.index((i + k, r)) for (i, r) in second]
    bk2 = torch.zeros_like(bk)
    bv2 = torch.zeros_like(bv)
    bk2[:, :, :, :6 - k] = bk[:, :, :, k:6]
    bv2[:, :, :, :6 - k] = bv[:, :, :, k:6]
    o2, l2 = cache.verify(0, second, q[:, idx2].contiguous(), bk2, bv2, 6 - k)
    torch.cuda.synchronize()
    so = torch.zeros_like(full_o)
    sl = torch.zeros_like(full_l)
    so[:, idx1], sl[:, idx1] = o1, l1
    so[:, idx2], sl[:, idx2] = o2, l2
    assert float((so - full_o).abs().max()) < 1e-5
    assert float((sl - full_l).abs().max()) < 1e-5


@pytest.mark.parametrize("d", [64, 96, 128])
def test_peaked_softmax_large_values(d):
    """Two deep-plane keys per KV head take nearly all of every row-head's
    softmax weight (scores ~8 sqrt(d) above the others and ~0.4 apart) and
    carry values of magnitude ~40 of opposite sign.  Their weights are not
    bf16 numbers: P.V with P rounded to bf16 alone would miss O by far more
    than the tolerance (checked below on the CPU, from the exact weights),
    while the hi/lo split of P stays within it (its own rounding, ~2^-18 of
    a weight, times value components up to ~150, leaves a few 1e-4).  Runs
    through every launch choice of the fixtures (the rows kernel's fast phase
    included)."""
    from synth import bf16_to_f32
    H = _h()
    R, HQ, HKV, W, D, L = 4, 4, 2, 8, 4, 600
    rows = grid_rows(D, R)
    wl = Workload(f"peak{d}", 81, 1, R, HQ, HKV, d, W, D, [L], 0.88, rows)
    rng = np.random.default_rng(81 + d)
    K = 0.05 * rng.standard_normal((HKV, L, d))
    V = rng.standard_normal((HKV, L, d))
    u = rng.standard_normal((HKV, d))
    pairs = [(100 + 7 * g, 350 + 11 * g) for g in range(HKV)]       # both below L - W
    for g, (a, b) in enumerate(pairs):
        K[g, a] = u[g]
        K[g, b] = u[g] + 0.05 * rng.standard_normal(d)
        V[g, a] = 40.0 * rng.standard_normal(d)
        V[g, b] = -V[g, a] + rng.standard_normal(d)
    kb, vb = f32_to_bf16(K.astype(np.float32)), f32_to_bf16(V.astype(np.float32))
    dk, dv = kb[None], vb[None]                                     # [1][Hkv][L][d]
    wk = np.repeat(kb[None, None, :, L - W:], R - 1, axis=1)        # [1][R-1][Hkv][W][d]
    wv = np.repeat(vb[None, None, :, L - W:], R - 1, axis=1)
    grp = [h * HKV // HQ for h in range(HQ)]
    q = f32_to_bf16(np.broadcast_to((8.0 * u[grp])[None, None], (1, len(rows), HQ, d)).astype(np.float32))
    bk = f32_to_bf16((0.05 * rng.standard_normal((1, R, HKV, D, d))).astype(np.float32))
    bv = f32_to_bf16(rng.standard_normal((1, R, HKV, D, d)).astype(np.float32))

    # the premise, from the exact weights of the dominant pair (row 0, head 0)
    # against the reference the kernels take there (key a's score: the tile
    # that holds it moves the reference, key b's score is within the margin)
    qf = bf16_to_f32(q[0, 0, 0]).astype(np.float64)
    a, b = pairs[0]
    s = np.array([bf16_to_f32(kb[0, a]) @ qf, bf16_to_f32(kb[0, b]) @ qf]) / np.sqrt(d)
    p = np.exp(s - s[0])
    p_bf = bf16_to_f32(f32_to_bf16(p.astype(np.float32))).astype(np.float64)
    va, vb_ = bf16_to_f32(vb[0, a]).astype(np.float64), bf16_to_f32(vb[0, b]).astype(np.float64)
    exact = (p[0] * va + p[1] * vb_) / p.sum()
    rounded = (p_bf[0] * va + p_bf[1] * vb_) / p.sum()
    assert np.max(np.abs(rounded - exact)) > 10 * TOL_O, "the inputs do not stress the weights' precision"

    cache = H.make_cache(wl)
    cache.append(0, [L], H.to_dev(dk), H.to_dev(dv), H.to_dev(wk), H.to_dev(wv))
    oc = oracle.OracleCache(oracle.config_of(wl))
    assert oc.append(0, [L], dk, dv, wk, wv) == oracle.ORA_OK
    torch.cuda.synchronize()
    assert np.array_equal(cache.storage.cpu().numpy(), oc.image), "layout differs from the oracle"
    out, lse = cache.verify(0, rows, H.to_dev(q), H.to_dev(bk), H.to_dev(bv), D)
    torch.cuda.synchronize()
    ref_o, ref_l = oc.verify(0, rows, q, bk, bv, D)
    assert float(np.max(np.abs(ref_o))) > 1.0                       # the pair dominates O
    assert_close(out, lse, ref_o, ref_l, f"peaked d={d}")


@pytest.mark.parametrize("d", [64, 96, 128])
def test_rising_scores_rescale_every_tile(d):
    """Committed keys whose scores rise by ~10 (log2 units) from one 32-key
    tile to the next: every tile passes the exponent reference by more than
    its margin, so the rescale of l and O (otherwise about once per row-head)
    runs on every tile of every launch choice.  Deepest plane only (W = 0);
    the last few committed keys dominate the softmax."""
    from synth import bf16_to_f32
    H = _h()
    R, HQ, HKV, W, D, L = 4, 4, 2, 0, 4, 500
    rows = grid_rows(D, R)
    wl = Workload(f"rise{d}", 82, 1, R, HQ, HKV, d, W, D, [L], 0.88, rows)
    rng = np.random.default_rng(82 + d)
    u = rng.standard_normal((HKV, d))
    step = 10.0 / 32 / (np.log2(np.e) / np.sqrt(d)) / d             # score rise per position / |u|^2
    t = step * np.arange(L)
    K = t[None, :, None] * u[:, None, :] + 0.05 * rng.standard_normal((HKV, L, d))
    V = rng.standard_normal((HKV, L, d))
    kb, vb = f32_to_bf16(K.astype(np.float32)), f32_to_bf16(V.astype(np.float32))
    dk, dv = kb[None], vb[None]
    wk = np.zeros((1, R - 1, HKV, 1, d), np.uint16)                 # no ring (W = 0)
    grp = [h * HKV // HQ for h in range(HQ)]
    q = f32_to_bf16(np.broadcast_to(u[grp][None, None], (1, len(rows), HQ, d)).astype(np.float32))
    bk = f32_to_bf16((0.05 * rng.standard_normal((1, R, HKV, D, d))).astype(np.float32))
    bv = f32_to_bf16(rng.standard_normal((1, R, HKV, D, d)).astype(np.float32))
    # the premise: consecutive tiles' maxima (log2 units) differ by more than 8
    qf = bf16_to_f32(q[0, 0, 0]).astype(np.float64)
    x = (bf16_to_f32(kb[0]).astype(np.float64) @ qf) * np.log2(np.e) / np.sqrt(d)
    tile_max = x[: L // 32 * 32].reshape(-1, 32).max(axis=1)
    assert np.all(np.diff(tile_max) > 8.0)

    cache = H.make_cache(wl)
    cache.append(0, [L], H.to_dev(dk), H.to_dev(dv), None, None)
    oc = oracle.OracleCache(oracle.config_of(wl))
    assert oc.append(0, [L], dk, dv, wk, wk) == oracle.ORA_OK
    torch.cuda.synchronize()
    assert np.array_equal(cache.storage.cpu().numpy(), oc.image), "layout differs from the oracle"
    out, lse = cache.verify(0, rows, H.to_dev(q), H.to_dev(bk), H.to_dev(bv), D)
    torch.cuda.synchronize()
    ref_o, ref_l = oc.verify(0, rows, q, bk, bv, D)
    assert_close(out, lse, ref_o, ref_l, f"rising d={d}")


@pytest.mark.parametrize("heads", [(6, 2), (5, 1), (16, 2), (32, 2)])
@pytest.mark.parametrize("d", [64, 128])
def test_group_sizes(heads, d):
    """Query heads per KV head of 3 and 5 (a 16-row-head tile then ends inside
    a row's group of heads), 8 and 16 (12 rows already give 96 and 192
    row-heads per KV head), at two head sizes and every launch choice."""
    hq, hkv = heads
    wl = Workload(f"g{hq}x{hkv}", 83 + hq, 1, 3, hq, hkv, d, 8, 4, [170, 33], 0.88, grid_rows(4, 3),
                  heavy_frac=0.02)
    run_case(wl)


@pytest.mark.parametrize("d", [96, 128])
def test_layers_with_different_lengths(d):
    """Three layers: the prefix on every layer, then accepted tokens on the
    middle layer only (evicting window positions there), so the layers'
    lengths differ.  Storage bit-exact against the oracle; every layer's call
    against the oracle's (each layer has its own data, lengths and sections)."""
    H = _h()
    wl = Workload(f"layers{d}", 84, 3, 4, 4, 2, d, 8, 4, [150, 40], 0.88, grid_rows(4, 4),
                  heavy_frac=0.02, capacity=200)
    cache = H.make_cache(wl)
    H.load_prefix(cache, wl)
    oc = oracle.prefix_cache(wl)
    n_new = [6, 3]
    arrs = step_arrays(wl, 1, wl.lens, n_new)
    cache.append(1, n_new, *[H.to_dev(a) for a in arrs])
    assert oc.append(1, n_new, *arrs) == oracle.ORA_OK
    torch.cuda.synchronize()
    assert [cache.lengths(k) for k in range(3)] == [[150, 40], [156, 43], [150, 40]]
    assert np.array_equal(cache.storage.cpu().numpy(), oc.image), "layout differs from the oracle"
    for layer in range(3):
        q, bk, bv = H.verify_inputs(wl, layer)
        out, lse = cache.verify(layer, wl.rows, q, bk, bv, wl.n_blk)
        torch.cuda.synchronize()
        ref_o, ref_l = oc.verify(layer, wl.rows, wl.queries(layer), *wl.block(layer), wl.n_blk)
        assert_close(out, lse, ref_o, ref_l, f"layers d={d} layer={layer}")
