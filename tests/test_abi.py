"""C-ABI contract checks that need no GPU: the library loads, exports every
symbol the header declares, sizes its storage exactly as the layout reader
does, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

from self_speculative_verify_amd import ripe
from layout_ref import sections

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "ripe.h")).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\*]+\s+)+\**(ripe_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = ripe.load()
    syms = declared_symbols()
    assert len(syms) >= 9, syms
    for s in syms:
        assert hasattr(lib, s), f"{s} is declared in include/ripe.h but not exported"


@pytest.mark.parametrize("cfg", [
    (1, 8, 2, 2, 64, 16, 1, 132, 4, 0),
    (4, 32, 55, 55, 96, 64, 1, 1032, 8, 0),
    (4, 32, 32, 8, 128, 0, 4, 4104, 8, 1),
    (4, 32, 32, 8, 128, ripe.RIPE_WINDOW_FULL, 4, 4104, 8, 0),
    (2, 1, 4, 2, 64, 10, 3, 77, 3, 0),
    (3, 5, 6, 3, 96, 1000, 2, 100, 16, 1),
])
def test_storage_size_and_sections_match_layout(cfg):
    c = ripe.config(*cfg)
    NL, R, Hq, Hkv, d, W, B, cap, Dmax, anchor = cfg
    s = sections(NL, R, Hkv, d, W, B, cap)
    assert ripe.ripe_cache_bytes(c) == s["total"]
    names = ["lens", "deep_k", "deep_v", "ring_k", "ring_v", "total"]
    for i, n in enumerate(names):
        assert ripe.ripe_section_offset(c, i) == s[n]


@pytest.mark.parametrize("bad", [
    dict(n_layers=0), dict(n_loops=0), dict(n_loops=256), dict(n_heads_q=3),
    dict(head_dim=80), dict(window=-1), dict(batch=0), dict(capacity=0),
    dict(max_block=0), dict(max_block=257), dict(anchor=2),
])
def test_invalid_configs_rejected_without_device(bad):
    base = dict(n_layers=1, n_loops=4, n_heads_q=4, n_heads_kv=2, head_dim=64, window=8,
                batch=2, capacity=64, max_block=4, anchor=0)
    base.update(bad)
    c = ripe.RipeConfig(**base)
    assert ripe.ripe_cache_bytes(c) == 0
    assert ripe.ripe_section_offset(c, 0) == -1
    h = ctypes.c_void_p()
    st = ripe.load().ripe_cache_create(ctypes.byref(c), ctypes.c_void_p(1 << 20), 1 << 30,
                                       None, ctypes.byref(h))
    assert st == ripe.RIPE_EINVAL and not h.value


def test_null_handles_and_pointers_rejected():
    L = ripe.load()
    v = ripe.null_view()
    n = (ctypes.c_int32 * 1)(1)
    assert L.ripe_append(None, 0, n, v, v, v, v, None) == ripe.RIPE_EINVAL
    assert L.ripe_verify_attn(None, 0, 1, n, n, None, v, v, 1, None, None, None, 0, None) == ripe.RIPE_EINVAL
    assert L.ripe_workspace_bytes(None, 4) == 0
    assert L.ripe_draft_attn(None, 0, 1, n, n, None, v, v, 1, 0, 4, None, None, None) == ripe.RIPE_EINVAL
    L.ripe_destroy(None)
    c = ripe.config(1, 4, 2, 2, 64, 8, 1, 64, 4)
    h = ctypes.c_void_p()
    # misaligned storage and undersized storage are refused before any HIP call
    assert L.ripe_cache_create(ctypes.byref(c), ctypes.c_void_p(4096 + 16), 1 << 30, None,
                               ctypes.byref(h)) == ripe.RIPE_EINVAL
    assert L.ripe_cache_create(ctypes.byref(c), ctypes.c_void_p(4096),
                               ripe.ripe_cache_bytes(c) - 1, None, ctypes.byref(h)) == ripe.RIPE_EINVAL


def test_status_strings():
    for s in range(4):
        assert ripe.ripe_status_string(s)
    assert "capacity" in ripe.ripe_status_string(ripe.RIPE_ECAPACITY)


# ---------------------------------------------------------------- binding views

def test_kv_view_strides_by_name():
    """kv_view maps each named dimension to its element stride; letters the
    string leaves out get stride 0; views of two layouts in turn stay apart."""
    import torch
    from self_speculative_verify_amd import ripe
    t5 = torch.zeros(2, 3, 4, 5, 64, dtype=torch.bfloat16)
    v = ripe.kv_view(t5, "bphtd")
    assert (v.s_b, v.s_plane, v.s_head, v.s_tok) == t5.stride()[:4]
    assert v.ptr == t5.data_ptr()
    t4 = torch.zeros(2, 6, 9, 32, dtype=torch.bfloat16)[:, :, 1:8]      # strided token dimension
    w = ripe.kv_view(t4, "bhtd")
    assert (w.s_b, w.s_plane, w.s_head, w.s_tok) == (t4.stride(0), 0, t4.stride(1), t4.stride(2))
    assert w.ptr == t4.data_ptr()
    t3 = torch.zeros(4, 7, 16, dtype=torch.bfloat16)
    x = ripe.kv_view(t3, "ptd")
    assert (x.s_b, x.s_plane, x.s_head, x.s_tok) == (0, t3.stride(0), 0, t3.stride(1))
    v2 = ripe.kv_view(t5, "bphtd")                                      # again, after other strings
    assert (v2.s_b, v2.s_plane, v2.s_head, v2.s_tok) == t5.stride()[:4]


def test_kv_view_rejects_bad_tensors():
    import torch
    from self_speculative_verify_amd import ripe
    with pytest.raises(TypeError):
        ripe.kv_view(torch.zeros(2, 64), "td")                          # not 16-bit
    with pytest.raises(ValueError):
        ripe.kv_view(torch.zeros(64, 2, dtype=torch.bfloat16).t(), "td")  # d not contiguous
    with pytest.raises(ValueError):
        ripe.kv_view(torch.zeros(2, 64, dtype=torch.bfloat16), "htd")   # rank differs
    with pytest.raises(ValueError):
        ripe.kv_view(torch.zeros(2, 64, dtype=torch.bfloat16), "dt")    # does not end in d


def test_stream_handle_passthrough():
    """A raw stream handle given as an integer goes through unchanged."""
    from self_speculative_verify_amd import ripe
    assert ripe._stream(0x1234).value == 0x1234
