"""Python binding of the RIPE C ABI (include/ripe.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libripe.so``.  PyTorch supplies device memory and streams.  The
binding raises if the library has not been built; there is no fallback.
"""
from __future__ import annotations

import array
import ctypes
import os
from typing import Optional, Sequence

import torch

__all__ = [
    "RIPE_OK", "RIPE_EINVAL", "RIPE_ECAPACITY", "RIPE_EDEVICE", "RIPE_ESCRATCH",
    "RIPE_NOALLOC_SCRATCH_BYTES", "ripe_verify_attn_noalloc",
    "RIPE_ANCHOR_QUERY", "RIPE_ANCHOR_CACHE", "RIPE_WINDOW_FULL",
    "RIPE_SECTION_LENS", "RIPE_SECTION_DEEP_K", "RIPE_SECTION_DEEP_V",
    "RIPE_SECTION_RING_K", "RIPE_SECTION_RING_V", "RIPE_SECTION_END",
    "RipeConfig", "RipeKVView", "RipeError", "library_path", "load",
    "ripe_cache_bytes", "ripe_section_offset", "ripe_max_batch", "ripe_cache_create",
    "ripe_cache_open", "ripe_destroy",
    "ripe_get_lengths", "ripe_append", "ripe_workspace_bytes", "ripe_verify_attn",
    "ripe_draft_attn", "RipeTuning", "ripe_set_tuning",
    "ripe_status_string", "kv_view", "null_view", "config",
]

RIPE_OK, RIPE_EINVAL, RIPE_ECAPACITY, RIPE_EDEVICE, RIPE_ESCRATCH = 0, 1, 2, 3, 4
RIPE_NOALLOC_SCRATCH_BYTES = 128 << 20
RIPE_ANCHOR_QUERY, RIPE_ANCHOR_CACHE = 0, 1
RIPE_WINDOW_FULL = 2**31 - 1
(RIPE_SECTION_LENS, RIPE_SECTION_DEEP_K, RIPE_SECTION_DEEP_V, RIPE_SECTION_RING_K,
 RIPE_SECTION_RING_V, RIPE_SECTION_END) = range(6)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def library_path() -> str:
    return os.path.join(_HERE, "libripe.so")


class RipeConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "n_loops", "n_heads_q", "n_heads_kv", "head_dim",
        "window", "batch", "capacity", "max_block", "anchor")]


class RipeKVView(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("s_b", ctypes.c_int64), ("s_plane", ctypes.c_int64),
                ("s_head", ctypes.c_int64), ("s_tok", ctypes.c_int64)]


class RipeTuning(ctypes.Structure):
    """Fixed launch choices of one handle (0 = the planner's choice)."""
    _fields_ = [(n, ctypes.c_int32) for n in (
        "kernel", "keys_waves", "row_tiles", "private_waves", "items_target", "min_chunk")]


class RipeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {ripe_status_string(status)} (status {status})")
        self.status = status


def load():
    """Load libripe.so (raises if it is not built)."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(path)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        CFG = ctypes.POINTER(RipeConfig)
        L.ripe_cache_bytes.restype = SZ
        L.ripe_cache_bytes.argtypes = [CFG]
        L.ripe_section_offset.restype = I64
        L.ripe_section_offset.argtypes = [CFG, I32]
        L.ripe_max_batch.restype = I32
        L.ripe_max_batch.argtypes = [CFG, SZ]
        L.ripe_cache_create.restype = I32
        L.ripe_cache_create.argtypes = [CFG, P, SZ, P, ctypes.POINTER(P)]
        L.ripe_cache_open.restype = I32
        L.ripe_cache_open.argtypes = [CFG, P, SZ, P, ctypes.POINTER(P)]
        L.ripe_destroy.restype = None
        L.ripe_destroy.argtypes = [P]
        L.ripe_get_lengths.restype = I32
        L.ripe_get_lengths.argtypes = [P, I32, P]
        L.ripe_append.restype = I32
        L.ripe_append.argtypes = [P, I32, P, RipeKVView, RipeKVView, RipeKVView, RipeKVView, P]
        L.ripe_workspace_bytes.restype = SZ
        L.ripe_workspace_bytes.argtypes = [P, I32]
        L.ripe_verify_attn.restype = I32
        L.ripe_verify_attn.argtypes = [P, I32, I32, P, P, P, RipeKVView, RipeKVView, I32,
                                       P, P, P, SZ, P]
        L.ripe_verify_attn_noalloc.restype = I32
        L.ripe_verify_attn_noalloc.argtypes = [P, I32, I32, P, P, P, RipeKVView, RipeKVView, I32,
                                               P, P, P]
        L.ripe_draft_attn.restype = I32
        L.ripe_draft_attn.argtypes = [P, I32, I32, P, P, P, RipeKVView, RipeKVView, I32, I32, I32,
                                      P, P, P]
        L.ripe_set_tuning.restype = I32
        L.ripe_set_tuning.argtypes = [P, ctypes.POINTER(RipeTuning)]
        L.ripe_status_string.restype = ctypes.c_char_p
        L.ripe_status_string.argtypes = [I32]
        _LIB = L
    return _LIB


def ripe_status_string(status: int) -> str:
    return load().ripe_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != RIPE_OK:
        raise RipeError(status, what)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        # the current device's current stream, read as a raw handle (no
        # Stream object is built on every call)
        return ctypes.c_void_p(torch._C._cuda_getCurrentRawStream(torch.cuda.current_device()))
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _i32_array(xs: Sequence[int]):
    """Host int32 array of xs (ints, or objects with __index__) for a pointer
    argument; built in C through array.array, which is several times faster
    than element-wise ctypes construction for the 256-row calls."""
    a = array.array("i", xs)
    return (ctypes.c_int32 * len(a)).from_buffer(a)


def config(n_layers, n_loops, n_heads_q, n_heads_kv, head_dim, window, batch, capacity,
           max_block, anchor=RIPE_ANCHOR_QUERY) -> RipeConfig:
    return RipeConfig(n_layers, n_loops, n_heads_q, n_heads_kv, head_dim, window, batch,
                      capacity, max_block, anchor)


_VIEW_TYPES = (torch.bfloat16, torch.int16, torch.uint16)
_VIEW_DIMS = {}      # dims string -> positions of b, p, h, t in it (-1: absent)


def kv_view(t: torch.Tensor, dims: str) -> RipeKVView:
    """A view of a bf16 tensor whose dimensions are named by ``dims``, a string
    over b (sequence), p (plane), h (KV head), t (token) ending in d (head
    dimension, stride 1).  Missing letters get stride 0."""
    if t.dtype not in _VIEW_TYPES:
        raise TypeError(f"expected a bfloat16 tensor, got {t.dtype}")
    st = t.stride()
    if len(st) != len(dims) or not dims.endswith("d") or st[-1] != 1:
        raise ValueError(f"tensor of shape {tuple(t.shape)} does not match '{dims}' with d contiguous")
    pos = _VIEW_DIMS.get(dims)
    if pos is None:
        pos = _VIEW_DIMS[dims] = tuple(dims.find(c) for c in "bpht")
    b, p, h, k = pos
    return RipeKVView(t.data_ptr(), st[b] if b >= 0 else 0, st[p] if p >= 0 else 0,
                      st[h] if h >= 0 else 0, st[k] if k >= 0 else 0)


def null_view() -> RipeKVView:
    return RipeKVView(None, 0, 0, 0, 0)


def ripe_cache_bytes(cfg: RipeConfig) -> int:
    return int(load().ripe_cache_bytes(ctypes.byref(cfg)))


def ripe_section_offset(cfg: RipeConfig, section: int) -> int:
    return int(load().ripe_section_offset(ctypes.byref(cfg), int(section)))


def ripe_max_batch(cfg: RipeConfig, budget_bytes: int) -> int:
    """Largest batch whose storage fits in budget_bytes (0: none; -1: invalid)."""
    return int(load().ripe_max_batch(ctypes.byref(cfg), int(budget_bytes)))


def ripe_cache_create(cfg: RipeConfig, storage: torch.Tensor, stream=None) -> ctypes.c_void_p:
    """Bind a handle to a uint8 device tensor of at least ripe_cache_bytes(cfg)."""
    if not storage.is_cuda or storage.dtype != torch.uint8 or not storage.is_contiguous():
        raise ValueError("storage must be a contiguous uint8 device tensor")
    h = ctypes.c_void_p()
    _check(load().ripe_cache_create(ctypes.byref(cfg), ctypes.c_void_p(storage.data_ptr()),
                                    storage.numel(), _stream(stream), ctypes.byref(h)),
           "ripe_cache_create")
    return h


def ripe_cache_open(cfg: RipeConfig, storage: torch.Tensor, stream=None) -> ctypes.c_void_p:
    """Bind a handle to a uint8 device tensor that already holds a cache image."""
    if not storage.is_cuda or storage.dtype != torch.uint8 or not storage.is_contiguous():
        raise ValueError("storage must be a contiguous uint8 device tensor")
    h = ctypes.c_void_p()
    _check(load().ripe_cache_open(ctypes.byref(cfg), ctypes.c_void_p(storage.data_ptr()),
                                  storage.numel(), _stream(stream), ctypes.byref(h)),
           "ripe_cache_open")
    return h


def ripe_destroy(handle) -> None:
    load().ripe_destroy(handle)


def ripe_set_tuning(handle, tuning: Optional[dict] = None) -> None:
    """Fix launch choices of a handle (keys of RipeTuning; None restores the planner)."""
    if tuning is None:
        _check(load().ripe_set_tuning(handle, None), "ripe_set_tuning")
        return
    t = RipeTuning(**tuning)
    _check(load().ripe_set_tuning(handle, ctypes.byref(t)), "ripe_set_tuning")


def ripe_get_lengths(handle, layer: int, batch: int):
    arr = (ctypes.c_int32 * batch)()
    _check(load().ripe_get_lengths(handle, layer, arr), "ripe_get_lengths")
    return list(arr)


def ripe_append(handle, layer: int, n_new: Sequence[int], deep_k: RipeKVView,
                deep_v: RipeKVView, win_k: RipeKVView, win_v: RipeKVView, stream=None) -> None:
    _check(load().ripe_append(handle, layer, _i32_array(n_new), deep_k, deep_v, win_k, win_v,
                              _stream(stream)), "ripe_append")


def ripe_workspace_bytes(handle, n_rows: int) -> int:
    return int(load().ripe_workspace_bytes(handle, n_rows))


def ripe_verify_attn(handle, layer: int, row_blk: Sequence[int], row_loop: Sequence[int],
                     q: torch.Tensor, blk_k: RipeKVView, blk_v: RipeKVView, n_blk: int,
                     out: torch.Tensor, lse: torch.Tensor, ws: Optional[torch.Tensor] = None,
                     stream=None) -> None:
    if len(row_blk) != len(row_loop):
        raise ValueError("row_blk and row_loop differ in length")
    for t, name, dt in ((q, "q", torch.bfloat16), (out, "out", torch.float32),
                        (lse, "lse", torch.float32)):
        if not t.is_cuda or t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} device tensor")
    ws_ptr = ctypes.c_void_p(ws.data_ptr()) if ws is not None else ctypes.c_void_p()
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(load().ripe_verify_attn(handle, layer, len(row_blk), _i32_array(row_blk),
                                   _i32_array(row_loop), ctypes.c_void_p(q.data_ptr()),
                                   blk_k, blk_v, n_blk, ctypes.c_void_p(out.data_ptr()),
                                   ctypes.c_void_p(lse.data_ptr()), ws_ptr, ws_bytes,
                                   _stream(stream)), "ripe_verify_attn")


def ripe_verify_attn_noalloc(handle, layer: int, row_blk: Sequence[int], row_loop: Sequence[int],
                             q: torch.Tensor, blk_k: RipeKVView, blk_v: RipeKVView, n_blk: int,
                             out: torch.Tensor, lse: torch.Tensor, stream=None) -> None:
    """ripe_verify_attn with the library's fixed scratch instead of a workspace."""
    if len(row_blk) != len(row_loop):
        raise ValueError("row_blk and row_loop differ in length")
    for t, name, dt in ((q, "q", torch.bfloat16), (out, "out", torch.float32),
                        (lse, "lse", torch.float32)):
        if not t.is_cuda or t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} device tensor")
    _check(load().ripe_verify_attn_noalloc(handle, layer, len(row_blk), _i32_array(row_blk),
                                           _i32_array(row_loop), ctypes.c_void_p(q.data_ptr()),
                                           blk_k, blk_v, n_blk, ctypes.c_void_p(out.data_ptr()),
                                           ctypes.c_void_p(lse.data_ptr()), _stream(stream)),
           "ripe_verify_attn_noalloc")


def ripe_draft_attn(handle, layer: int, row_blk: Sequence[int], row_loop: Sequence[int],
                    q: torch.Tensor, blk_k: RipeKVView, blk_v: RipeKVView, n_blk: int,
                    n_sink: int, w_draft: int, out: torch.Tensor, lse: torch.Tensor,
                    stream=None) -> None:
    if len(row_blk) != len(row_loop):
        raise ValueError("row_blk and row_loop differ in length")
    for t, name, dt in ((q, "q", torch.bfloat16), (out, "out", torch.float32),
                        (lse, "lse", torch.float32)):
        if not t.is_cuda or t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} device tensor")
    _check(load().ripe_draft_attn(handle, layer, len(row_blk), _i32_array(row_blk),
                                  _i32_array(row_loop), ctypes.c_void_p(q.data_ptr()),
                                  blk_k, blk_v, n_blk, int(n_sink), int(w_draft),
                                  ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
                                  _stream(stream)), "ripe_draft_attn")
