"""CPU oracle for RIPE verification attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never calls it.

Contents
  * ``ripe_oracle.c`` -- the fp64 layout writer and masked attention (plain C,
    OpenMP over output rows), loaded here through ctypes;
  * ``brute.py``      -- an independent pure-Python simulation of the RIPE
    cache as a dictionary of (position, plane) entries, for tiny inputs;
  * ``memory.py``     -- closed forms of the cache's memory footprint.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
brute force, closed forms, special cases that reduce to ordinary attention,
and the 11.9% memory figure the RIPE abstract prints.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ripe_oracle.c")
# RIPE_ORACLE_LIB: load another build of ripe_oracle.c instead (the test
# suite's sanitizer run points it at an instrumented build)
_LIB_PATH = os.environ.get("RIPE_ORACLE_LIB") or os.path.join(_HERE, "libripe_oracle.so")
_lib = None

ORA_OK, ORA_EINVAL, ORA_ECAPACITY, ORA_EMISSING = 0, 1, 2, 4


def build(force: bool = True, out: Optional[str] = None, extra_flags: Sequence[str] = ()) -> str:
    """Compile the C oracle (gcc, -O2, OpenMP), in place unless ``out`` names
    another file (extra_flags: e.g. sanitizers)."""
    path = out or _LIB_PATH
    stale = not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC)
    if force or stale:
        tmp = f"{path}.{os.getpid()}.tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                               *extra_flags, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, path)
    return path


class OraConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "n_loops", "n_heads_q", "n_heads_kv", "head_dim",
        "window", "batch", "capacity", "max_block", "anchor")]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        L.ora_storage_bytes.restype = ctypes.c_int64
        L.ora_storage_bytes.argtypes = [ctypes.POINTER(OraConfig)]
        L.ora_layout_value.restype = ctypes.c_int64
        L.ora_layout_value.argtypes = [ctypes.POINTER(OraConfig), ctypes.c_int32]
        L.ora_append.restype = ctypes.c_int32
        L.ora_append.argtypes = [ctypes.POINTER(OraConfig), P, ctypes.c_int32, P, P, P, P, P, P, P]
        L.ora_verify.restype = ctypes.c_int32
        L.ora_verify.argtypes = [ctypes.POINTER(OraConfig), P, ctypes.c_int32, ctypes.c_int32,
                                 P, P, P, P, P, P, ctypes.c_int32, P, P, P]
        L.ora_draft.restype = ctypes.c_int32
        L.ora_draft.argtypes = [ctypes.POINTER(OraConfig), P, ctypes.c_int32, ctypes.c_int32,
                                P, P, P, P, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                P, P, P]
        L.ora_threads.restype = ctypes.c_int32
        L.ora_set_threads.restype = None
        L.ora_set_threads.argtypes = [ctypes.c_int32]
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def config(n_layers, n_loops, n_heads_q, n_heads_kv, head_dim, window, batch,
           capacity, max_block, anchor=0) -> OraConfig:
    return OraConfig(n_layers, n_loops, n_heads_q, n_heads_kv, head_dim,
                     window, batch, capacity, max_block, anchor)


def config_of(wl, anchor: Optional[int] = None, window: Optional[int] = None) -> OraConfig:
    """Oracle configuration of a ``synth.Workload``."""
    return config(wl.n_layers, wl.n_loops, wl.n_heads_q, wl.n_heads_kv, wl.head_dim,
                  wl.window if window is None else window, wl.batch, wl.capacity,
                  wl.max_block, wl.anchor if anchor is None else anchor)


def layout_value(cfg: OraConfig, which: str) -> int:
    names = ["lens", "deep_k", "deep_v", "ring_k", "ring_v", "total", "cp", "wr", "wp"]
    return int(lib().ora_layout_value(ctypes.byref(cfg), names.index(which)))


def threads() -> int:
    return int(lib().ora_threads())


def set_threads(n: int) -> None:
    """Threads the oracle uses from now on (OpenMP)."""
    lib().ora_set_threads(int(n))


class OracleCache:
    """A host image of the RIPE storage, written and read by the C oracle."""

    def __init__(self, cfg: OraConfig):
        self.cfg = cfg
        n = lib().ora_storage_bytes(ctypes.byref(cfg))
        if n < 0:
            raise ValueError("invalid oracle configuration")
        self.image = np.zeros(int(n), dtype=np.uint8)

    def lens(self, layer: int) -> np.ndarray:
        off = layout_value(self.cfg, "lens")
        B = self.cfg.batch
        return self.image[off:off + 4 * self.cfg.n_layers * B].view(np.int32).reshape(
            self.cfg.n_layers, B)[layer].copy()

    def append(self, layer: int, n_new: Sequence[int], deep_k: np.ndarray, deep_v: np.ndarray,
               win_k: np.ndarray, win_v: np.ndarray) -> int:
        """Append tokens to every sequence of one layer.

        deep_k/deep_v: uint16 [B][Hkv][T][d] (plane R of token t < n_new[b]);
        win_k/win_v:   uint16 [B][R-1][Hkv][U][d] (planes 1..R-1 of the last
        min(n_new[b], ring slots) tokens, oldest first).
        """
        nn = np.ascontiguousarray(n_new, dtype=np.int32)
        dk = np.ascontiguousarray(deep_k, dtype=np.uint16)
        dv = np.ascontiguousarray(deep_v, dtype=np.uint16)
        wk = np.ascontiguousarray(win_k, dtype=np.uint16)
        wv = np.ascontiguousarray(win_v, dtype=np.uint16)
        ds = np.array([dk.shape[1] * dk.shape[2] * dk.shape[3], dk.shape[2] * dk.shape[3],
                       dk.shape[3]], dtype=np.int64)
        ws = np.array([wk.shape[1] * wk.shape[2] * wk.shape[3] * wk.shape[4],
                       wk.shape[2] * wk.shape[3] * wk.shape[4], wk.shape[3] * wk.shape[4],
                       wk.shape[4]], dtype=np.int64)
        return int(lib().ora_append(ctypes.byref(self.cfg), _ptr(self.image), layer, _ptr(nn),
                                    _ptr(dk), _ptr(dv), _ptr(ds), _ptr(wk), _ptr(wv), _ptr(ws)))

    def verify(self, layer: int, rows: Sequence[Tuple[int, int]], q: np.ndarray,
               blk_k: np.ndarray, blk_v: np.ndarray, n_blk: int,
               want: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
        """fp64 verification attention.

        q: uint16 [B][n_rows][Hq][d]; blk_k/blk_v: uint16 [B][R][Hkv][Dmax][d].
        Returns (out [B][n_rows][Hq][d], lse [B][n_rows][Hq]) as float64.
        """
        return self._attend(layer, rows, q, blk_k, blk_v, n_blk, None, want)

    def draft(self, layer: int, rows: Sequence[Tuple[int, int]], q: np.ndarray,
              blk_k: np.ndarray, blk_v: np.ndarray, n_blk: int, n_sink: int, w_draft: int,
              want: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
        """fp64 windowed draft attention: committed keys are the first n_sink
        positions and the w_draft positions before the query."""
        return self._attend(layer, rows, q, blk_k, blk_v, n_blk, (n_sink, w_draft), want)

    def _attend(self, layer, rows, q, blk_k, blk_v, n_blk, window, want):
        c = self.cfg
        rb = np.ascontiguousarray([i for i, _ in rows], dtype=np.int32)
        rl = np.ascontiguousarray([r for _, r in rows], dtype=np.int32)
        q = np.ascontiguousarray(q, dtype=np.uint16)
        bk = np.ascontiguousarray(blk_k, dtype=np.uint16)
        bv = np.ascontiguousarray(blk_v, dtype=np.uint16)
        bs = np.array([bk.shape[1] * bk.shape[2] * bk.shape[3] * bk.shape[4],
                       bk.shape[2] * bk.shape[3] * bk.shape[4], bk.shape[3] * bk.shape[4],
                       bk.shape[4]], dtype=np.int64)
        nr = len(rows)
        out = np.zeros((c.batch, nr, c.n_heads_q, c.head_dim), dtype=np.float64)
        lse = np.zeros((c.batch, nr, c.n_heads_q), dtype=np.float64)
        w = None if want is None else np.ascontiguousarray(want, dtype=np.uint8)
        if window is None:
            st = lib().ora_verify(ctypes.byref(c), _ptr(self.image), layer, nr, _ptr(rb), _ptr(rl),
                                  _ptr(q), _ptr(bk), _ptr(bv), _ptr(bs), n_blk, _ptr(w),
                                  _ptr(out), _ptr(lse))
        else:
            st = lib().ora_draft(ctypes.byref(c), _ptr(self.image), layer, nr, _ptr(rb), _ptr(rl),
                                 _ptr(q), _ptr(bk), _ptr(bv), _ptr(bs), n_blk, int(window[0]),
                                 int(window[1]), _ptr(w), _ptr(out), _ptr(lse))
        if st != ORA_OK:
            raise RuntimeError(f"oracle attention failed with status {st}")
        return out, lse


def prefix_cache(wl, layers: Optional[Sequence[int]] = None, anchor: Optional[int] = None,
                 window: Optional[int] = None) -> OracleCache:
    """An oracle cache holding the committed prefix of every sequence of ``wl``
    (one append of all L_b tokens per layer)."""
    cfg = config_of(wl, anchor=anchor, window=window)
    oc = OracleCache(cfg)
    R, H, d, B = wl.n_loops, wl.n_heads_kv, wl.head_dim, wl.batch
    wr = layout_value(cfg, "wr")
    for layer in (range(wl.n_layers) if layers is None else layers):
        T = max(wl.lens)
        U = min(T, wr) if R > 1 else 0
        dk = np.zeros((B, H, T, d), np.uint16)
        dv = np.zeros_like(dk)
        wk = np.zeros((B, max(R - 1, 0), H, max(U, 0), d), np.uint16)
        wv = np.zeros_like(wk)
        for b in range(B):
            L = wl.lens[b]
            nw = min(L, wr) if R > 1 else 0
            a, bb, c_, e = wl.prefix(layer, b, n_win=nw)
            dk[b, :, :L] = a
            dv[b, :, :L] = bb
            if nw:
                wk[b, :, :, :nw] = c_
                wv[b, :, :, :nw] = e
        st = oc.append(layer, wl.lens, dk, dv, wk, wv)
        if st != ORA_OK:
            raise RuntimeError(f"oracle append failed with status {st}")
    return oc
