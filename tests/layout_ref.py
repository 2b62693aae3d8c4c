"""Reader of the RIPE storage byte layout, written separately from both the C
oracle's writer and the HIP library, for the layout pins.

Layout (sections 256-byte aligned, in order):
  lens   int32 [NL][B]
  deep_k bf16  [NL][B][Hkv][CP*d]      CP = ceil(capacity / 32) * 32
  deep_v bf16  [NL][B][Hkv][CP*d]
  ring_k bf16  [NL][B][Hkv][R-1][WP*d] WR = min(W, capacity) (0 if R == 1), WP = ceil(WR/32)*32
  ring_v bf16  [NL][B][Hkv][R-1][WP*d]
Row p of a region (position, or ring slot p mod WR) splits into 32-row tiles of
32*d elements. Keys: [d/32 column blocks][32 rows][32 columns]; values:
[d columns][32 rows], with row k stored at column slot(k) where
slot(k) = 8*((k%16)//4) + 4*(k//16) + k%4.
"""
import numpy as np


def _ceil(x, a):
    return -(-x // a) * a


def sections(NL, R, Hkv, d, W, B, cap):
    CP = _ceil(cap, 32)
    WR = 0 if R == 1 else min(W, cap)
    WP = _ceil(WR, 32)
    sizes = [NL * B * 4, NL * B * Hkv * CP * d * 2, NL * B * Hkv * CP * d * 2,
             NL * B * Hkv * (R - 1) * WP * d * 2, NL * B * Hkv * (R - 1) * WP * d * 2]
    offs, o = [], 0
    for s in sizes:
        offs.append(o)
        o = _ceil(o + s, 256)
    return dict(lens=offs[0], deep_k=offs[1], deep_v=offs[2], ring_k=offs[3], ring_v=offs[4],
                total=o, CP=CP, WR=WR, WP=WP)


def _slot(k):
    return 8 * ((k % 16) // 4) + 4 * (k // 16) + k % 4


def key_elems(row, d):
    """Element offsets of row `row` (all d dims) of a key region."""
    e = np.arange(d)
    return (row // 32) * 32 * d + (e // 32) * 1024 + (row % 32) * 32 + e % 32


def value_elems(row, d):
    e = np.arange(d)
    return (row // 32) * 32 * d + e * 32 + _slot(row % 32)


class Image:
    def __init__(self, raw: np.ndarray, NL, R, Hkv, d, W, B, cap):
        self.raw = raw.view(np.uint8)
        self.NL, self.R, self.H, self.d, self.W, self.B, self.cap = NL, R, Hkv, d, W, B, cap
        self.s = sections(NL, R, Hkv, d, W, B, cap)
        assert self.raw.size == self.s["total"], (self.raw.size, self.s["total"])

    def _u16(self, name):
        o = self.s[name]
        return self.raw[o:].view(np.uint16) if (o % 2 == 0) else None

    def lens(self):
        o = self.s["lens"]
        return self.raw[o:o + 4 * self.NL * self.B].view(np.int32).reshape(self.NL, self.B)

    def deep(self, layer, b, g, p):
        """(key, value) uint16 vectors of position p, plane R."""
        d = self.d
        base = ((layer * self.B + b) * self.H + g) * self.s["CP"] * d
        k = self._u16("deep_k")[base + key_elems(p, d)]
        v = self._u16("deep_v")[base + value_elems(p, d)]
        return k, v

    def ring(self, layer, b, g, r, p):
        """(key, value) of plane r < R for the position p (slot p mod WR)."""
        d, WR, WP = self.d, self.s["WR"], self.s["WP"]
        slot = p % WR
        base = (((layer * self.B + b) * self.H + g) * (self.R - 1) + (r - 1)) * WP * d
        k = self._u16("ring_k")[base + key_elems(slot, d)]
        v = self._u16("ring_v")[base + value_elems(slot, d)]
        return k, v

    def written_mask(self, entries):
        """Byte mask of every location the given (layer, b, g, p, plane) entries
        occupy, plus the lens section."""
        m = np.zeros(self.raw.size, dtype=bool)
        o = self.s["lens"]
        m[o:o + 4 * self.NL * self.B] = True
        d, WR, WP, CP = self.d, self.s["WR"], self.s["WP"], self.s["CP"]
        for (layer, b, g, p, plane) in entries:
            if plane == self.R:
                base = ((layer * self.B + b) * self.H + g) * CP * d
                ke, ve = key_elems(p, d), value_elems(p, d)
                ks, vs = self.s["deep_k"], self.s["deep_v"]
            else:
                base = (((layer * self.B + b) * self.H + g) * (self.R - 1) + plane - 1) * WP * d
                ke, ve = key_elems(p % WR, d), value_elems(p % WR, d)
                ks, vs = self.s["ring_k"], self.s["ring_v"]
            for sec, el in ((ks, ke), (vs, ve)):
                byte = sec + 2 * (base + el)
                m[byte] = True
                m[byte + 1] = True
        return m
