"""RIPE verification attention on MI355X (gfx950).

``ripe``  -- the Python binding of the C ABI in include/ripe.h (libripe.so);
``cache`` -- RipeCache, PyTorch-owned storage bound to a library handle.
"""
from . import ripe  # noqa: F401
from .cache import RipeCache  # noqa: F401
