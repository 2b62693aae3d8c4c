"""Seeded synthetic inputs for RIPE verification workloads.

This package is shared by the HIP path (tests, bench) and by the CPU oracle.
It only draws random numbers and rounds them to bfloat16; it holds none of the
cache-layout or attention arithmetic.
"""
from .gen import *  # noqa: F401,F403
