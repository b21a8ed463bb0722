"""Seeded synthetic inputs for paged attention.

This package is shared by the tests, the benchmark and the CPU oracle's
callers.  It draws random numbers, rounds them to storage precisions and lays
them out in a block pool; it holds none of the attention, allocator or cache
arithmetic.  Neither the HIP library nor the oracle is imported here.
"""
from .workloads import *  # noqa: F401,F403
