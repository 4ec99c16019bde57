"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

Holds only input construction (random draws, quantisation into the cache
formats, placement into the block-packed pool); none of the method's
arithmetic.
"""
from . import formats, workloads  # noqa: F401
