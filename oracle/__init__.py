"""Test infrastructure: a plain fp64 CPU oracle for deferred-RoPE paged attention.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package.  The library under test never calls it, and it
imports nothing from the library.
"""
from .lazyattn_oracle import *  # noqa: F401,F403
