"""MI355X-native deferred-RoPE attention over a position-agnostic paged KV pool.

The compute lives in liblazyattn.so (hand-written HIP kernels for gfx950)
behind the C interface in include/lazyattn.h; ``_abi`` is its ctypes binding
and ``staging`` moves host inputs into the library's device layouts.
"""
from . import _abi  # noqa: F401
from ._abi import LazyAttnError, lib  # noqa: F401

__all__ = ["_abi", "lib", "LazyAttnError"]
