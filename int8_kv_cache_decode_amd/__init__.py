"""MI355X (gfx950) single-query decode attention over a head-major f32 or
int8 (q8_2f) KV cache, behind the C ABI in include/kvq.h.

`kvq` is the Python binding (ctypes marshalling of libkvq.so); `build`
compiles the HIP library.
"""
from . import kvq  # noqa: F401

__all__ = ["kvq"]
