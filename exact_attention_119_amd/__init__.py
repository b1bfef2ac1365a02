"""Fused exact-attention forward pass for AMD MI355X (gfx950).

The computation lives in libattn119.so (hand-written HIP kernels behind the C ABI
of include/attn119.h); `lib` is its ctypes binding (argument marshalling only).
"""

from . import lib  # noqa: F401
