"""MI355X-native MoE expert layer: HIP kernels behind a C ABI (libmoe.so).

``ops`` holds the Python binding (one function per C entry point, plus a
preallocated ``MoELayer``); ``accounting`` the algorithmic FLOP/byte counts.
"""
from . import accounting  # noqa: F401
