"""MI355X-native Q4_0 x Q8_1 mixture-of-experts expert matmul.

The computation lives in libftq.so (HIP kernels for gfx950 behind the C ABI in
include/ftq.h); ``ftq`` is its Python binding and ``inputs`` the seeded
synthetic input generator.  Importing the package loads nothing: the library
is opened on first use, and a missing library raises instead of falling back.
"""
__all__ = ["ftq", "inputs", "build"]
