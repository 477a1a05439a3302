"""MI355X-native forward pass of a DeepSeek-V3-style Mixture-of-Experts layer.

The compute path lives in ``libmoe.so`` (hand-written HIP kernels for gfx950
behind a C ABI declared in ``include/moe.h``).  ``moe`` is the ctypes binding;
``inputs`` draws the seeded synthetic inputs.  Importing this package loads
nothing: the shared library is opened on first use by ``moe``.
"""

__all__ = ["inputs", "moe"]
