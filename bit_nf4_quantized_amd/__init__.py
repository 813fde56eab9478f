"""MI355X (gfx950) library for the QLoRA NF4 hot path.

The compute lives in a C-ABI shared library of hand-written HIP kernels
(``libqlora_nf4.so``, built from ``csrc/``); ``api`` is a thin ctypes
binding that passes torch device pointers and the current HIP stream.
Importing this package does not load the library; the first call does, and
it raises if the library is missing.
"""

__all__ = ["api", "workloads"]
