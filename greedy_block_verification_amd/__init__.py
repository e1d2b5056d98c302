"""Greedy block verification on MI355X: a C-ABI HIP library (libsv.so) and its binding.

The compute path lives entirely in ``csrc/`` (HIP kernels for gfx950 behind the
``sv_*`` C ABI declared in ``include/sv.h``).  ``binding`` marshals arguments
through ctypes; PyTorch only provides device memory and the stream.  Importing
this package does not load the library; ``binding.lib()`` does, and raises if it
is missing.
"""
