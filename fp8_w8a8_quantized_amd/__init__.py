"""MI355X-native FP8 W8A8 linear layer (gfx950 HIP kernels behind a C ABI).

The compute path lives in ``libfp8w8a8.so`` (built from ``csrc/``); the
Python layer only marshals torch device tensors and the current HIP stream
into the C calls.  Importing this package does not load the library; the
first call does, and raises if the library is missing.
"""
