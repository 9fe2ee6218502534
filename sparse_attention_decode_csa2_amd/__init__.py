"""MI355X-native CSA2 FP4 sparse-attention decode.

The compute path is the C-ABI library ``libcsa2.so`` (hand-written HIP
kernels for gfx950) declared in ``include/csa2.h``; ``csa2`` is its thin
ctypes binding.  Importing this package loads nothing: ``workloads`` (seeded
inputs) is usable without a GPU, and the binding loads the library on first
use and raises if it is missing.
"""
