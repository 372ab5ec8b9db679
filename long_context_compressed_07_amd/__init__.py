"""MI355X-native CSA/HCA hybrid compressed attention.

The compute path is the C-ABI library `libcsa.so` (HIP kernels for gfx950) under `csrc/`; `lib`
is its thin ctypes binding. `configs` and `inputs` describe and draw the synthetic workloads.
Nothing is loaded at import time: `lib.load()` opens the shared library on first use and raises if
it is missing.
"""
__all__ = ["configs", "inputs", "lib"]
