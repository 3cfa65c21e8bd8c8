"""MI355X-native mHC (Manifold-Constrained Hyper-Connections) layer operator.

The operator lives in a HIP shared library (``libmhc.so``, C ABI declared in
``include/mhc.h``); ``manifold_constrained_residuals_amd.mhc`` is its thin ctypes
binding.  Importing this package does not load the library, so the seeded input
generators (``.inputs``) stay usable on machines without a GPU.
"""
__all__ = ["inputs", "mhc"]
