"""MI355X-native Float8 training linear layer.

The compute path is a HIP library (``csrc/``) behind a C ABI declared in
``include/fp8_linear.h``; ``ops`` is a thin ctypes binding with the same
entry-point names.  Importing the package loads nothing: the binding loads
the shared library on first use and raises if it is missing.
"""
__all__ = ["ops", "workloads"]
