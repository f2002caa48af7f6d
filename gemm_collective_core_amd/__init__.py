"""MI355X (gfx950) compute core of the MC2 fused compute/communication operators.

The HIP library ``libmc2.so`` (built from ``csrc/`` by ``build.py``) does all
the work; :mod:`gemm_collective_core_amd.mc2` is a thin ctypes binding over its
C ABI (``include/mc2.h``) that takes torch tensors for device memory and the
current HIP stream. Importing this package loads nothing; the library is
loaded on first use and its absence is an error, never a fallback.
"""
__all__ = ["mc2"]
