"""MI355X-native block-quantized decode GEMV (Q8G64 / Q4G32).

The compute path is the HIP library ``libqgemv.so`` built from ``csrc/`` for
gfx950; ``qgemv`` holds the thin ctypes binding with the same names as the
C ABI in ``include/qgemv.h``.  ``synth`` holds the seeded input generators.
"""
from . import synth  # noqa: F401

__all__ = ["synth"]
