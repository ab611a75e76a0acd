"""MI355X-native exact attention (FlashAttention forward and backward) for gfx950.

The compute path is the HIP library ``libfa.so`` built from ``csrc/``;
``fwd``, ``fwd_fp8`` and ``bwd`` are thin ctypes bindings over its C ABI (``include/fa.h``)
that only marshal arguments. Importing this package loads nothing: the library is
opened on the first call, and that call raises if the library is missing.
"""
from .binding import FaError, bwd, fwd, fwd_fp8, library_path, load_library  # noqa: F401

__all__ = ["fwd", "fwd_fp8", "bwd", "FaError", "load_library", "library_path"]
