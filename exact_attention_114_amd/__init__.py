"""MI355X-native exact attention (FlashAttention forward) for gfx950.

The compute path is the HIP library ``libfa_fwd.so`` built from ``csrc/``;
``fwd`` is a thin ctypes binding over its C ABI (``include/fa.h``) that only
marshals arguments. Importing this package loads nothing: the library is
opened on the first call, and that call raises if the library is missing.
"""
from .binding import FaError, fwd, library_path, load_library  # noqa: F401

__all__ = ["fwd", "FaError", "load_library", "library_path"]
