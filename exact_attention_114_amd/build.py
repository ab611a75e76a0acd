"""Builds libfa.so (gfx950 code objects inside a host shared library) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = [os.path.join(HERE, "csrc", "fa_fwd.hip"), os.path.join(HERE, "csrc", "fa_bwd.hip")]
DEPENDS = [os.path.join(HERE, "csrc", "fa_fwd_kernel.hpp"), os.path.join(HERE, "csrc", "fa_bwd_kernel.hpp"),
           os.path.join(HERE, "csrc", "fa_status.hpp"), os.path.join(HERE, "csrc", "fa_mask.hpp"),
           os.path.join(HERE, "csrc", "fa_mask_kernel.hpp"),
           os.path.join(os.path.dirname(HERE), "include", "fa.h")]
OUTPUT = os.path.join(HERE, "libfa.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
    # Non-finite inputs give undefined results (include/fa.h); without NaNs to honour, the
    # row maxima need no NaN-quieting instructions around v_max3_f32.
    "-fno-honor-nans",
    # Packed fp32 VALU forms are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build_library(verbose: bool = False) -> str:
    """Compile every HIP source into libfa.so (always recompiles)."""
    tmp = OUTPUT + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs:
        print(errs, file=sys.stderr)
    # A kernel whose host stub was not emitted leaves an undefined symbol behind: refuse a
    # library that the dynamic loader cannot resolve.
    import ctypes

    try:
        ctypes.CDLL(tmp)
    except OSError as e:
        os.remove(tmp)
        raise RuntimeError(f"built library does not load: {e}") from None
    os.replace(tmp, OUTPUT)
    return OUTPUT


if __name__ == "__main__":
    print(build_library(verbose=True))
