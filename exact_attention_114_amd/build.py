"""Builds libfa.so (gfx950 code objects inside a host shared library) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = [os.path.join(HERE, "csrc", "fa_fwd.hip"), os.path.join(HERE, "csrc", "fa_bwd.hip"),
           os.path.join(HERE, "csrc", "fa_fwd_f32.hip"), os.path.join(HERE, "csrc", "fa_fwd_fp8.hip")]
# The forward and backward kernel instances, one object per (input type, head dimension) slice of
# one source each, so that they compile in parallel.
SLICE_SOURCE = os.path.join(HERE, "csrc", "fa_fwd_inst.hip")
BWD_SLICE_SOURCE = os.path.join(HERE, "csrc", "fa_bwd_inst.hip")
SLICES = [(bf16, d) for bf16 in (0, 1) for d in (32, 48, 64, 80, 96, 112, 128)]
DEPENDS = [os.path.join(HERE, "csrc", "fa_fwd_kernel.hpp"), os.path.join(HERE, "csrc", "fa_fwd_launch.hpp"),
           os.path.join(HERE, "csrc", "fa_fwd_f32_kernel.hpp"), os.path.join(HERE, "csrc", "fa_fwd_fp8_kernel.hpp"), os.path.join(HERE, "csrc", "fa_bwd_kernel.hpp"),
           os.path.join(HERE, "csrc", "fa_bwd_launch.hpp"),
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
    """Compile every HIP source into libfa.so (always recompiles): one hipcc process per source or
    slice, run in parallel, then one link."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    objs = []
    units = [(src, [], os.path.basename(src)) for src in SOURCES]
    units += [(SLICE_SOURCE, [f"-DFA_INST_BF16={bf}", f"-DFA_INST_D={d}"], f"fa_fwd_inst_{'bf16' if bf else 'f16'}_d{d}")
              for bf, d in SLICES]
    units += [(BWD_SLICE_SOURCE, [f"-DFA_INST_BF16={bf}", f"-DFA_INST_D={d}"], f"fa_bwd_inst_{'bf16' if bf else 'f16'}_d{d}")
              for bf, d in SLICES]
    # at most one compiler per CPU (each can take a few GiB); the backward slices (the slowest),
    # largest head dimension first, start at once
    def cost(i):
        d = next((int(f.split("=")[1]) for f in units[i][1] if f.startswith("-DFA_INST_D=")), 0)
        return (units[i][0] != BWD_SLICE_SOURCE, -d)

    order = sorted(range(len(units)), key=cost)
    jobs = max(1, min(len(units), os.cpu_count() or 8))

    def compile_unit(i):
        src, defs, name = units[i]
        cmd = [hipcc()] + compile_flags + defs + ["-c", src, "-o", objs[i]]
        if verbose:
            print(" ".join(cmd), flush=True)
        return subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)

    for src, defs, name in units:
        objs.append(os.path.join(objdir, name + ".o"))
    from concurrent.futures import ThreadPoolExecutor

    with ThreadPoolExecutor(max_workers=jobs) as pool:
        results = dict(zip(order, pool.map(compile_unit, order)))
    failed = []
    for i, (src, _, name) in enumerate(units):
        p = results[i]
        errs = "\n".join(l for l in p.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
        if p.returncode != 0:
            failed.append(f"{name} ({p.returncode}):\n{errs}")
        elif verbose and errs:
            print(errs, file=sys.stderr)
    if failed:
        raise RuntimeError("hipcc failed: " + "\n".join(failed))
    tmp = OUTPUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed ({res.returncode}):\n{res.stderr}")
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
