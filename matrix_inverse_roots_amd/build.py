"""Compile the HIP library ``libshampoo.so`` for gfx950, in the package directory.

Usage: ``python matrix_inverse_roots_amd/build.py`` (run as a file: importing
the package would load the library before it is rebuilt), or
``__graft_entry__.build()``.  hipcc cross-compiles for gfx950 without a GPU.
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libshampoo.so")
SOURCES = [os.path.join(PKG, "csrc", "shampoo.hip")]
HEADERS = [os.path.join(PKG, "csrc", f) for f in ("gemm_common.hpp", "gemm.hpp", "gemm_hsym.hpp", "gemm_nn256.hpp",
                                                  "kernels.hpp")] + [
    os.path.join(ROOT, "include", "shampoo.h")]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed FP32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-pass-failed",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def build(verbose=False):
    """Compile libshampoo.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, err))
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
