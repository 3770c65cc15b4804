"""Build libcpring.so for gfx950 with hipcc, in-tree.

    python -m context_ring_attention_zigzag_amd.build

compiles every HIP source under ``csrc/`` into
``context_ring_attention_zigzag_amd/libcpring.so``. hipcc cross-compiles, so
this works on a machine without a GPU.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libcpring.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

# Packed fp32 VALU forms are kept out of the generated code; plain fp32 ops only.
HIP_FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-result"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libcpring)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile libcpring.so and return its path. Always recompiles."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *(extra_flags or []), f"-I{INCLUDE}", f"-I{CSRC}", *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name; that warning is harmless.
    noise = "not a recognized feature for this target"
    errs = "\n".join(x for x in (res.stdout + res.stderr).splitlines() if noise not in x)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs)
    # A kernel whose host pass fails leaves an undefined launch stub behind
    # without a compiler error; refuse such a library here.
    import ctypes
    try:
        ctypes.CDLL(tmp)
    except OSError as e:
        raise RuntimeError(f"built library does not load: {e}") from e
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
