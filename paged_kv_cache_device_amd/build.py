"""Build libpkvg.so (the HIP library) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", "pkvg_capi.hip")]
DEPENDS = SOURCES + [os.path.join(PKG, "csrc", "gather_kernels.hpp"),
                     os.path.join(PKG, "csrc", "indexer_kernels.hpp"),
                     os.path.join(REPO, "include", "pkvg.h")]
LIBRARY = os.path.join(PKG, "libpkvg.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    # packed fp32 VALU forms stay off: hipcc emits them on its own otherwise
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the gather kernel's 14 leading scalar argument dwords arrive in SGPRs
    "-mllvm", "-amdgpu-kernarg-preload-count=14",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(extra_flags=(), output: str = LIBRARY, verbose: bool = False) -> str:
    """Compile every source into ``output`` (always recompiles)."""
    tmp = output + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", os.path.join(REPO, "include"),
           "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in proc.stderr.splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, output)
    return output


def is_stale(path: str = LIBRARY) -> bool:
    if not os.path.exists(path):
        return True
    t = os.path.getmtime(path)
    return any(os.path.getmtime(d) > t for d in DEPENDS)


if __name__ == "__main__":
    print(build(verbose=True))
