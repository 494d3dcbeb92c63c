"""Build the native C-ABI test program (tests/native/capi_native) with hipcc,
linked against the in-tree libpkvg.so and the oracle's liboracle.so (the
checker) through $ORIGIN-relative run paths, so it runs from any checkout."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(os.path.dirname(HERE))
SOURCE = os.path.join(HERE, "capi_native.cpp")
PROGRAM = os.path.join(HERE, "capi_native")


def build() -> str:
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    cmd = [hipcc, "-O2", "-std=c++17", "-I", os.path.join(REPO, "include"), SOURCE, "-o", PROGRAM,
           "-L", os.path.join(REPO, "paged_kv_cache_device_amd"), "-lpkvg",
           "-L", os.path.join(REPO, "oracle"), "-loracle",
           "-Wl,-rpath,$ORIGIN/../../paged_kv_cache_device_amd", "-Wl,-rpath,$ORIGIN/../../oracle"]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{' '.join(cmd)}\n{proc.stderr}")
    return PROGRAM


if __name__ == "__main__":
    print("built", build())
