"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Two builds, each loaded into a child Python process that preloads its
compiler's sanitizer runtime:

- the oracle (plain C, gcc), run through every oracle pin;
- the C-ABI library with its host code instrumented (hipcc; nothing is
  launched), run through the host-side argument checks of
  test_capi_host.py and the launch planning of test_plan_host.py.

A planted out-of-bounds call (a destination one row short, handed to the
oracle) checks that the sanitizer is live in the child.
"""
import os
import shutil
import subprocess
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(REPO, "tests")


def _gcc_runtime(name):
    gcc = shutil.which("gcc")
    if not gcc:
        return None
    path = subprocess.run([gcc, f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _child(code, env_extra, timeout=600):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", **env_extra)
    return subprocess.run([sys.executable, "-c", code], cwd=REPO, env=env, capture_output=True,
                          text=True, timeout=timeout)


@pytest.fixture(scope="module")
def oracle_asan(tmp_path_factory):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not found")
    out = str(tmp_path_factory.mktemp("asan") / "liboracle_asan.so")
    src = os.path.join(REPO, "oracle", "oracle.c")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out, {"LD_PRELOAD": f"{asan}:{ubsan}"}


ORACLE_PINS = """
import sys
sys.path.insert(0, {tests!r})
import oracle, oracle_pins
o = oracle.Oracle({lib!r})
for check in oracle_pins.ALL_CHECKS:
    check(o)
print("pins passed")
"""

PLANTED = """
import numpy as np, oracle
o = oracle.Oracle({lib!r})
src = np.zeros(4 * 2 * 2, dtype=np.uint8)   # 4 blocks of 2 tokens, one int16 each
dst = np.zeros(3 * 2, dtype=np.uint8)       # 3 int16 rows for a 4-token request
o.gather(0, src, 2, 4, 2, 1, 2, 1, dst, 2, 4, 1, np.array([[0, 1]], dtype=np.int32), 2, 2,
         np.array([0, 4], dtype=np.int32), None, 1)
print("not detected")
"""


def test_oracle_pins_under_sanitizers(oracle_asan):
    lib, env = oracle_asan
    r = _child(ORACLE_PINS.format(tests=TESTS, lib=lib), env)
    assert r.returncode == 0 and "pins passed" in r.stdout, r.stderr[-3000:]
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]


def test_sanitizer_is_live(oracle_asan):
    lib, env = oracle_asan
    r = _child(PLANTED.format(lib=lib), env)
    assert r.returncode != 0 and "not detected" not in r.stdout
    assert "AddressSanitizer: heap-buffer-overflow" in r.stderr, r.stderr[-3000:]


def _clang_asan_runtime():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    clang = os.path.join(rocm, "llvm", "bin", "clang")
    if not os.path.exists(clang):
        return None
    path = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                          capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        path = subprocess.run([clang, "--print-runtime-dir"], capture_output=True,
                              text=True).stdout.strip() + "/libclang_rt.asan-x86_64.so"
    return path if os.path.exists(path) else None


def test_host_library_under_sanitizers(tmp_path):
    from paged_kv_cache_device_amd import build

    runtime = _clang_asan_runtime()
    if runtime is None or not os.path.exists(build.hipcc()):
        pytest.skip("hipcc or clang's ASan runtime not found")
    out = str(tmp_path / "libpkvg_host_asan.so")
    # the product's flags at -O1 (quicker to build); every -fsanitize= applies
    # to host code only, and the device code built alongside is never launched
    cmd = [build.hipcc(), *build.HIPCC_FLAGS, "-O1", "-g",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-I", os.path.join(REPO, "include"),
           "-o", out, *build.SOURCES]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, LD_PRELOAD=runtime, PKVG_TEST_LIBRARY=out,
               ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(TESTS, "test_capi_host.py"), os.path.join(TESTS, "test_plan_host.py")],
                       cwd=REPO, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]
