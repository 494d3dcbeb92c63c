"""The C ABI from a native program (tests/native/capi_native.cpp): no Python
or torch in the path, device memory from hipMalloc.  Every compute entry point
is called: the four paged gathers (gather_cache, gather_upconvert_fp8,
gather_maybe_dequant auto and fp8, and its no-allocation variant) on a small
batch and on 1,500 short requests, gather_page_tasks and
gather_indexer_quant_cache; the program checks every output byte against the
C oracle."""
import os
import subprocess

import pytest

from gpu_util import log

pytestmark = pytest.mark.gpu

PROGRAM = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "capi_native")


def test_native_program_matches_the_oracle():
    if not os.path.exists(PROGRAM):
        pytest.fail(f"{PROGRAM} is not built: run __graft_entry__.build()")
    log("[native] running tests/native/capi_native")
    proc = subprocess.run([PROGRAM], capture_output=True, text=True, timeout=120)
    log(proc.stdout)
    assert proc.returncode == 0, proc.stdout + proc.stderr
    assert "native C-ABI parity ok" in proc.stdout
