"""Host-side checks of the C-ABI library that need no GPU: the library loads,
exports every entry point include/pkvg.h declares, and rejects bad arguments
(or returns early when there is no work) before any HIP call."""
import ctypes
import os
import re

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(REPO, "include", "pkvg.h")

pkvg = pytest.importorskip("paged_kv_cache_device_amd")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


@pytest.fixture(scope="module")
def lib():
    from paged_kv_cache_device_amd import build

    # another build of the same sources (the sanitizer test's host-only one)
    other = os.environ.get("PKVG_TEST_LIBRARY")
    if other:
        return pkvg.library(other)
    if build.is_stale():
        build.build()
    return pkvg.library()


def test_header_declares_the_entry_points():
    names = set(_declared_functions())
    assert {"gather_cache", "gather_maybe_dequant", "gather_upconvert_fp8",
            "gather_page_tasks", "pkvg_status_string", "pkvg_last_hip_error"} <= names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert set(_declared_functions()) == set(pkvg.SIGNATURES)


def test_status_strings(lib):
    for code in range(8):
        assert pkvg.status_string(code).startswith("PKVG_")
    assert "unknown" in pkvg.status_string(99)
    assert lib.pkvg_last_hip_error() == 0


FAKE = 0x10000  # never dereferenced: every call below returns before any HIP call


def _gc(lib, **kw):
    a = dict(src=FAKE, elem=2, nb=4, bs=16, entry=8, sbs=128, sts=8, dst=FAKE, T=10, drs=8,
             bt=FAKE, W=2, ld=2, cu=FAKE, term=1, ss=None, R=1)
    a.update(kw)
    return lib.gather_cache(a["src"], a["elem"], a["nb"], a["bs"], a["entry"], a["sbs"], a["sts"],
                            a["dst"], a["T"], a["drs"], a["bt"], a["W"], a["ld"], a["cu"], a["term"],
                            a["ss"], a["R"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(elem=3), pkvg.PKVG_E_DTYPE),
    (dict(elem=0), pkvg.PKVG_E_DTYPE),
    (dict(bs=0), pkvg.PKVG_E_SHAPE),
    (dict(entry=0), pkvg.PKVG_E_SHAPE),
    (dict(R=-1), pkvg.PKVG_E_SHAPE),
    (dict(T=-1), pkvg.PKVG_E_SHAPE),
    (dict(nb=-1), pkvg.PKVG_E_SHAPE),
    (dict(W=-1), pkvg.PKVG_E_SHAPE),
    (dict(term=2), pkvg.PKVG_E_SHAPE),
    (dict(term=-1), pkvg.PKVG_E_SHAPE),
    (dict(drs=7), pkvg.PKVG_E_STRIDE),
    (dict(sts=-1), pkvg.PKVG_E_STRIDE),
    (dict(sbs=-1), pkvg.PKVG_E_STRIDE),
    (dict(ld=1), pkvg.PKVG_E_STRIDE),
    (dict(src=None), pkvg.PKVG_E_NULL),
    (dict(dst=None), pkvg.PKVG_E_NULL),
    (dict(bt=None), pkvg.PKVG_E_NULL),
    (dict(cu=None), pkvg.PKVG_E_NULL),
    (dict(T=(1 << 31) * 16), pkvg.PKVG_E_LIMIT),        # too many page tasks
    (dict(T=1 << 31, bs=1 << 20, entry=1), pkvg.PKVG_E_LIMIT),  # rows past int32
    (dict(bs=1 << 20, entry=1 << 10, drs=1 << 10), pkvg.PKVG_E_LIMIT),  # a page spans >= 2^31 bytes
    (dict(R=0, src=None, dst=None, bt=None, cu=None), pkvg.PKVG_OK),   # no work: nothing enqueued
    (dict(T=0, src=None, dst=None, bt=None, cu=None), pkvg.PKVG_OK),
])
def test_gather_cache_argument_checks(lib, kw, code):
    assert _gc(lib, **kw) == code


def test_maybe_dequant_argument_checks(lib):
    args = [4, 16, 8, 128, 8, FAKE, 10, 8, FAKE, 2, 2, FAKE, 1, None, 1]
    assert lib.gather_maybe_dequant(FAKE, 7, *args, FAKE, None) == pkvg.PKVG_E_DTYPE
    assert lib.gather_maybe_dequant(FAKE, pkvg.PKVG_KV_FP8_E4M3, *args, None, None) == pkvg.PKVG_E_NULL
    assert lib.gather_upconvert_fp8(FAKE, *args, None, None) == pkvg.PKVG_E_NULL
    no_work = [4, 16, 8, 128, 8, None, 0, 8, None, 2, 2, None, 1, None, 1]
    assert lib.gather_upconvert_fp8(None, *no_work, None, None) == pkvg.PKVG_OK
    bad_stride = [4, 16, 8, 128, 8, FAKE, 10, 7, FAKE, 2, 2, FAKE, 1, None, 1]
    assert lib.gather_upconvert_fp8(FAKE, *bad_stride, FAKE, None) == pkvg.PKVG_E_STRIDE


def test_page_tasks_argument_checks(lib):
    def f(*a):
        return lib.gather_page_tasks(a[0], 1, *a[1:])

    assert f(FAKE, None, 1, 10, 0, FAKE, 2, 2, 4, FAKE, 8, FAKE, None) == pkvg.PKVG_E_SHAPE
    assert f(FAKE, None, 1, 10, 16, FAKE, 2, 1, 4, FAKE, 8, FAKE, None) == pkvg.PKVG_E_STRIDE
    assert f(FAKE, None, 1, 10, 16, FAKE, 2, 2, 4, FAKE, 8, None, None) == pkvg.PKVG_E_NULL
    assert f(None, None, 1, 10, 16, FAKE, 2, 2, 4, FAKE, 8, FAKE, None) == pkvg.PKVG_E_NULL
    assert f(FAKE, None, 1, 10, 16, FAKE, 2, 2, 4, None, 8, FAKE, None) == pkvg.PKVG_E_NULL
    assert f(FAKE, None, 1, 10, 16, FAKE, 2, 2, 4, FAKE, 1 << 31, FAKE, None) == pkvg.PKVG_E_LIMIT
    assert f(FAKE, None, -1, 10, 16, FAKE, 2, 2, 4, FAKE, 8, FAKE, None) == pkvg.PKVG_E_SHAPE
    assert lib.gather_page_tasks(FAKE, 3, None, 1, 10, 16, FAKE, 2, 2, 4, FAKE, 8, FAKE,
                                 None) == pkvg.PKVG_E_SHAPE


def test_binding_rejects_host_tensors():
    import torch

    cache = torch.zeros(4, 16, 8, dtype=torch.bfloat16)
    dst = torch.zeros(10, 8, dtype=torch.bfloat16)
    bt = torch.zeros(1, 2, dtype=torch.int32)
    cu = torch.tensor([0, 10], dtype=torch.int32)
    with pytest.raises(ValueError):
        pkvg.gather_cache(cache, dst, bt, cu, 1)


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(ImportError):
        pkvg.library(str(tmp_path / "missing.so"))


def _ix(lib, **kw):
    a = dict(cache=FAKE, nb=4, bs=16, bstride=16 * 132, layout=pkvg.PKVG_INDEXER_FLAT, hd=128,
             bt_=16, ht=16, vals=FAKE, vstride=128, scales=FAKE, sstride=1, T=10, t2s=FAKE, cu=FAKE,
             B=2, table=FAKE, W=3, ld=3)
    a.update(kw)
    return lib.gather_indexer_quant_cache(
        a["cache"], a["nb"], a["bs"], a["bstride"], a["layout"], a["hd"], a["bt_"], a["ht"], a["vals"],
        a["vstride"], a["scales"], a["sstride"], a["T"], a["t2s"], a["cu"], a["B"], a["table"],
        a["W"], a["ld"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(layout=2), pkvg.PKVG_E_DTYPE),                       # unknown record layout
    (dict(hd=96), pkvg.PKVG_E_DTYPE),                          # head_dim not built
    (dict(layout=pkvg.PKVG_INDEXER_TILED, bt_=8), pkvg.PKVG_E_DTYPE),   # tile shape not built
    (dict(layout=pkvg.PKVG_INDEXER_TILED, bs=8, bstride=8 * 132), pkvg.PKVG_E_SHAPE),  # bs % 16
    (dict(bs=0), pkvg.PKVG_E_SHAPE),
    (dict(T=-1), pkvg.PKVG_E_SHAPE),
    (dict(B=-1), pkvg.PKVG_E_SHAPE),
    (dict(nb=-1), pkvg.PKVG_E_SHAPE),
    (dict(W=-1), pkvg.PKVG_E_SHAPE),
    (dict(bstride=16 * 132 - 4), pkvg.PKVG_E_STRIDE),         # record shorter than values + scales
    (dict(vstride=127), pkvg.PKVG_E_STRIDE),
    (dict(sstride=0), pkvg.PKVG_E_STRIDE),
    (dict(ld=2), pkvg.PKVG_E_STRIDE),
    (dict(bstride=16 * 132 + 2), pkvg.PKVG_E_STRIDE),         # records not dword-aligned
    (dict(cache=FAKE + 2), pkvg.PKVG_E_STRIDE),
    (dict(scales=FAKE + 2), pkvg.PKVG_E_STRIDE),
    (dict(cache=None), pkvg.PKVG_E_NULL),
    (dict(vals=None), pkvg.PKVG_E_NULL),
    (dict(scales=None), pkvg.PKVG_E_NULL),
    (dict(t2s=None), pkvg.PKVG_E_NULL),
    (dict(cu=None), pkvg.PKVG_E_NULL),
    (dict(table=None), pkvg.PKVG_E_NULL),
    (dict(T=1 << 31), pkvg.PKVG_E_LIMIT),
    (dict(bstride=1 << 31), pkvg.PKVG_E_LIMIT),
    (dict(T=0, cache=None, vals=None, scales=None, t2s=None, cu=None, table=None), pkvg.PKVG_OK),
    (dict(B=0, cache=None, vals=None, scales=None, t2s=None, cu=None, table=None), pkvg.PKVG_OK),
    # no row can pass the block-id or column masks: nothing is enqueued
    (dict(nb=0, cache=None, vals=None, scales=None, t2s=None, cu=None, table=None), pkvg.PKVG_OK),
    (dict(W=0, cache=None, vals=None, scales=None, t2s=None, cu=None, table=None), pkvg.PKVG_OK),
])
def test_indexer_argument_checks(lib, kw, code):
    assert _ix(lib, **kw) == code


def test_noalloc_rejects_batches_beyond_its_scratch(lib):
    """The no-allocation entry point checks its fixed scratch's limits before
    any HIP call: too many requests, or too many task units."""
    def call(R, T, bs, width):
        return lib.gather_maybe_dequant_noalloc(FAKE, pkvg.PKVG_KV_AUTO, 10 ** 6, bs, 576, bs * 576,
                                                576, FAKE, T, 576, FAKE, width, width, FAKE, 1, None, R,
                                                None, None)
    # sparse tables (far wider than the rows need): the task-table path
    assert call(pkvg.PKVG_NOALLOC_MAX_REQS + 1, 10 ** 6, 64, 4) == pkvg.PKVG_E_SCRATCH
    assert call(2000, 64 * 16 * pkvg.PKVG_NOALLOC_MAX_TASKS, 64, 4096) == pkvg.PKVG_E_SCRATCH
    # a dense table is walked directly and needs no scratch (planned only: no launch here)
    info = pkvg.pkvg_plan(pkvg.PKVG_OP_GATHER_MAYBE_DEQUANT, pkvg.PKVG_KV_AUTO, FAKE, 10 ** 6, 64, 576,
                          64 * 576, 576, FAKE, 64 * 16 * pkvg.PKVG_NOALLOC_MAX_TASKS, 576, FAKE, 4, 4,
                          FAKE, 1, None, 2000, None)
    assert info["task_mode"] == pkvg.PKVG_TASKS_WALK
    # argument errors still come first
    assert lib.gather_maybe_dequant_noalloc(FAKE, 9, 100, 64, 576, 64 * 576, 576, FAKE, 10, 576,
                                            FAKE, 4, 4, FAKE, 1, None, 2000, None,
                                            None) == pkvg.PKVG_E_DTYPE


def test_native_program_loads_without_a_gpu():
    """The native C-ABI program links the library and the oracle through
    relative run paths; where no GPU is visible it says so and exits 2
    (no compute call is made)."""
    import os
    import subprocess

    import torch

    program = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "capi_native")
    if not os.path.exists(program):
        pytest.fail(f"{program} is not built: run __graft_entry__.build()")
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: the GPU test runs the program")
    proc = subprocess.run([program], capture_output=True, text=True, timeout=60)
    assert proc.returncode == 2 and "no GPU" in proc.stdout, proc.stdout + proc.stderr
