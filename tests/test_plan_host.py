"""The host's launch decisions, on the CPU: pkvg_plan runs the same argument
checks and planning as the gather calls (access width, task units, kernel,
workgroup shape, grid) and reports them without touching a device.  Addresses
below are fake (never read), aligned to 64 KiB unless a case needs otherwise."""
import ctypes
import os

import pytest

pkvg = pytest.importorskip("paged_kv_cache_device_amd")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    # another build of the same sources (the sanitizer test's instrumented one)
    other = os.environ.get("PKVG_TEST_LIBRARY")
    if other:
        pkvg._lib = pkvg.library(other)
        yield
        pkvg._lib = None
        return
    from paged_kv_cache_device_amd import build

    if build.is_stale():
        build.build()
    yield


F = 0x10000
RAW, DEQ, UP = pkvg.PKVG_OP_GATHER_CACHE, pkvg.PKVG_OP_GATHER_MAYBE_DEQUANT, pkvg.PKVG_OP_GATHER_UPCONVERT_FP8
FP8 = pkvg.PKVG_KV_FP8_E4M3


def plan(op=RAW, kind=2, bs=64, entry=576, T=61440, R=1, nb=None, ccols=None, dcols=None, starts=False,
         width=None, src=F, dst=F, scale=F):
    """A call over a [nb, bs, ccols] cache and a [T, dcols] destination; strides
    in elements of each tensor (fp8 caches: bytes)."""
    ccols = entry if ccols is None else ccols
    dcols = entry if dcols is None else dcols
    width = -(-T // bs) if width is None else width
    nb = width * R + 8 if nb is None else nb
    return pkvg.pkvg_plan(op, kind, src, nb, bs, entry, bs * ccols, ccols, dst, T, dcols, F, width, width, F, 1,
                          F if starts else None, R, scale)


def test_headline_gathers():
    # one request of 61,440 raw tokens: 64-token pages moved as 8-token units, small shape
    p = plan()
    assert (p["kernel"], p["task_mode"], p["threads"], p["batch_bytes"]) == (
        pkvg.PKVG_KERNEL_PAGES, pkvg.PKVG_TASKS_SINGLE, 256, 20480)
    assert (p["access_width"], p["flat"], p["task_tokens"], p["split_shift"], p["group_shift"]) == (16, 1, 8, 3, 0)
    assert p["grid"] == p["task_capacity"] == 61440 // 8 + 3
    # one request of 307,200 fp8 tokens to bf16: whole 64-token pages, wide shape
    p = plan(op=UP, kind=0, T=307200)
    assert (p["threads"], p["batch_bytes"], p["convert"], p["access_width"], p["src_vector"]) == (1024, 81920, 1, 8, 1)
    assert (p["task_tokens"], p["split_shift"], p["grid"]) == (64, 0, 307200 // 64 + 3)
    # skew-8: wave-register prefix, 72 KiB pages, wide shape (>= 1024 tasks)
    p = plan(T=141101, R=8, starts=True, width=2048)
    assert (p["task_mode"], p["task_tokens"], p["threads"]) == (pkvg.PKVG_TASKS_WAVE, 64, 1024)
    # the strided fp8 batch: 577-byte code rows (windowed loads), 1160-byte bf16 rows
    p = plan(op=DEQ, kind=FP8, T=298156, R=64, ccols=577, dcols=580, width=1024)
    assert (p["flat"], p["src_vector"], p["access_width"], p["task_mode"], p["threads"]) == (
        0, 0, 8, pkvg.PKVG_TASKS_WAVE, 1024)


@pytest.mark.parametrize("op,kind,bs,R,kernel,tokens,split,group,threads", [
    (RAW, 2, 1, 1, pkvg.PKVG_KERNEL_GROUPS, 8, 0, 3, 256),      # 9 KiB groups of one-token pages
    (UP, 0, 1, 1, pkvg.PKVG_KERNEL_GROUPS, 16, 0, 4, 256),      # 18 KiB groups (fp8)
    (RAW, 2, 1, 512, pkvg.PKVG_KERNEL_GROUPS, 16, 0, 4, 256),   # 18 KiB groups (batch)
    (RAW, 2, 3, 1, pkvg.PKVG_KERNEL_GROUPS, 6, 0, 1, 256),      # 3-token pages in pairs
    (RAW, 2, 8, 1, pkvg.PKVG_KERNEL_PAGES, 8, 0, 0, 256),       # 9 KiB pages: one per workgroup
    (UP, 0, 8, 1, pkvg.PKVG_KERNEL_GROUPS, 16, 0, 1, 256),      # ... but grouped for fp8
    (RAW, 2, 8, 70, pkvg.PKVG_KERNEL_GROUPS, 16, 0, 1, 256),    # ... and for batches (pairs)
    (RAW, 2, 16, 1, pkvg.PKVG_KERNEL_PAGES, 8, 1, 0, 256),      # one request: 8-token units
    (RAW, 2, 96, 1, pkvg.PKVG_KERNEL_PAGES, 6, 4, 0, 256),      # 96 -> 48 -> 24 -> 12 -> 6
    (RAW, 2, 1024, 1, pkvg.PKVG_KERNEL_PAGES, 8, 7, 0, 256),
    (UP, 0, 1024, 1, pkvg.PKVG_KERNEL_PAGES, 64, 4, 0, 1024),   # fp8 keeps 72 KiB units
    (RAW, 2, 1024, 4, pkvg.PKVG_KERNEL_PAGES, 8, 7, 0, 256),    # small batch, < 1024 pages: 9 KiB units
    (RAW, 2, 64, 8, pkvg.PKVG_KERNEL_PAGES, 8, 3, 0, 256),      # 8 x 7,680 tokens: 9 KiB units
    (RAW, 2, 64, 64, pkvg.PKVG_KERNEL_PAGES, 64, 0, 0, 1024),   # 64 requests: 1,089 tasks, 72 KiB wide
    (UP, 0, 1024, 4, pkvg.PKVG_KERNEL_PAGES, 64, 4, 0, 1024),   # fp8 small batch: 72 KiB units, wide
    (RAW, 2, 64, 100, pkvg.PKVG_KERNEL_PAGES, 16, 2, 0, 256),   # > 64 requests: 18 KiB units, small
    (UP, 0, 64, 100, pkvg.PKVG_KERNEL_PAGES, 16, 2, 0, 256),    # ... also for fp8 (18 KiB of bf16)
    (UP, 0, 64, 64, pkvg.PKVG_KERNEL_PAGES, 64, 0, 0, 1024),    # fp8, <= 64 requests: whole pages, wide
    (RAW, 2, 127, 1, pkvg.PKVG_KERNEL_PAGES, 127, 0, 0, 256),   # odd: no split, narrow
])
def test_task_units_and_kernels(op, kind, bs, R, kernel, tokens, split, group, threads):
    p = plan(op=op, kind=kind, bs=bs, R=R, T=61440)
    assert (p["kernel"], p["task_tokens"], p["split_shift"], p["group_shift"], p["threads"]) == (
        kernel, tokens, split, group, threads), p
    # a task unit is a power-of-two part of a page, or a power-of-two group of pages
    assert p["split_shift"] == 0 or p["group_shift"] == 0
    assert p["task_tokens"] << p["split_shift"] == bs << p["group_shift"]
    # one workgroup per task unit (capacity bound: T / unit + 2R + 1)
    assert p["task_capacity"] == 61440 // p["task_tokens"] + 2 * R + 1 == p["grid"]


def test_task_modes():
    # these tables are as wide as all the rows (sparse): prefix modes by batch size
    assert plan(R=1)["task_mode"] == pkvg.PKVG_TASKS_SINGLE
    assert plan(R=2)["task_mode"] == pkvg.PKVG_TASKS_WAVE
    assert plan(R=64)["task_mode"] == pkvg.PKVG_TASKS_WAVE
    assert plan(R=65)["task_mode"] == pkvg.PKVG_TASKS_LDS
    assert plan(R=1024)["task_mode"] == pkvg.PKVG_TASKS_LDS
    assert plan(R=1025)["task_mode"] == pkvg.PKVG_TASKS_TABLE
    for p in (plan(R=3), plan(R=100), plan(R=2000)):
        assert p["grid_rows"] == 1


@pytest.mark.parametrize("R,T,bs,width,walk", [
    (8, 61440, 64, 120, True),       # 8 x 7,680 tokens: a table exactly as wide as the pages
    (2, 61440, 64, 480, True),
    (64, 61440, 64, 15, True),
    (512, 102400, 64, 4, True),      # 512 x 200 tokens: 4 pages a row, 3.1 used
    (2000, 80000, 16, 3, True),      # beyond the fused limit: walked, no task table
    (8, 141101, 64, 2048, False),    # skew-8: rows far wider than most requests
    (64, 298156, 64, 1024, False),   # the mixed batch
    (8, 61440, 64, 153, False),      # just past 5/4 of the pages
    (8, 61440, 64, 0, False),        # no columns: nothing to walk
    (70000, 10 ** 6, 16, 1, False),  # beyond the grid's y extent
])
def test_walk_decision(R, T, bs, width, walk):
    p = plan(R=R, T=T, bs=bs, width=width)
    if walk:
        assert p["task_mode"] == pkvg.PKVG_TASKS_WALK and p["grid_rows"] == R, p
        # one workgroup per unit of each table row: split parts, or groups of pages
        units = -(-width // (1 << p["group_shift"])) if p["group_shift"] else width << p["split_shift"]
        assert p["grid"] == units
    else:
        assert p["task_mode"] != pkvg.PKVG_TASKS_WALK and p["grid_rows"] == 1, p


def test_walk_units_follow_the_single_request_rules():
    """A walked batch moves the same units as one request: 9 KiB raw units,
    whole 64-token fp8 pages, 9 KiB groups of one-token raw pages."""
    assert plan(R=8, width=120)["task_tokens"] == plan(R=1)["task_tokens"] == 8
    assert plan(op=UP, kind=0, R=8, width=120)["task_tokens"] == 64
    p = plan(R=512, T=102400, bs=1, width=200)
    assert (p["task_mode"], p["kernel"], p["group_shift"], p["grid"]) == (
        pkvg.PKVG_TASKS_WALK, pkvg.PKVG_KERNEL_GROUPS, 3, 25)


def test_access_widths():
    assert plan(entry=575)["access_width"] == 2                       # 1150-byte rows
    assert plan(entry=578, ccols=578, dcols=580)["access_width"] == 4  # 1156-byte rows, dword strides
    assert plan(kind=4, entry=6)["access_width"] == 8                  # 24-byte fp32 rows
    assert plan(kind=1, entry=7)["access_width"] == 1
    assert plan(dst=F + 2)["access_width"] == 2                        # destination only 2-byte aligned
    p = plan(op=UP, kind=0, entry=12)                                  # 12 codes per row
    assert (p["access_width"], p["src_vector"]) == (4, 1)
    p = plan(op=UP, kind=0, entry=576, ccols=577)                      # odd code-row pitch: windows
    assert (p["access_width"], p["src_vector"], p["flat"]) == (8, 0, 0)


def test_no_work_and_errors():
    assert plan(T=0) == {k: 0 for k in plan(T=0)}
    assert plan(R=0)["grid"] == 0
    with pytest.raises(pkvg.PkvgError) as e:
        plan(kind=3)
    assert e.value.status == pkvg.PKVG_E_DTYPE
    with pytest.raises(pkvg.PkvgError) as e:
        plan(op=7)
    assert e.value.status == pkvg.PKVG_E_SHAPE
    with pytest.raises(pkvg.PkvgError) as e:
        plan(op=UP, kind=0, scale=None)
    assert e.value.status == pkvg.PKVG_E_NULL
    with pytest.raises(pkvg.PkvgError) as e:
        plan(op=DEQ, kind=9)
    assert e.value.status == pkvg.PKVG_E_DTYPE
    with pytest.raises(pkvg.PkvgError) as e:
        plan(dcols=500)
    assert e.value.status == pkvg.PKVG_E_STRIDE
    lib = pkvg.library()
    assert lib.pkvg_plan(RAW, 2, F, 4, 16, 8, 128, 8, F, 10, 8, F, 2, 2, F, 1, None, 1, None, None) == \
        pkvg.PKVG_E_NULL


@pytest.mark.parametrize("bad", [dict(kind=3), dict(bs=0), dict(entry=0), dict(dcols=100), dict(src=None),
                                 dict(T=1 << 31)])
def test_plan_status_matches_the_call(bad):
    """pkvg_plan returns exactly what gather_cache returns from its checks
    (both return before any HIP call for these)."""
    a = dict(kind=2, bs=16, entry=128, T=1000, R=1, src=F, dcols=None)
    a.update(bad)
    dcols = a["entry"] if a["dcols"] is None else a["dcols"]
    width = max(-(-a["T"] // max(a["bs"], 1)), 1)
    lib = pkvg.library()
    args = (a["src"], 64, a["bs"], a["entry"], a["bs"] * a["entry"], a["entry"], F, a["T"], dcols, F, width,
            width, F, 1, None, a["R"])
    want = lib.gather_cache(args[0], a["kind"], *args[1:], None)
    info = pkvg.PlanInfo()
    got = lib.pkvg_plan(RAW, a["kind"], *args, None, ctypes.byref(info))
    assert got == want != pkvg.PKVG_OK


# --- property test: the host checks and the launch plan on random arguments ---

from hypothesis import HealthCheck, given, settings, strategies as st  # noqa: E402

_STATUSES = {pkvg.PKVG_OK, pkvg.PKVG_E_NULL, pkvg.PKVG_E_SHAPE, pkvg.PKVG_E_STRIDE, pkvg.PKVG_E_DTYPE,
             pkvg.PKVG_E_LIMIT}
_POINTERS = [None, F, F + 1, F + 2, F + 4, F + 8]


@settings(max_examples=400, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(data=st.data())
def test_plan_on_random_arguments(data):
    """pkvg_plan runs the calls' own checks and launch planning without touching
    a device: on any arguments it returns one of the documented statuses, and
    every plan it accepts respects the launch rules (grid cap, walked grids,
    shapes, access widths, unit sizes).  Fake addresses are never read."""
    draw = data.draw

    def mostly(valid, odd):
        # a valid value seven times in eight, else one from the edges
        return draw(valid if draw(st.integers(0, 7)) else odd)

    op = draw(st.sampled_from([RAW, DEQ, UP]))
    kinds = {RAW: [1, 2, 4, 8], DEQ: [0, 1], UP: [0]}
    kind = mostly(st.sampled_from(kinds[op]), st.sampled_from([-1, 0, 3, 9, 16]))
    bs = mostly(st.sampled_from([1, 2, 3, 4, 8, 16, 32, 64, 128, 1024]),
                st.one_of(st.integers(-2, 70), st.sampled_from([1 << 16, 1 << 20])))
    entry = mostly(st.integers(1, 1200), st.sampled_from([-2, 0, 4096, 1 << 20]))
    pad_c = draw(st.integers(0, 9))
    sts = mostly(st.just(entry + pad_c), st.integers(-3, 1 << 34))
    sbs = mostly(st.just(max(bs, 0) * (entry + pad_c)), st.integers(-3, 1 << 40))
    drs = mostly(st.just(entry + draw(st.integers(0, 9))), st.integers(-3, 1 << 34))
    T = mostly(st.integers(0, 400000), st.sampled_from([-2, -1, (1 << 31) - 1, (1 << 31) + 5, 1 << 40]))
    R = mostly(st.one_of(st.integers(0, 80), st.integers(1000, 70000)), st.sampled_from([-2, -1, 1 << 20]))
    width = mostly(st.integers(1, 5000), st.sampled_from([-2, 0, 1 << 20]))
    ld = width + mostly(st.just(0), st.integers(-3, 64))
    nb = mostly(st.integers(1, 1 << 20), st.sampled_from([-2, 0, 1 << 40]))
    term = mostly(st.just(1), st.sampled_from([0, 2]))
    ptr = lambda: mostly(st.just(F), st.sampled_from(_POINTERS))  # noqa: E731
    src, dst, table, cu, starts, scale = ptr(), ptr(), ptr(), ptr(), ptr(), ptr()

    info = pkvg.PlanInfo()
    status = pkvg.library().pkvg_plan(op, kind, src, nb, bs, entry, sbs, sts, dst, T, drs, table, width,
                                      ld, cu, term, starts, R, scale, ctypes.byref(info))
    assert status in _STATUSES, status
    if status != pkvg.PKVG_OK:
        return
    p = info.as_dict()
    if p["grid"] == 0:  # no work: nothing is planned
        assert all(v == 0 for v in p.values()), p
        return
    assert p["kernel"] in (pkvg.PKVG_KERNEL_PAGES, pkvg.PKVG_KERNEL_GROUPS), p
    assert p["threads"] in (256, 1024) and p["access_width"] in (1, 2, 4, 8, 16), p
    assert 1 <= p["grid"] <= 1 << 16, p
    if p["task_mode"] == pkvg.PKVG_TASKS_WALK:
        assert p["grid_rows"] == R and 1 <= R <= 65535, p
    else:
        assert p["grid_rows"] == 1 and p["grid"] == min(p["task_capacity"], 1 << 16), p
    assert 0 <= p["group_shift"] <= 6 and p["split_shift"] >= 0, p
    if p["group_shift"] > 0:
        assert p["kernel"] == pkvg.PKVG_KERNEL_GROUPS and p["task_tokens"] == bs << p["group_shift"], p
    else:
        assert p["kernel"] == pkvg.PKVG_KERNEL_PAGES, p
        assert p["task_tokens"] << p["split_shift"] == bs, p
