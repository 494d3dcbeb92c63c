"""Parity of the HIP gather (through the C ABI) with the CPU oracle, bit for
bit, on MI355X: the five named workloads at full size, seeded random small
workloads spanning every edge case, every access-width path, the exhaustive
fp8 code table, the page-task builder, the large-batch (tabled) path, and byte
offsets beyond 2^31."""
import numpy as np
import pytest
import torch

import oracle
import oracle_pins
import paged_kv_cache_device_amd as pkvg
import workloads
from gpu_util import byte_diff, check_parity, log, plan_of, run_hip

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_device_amd as pkvg

    pkvg.library()  # fail loudly if the HIP library is missing


# ---------------------------------------------------------------------------
# the five named workloads, full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(workloads.NAMED))
def test_named_workload_parity(name):
    check_parity(workloads.named(name), DEV)


# ---------------------------------------------------------------------------
# the page's own kernel test shape: 17 / 32,768 / 71 rows, starts 3 / 17 / 5,
# block 64, entry 576, each table row a permutation of all 1,024 blocks
# ---------------------------------------------------------------------------

PAGES_TEST_CALLS = [
    (workloads.RAW, torch.bfloat16),        # gather_cache, 'auto' (bf16) cache
    (workloads.RAW, torch.uint8),           # gather_cache, one-byte fp8 cache copied as bytes
    (workloads.DEQUANT_AUTO, torch.bfloat16),
    (workloads.DEQUANT_FP8, None),
    (workloads.UPCONVERT, None),
]


@pytest.mark.parametrize("use_starts", [False, True])
@pytest.mark.parametrize("kind,cache_dtype", PAGES_TEST_CALLS,
                         ids=["raw_bf16", "raw_u8", "auto", "fp8", "upconvert"])
def test_pages_large_uneven_sequences(kind, cache_dtype, use_starts):
    check_parity(workloads.pages_uneven_test(kind, use_starts, cache_dtype or torch.bfloat16), DEV)


# ---------------------------------------------------------------------------
# random small workloads: partial pages, seq_starts, zero-length requests,
# aliased blocks, strided rows, num_tokens clamping, guard-skipped pages
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [101, 102, 103])
def test_random_small_workloads(seed):
    for wl in oracle_pins.random_small_workloads(seed, 40):
        check_parity(wl, DEV)


@pytest.mark.parametrize("R,bs", [(64, 16), (300, 16), (1024, 4), (1025, 4), (3000, 2), (20000, 1),
                                  (70000, 2)])
def test_many_requests(R, bs):
    """Fused builder with several requests per thread (R > 256), the largest fused
    batch, and the tabled builder beyond it (its scan carries across up to 69
    chunks of 1024 requests; one-token pages go through the group kernel)."""
    g = torch.Generator("cpu").manual_seed(R)
    lens = torch.randint(0, 5 * bs, (R,), generator=g)
    lens[torch.rand(R, generator=g) < 0.15] = 0
    lens = lens.tolist()
    starts = [int(torch.randint(0, n + 1, (1,), generator=g)) for n in lens]
    pages = sum(-(-n // bs) for n in lens)
    for kind, use_starts in ((workloads.RAW, True), (workloads.UPCONVERT, False)):
        wl = workloads.make_workload(f"many_{R}_{kind}", kind, lens, bs, 72, pages + 3,
                                     seed=R + 1, starts=starts if use_starts else None,
                                     scale=0.05)
        check_parity(wl, DEV)


# ---------------------------------------------------------------------------
# every access path: widths 16/8/4/2/1 x flat/rows for raw copies; 8/4/2/1
# codes per lane x vector/byte loads x flat/rows for fp8
# ---------------------------------------------------------------------------

RAW_PATHS = [
    # (cache dtype, entry, cache cols, dst cols)
    (torch.bfloat16, 576, 576, 576),   # 16 B, flat
    (torch.bfloat16, 576, 640, 576),   # 16 B, rows (padded cache rows)
    (torch.bfloat16, 576, 576, 584),   # 16 B, rows (padded dst rows)
    (torch.bfloat16, 576, 578, 580),   # 16 B, dword-aligned rows (1156 / 1160-byte pitch)
    (torch.bfloat16, 576, 578, 578),   # 16 B, rows at every dword offset mod 16
    (torch.bfloat16, 12, 12, 12),      # 8 B (24-byte rows), flat
    (torch.bfloat16, 12, 16, 12),      # 8 B, rows
    (torch.bfloat16, 12, 14, 14),      # 8 B, dword-aligned rows (28-byte pitch)
    (torch.bfloat16, 6, 6, 6),         # 4 B, flat
    (torch.bfloat16, 6, 8, 10),        # 4 B, rows
    (torch.bfloat16, 7, 7, 7),         # 2 B, flat
    (torch.bfloat16, 7, 9, 8),         # 2 B, rows
    (torch.uint8, 577, 577, 577),      # 1 B, flat
    (torch.uint8, 577, 579, 580),      # 1 B, rows
    (torch.uint8, 576, 580, 588),      # 16 B, dword-aligned byte rows
    (torch.float32, 576, 576, 576),    # fp32 entries, 16 B flat
    (torch.float32, 3, 5, 3),          # fp32, 4 B rows
]


@pytest.mark.parametrize("dtype,entry,ccols,dcols", RAW_PATHS)
def test_raw_access_paths(dtype, entry, ccols, dcols):
    lens = [0, 1, 63, 64, 65, 200, 17]
    starts = [5, 0, 1, 0, 63, 7, 16]
    for use_starts in (False, True):
        wl = workloads.make_workload(f"raw_{dtype}_{entry}_{ccols}_{dcols}", workloads.RAW, lens,
                                     16, entry, 40, seed=entry + ccols,
                                     starts=starts if use_starts else None, cache_cols=ccols,
                                     dst_cols=dcols, cache_dtype=dtype,
                                     workspace_rows=sum(lens) + 3)
        check_parity(wl, DEV)


FP8_PATHS = [
    # (entry, cache cols, dst cols)
    (576, 576, 576),   # 8 codes, vector loads, flat
    (576, 584, 576),   # 8 codes, vector loads, rows
    (576, 577, 576),   # 8 codes, unaligned code rows (dword windows), rows
    (576, 577, 580),   # 8 codes, windows, 1160-byte dst pitch (the strided mixed workload)
    (576, 580, 580),   # 8 codes, dword-aligned code rows, 1160-byte dst pitch
    (576, 578, 578),   # 8 codes, windows, dst rows at every dword offset mod 16
    (20, 21, 22),      # 4 codes, windows, 44-byte dst pitch
    (12, 12, 12),      # 4 codes (24-byte dst rows), flat
    (6, 6, 6),         # 2 codes, flat
    (6, 7, 7),         # 1 code
    (5, 5, 5),         # 1 code, flat
]


@pytest.mark.parametrize("entry,ccols,dcols", FP8_PATHS)
@pytest.mark.parametrize("kind", [workloads.DEQUANT_FP8, workloads.UPCONVERT])
def test_fp8_access_paths(kind, entry, ccols, dcols):
    lens = [0, 1, 63, 64, 65, 200, 17]
    starts = [5, 0, 1, 0, 63, 7, 16]
    for use_starts in (False, True):
        wl = workloads.make_workload(f"fp8_{entry}_{ccols}_{dcols}", kind, lens, 16, entry, 40,
                                     seed=entry * 7 + ccols, starts=starts if use_starts else None,
                                     cache_cols=ccols, dst_cols=dcols, scale=0.05,
                                     workspace_rows=sum(lens) + 3)
        check_parity(wl, DEV)


@pytest.mark.parametrize("seed", range(6))
def test_wide_shape_random(seed):
    """Random batches big enough for the wide workgroup shape (>= 1024 pages, or
    any flat fp8 gather): block sizes whose pages have 64-multiple or ragged
    chunk counts, entries of several widths, seq_starts, partial pages; the
    wave-uniform store bursts and write-through stores against the oracle."""
    g = torch.Generator("cpu").manual_seed(9000 + seed)
    pick = lambda xs: xs[int(torch.randint(0, len(xs), (1,), generator=g))]
    kind = pick([workloads.RAW, workloads.UPCONVERT, workloads.DEQUANT_FP8])
    bs = pick([16, 32, 64, 128])
    entry = pick([64, 136, 512, 576, 1000])
    R = int(torch.randint(1, 9, (1,), generator=g))
    target_pages = 1100 + int(torch.randint(0, 600, (1,), generator=g))
    lens = [int(x) for x in torch.randint(1, 2 * target_pages * bs // R + 2, (R,), generator=g)]
    starts = [int(torch.randint(0, n // 3 + 1, (1,), generator=g)) for n in lens]
    pages = sum(-(-n // bs) for n in lens)
    wl = workloads.make_workload(f"wide_rand_{seed}", kind, lens, bs, entry, pages + 5, seed=9100 + seed,
                                 starts=starts, scale=0.05)
    check_parity(wl, DEV)


WIDE_NARROW = [
    # (cache dtype, entry, block size, pages, chunk bytes): raw pages of more than 36 KiB, at
    # least 1,024 of them, in a batch of 4 requests with a sparse table (not walked)
    (torch.bfloat16, 12, 2048, 1100, 8),   # 24-byte rows, 48 KiB pages
    (torch.bfloat16, 6, 8192, 1030, 4),    # 12-byte rows, 96 KiB pages in two parts
    (torch.bfloat16, 7, 4096, 1030, 2),    # 14-byte rows, 56 KiB pages
    (torch.uint8, 577, 128, 1100, 1),      # 577-byte rows, 72 KiB pages in two parts
]


@pytest.mark.parametrize("dtype,entry,bs,pages,width", WIDE_NARROW)
def test_wide_shape_narrow_chunks(dtype, entry, bs, pages, width):
    """The wide shape with 8-, 4-, 2- and 1-byte raw chunks: its store bursts
    on whole waves and, on the waves a ragged page leaves partly filled,
    buffer stores whose chunks past the page's end take an out-of-range
    offset.  Ragged lengths and seq_starts give partial first and last pages."""
    R = 4
    per = pages // R
    lens = [per * bs - 5, per * bs + bs // 3, per * bs - bs // 2 + 1, per * bs + 7]
    starts = [3, 0, bs // 2 + 1, 1]
    need = [-(-n // bs) for n in lens]
    wl = workloads.make_workload(f"wide_narrow_{entry}_{bs}", workloads.RAW, lens, bs, entry,
                                 sum(need) + 8, seed=entry + bs, starts=starts,
                                 width=2 * max(need) + 3, cache_dtype=dtype)
    plan = plan_of(wl.to(DEV))
    log(f"[wide narrow] entry={entry} bs={bs} T={wl.num_tokens} plan={plan}")
    assert (plan["threads"], plan["access_width"], plan["flat"]) == (1024, width, 1), plan
    check_parity(wl, DEV)


@pytest.mark.parametrize("case", ["pages", "one_token_groups"])
def test_tasks_beyond_the_grid(case):
    """More task units than the launch has workgroups (the grid is capped at
    65,536): workgroups stride over the tasks, and every task after a
    workgroup's first looks its block-table entries up inside the loop
    instead of taking the ones fetched with the request extent.  One request
    of 614,400 tokens in 9 KiB units (76,798 units) and one of 600,000
    one-token pages in 8-page groups (75,002 groups), with seq_starts; the
    whole workspace against the oracle."""
    if case == "pages":
        wl = workloads.make_workload("grid_cap_pages", workloads.RAW, [614400], 64, 576,
                                     614400 // 64 + 9, seed=71, starts=[37])
    else:
        wl = workloads.make_workload("grid_cap_groups", workloads.RAW, [600000], 1, 576, 600017,
                                     seed=73, starts=[5])
    plan = plan_of(wl.to(DEV))
    log(f"[grid cap] {case}: T={wl.num_tokens} plan={plan}")
    assert plan["task_mode"] == pkvg.PKVG_TASKS_SINGLE
    assert plan["grid"] < plan["task_capacity"], plan
    check_parity(wl, DEV)


@pytest.mark.parametrize("bs,lens,kind", [
    (1024, [20000], workloads.RAW),
    (1024, [20000], workloads.UPCONVERT),
    (4096, [9000, 0, 17, 5000], workloads.RAW),
    (4096, [9000, 4097], workloads.DEQUANT_FP8),
    (2048, [3000] * 70, workloads.RAW),
])
def test_large_pages(bs, lens, kind):
    """Pages of 1,024-4,096 tokens (1.2-4.7 MB of output each): every workgroup
    moves its page in several batches, with seq_starts and partial pages."""
    starts = [n // 3 for n in lens]
    pages = sum(-(-n // bs) for n in lens)
    wl = workloads.make_workload(f"large_pages_{bs}_{kind}_{len(lens)}", kind, lens, bs, 576, pages + 3,
                                 seed=bs + len(lens), starts=starts, scale=0.05)
    check_parity(wl, DEV)


def _with_holes(wl, seed):
    """A copy of `wl` with guard-skipped pages: a few table entries set to -1 or
    past the cache, and the table cut a few columns short."""
    g = torch.Generator("cpu").manual_seed(seed)
    bt = wl.block_table.clone()
    flat = bt.view(-1)
    if flat.numel() > 0:
        for k in range(min(7, flat.numel())):
            flat[int(torch.randint(0, flat.numel(), (1,), generator=g))] = [-1, wl.num_blocks, 1 << 30][k % 3]
    wl.block_table = bt[:, : max(bt.shape[1] - 3, 0)].contiguous()
    return wl


@pytest.mark.parametrize("bs,R,kind,pad", [
    (1, 1, workloads.RAW, False),
    (1, 1, workloads.UPCONVERT, False),
    (1, 300, workloads.DEQUANT_FP8, True),
    (2, 5, workloads.RAW, True),
    (3, 1, workloads.DEQUANT_FP8, True),
    (4, 70, workloads.RAW, False),
    (5, 1200, workloads.RAW, False),
    (8, 1, workloads.UPCONVERT, False),
    (7, 40, workloads.UPCONVERT, True),
])
def test_small_page_groups(bs, R, kind, pad):
    """Pages of one to eight tokens, moved as groups of consecutive pages per
    workgroup: requests that start and end inside a group, every task path,
    padded rows (strided copies, unaligned fp8 code rows), then guard-skipped
    pages inside groups and a table that ends mid-request."""
    g = torch.Generator("cpu").manual_seed(bs * 1000 + R)
    hi = max(40_000 // R, 3)
    lens = [int(x) for x in torch.randint(0, hi, (R,), generator=g)]
    starts = [int(torch.randint(0, n // 2 + 1, (1,), generator=g)) for n in lens]
    pages = sum(-(-n // bs) for n in lens)
    wl = workloads.make_workload(f"groups_{bs}_{R}_{kind}", kind, lens, bs, 576, pages + 11, seed=bs + R,
                                 starts=starts, scale=0.05, cache_cols=577 if pad else 576,
                                 dst_cols=580 if pad else 576)
    check_parity(wl, DEV)
    check_parity(_with_holes(wl, bs + R), DEV)


@pytest.mark.parametrize("bs,lens,kind", [
    (128, [61440], workloads.RAW),
    (256, [30000, 5, 0, 777], workloads.UPCONVERT),
    (512, [100000], workloads.DEQUANT_FP8),
    (256, [2000] * 100, workloads.RAW),
    (128, [300] * 1100, workloads.RAW),
    (96, [20000, 3], workloads.UPCONVERT),
])
def test_split_pages(bs, lens, kind):
    """Pages of more than 64 rows of 1152 output bytes, split into 2^k task
    units of one page each: seq_starts inside a unit, every task path, then
    guard-skipped pages (all units of a skipped page stay untouched)."""
    starts = [n // 5 for n in lens]
    pages = sum(-(-n // bs) for n in lens)
    wl = workloads.make_workload(f"split_{bs}_{len(lens)}_{kind}", kind, lens, bs, 576, pages + 3,
                                 seed=bs + len(lens), starts=starts, scale=0.05)
    check_parity(wl, DEV)
    check_parity(_with_holes(wl, bs), DEV)


def medium_random_workload(seed: int) -> workloads.Workload:
    """A seeded mid-size batch: every workgroup shape (page sizes from a few KiB
    to over 72 KiB), every task path (one request, wave registers, LDS prefix,
    task table), raw widths and fp8 code widths, strided rows, seq_starts,
    aliased blocks, guard-skipped pages, clamped and open-ended extents."""
    g = torch.Generator("cpu").manual_seed(seed)
    ri = lambda lo, hi: int(torch.randint(lo, hi + 1, (1,), generator=g))
    kind = [workloads.RAW, workloads.DEQUANT_FP8, workloads.UPCONVERT, workloads.DEQUANT_AUTO][seed % 4]
    R = [1, 3, 20, 64, 65, 200, 1100][ri(0, 6)]
    bs = [8, 16, 32, 64, 128][ri(0, 4)]
    entry = [64, 136, 256, 512, 576, 1000][ri(0, 5)]
    cache_dtype = [torch.bfloat16, torch.float32, torch.uint8][ri(0, 2)]
    max_tokens = max(40_000 // R, 2)
    lens = [0 if ri(0, 9) == 0 else ri(1, max_tokens) for _ in range(R)]
    starts = [ri(0, n // 2) for n in lens] if ri(0, 1) else None
    pages = sum(-(-n // bs) for n in lens)
    alias = ri(0, 3) == 0
    nb = max(pages, 1) + ri(0, 8) if not alias else max([-(-n // bs) for n in lens] + [1]) + 2
    wl = workloads.make_workload(f"medium_{seed}", kind, lens, bs, entry, nb, seed=seed + 77,
                                 starts=starts, cache_cols=entry + [0, 0, 1, 4][ri(0, 3)],
                                 dst_cols=entry + [0, 0, 2, 4][ri(0, 3)], scale=[0.0625, 0.05][ri(0, 1)],
                                 allow_alias=alias, cache_dtype=cache_dtype)
    total = int(wl.cu_seq_lens[-1])
    if ri(0, 4) == 0 and total > 0:
        T = ri(0, total)
        wl.num_tokens = T
        wl.workspace = wl.workspace[: max(T, 1)].clone()
    if ri(0, 4) == 0:
        wl = wl.open_ended()
    if ri(0, 2) == 0 and wl.block_table.numel() > 0:
        flat = wl.block_table.view(-1)
        for _ in range(ri(1, 5)):
            flat[ri(0, flat.numel() - 1)] = [nb, nb + 9, -1][ri(0, 2)]
    return wl


@pytest.mark.parametrize("seed", range(24))
def test_medium_random(seed):
    check_parity(medium_random_workload(seed), DEV)


def dense_random_workload(seed: int) -> workloads.Workload:
    """A seeded batch whose lengths stay within 15% of each other, so its block
    table is about as wide as its pages and the batch is walked (the host's
    density rule decides; clamping, starts and narrow tables can tip it back):
    every page size from one token to 256, raw and fp8 kinds, strided rows,
    seq_starts, aliased blocks, guard-skipped pages, clamped and open-ended
    extents, batches past the fused limit."""
    g = torch.Generator("cpu").manual_seed(seed)
    ri = lambda lo, hi: int(torch.randint(lo, hi + 1, (1,), generator=g))
    kind = [workloads.RAW, workloads.DEQUANT_FP8, workloads.UPCONVERT, workloads.DEQUANT_AUTO][seed % 4]
    R = [2, 5, 16, 64, 100, 700, 1500][ri(0, 6)]
    bs = [1, 2, 4, 16, 64, 256][ri(0, 5)]
    entry = [64, 136, 576][ri(0, 2)]
    base = max(ri(1, 60_000 // R), 1)
    lens = [max(base + ri(-base // 8, base // 8), 0) for _ in range(R)]
    starts = [ri(0, min(n // 8, 3 * bs)) for n in lens] if ri(0, 1) else None
    pages = sum(-(-n // bs) for n in lens)
    alias = ri(0, 4) == 0
    nb = pages + ri(0, 8) if not alias else max([-(-n // bs) for n in lens] + [1]) + 3
    wl = workloads.make_workload(f"dense_{seed}", kind, lens, bs, entry, max(nb, 1), seed=seed + 91,
                                 starts=starts, cache_cols=entry + [0, 0, 1, 4][ri(0, 3)],
                                 dst_cols=entry + [0, 0, 2][ri(0, 2)], scale=[0.0625, 0.05][ri(0, 1)],
                                 allow_alias=alias)
    total = int(wl.cu_seq_lens[-1])
    if ri(0, 5) == 0 and total > 0:
        T = ri(total * 4 // 5, total)
        wl.num_tokens = T
        wl.workspace = wl.workspace[: max(T, 1)].clone()
    if ri(0, 4) == 0:
        wl = wl.open_ended()
    if ri(0, 2) == 0 and wl.block_table.numel() > 0:
        flat = wl.block_table.view(-1)
        for _ in range(ri(1, 5)):
            flat[ri(0, flat.numel() - 1)] = [wl.num_blocks, wl.num_blocks + 9, -1][ri(0, 2)]
    return wl


@pytest.mark.parametrize("seed", range(40))
def test_dense_random(seed):
    wl = dense_random_workload(30000 + seed)
    log(f"[dense] seed {30000 + seed}: mode {plan_of(wl.to(DEV))['task_mode']}")
    check_parity(wl, DEV)


def page_size_random_workload(seed: int) -> workloads.Workload:
    """A seeded batch over the whole page-size range: block sizes from 1 to
    1,000 tokens and rows from 1 element to 1,000, so that pages go whole,
    split into parts or grouped (every task path for each), with every element
    size, padded rows, seq_starts, clamped and open-ended extents and guard-
    skipped pages."""
    g = torch.Generator("cpu").manual_seed(seed)
    ri = lambda lo, hi: int(torch.randint(lo, hi + 1, (1,), generator=g))
    kind = [workloads.RAW, workloads.DEQUANT_FP8, workloads.UPCONVERT, workloads.DEQUANT_AUTO][seed % 4]
    R = [1, 1, 2, 9, 64, 65, 300, 1100][ri(0, 7)]
    bs = [1, 2, 3, 4, 5, 7, 8, 16, 24, 64, 96, 128, 256, 1000][ri(0, 13)]
    entry = [1, 2, 7, 16, 64, 136, 576, 1000][ri(0, 7)]
    cache_dtype = [torch.bfloat16, torch.float32, torch.uint8][ri(0, 2)]
    max_tokens = max(24_000 // R, 2)
    lens = [0 if ri(0, 9) == 0 else ri(1, max_tokens) for _ in range(R)]
    starts = [ri(0, n // 2) for n in lens] if ri(0, 1) else None
    pages = sum(-(-n // bs) for n in lens)
    wl = workloads.make_workload(f"page_size_{seed}", kind, lens, bs, entry, max(pages, 1) + ri(0, 5),
                                 seed=seed + 31, starts=starts, cache_cols=entry + [0, 0, 1, 3][ri(0, 3)],
                                 dst_cols=entry + [0, 0, 2, 4][ri(0, 3)], scale=0.05, cache_dtype=cache_dtype)
    total = int(wl.cu_seq_lens[-1])
    if ri(0, 4) == 0 and total > 0:
        T = ri(0, total)
        wl.num_tokens = T
        wl.workspace = wl.workspace[: max(T, 1)].clone()
    if ri(0, 4) == 0:
        wl = wl.open_ended()
    if ri(0, 2) == 0 and wl.block_table.numel() > 0:
        flat = wl.block_table.view(-1)
        for _ in range(ri(1, 9)):
            flat[ri(0, flat.numel() - 1)] = [wl.num_blocks, -1, 1 << 29][ri(0, 2)]
    return wl


@pytest.mark.parametrize("seed", range(40))
def test_random_page_sizes(seed):
    check_parity(page_size_random_workload(5000 + seed), DEV)


# ---------------------------------------------------------------------------
# task-unit rules by batch size, each case pinned to its plan, with seq_starts,
# zero-length requests, partial pages and guard-skipped pages
# ---------------------------------------------------------------------------

def sparse_width(lens, bs):
    """A block-table width four times the longest request's pages (plus 8): far
    from dense, so a batch takes a prefix mode rather than the table walk."""
    return 4 * max([-(-n // bs) for n in lens] + [1]) + 8


@pytest.mark.parametrize("name,kind,R,bs,mode,unit,split,group", [
    # at most 64 requests and fewer than 1024 whole-page tasks: raw 9 KiB units
    ("small_batch_raw", workloads.RAW, 8, 64, "wave", 8, 3, 0),
    ("small_batch_raw_big_pages", workloads.RAW, 5, 1024, "wave", 8, 7, 0),
    # ... fp8 keeps whole pages
    ("small_batch_fp8", workloads.UPCONVERT, 8, 64, "wave", 64, 0, 0),
    # more than 64 requests: 18 KiB units, raw and fp8 (LDS prefix and task table)
    ("lds_batch_raw", workloads.RAW, 65, 64, "lds", 16, 2, 0),
    ("lds_batch_fp8", workloads.DEQUANT_FP8, 200, 64, "lds", 16, 2, 0),
    ("table_batch_fp8", workloads.UPCONVERT, 1100, 64, "table", 16, 2, 0),
    # small pages of batches: 18 KiB groups
    ("lds_batch_groups", workloads.RAW, 300, 1, "lds", 16, 0, 4),
    ("wave_batch_groups", workloads.RAW, 20, 2, "wave", 16, 0, 3),
])
def test_batch_unit_rules(name, kind, R, bs, mode, unit, split, group):
    g = torch.Generator("cpu").manual_seed(len(name) * 1000 + R)
    ri = lambda lo, hi: int(torch.randint(lo, hi + 1, (1,), generator=g))
    max_tokens = max(30_000 // R, 40)
    lens = [0 if ri(0, 7) == 0 else ri(1, max_tokens) for _ in range(R)]
    starts = [ri(0, n // 3) for n in lens]
    pages = sum(-(-n // bs) for n in lens)
    # a table four times wider than the longest request: the prefix modes, not the walk
    wl = workloads.make_workload(name, kind, lens, bs, 576, pages + 7, seed=R + bs, starts=starts,
                                 scale=0.05, width=sparse_width(lens, bs))
    flat = wl.block_table.view(-1)
    for _ in range(5):  # guard-skipped pages: past the cache, negative
        flat[ri(0, flat.numel() - 1)] = [wl.num_blocks, -1][ri(0, 1)]
    p = plan_of(wl.to(DEV))
    modes = {"wave": pkvg.PKVG_TASKS_WAVE, "lds": pkvg.PKVG_TASKS_LDS, "table": pkvg.PKVG_TASKS_TABLE}
    assert (p["task_mode"], p["task_tokens"], p["split_shift"], p["group_shift"]) == (
        modes[mode], unit, split, group), p
    check_parity(wl, DEV)


@pytest.mark.parametrize("R", [256, 257, 512, 513])
@pytest.mark.parametrize("kind", [workloads.RAW, workloads.UPCONVERT])
def test_lds_prefix_share_boundaries(R, kind):
    """The LDS prefix gives each of a workgroup's 256 lanes 1, 2 or 4 requests,
    the smallest share that covers the batch: batches on both sides of each
    switch, with seq_starts, zero-length requests and guard-skipped pages."""
    g = torch.Generator("cpu").manual_seed(R * 10 + len(kind))
    ri = lambda lo, hi: int(torch.randint(lo, hi + 1, (1,), generator=g))
    lens = [0 if ri(0, 6) == 0 else ri(1, 300) for _ in range(R)]
    starts = [ri(0, n // 3) for n in lens]
    pages = sum(-(-n // 16) for n in lens)
    wl = workloads.make_workload(f"lds_share_{R}_{kind}", kind, lens, 16, 576, pages + 5, seed=R,
                                 starts=starts, scale=0.05, width=sparse_width(lens, 16))
    flat = wl.block_table.view(-1)
    for _ in range(4):
        flat[ri(0, flat.numel() - 1)] = [wl.num_blocks, -1][ri(0, 1)]
    assert plan_of(wl.to(DEV))["task_mode"] == pkvg.PKVG_TASKS_LDS
    check_parity(wl, DEV)


@pytest.mark.parametrize("block", range(10))
def test_random_sweep(block):
    """Both random generators above at 15 more seeds per block (300 cases in
    all): every task path, unit rule, access width and edge case, many times."""
    for seed in range(20000 + 15 * block, 20000 + 15 * (block + 1)):
        check_parity(medium_random_workload(seed), DEV)
        check_parity(page_size_random_workload(seed), DEV)


# ---------------------------------------------------------------------------
# the fp8 arithmetic on every code, NaN codes included
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("scale", [0.0625, 0.05, 1.0, 9.7, 0.5395833253860474, -3.0, 1e-38,
                                   1.7e38, 7.62939453125e-06])
def test_fp8_every_code(scale):
    """One block holds all 256 codes; compare with the oracle element by element
    (bit-exact), NaN codes only for NaN-ness."""
    import paged_kv_cache_device_amd as pkvg

    log(f"[fp8 codes] scale={scale}")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(1, 4, 64)  # 1 block, bs 4
    bt = torch.tensor([[0]], dtype=torch.int32)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    sc = torch.tensor([scale], dtype=torch.float32)
    dst = torch.full((4, 64), -1, dtype=torch.int16).view(torch.bfloat16)
    o = oracle.load()
    want = torch.tensor([o.dequant_e4m3fn_bf16(c, scale) for c in range(256)], dtype=torch.int32)
    nan = torch.tensor([c in (0x7F, 0xFF) for c in range(256)])
    # the cache as raw bytes and as torch's float8_e4m3fn (same bits), through both fp8 calls
    for cache in (codes.to(DEV), codes.to(DEV).view(torch.float8_e4m3fn)):
        for call in ("upconvert", "maybe_dequant"):
            d = dst.to(DEV)
            if call == "upconvert":
                pkvg.gather_upconvert_fp8(cache, d, bt.to(DEV), cu.to(DEV), 1, sc.to(DEV))
            else:
                pkvg.gather_maybe_dequant(cache, d, bt.to(DEV), cu.to(DEV), 1, "fp8", sc.to(DEV))
            torch.cuda.synchronize()
            got = d.cpu().view(torch.int16).flatten().to(torch.int32) & 0xFFFF
            assert torch.equal(got[~nan], want[~nan]), (call, cache.dtype,
                                                        (got[~nan] != want[~nan]).nonzero().flatten()[:8])
            assert torch.isnan(d.cpu().flatten().float()[nan]).all()


# ---------------------------------------------------------------------------
# the page-task builder on its own
# ---------------------------------------------------------------------------

def test_page_tasks_match_oracle():
    import paged_kv_cache_device_amd as pkvg

    o = oracle.load()
    g = torch.Generator("cpu").manual_seed(5)
    for k in range(40):
        R = int(torch.randint(1, 40 if k % 4 else 1500, (1,), generator=g))
        bs = [1, 2, 16, 64][k % 4]
        lens = torch.randint(0, 4 * bs + 3, (R,), generator=g)
        lens[torch.rand(R, generator=g) < 0.2] = 0
        starts = torch.randint(0, 3 * bs, (R,), generator=g) if k % 2 else None
        cu = torch.cat([torch.zeros(1, dtype=torch.int64), lens.cumsum(0)]).to(torch.int32)
        T = int(cu[-1]) if k % 3 else int(cu[-1]) // 2
        W = int(((starts if starts is not None else 0) + lens).max()) // bs + 1
        nb = 50
        bt = torch.randint(-2, nb + 3, (R, W + 2), generator=g, dtype=torch.int32)
        log(f"[page tasks] case {k} R={R} bs={bs} T={T} starts={starts is not None}")
        want = o.page_tasks(cu, None if starts is None else starts.to(torch.int32), R, T, bs)
        tasks, count = pkvg.gather_page_tasks(
            cu.to(DEV), None if starts is None else starts.to(torch.int32).to(DEV), R, T, bs,
            bt.to(DEV)[:, :W], nb)
        torch.cuda.synchronize()
        n = int(count.item())
        got = tasks[:n].cpu().numpy()
        assert n == len(want), (k, n, len(want))
        assert np.array_equal(got[:, :5], want), k
        btn = bt.numpy()
        for row in got:
            r, lb = row[0], row[1]
            phys = btn[r, lb] if lb < W else -1
            phys = phys if 0 <= phys < nb else -1
            assert row[5] == phys


# ---------------------------------------------------------------------------
# no work, block table pitch, byte offsets beyond 2^31
# ---------------------------------------------------------------------------

def test_no_work_leaves_destination_untouched():
    import paged_kv_cache_device_amd as pkvg

    cache = torch.randn(4, 16, 8).to(torch.bfloat16).to(DEV)
    ws = torch.full((10, 8), 7.0, dtype=torch.bfloat16, device=DEV)
    bt = torch.zeros(1, 2, dtype=torch.int32, device=DEV)
    cu = torch.tensor([0, 10], dtype=torch.int32, device=DEV)
    pkvg.gather_cache(cache, ws[:0], bt, cu, 1)          # num_tokens == 0
    pkvg.gather_cache(cache, ws, bt, cu, 0)              # num_reqs == 0
    torch.cuda.synchronize()
    assert bool((ws == 7.0).all())


def test_block_table_row_pitch():
    """A block table that is a column slice of a wider table (row pitch > width)."""
    import paged_kv_cache_device_amd as pkvg

    wl = workloads.make_workload("pitch", workloads.RAW, [40, 70, 5], 16, 64, 20, seed=3,
                                 width=5)
    want, _ = oracle.run_workload(wl)
    wide = torch.full((3, 9), 12345, dtype=torch.int32)
    wide[:, :5] = wl.block_table
    g = wl.to(DEV)
    ws = g.fresh_workspace()
    pkvg.gather_cache(g.src_cache(), ws[: g.num_tokens, : g.entry], wide.to(DEV)[:, :5],
                      g.cu_seq_lens, 3, None)
    torch.cuda.synchronize()
    assert torch.equal(ws.cpu().view(torch.uint8), want.view(torch.uint8))


def test_offsets_beyond_2_to_31_bytes():
    """One request of 1,000,000 tokens of fp32 entries (2304-byte rows): output row
    offsets and physical page offsets both pass 2^31 bytes (the int32 product
    the page's review flags would overflow near 932K tokens)."""
    import paged_kv_cache_device_amd as pkvg

    T, bs, entry = 1_000_000, 64, 576
    nb = T // bs + 1 + 40
    log(f"[int64] T={T} bytes per side ~{T * entry * 4 / 2**30:.2f} GiB")
    g = torch.Generator("cpu").manual_seed(64)
    perm = torch.randperm(nb, generator=g).to(torch.int32)
    pages = -(-T // bs)
    bt = perm[:pages].view(1, pages).contiguous()
    # self-identifying fp32 bit patterns, generated on the device
    ids = ((torch.arange(nb, device=DEV, dtype=torch.int32).view(nb, 1, 1) << 16)
           | (torch.arange(bs, device=DEV, dtype=torch.int32).view(1, bs, 1) << 10)
           | torch.arange(entry, device=DEV, dtype=torch.int32).view(1, 1, entry))
    cache = ids.view(torch.float32)
    ws = torch.full((T + 2, entry), -1, dtype=torch.int32, device=DEV).view(torch.float32)
    cu = torch.tensor([0, T], dtype=torch.int32)
    pkvg.gather_cache(cache, ws[:T], bt.to(DEV), cu.to(DEV), 1, None)
    torch.cuda.synchronize()
    got = ws.cpu()
    del ws
    want = torch.full((T + 2, entry), -1, dtype=torch.int32).view(torch.float32)
    o = oracle.load()
    rows = o.gather_tensors(oracle.MODE_COPY, cache.cpu(), want[:T], bt, cu, None, 1)
    assert rows == T
    assert torch.equal(got.view(torch.int32), want.view(torch.int32))


def test_fp8_offsets_beyond_2_to_31_bytes():
    """The fp8 flat path (wide shape, write-through stores through a buffer
    resource based at each page's first output row): 2,000,000 tokens of 576
    codes write 2.3 GB of bf16, so page bases pass 2^31 bytes."""
    import paged_kv_cache_device_amd as pkvg

    T, bs, entry = 2_000_000, 64, 576
    nb = T // bs + 1 + 40
    log(f"[int64 fp8] T={T} output ~{T * entry * 2 / 2**30:.2f} GiB")
    g = torch.Generator("cpu").manual_seed(65)
    perm = torch.randperm(nb, generator=g).to(torch.int32)
    pages = -(-T // bs)
    bt = perm[:pages].view(1, pages).contiguous()
    gd = torch.Generator(DEV).manual_seed(66)
    codes = torch.randint(0, 256, (nb, bs, entry), dtype=torch.uint8, device=DEV, generator=gd)
    codes[(codes & 0x7F) == 0x7F] -= 1  # no NaN codes
    scale = torch.tensor([0.0625], dtype=torch.float32)
    ws = torch.full((T + 2, entry), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    cu = torch.tensor([0, T], dtype=torch.int32)
    pkvg.gather_upconvert_fp8(codes, ws[:T], bt.to(DEV), cu.to(DEV), 1, scale.to(DEV), None)
    torch.cuda.synchronize()
    got = ws.cpu()
    del ws
    want = torch.full((T + 2, entry), -1, dtype=torch.int16).view(torch.bfloat16)
    rows = oracle.load().gather_tensors(oracle.MODE_E4M3FN_TO_BF16, codes.cpu(), want[:T], bt, cu, None, 1,
                                        float(scale[0]))
    assert rows == T
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))


# ---------------------------------------------------------------------------
# one request: the path that requests the first block-table entry early
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("tokens,start,bs,kind", [
    (61440, 0, 64, workloads.RAW),            # narrow shape, whole pages
    (5000, 37, 16, workloads.RAW),            # partial first and last pages
    (130000, 1000, 64, workloads.UPCONVERT),  # wide shape (>= 1024 pages)
    (70000, 63, 64, workloads.DEQUANT_FP8),
])
def test_single_request(tokens, start, bs, kind):
    wl = workloads.make_workload(f"single_{tokens}_{start}", kind, [tokens], bs, 576,
                                 -(-tokens // bs) + 9, seed=tokens, starts=[start], scale=0.05)
    check_parity(wl, DEV)
    # guards on the single-request path: a hole in the table, an id past the
    # cache, and a table narrower than the request
    bt = wl.block_table
    bt[0, 1] = -1
    bt[0, 2] = wl.num_blocks + 3
    wl.block_table = bt[:, : bt.shape[1] - 2].contiguous()
    check_parity(wl, DEV)
    # fewer destination rows than the request's extent
    wl.num_tokens = tokens // 3
    wl.workspace = wl.workspace[: tokens // 3 + 5].clone()
    check_parity(wl, DEV)


@pytest.mark.parametrize("bs", [64, 128, 24, 40, 1000])
def test_single_request_units(bs):
    """One request's raw pages move as units of at most 9 KiB (1152-byte rows:
    8 tokens of a 64-token page, 6 of a 24-token page, 5 of a 40-token page,
    125 of a 1,000-token page after three halvings): seq_starts on and beside
    unit and page boundaries, a table narrower than the request, holes."""
    for start in (1, 4, 5, 6, 7, 8, 9, bs - 1, bs, bs + 1, 3 * bs + 5):
        wl = workloads.make_workload(f"units_{bs}_{start}", workloads.RAW, [start + 3000 + bs // 3], bs, 576,
                                     -(-(start + 3000 + bs) // bs) + 4, seed=bs * 100 + start, starts=[start])
        check_parity(wl, DEV)
    check_parity(_with_holes(wl, bs), DEV)


@pytest.mark.parametrize("kind", [workloads.RAW, workloads.UPCONVERT])
def test_single_request_prologue_edges(kind):
    """The single-request prologue reads its three metadata values without a
    branch: no seq_starts with a partial last page, a request whose first
    output row is not 0, a start past the end of the table row, and a table
    with no columns (never read; torch passes a null pointer for it)."""
    mk = lambda name, **kw: workloads.make_workload(name, kind, [5000], 16, 576, 330, seed=77,
                                                    scale=0.05, **kw)
    check_parity(mk("single_no_starts_partial"), DEV)
    wl = mk("single_offset_rows", workspace_rows=5000 + 40)
    wl.cu_seq_lens = torch.tensor([23, 23 + 5000], dtype=torch.int32)
    wl.num_tokens = 5000 + 23
    check_parity(wl, DEV)
    wl.num_tokens = 2000  # the extent clamps to the destination
    check_parity(wl, DEV)
    wl = mk("single_start_past_table", starts=[4000])
    wl.block_table = wl.block_table[:, :100].contiguous()  # pages 250.. lie past the row
    check_parity(wl, DEV)
    wl = mk("single_empty_table")
    wl.block_table = wl.block_table[:, :0].contiguous()
    check_parity(wl, DEV)


@pytest.mark.parametrize("R", [3, 100, 1500])
def test_empty_block_table(R):
    """A table with no columns on the batched paths (wave registers, LDS
    prefix, prebuilt task table): every page is skipped, nothing is written."""
    lens = [(37 * r) % 300 for r in range(R)]
    wl = workloads.make_workload(f"empty_table_{R}", workloads.RAW, lens, 16, 64, sum(lens) // 16 + 2 * R,
                                 seed=R)
    wl.block_table = wl.block_table[:, :0].contiguous()
    check_parity(wl, DEV)


# ---------------------------------------------------------------------------
# capture in a HIP graph: every replay recomputes from the current inputs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("entry", [64, 576])
@pytest.mark.parametrize("kind,R", [(workloads.RAW, 1), (workloads.UPCONVERT, 5),
                                    (workloads.DEQUANT_FP8, 100), (workloads.RAW, 1500)])
def test_graph_replays(kind, R, entry):
    """The calls enqueue only kernel launches (up to 1024 requests) or kernel
    launches between a stream-ordered allocation and its free (more requests),
    and no memset, so they can be captured.  Between replays the cache
    contents change and eager work runs; each replay must match the oracle on
    the inputs of that moment.  16-token pages of 64-element rows go to the
    group kernel, of 576-element rows to the page kernel."""
    import paged_kv_cache_device_amd as pkvg

    g = torch.Generator("cpu").manual_seed(R)
    lens = torch.randint(1, 300, (R,), generator=g).tolist()
    starts = [int(torch.randint(0, n + 1, (1,), generator=g)) for n in lens]
    wl = workloads.make_workload(f"graph_{kind}_{R}_{entry}", kind, lens, 16, entry,
                                 sum(-(-n // 16) for n in lens) + 2, seed=R, starts=starts,
                                 scale=0.05, workspace_rows=sum(lens) + 4)
    d = wl.to(DEV)
    ws = d.fresh_workspace()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            if kind == workloads.RAW:
                pkvg.gather_cache(d.src_cache(), ws[: d.num_tokens, : d.entry], d.block_table,
                                  d.cu_seq_lens, R, d.seq_starts)
            elif kind == workloads.UPCONVERT:
                pkvg.gather_upconvert_fp8(d.src_cache(), ws[: d.num_tokens, : d.entry],
                                          d.block_table, d.cu_seq_lens, R, d.scale_tensor,
                                          d.seq_starts)
            else:
                pkvg.gather_maybe_dequant(d.src_cache(), ws[: d.num_tokens, : d.entry],
                                          d.block_table, d.cu_seq_lens, R, "fp8", d.scale_tensor,
                                          d.seq_starts)
    torch.cuda.synchronize()
    for rep in range(4):
        log(f"[graph] {kind} R={R} replay {rep}")
        # new cache contents in place (the graph holds the same pointers)
        fresh = workloads.make_workload("tmp", kind, lens, 16, entry, wl.num_blocks, seed=100 + rep,
                                        starts=starts, scale=0.05)
        wl.cache_base.copy_(fresh.cache_base)
        d.cache_base.copy_(fresh.cache_base)
        ws.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        _ = (d.cache_base.float().sum() if d.cache_base.is_floating_point() else d.cache_base.sum())
        torch.cuda.synchronize()
        want, _ = oracle.run_workload(wl, ws=torch.full_like(wl.workspace, -1.0))
        assert torch.equal(ws.cpu().view(torch.uint8), want.view(torch.uint8)), rep


# ---------------------------------------------------------------------------
# the open-ended cu_seq_lens convention (no terminal entry)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("entry", [64, 576])
@pytest.mark.parametrize("R,kind", [(1, workloads.RAW), (7, workloads.UPCONVERT),
                                    (200, workloads.DEQUANT_FP8), (1500, workloads.RAW)])
def test_open_ended_cu_seq_lens(R, kind, entry):
    """cu_seq_lens holds only the R starts; the last request runs to num_tokens.
    On the device the array is followed by a poisoned entry, so a kernel that
    read a terminal entry would write the wrong rows.  Covers the single-request,
    wave-register, LDS-prefix and task-table paths, in the group kernel (64-
    element rows) and the page kernel (576-element rows)."""
    import paged_kv_cache_device_amd as pkvg

    g = torch.Generator("cpu").manual_seed(R + 7)
    lens = torch.randint(1, 200, (R,), generator=g).tolist()
    starts = [int(torch.randint(0, n + 1, (1,), generator=g)) for n in lens]
    wl = workloads.make_workload(f"open_{R}_{kind}_{entry}", kind, lens, 16, entry,
                                 sum(-(-n // 16) for n in lens) + 2, seed=R, starts=starts,
                                 scale=0.05, workspace_rows=sum(lens) + 8).open_ended()
    want, _ = oracle.run_workload(wl)
    for poison in (0, 1 << 30):
        log(f"[open-ended] R={R} kind={kind} poison={poison}")
        d = wl.to(DEV)
        padded = torch.full((R + 1,), poison, dtype=torch.int32, device=DEV)
        padded[:R] = d.cu_seq_lens
        d.cu_seq_lens = padded[:R]
        ws = run_hip(d)
        torch.cuda.synchronize()
        assert torch.equal(ws.cpu().view(torch.uint8), want.view(torch.uint8))
    # the builder alone, against the oracle's task list in the same convention
    o = oracle.load()
    tw = o.page_tasks(wl.cu_seq_lens, wl.seq_starts, R, wl.num_tokens, 16, terminal=False)
    d = wl.to(DEV)
    tasks, count = pkvg.gather_page_tasks(d.cu_seq_lens, d.seq_starts, R, wl.num_tokens, 16,
                                          d.block_table, wl.num_blocks)
    torch.cuda.synchronize()
    n = int(count.item())
    assert n == len(tw)
    assert np.array_equal(tasks[:n].cpu().numpy()[:, :5], tw)


# ---------------------------------------------------------------------------
# calls from several host threads at once, each on its own stream
# ---------------------------------------------------------------------------

def test_concurrent_calls_from_threads():
    """The library keeps no shared mutable state (its error slot is per thread):
    eight threads, each on its own stream, run different gathers repeatedly
    and every result matches the oracle."""
    import threading

    cases = []
    for i, (kind, lens) in enumerate([(workloads.RAW, [700, 0, 33]), (workloads.UPCONVERT, [5000]),
                                      (workloads.DEQUANT_FP8, [17] * 80), (workloads.RAW, [9] * 1200),
                                      (workloads.RAW, [4096]), (workloads.UPCONVERT, [100, 200, 300]),
                                      (workloads.DEQUANT_AUTO, [257, 64]), (workloads.DEQUANT_FP8, [31] * 1100)]):
        wl = workloads.make_workload(f"threads_{i}", kind, lens, 16, 64, sum(-(-n // 16) for n in lens) + 3,
                                     seed=500 + i, scale=0.05)
        want, _ = oracle.run_workload(wl)
        cases.append((wl.to(DEV), want))
    errors = []

    def worker(idx):
        try:
            d, want = cases[idx]
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for _ in range(20):
                    ws = d.fresh_workspace()
                    run_hip(d, ws)
                stream.synchronize()
            if not torch.equal(ws.cpu().view(torch.uint8), want.view(torch.uint8)):
                errors.append(f"case {idx}: " + byte_diff(ws.cpu(), want))
        except Exception as e:  # reported below with the case that raised
            errors.append(f"case {idx}: {e!r}")

    log("[threads] 8 threads x 20 calls")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors


# ---------------------------------------------------------------------------
# batches walked straight through a dense block table
# ---------------------------------------------------------------------------

def _walk_cases():
    W = workloads
    g = torch.Generator("cpu").manual_seed(31)
    cases = []
    # the single-60K bytes over 8 requests (raw), with starts, and fp8 / strided fp8
    cases.append(W.make_workload("walk_8x7680", W.RAW, [7680] * 8, 64, 576, 1000, seed=41))
    lens = [300] * 10
    starts = [int(torch.randint(0, 100, (1,), generator=g)) for _ in lens]
    cases.append(W.make_workload("walk_starts", W.RAW, lens, 16, 64, 250, seed=42, starts=starts))
    cases.append(W.make_workload("walk_fp8", W.UPCONVERT, [500, 480, 499, 470], 16, 576, 140, seed=43,
                                 starts=[7, 0, 16, 33], scale=0.0625))
    cases.append(W.make_workload("walk_fp8_strided", W.DEQUANT_FP8, [200] * 20, 64, 576, 90, seed=44,
                                 cache_cols=577, dst_cols=580, scale=0.05, workspace_rows=4004))
    cases.append(W.make_workload("walk_auto", W.DEQUANT_AUTO, [129] * 40, 32, 576, 200, seed=45))
    # one-token pages through the group kernel, raw and fp8
    cases.append(W.make_workload("walk_bs1", W.RAW, [200] * 64, 1, 576, 12900, seed=46))
    cases.append(W.make_workload("walk_bs1_fp8", W.UPCONVERT, [100] * 30, 1, 576, 3010, seed=47,
                                 starts=[3] * 30, scale=0.05))
    cases.append(W.make_workload("walk_bs2", W.RAW, [64, 65, 63, 60] * 16, 2, 64, 2200, seed=48))
    # beyond the fused batch limit: walked without a task table
    cases.append(W.make_workload("walk_1500", W.RAW, [40] * 1500, 16, 64, 4600, seed=49))
    # num_tokens cuts the batch short; open-ended cu_seq_lens; guard-failing entries
    wl = W.make_workload("walk_clamped", W.RAW, [64] * 12, 16, 64, 60, seed=50, workspace_rows=768)
    wl.num_tokens = 500
    cases.append(wl)
    cases.append(W.make_workload("walk_open", W.RAW, [70] * 6, 16, 64, 40, seed=51,
                                 workspace_rows=430).open_ended())
    wl = W.make_workload("walk_guards", W.UPCONVERT, [90] * 9, 16, 64, 60, seed=52, scale=0.05)
    flat = wl.block_table.view(-1)
    flat[3], flat[17], flat[30] = -1, wl.num_blocks, wl.num_blocks + 4
    cases.append(wl)
    return cases


@pytest.mark.parametrize("idx", range(12))
def test_walk_mode_parity(idx):
    wl = _walk_cases()[idx]
    plan = plan_of(wl.to(DEV))
    assert plan["task_mode"] == pkvg.PKVG_TASKS_WALK, (wl.name, plan)
    check_parity(wl, DEV)
