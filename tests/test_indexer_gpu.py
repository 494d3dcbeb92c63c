"""Parity of the HIP indexer quant-cache gather (through the C ABI) with the
CPU oracle, byte for byte, on MI355X: the named indexer workloads at full
size, seeded random cases with every mask (padding rows, batch ids past the
batch count, rows outside their batch, narrowed tables, out-of-range blocks),
both record layouts, three head dimensions, 16-byte and byte-wise destination
rows, and block addresses past 2^31 bytes."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_device_amd as pkvg
import workloads
from gpu_util import log

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LAYOUT_NAMES = {workloads.INDEXER_LAYOUT_FLAT: "flat", workloads.INDEXER_LAYOUT_TILED: "tiled"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkvg.library()  # fail loudly if the HIP library is missing


def run_indexer_hip(iw_dev, values, scales):
    pkvg.gather_indexer_quant_cache(
        iw_dev.cache, iw_dev.dst_values(values), iw_dev.dst_scales(scales), iw_dev.token_to_seq,
        iw_dev.cu_seqlen, iw_dev.block_table, iw_dev.block_size, LAYOUT_NAMES[iw_dev.layout],
        block_tile=iw_dev.block_tile, head_tile=iw_dev.head_tile,
        block_table_width=iw_dev.block_table_width)


def check_indexer_parity(iw):
    log(f"[indexer parity] {iw.name} layout={iw.layout} T={iw.num_tokens} B={iw.num_batches} "
        f"bs={iw.block_size} hd={iw.head_dim} nb={iw.num_blocks} stride={iw.block_stride} "
        f"values={tuple(iw.values.shape)} scales={tuple(iw.scales.shape)}")
    want_v, want_s, _ = oracle.run_indexer_workload(iw)
    d = iw.to(DEV)
    got_v, got_s = d.fresh_values(), d.fresh_scales()
    run_indexer_hip(d, got_v, got_s)
    torch.cuda.synchronize()
    gv, gs = got_v.cpu(), got_s.cpu()
    bad_v = (gv != want_v).any(dim=1).nonzero().flatten()
    assert bad_v.numel() == 0, f"{iw.name}: value rows differ: {bad_v[:8].tolist()}"
    bad_s = (gs.view(torch.uint8) != want_s.view(torch.uint8)).any(dim=1).nonzero().flatten()
    assert bad_s.numel() == 0, f"{iw.name}: scale rows differ: {bad_s[:8].tolist()}"


@pytest.mark.parametrize("name", list(workloads.INDEXER_NAMED))
def test_indexer_named_workload_parity(name):
    check_indexer_parity(workloads.named(name))


def corrupt(iw, rng):
    """Masks of every kind: padding ids, ids past the batch count, a batch's
    first row claiming the previous batch, table entries out of range, and a
    narrowed table width."""
    t2s = iw.token_to_seq
    T, B = iw.num_tokens, iw.num_batches
    cu = iw.cu_seqlen.tolist()
    for _ in range(int(rng.integers(0, 5))):
        if T:
            t2s[int(rng.integers(0, T))] = int(rng.choice([-1, -9, B, B + 7]))
    for b in range(1, B):
        if cu[b + 1] > cu[b] and rng.random() < 0.5:
            t2s[cu[b]] = b - 1
    flat = iw.block_table.view(-1)
    for _ in range(int(rng.integers(0, 4))):
        if flat.numel():
            flat[int(rng.integers(0, flat.numel()))] = int(rng.choice([-1, -3, iw.num_blocks,
                                                                        iw.num_blocks + 11]))
    if rng.random() < 0.3 and iw.block_table.shape[1] > 1:
        iw.block_table_width = int(rng.integers(0, iw.block_table.shape[1]))
    return iw


@pytest.mark.parametrize("seed", range(8))
def test_indexer_random_small(seed):
    rng = np.random.default_rng(4000 + seed)
    for k in range(12):
        B = int(rng.integers(1, 9))
        layout = int(rng.integers(0, 2))
        bs = int(rng.choice([16, 32, 64])) if layout else int(rng.choice([1, 2, 7, 16, 64]))
        hd = int(rng.choice([64, 128, 256]))
        lens = rng.integers(0, 5 * bs + 3, size=B).tolist()
        lens = [0 if rng.random() < 0.15 else n for n in lens]
        pages = sum(-(-n // bs) for n in lens)
        iw = workloads.make_indexer_workload(
            f"ix_rand{seed}_{k}", lens, bs, hd, max(pages, 1) + int(rng.integers(0, 5)),
            seed=seed * 100 + k, layout=layout, record_pad=4 * int(rng.integers(0, 9)),
            pad_rows=int(rng.integers(0, 70)),
            value_cols=hd + int(rng.choice([0, 0, 1, 3, 16])),   # odd pitches: byte path
            scale_cols=int(rng.choice([1, 2, 3])), allow_alias=bool(rng.random() < 0.3))
        check_indexer_parity(corrupt(iw, rng))


def with_leading_rows(iw, lead: int, claim_first: bool):
    """``iw`` behind ``lead`` rows that belong to no batch: every batch extent
    moves down by ``lead`` (so cu_seqlen[0] == lead), and the new rows carry
    batch id -1, or 0 with ``claim_first`` (outside batch 0's extent, masked)."""
    sent = workloads.SENTINEL_BYTE
    head = torch.full((lead,), 0 if claim_first else -1, dtype=torch.int32)
    values = torch.cat([torch.full((lead, iw.values.shape[1]), sent, dtype=torch.uint8), iw.values])
    scales = torch.cat([torch.full((lead, iw.scales.shape[1] * 4), sent, dtype=torch.uint8).view(torch.float32),
                        iw.scales])
    return dataclasses.replace(iw, name=f"{iw.name}_lead{lead}", token_to_seq=torch.cat([head, iw.token_to_seq]),
                               cu_seqlen=iw.cu_seqlen + lead, num_tokens=iw.num_tokens + lead, values=values,
                               scales=scales)


@pytest.mark.parametrize("lead,claim_first", [(1, False), (63, True), (64, False), (100, True), (4097, False)])
@pytest.mark.parametrize("layout", [workloads.INDEXER_LAYOUT_FLAT, workloads.INDEXER_LAYOUT_TILED])
def test_indexer_first_batch_after_leading_rows(lead, claim_first, layout):
    """A first batch that starts after row 0 (cu_seqlen[0] > 0): row r of batch 0
    then lies at position r - cu_seqlen[0], not r, so the table column the kernel
    requests ahead for first-batch rows (r / block_size) is theirs only where the
    two columns coincide; every row must still take its own block."""
    iw = workloads.make_indexer_workload(f"ix_lead_{layout}", [5000, 700, 0, 300], 64, 128, 120,
                                         seed=4300 + lead, layout=layout, pad_rows=9)
    check_indexer_parity(with_leading_rows(iw, lead, claim_first))


@pytest.mark.parametrize("layout", [workloads.INDEXER_LAYOUT_FLAT, workloads.INDEXER_LAYOUT_TILED])
@pytest.mark.parametrize("hd", [64, 128, 256])
def test_indexer_head_dims(layout, hd):
    """Each structural instantiation, with a batch spanning several workgroups
    and a ragged tail (rows past the last full wave)."""
    lens = [3000, 17, 0, 1290, 64]
    pages = sum(-(-n // 64) for n in lens)
    iw = workloads.make_indexer_workload(f"ix_hd{hd}_{layout}", lens, 64, hd, pages + 9,
                                         seed=hd + layout, layout=layout, pad_rows=37)
    check_indexer_parity(iw)


def test_indexer_empty_and_single_row():
    for lens, pad in (([1], 0), ([0], 3), ([0, 0, 5], 0), ([63], 1), ([64], 0), ([65], 0)):
        iw = workloads.make_indexer_workload(f"ix_small_{lens}_{pad}", lens, 16, 128, 8, seed=7,
                                             pad_rows=pad)
        if iw.num_tokens == 0:
            continue
        check_indexer_parity(iw)


def test_indexer_no_work_launches_nothing():
    """num_tokens == 0 and num_batches == 0 return at once; the destination is untouched."""
    iw = workloads.make_indexer_workload("ix_nowork", [5, 3], 16, 128, 4, seed=9).to(DEV)
    v, s = iw.fresh_values(), iw.fresh_scales()
    pkvg.gather_indexer_quant_cache(iw.cache, iw.dst_values(v)[:0], iw.dst_scales(s)[:0],
                                    iw.token_to_seq, iw.cu_seqlen, iw.block_table, 16)
    pkvg.gather_indexer_quant_cache(iw.cache, iw.dst_values(v), iw.dst_scales(s), iw.token_to_seq,
                                    iw.cu_seqlen[:1], iw.block_table[:0], 16, num_batches=0)
    torch.cuda.synchronize()
    assert bool((v == workloads.SENTINEL_BYTE).all())
    assert bool((s.view(torch.uint8) == workloads.SENTINEL_BYTE).all())


def test_indexer_block_addresses_beyond_2_to_31():
    """Records of 96 MiB: block ids above 21 put a record past 2^31 bytes, so
    the clamp-then-widen addressing must be 64-bit.  The device cache holds
    only seeded bytes in the records the table names; the oracle runs on a
    compact copy of exactly those records with the table renumbered, which
    gathers the same bytes."""
    bs, hd = 64, 128
    stride = 96 << 20
    nb = 26
    lens = [200, 130, 100]
    g = torch.Generator("cpu").manual_seed(77)
    iw = workloads.make_indexer_workload("ix_big_small", lens, bs, hd, 16, seed=78, pad_rows=3)
    # the table names high blocks 20 .. 25, one id past the cache (26) and
    # unused slots (-1): batch 0 reads 3 of its 4 pages, batch 1 2 of 3, batch 2 1 of 2
    used = [25, 21, 22, 24, 20, 23, 26]
    bt = torch.tensor([[used[0], used[1], used[2], -1], [used[3], used[4], -1, -1],
                       [used[5], used[6], -1, -1]], dtype=torch.int32)
    cache_dev = torch.empty((nb, stride), dtype=torch.uint8, device=DEV)
    compact = torch.randint(0, 256, (len(used), stride), generator=g, dtype=torch.uint8)
    for i, blk in enumerate(used):
        if blk < nb:
            cache_dev[blk].copy_(compact[i].to(DEV))
    log(f"[indexer parity] 64-bit records: nb={nb} stride={stride} bytes={nb * stride}")
    # oracle on the compact cache (renumbered table: entry i for block used[i];
    # the out-of-range id stays out of range)
    small = workloads.make_indexer_workload("ix_big_small", lens, bs, hd, 16, seed=78,
                                            pad_rows=3)
    small.cache = compact
    remap = {blk: i for i, blk in enumerate(used) if blk < nb}
    small.block_table = torch.tensor([[remap.get(int(x), len(used) + 5) if x >= 0 else -1
                                       for x in row] for row in bt.tolist()], dtype=torch.int32)
    small.block_table_width = 4
    want_v, want_s, rows = oracle.run_indexer_workload(small)
    assert rows == 192 + 128 + 64
    d = iw.to(DEV)
    d.cache = cache_dev
    d.block_table = bt.to(DEV)
    d.block_table_width = 4
    got_v, got_s = d.fresh_values(), d.fresh_scales()
    run_indexer_hip(d, got_v, got_s)
    torch.cuda.synchronize()
    assert torch.equal(got_v.cpu(), want_v)
    assert torch.equal(got_s.cpu().view(torch.uint8), want_s.view(torch.uint8))


@pytest.mark.parametrize("B", [63, 64, 100, 4095, 4096, 6000])
def test_indexer_many_batches(B):
    """Batch extents from wave registers (up to 63 batches) and from per-row
    loads (more): both sides of the switch and batch counts far past it, with
    rows claiming other batches and padding rows."""
    rng = np.random.default_rng(B)
    lens = rng.integers(0, 40, size=B).tolist()
    pages = sum(-(-n // 16) for n in lens)
    iw = workloads.make_indexer_workload(f"ix_batches_{B}", lens, 16, 128, pages + 7, seed=B,
                                         pad_rows=13, layout=B % 2 * workloads.INDEXER_LAYOUT_TILED)
    check_indexer_parity(corrupt(iw, rng))


def test_indexer_graph_replays():
    """The call enqueues one kernel launch and no allocation or memset, so a
    decode loop can capture it.  Between replays the cache bytes, the
    token-to-batch ids and the table change in place and eager work runs;
    each replay must match the oracle on the inputs of that moment."""
    lens = [700, 0, 130, 2100, 64]
    pages = sum(-(-n // 64) for n in lens)
    iw = workloads.make_indexer_workload("ix_graph", lens, 64, 128, pages + 5, seed=31,
                                         pad_rows=9, layout=workloads.INDEXER_LAYOUT_TILED)
    d = iw.to(DEV)
    got_v, got_s = d.fresh_values(), d.fresh_scales()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            run_indexer_hip(d, got_v, got_s)
    torch.cuda.synchronize()
    rng = np.random.default_rng(32)
    for rep in range(4):
        log(f"[indexer graph] replay {rep}")
        fresh = workloads.make_indexer_workload("ix_graph", lens, 64, 128, pages + 5,
                                                seed=100 + rep, pad_rows=9,
                                                layout=workloads.INDEXER_LAYOUT_TILED)
        iw.cache.copy_(fresh.cache)
        iw.token_to_seq.copy_(fresh.token_to_seq)
        iw.block_table.copy_(fresh.block_table)
        if rep >= 2:   # masks of every kind, the table width left as captured
            width = iw.block_table_width
            corrupt(iw, rng)
            iw.block_table_width = width
        for f in ("cache", "token_to_seq", "block_table"):
            getattr(d, f).copy_(getattr(iw, f))
        got_v.fill_(workloads.SENTINEL_BYTE)
        got_s.view(torch.uint8).fill_(workloads.SENTINEL_BYTE)
        torch.cuda.synchronize()
        graph.replay()
        _ = d.cache.sum()
        torch.cuda.synchronize()
        want_v, want_s, _ = oracle.run_indexer_workload(iw)
        assert torch.equal(got_v.cpu(), want_v), f"replay {rep}: values differ"
        assert torch.equal(got_s.cpu().view(torch.uint8), want_s.view(torch.uint8)), \
            f"replay {rep}: scales differ"


@pytest.mark.parametrize("pitch", [(1 << 25) - 16, 1 << 25])
def test_indexer_destination_pitch_at_the_store_range(pitch):
    """16-byte chunks are stored through a resource over a wave's 64
    destination rows, which must span fewer than 2^31 bytes: at a pitch just
    under 32 MiB the 64 rows of the first wave span 2^31 - 1 KiB; at 32 MiB
    the host takes byte chunks instead.  Rows 0..63 fill the first wave (two
    batches), row 64 (padding) the second.  The gathered columns match the
    oracle and every byte past them stays untouched."""
    hd = 128
    iw = workloads.make_indexer_workload(f"ix_pitch_{pitch}", [40, 24], 16, hd, 8, seed=pitch % 997,
                                         pad_rows=1, value_cols=pitch)
    log(f"[indexer parity] destination pitch {pitch}: T={iw.num_tokens} bytes={iw.num_tokens * pitch}")
    want_v, want_s, rows = oracle.run_indexer_workload(iw)
    assert rows == 64
    d = iw.to(DEV)
    got_v, got_s = d.fresh_values(), d.fresh_scales()
    run_indexer_hip(d, got_v, got_s)
    torch.cuda.synchronize()
    assert torch.equal(got_v[:, :hd].cpu(), want_v[:, :hd])
    assert bool((got_v[:, hd:] == workloads.SENTINEL_BYTE).all())
    assert torch.equal(got_s.cpu().view(torch.uint8), want_s.view(torch.uint8))


def test_indexer_rows_beyond_the_grid():
    """More rows than one pass of the capped grid covers (65,536 workgroups of
    64 rows = 4,194,304 rows): waves stride to their next 64 rows and load
    those rows' batch ids inside the loop.  One sequence of 4,300,000 tokens
    and padding rows past it."""
    n = 4_300_000
    iw = workloads.make_indexer_workload("ix_grid_cap", [n], 64, 128, -(-n // 64) + 5, seed=81,
                                         pad_rows=70)
    assert iw.num_tokens > 65536 * 64
    check_indexer_parity(iw)
