"""gather_maybe_dequant_noalloc (the entry point that allocates nothing)
against gather_maybe_dequant, byte for byte, through the C ABI: two calls in a
row on batches beyond the fused limit (its fixed scratch holds their task
tables), the second smaller than the first, both cache kinds, and a batch
within the fused limit (no scratch)."""
import pytest
import torch

import paged_kv_cache_device_amd as pkvg
import workloads
from gpu_util import log, plan_of

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkvg.library()


def batch(R, seed, kind, bs=16, max_len=90):
    """R requests with a block table twice as wide as the longest needs (a
    batch past the fused limit with a sparse table takes the task-table path,
    the one that uses scratch; a dense one would be walked without any)."""
    g = torch.Generator("cpu").manual_seed(seed)
    lens = torch.randint(0, max_len, (R,), generator=g)
    lens[torch.rand(R, generator=g) < 0.1] = 0
    lens = lens.tolist()
    starts = [int(torch.randint(0, n + 1, (1,), generator=g)) for n in lens]
    pages = sum(-(-n // bs) for n in lens)
    return workloads.make_workload(f"noalloc_{R}_{kind}", kind, lens, bs, 64, pages + 5, seed=seed,
                                   starts=starts, scale=0.05, workspace_rows=sum(lens) + 4,
                                   width=2 * -(-max_len // bs) + 2)


def both(wl):
    """(existing entry point's workspace, no-allocation entry point's workspace)."""
    d = wl.to(DEV)
    kv = "fp8" if wl.kind == workloads.DEQUANT_FP8 else "auto"
    sc = d.scale_tensor if kv == "fp8" else None
    want = d.fresh_workspace()
    pkvg.gather_maybe_dequant(d.src_cache(), want[: d.num_tokens, : d.entry], d.block_table,
                              d.cu_seq_lens, d.num_reqs, kv, sc, d.seq_starts)
    got = d.fresh_workspace()
    pkvg.gather_maybe_dequant_noalloc(d.src_cache(), got[: d.num_tokens, : d.entry], d.block_table,
                                      d.cu_seq_lens, d.num_reqs, kv, sc, d.seq_starts)
    torch.cuda.synchronize()
    return want.cpu(), got.cpu()


@pytest.mark.parametrize("first,second", [
    ((3000, workloads.DEQUANT_FP8), (1500, workloads.DEQUANT_AUTO)),
    ((5000, workloads.DEQUANT_AUTO), (1100, workloads.DEQUANT_FP8)),
    ((2500, workloads.DEQUANT_FP8), (300, workloads.DEQUANT_FP8)),   # then a fused batch
])
def test_noalloc_matches_gather_maybe_dequant(first, second):
    for i, (R, kind) in enumerate((first, second)):
        wl = batch(R, 9000 + R + i, kind)
        mode = plan_of(wl.to(DEV))["task_mode"]
        assert mode == (pkvg.PKVG_TASKS_TABLE if R > 1024 else pkvg.PKVG_TASKS_LDS), mode
        log(f"[noalloc] call {i + 1}: R={R} kind={kind} T={wl.num_tokens} mode={mode}")
        want, got = both(wl)
        assert torch.equal(want.view(torch.uint8), got.view(torch.uint8)), (R, kind)
        assert not bool((want.view(torch.uint8) == workloads.SENTINEL_BYTE).all())


def test_noalloc_prepared_call():
    """The binding's prepare() of the no-allocation entry point: marshalled once,
    issued twice on a 2,000-request batch with another batch's no-allocation call
    between them (which leaves its own task table in the shared scratch); each
    issue matches gather_maybe_dequant byte for byte."""
    wl = batch(2000, 9100, workloads.DEQUANT_FP8)
    other = batch(1200, 9101, workloads.DEQUANT_AUTO)
    d, o = wl.to(DEV), other.to(DEV)
    want = d.fresh_workspace()
    pkvg.gather_maybe_dequant(d.src_cache(), want[: d.num_tokens, : d.entry], d.block_table,
                              d.cu_seq_lens, d.num_reqs, "fp8", d.scale_tensor, d.seq_starts)
    got = d.fresh_workspace()
    call = pkvg.prepare("gather_maybe_dequant_noalloc", d.src_cache(), got[: d.num_tokens, : d.entry],
                        d.block_table, d.cu_seq_lens, d.num_reqs, "fp8", scale=d.scale_tensor,
                        seq_starts=d.seq_starts)
    for rep in range(2):
        got.view(torch.uint8).fill_(workloads.SENTINEL_BYTE)
        call()
        ows = o.fresh_workspace()
        pkvg.gather_maybe_dequant_noalloc(o.src_cache(), ows[: o.num_tokens, : o.entry], o.block_table,
                                          o.cu_seq_lens, o.num_reqs, "auto", None, o.seq_starts)
        torch.cuda.synchronize()
        log(f"[noalloc] prepared call, issue {rep + 1}: R={d.num_reqs} T={d.num_tokens}")
        assert torch.equal(want.view(torch.uint8).cpu(), got.view(torch.uint8).cpu()), rep


def test_noalloc_full_size_named_workload():
    """A named workload at full size through both entry points (fused path)."""
    wl = workloads.named("mixed_fp8_dequant_strided")
    log(f"[noalloc] {wl.name} R={wl.num_reqs} T={wl.num_tokens}")
    want, got = both(wl)
    assert torch.equal(want.view(torch.uint8), got.view(torch.uint8))


def test_noalloc_dense_batch_is_walked():
    """A dense batch past the fused limit is walked through its table and needs
    no scratch at all; both entry points agree."""
    lens = [48] * 1800
    wl = workloads.make_workload("noalloc_dense", workloads.DEQUANT_FP8, lens, 16, 64, 5500, seed=77,
                                 scale=0.05)
    assert plan_of(wl.to(DEV))["task_mode"] == pkvg.PKVG_TASKS_WALK
    log(f"[noalloc] dense R={wl.num_reqs} T={wl.num_tokens}")
    want, got = both(wl)
    assert torch.equal(want.view(torch.uint8), got.view(torch.uint8))


def test_noalloc_graph_replays():
    """Callers that cannot allocate include graph capture: the scratch path
    (a sparse batch past the fused limit: task builder, then gather, both on
    the fixed scratch) is captured once and replayed with new cache contents
    in place; every replay matches the allocating entry point run eagerly on
    the inputs of that moment."""
    wl = batch(2200, 9500, workloads.DEQUANT_FP8)
    d = wl.to(DEV)
    assert plan_of(d)["task_mode"] == pkvg.PKVG_TASKS_TABLE
    got = d.fresh_workspace()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            pkvg.gather_maybe_dequant_noalloc(d.src_cache(), got[: d.num_tokens, : d.entry],
                                              d.block_table, d.cu_seq_lens, d.num_reqs, "fp8",
                                              d.scale_tensor, d.seq_starts)
    torch.cuda.synchronize()
    base = d.cache_base.view(torch.uint8).clone()
    for rep in range(3):
        log(f"[noalloc graph] replay {rep}")
        d.cache_base.view(torch.uint8).copy_(torch.roll(base, 37 * rep + 1))
        got.view(torch.uint8).fill_(workloads.SENTINEL_BYTE)
        torch.cuda.synchronize()
        graph.replay()
        _ = d.cache_base.sum()
        torch.cuda.synchronize()
        want = d.fresh_workspace()
        pkvg.gather_maybe_dequant(d.src_cache(), want[: d.num_tokens, : d.entry], d.block_table,
                                  d.cu_seq_lens, d.num_reqs, "fp8", d.scale_tensor, d.seq_starts)
        torch.cuda.synchronize()
        assert torch.equal(want.view(torch.uint8), got.view(torch.uint8)), rep
        assert not bool((want.view(torch.uint8) == workloads.SENTINEL_BYTE).all())
