"""CPU checks of the seeded workloads and of bench.py's host-side logic."""
import json
import os
import subprocess
import sys

import pytest
import torch

import oracle
import workloads

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_tiny_workload_shape_and_oracle():
    wl = workloads.tiny_raw()
    assert wl.num_reqs == 3 and wl.num_tokens == 88 and wl.block_size == 16
    assert tuple(wl.block_table.shape) == (3, 8)
    assert wl.cu_seq_lens.tolist() == [0, 17, 88, 88]
    assert len(oracle.load().page_tasks(wl.cu_seq_lens, None, 3, 88, 16)) == 7
    ws, rows = oracle.run_workload(wl)
    assert rows == 88
    assert wl.algorithmic_bytes() == 88 * 576 * 4 + 16


def test_workloads_are_deterministic():
    a, b = workloads.tiny_raw(), workloads.tiny_raw()
    assert torch.equal(a.cache_base.view(torch.uint8), b.cache_base.view(torch.uint8))
    assert torch.equal(a.block_table, b.block_table)


def test_named_workload_sizes():
    """The headline shapes: 960 and 4800 pages, the skew and mixed batches."""
    o = oracle.load()
    wl = workloads.single_60k_raw()
    assert (wl.num_tokens, wl.num_blocks, wl.block_table.shape[1]) == (61440, 1200, 960)
    assert wl.algorithmic_bytes() == 141557768
    assert len(o.page_tasks(wl.cu_seq_lens, None, 1, 61440, 64)) == 960
    wl = workloads.single_300k_upconvert()
    assert (wl.num_tokens, wl.num_blocks, wl.cache_base.dtype) == (307200, 6000, torch.uint8)
    assert wl.algorithmic_bytes() == 530841608
    codes = wl.cache_base.flatten()[:1 << 20]
    assert not bool(((codes == 0x7F) | (codes == 0xFF)).any())   # no NaN codes drawn
    wl = workloads.skew8_raw_starts()
    lens = workloads.SKEW8_LENS
    starts = wl.seq_starts.tolist()
    assert all(0 <= s <= n // 4 for s, n in zip(starts, lens))
    assert wl.num_tokens == sum(n - s for n, s in zip(lens, starts))
    assert wl.workspace.shape[0] == sum(lens)
    for k, wl in ((2, workloads.skew2_raw_starts()), (4, workloads.skew4_raw_starts())):
        lens = workloads.SKEW8_LENS[:k]
        starts = wl.seq_starts.tolist()
        assert wl.num_reqs == k and wl.context_lens == lens
        assert all(0 <= s <= n // 4 for s, n in zip(starts, lens))
        assert wl.num_tokens == sum(n - s for n, s in zip(lens, starts))
        assert wl.workspace.shape[0] == sum(lens)
    wl = workloads.mixed_dequant_strided()
    assert wl.num_reqs == 64 and wl.cache_base.shape[2] == 577 and wl.workspace.shape[1] == 580
    assert wl.src_cache().stride() == (64 * 577, 577, 1) and wl.dst().stride() == (580, 1)
    assert all(0 <= n <= 65536 for n in wl.context_lens)
    # page-size variants: 61,440 one-token pages, 60 pages of 1,024 tokens,
    # 512 requests of 200 one-token pages
    for name, tokens, bs, width in (("single_60k_bs1_raw", 61440, 1, 61440),
                                    ("single_60k_bs1024_raw", 61440, 1024, 60),
                                    ("batch512x200_bs1_raw", 512 * 200, 1, 200)):
        wl = workloads.named(name)
        assert (wl.num_tokens, wl.block_size, wl.block_table.shape[1]) == (tokens, bs, width), name
        assert wl.algorithmic_bytes() == 2304 * tokens + 4 * (wl.num_reqs + 1), name
    # the single-60K bytes split evenly over 2, 8 and 64 requests
    for R in (2, 8, 64):
        wl = workloads.named(f"batch{R}_60k_raw")
        assert wl.num_reqs == R and wl.num_tokens == 61440 and wl.seq_starts is None
        assert wl.context_lens == [61440 // R] * R and wl.num_blocks == 1200
        assert wl.algorithmic_bytes() == 2304 * 61440 + 4 * (R + 1)


def test_bench_refuses_more_than_one_gpu():
    proc = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr


def test_bench_counter_summary(tmp_path, monkeypatch):
    """Counter scaling: each counter is divided by its reading for the
    calibration copies (the last 10 copy dispatches) of the same run."""
    sys.path.insert(0, REPO)
    import bench

    monkeypatch.setattr(bench, "TRAFFIC_DIR", str(tmp_path))
    head = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n"
    for kind, counter, gather_kib, copy_kib in (("fetch", "FETCH_SIZE", 34643.5, 131072.0),
                                                ("write", "WRITE_SIZE", 69121.0, 262144.0)):
        lines = [head]
        d = 0
        for _ in range(5):
            d += 1
            lines.append(f'{d},"pkvg::gather_pages_kernel<...>",{counter},{gather_kib}\n')
        for _ in range(10):
            d += 1
            lines.append(f'{d},"__amd_rocclr_copyBuffer",{counter},{copy_kib}\n')
        (tmp_path / f"{kind}_counter_collection.csv").write_text("".join(lines))
    res = bench.summarize_counters(str(tmp_path), "tiny_raw", 256, "cmd")
    assert res["fetch"]["scale"] == pytest.approx(2.0)
    assert res["write"]["scale"] == pytest.approx(1.0)
    assert res["hbm_bytes_per_launch"] == round(34643.5 * 1024 * 2 + 69121.0 * 1024)
    saved = json.loads((tmp_path / "traffic_tiny_raw.json").read_text())
    assert saved["kernel_source_sha"] == bench.kernel_source_hash()


@pytest.mark.parametrize("name,parts", [("tiny_raw", 5), ("skew8_raw_seq_starts", 16)])
def test_threaded_oracle_baseline_matches_oracle(name, parts):
    """The CPU baseline's row-range split reproduces the oracle's output."""
    from concurrent.futures import ThreadPoolExecutor

    sys.path.insert(0, REPO)
    import bench

    wl = workloads.named(name)
    want, rows = oracle.run_workload(wl)
    ws = wl.fresh_workspace()
    with ThreadPoolExecutor(max_workers=4) as pool:
        got_rows = bench.oracle_threaded(wl, parts, ws)(pool)
    assert got_rows == rows
    assert torch.equal(ws.view(torch.uint8), want.view(torch.uint8))
    open_wl = workloads.tiny_raw().open_ended()
    want, _ = oracle.run_workload(open_wl)
    ws = open_wl.fresh_workspace()
    with ThreadPoolExecutor(max_workers=2) as pool:
        bench.oracle_threaded(open_wl, 3, ws)(pool)
    assert torch.equal(ws.view(torch.uint8), want.view(torch.uint8))


@pytest.mark.parametrize("kind", ["raw", "fp8_upconvert", "fp8_dequant", "auto"])
def test_bench_custom_workload(kind):
    """bench.py --lens/--kind/--block-size/--entry/--starts builds a seeded
    workload of exactly that shape, with the library kind of that name."""
    import argparse

    sys.path.insert(0, REPO)
    import bench

    ns = argparse.Namespace(lens="300,0,77", kind=kind, block_size=16, entry=64, starts=True,
                            scale=0.05, seed=5)
    wl = bench.custom_workload(ns)
    want_kind = {"raw": workloads.RAW, "fp8_upconvert": workloads.UPCONVERT,
                 "fp8_dequant": workloads.DEQUANT_FP8, "auto": workloads.DEQUANT_AUTO}[kind]
    assert wl.kind == want_kind and wl.name == bench.custom_workload_name(ns)
    assert wl.context_lens == [300, 0, 77] and (wl.block_size, wl.entry) == (16, 64)
    starts = wl.seq_starts.tolist()
    assert all(0 <= s <= n // 4 for s, n in zip(starts, [300, 0, 77]))
    assert wl.num_tokens == sum(n - s for n, s in zip([300, 0, 77], starts))
    assert wl.num_blocks >= 19 + 5


@pytest.mark.parametrize("use_starts", [False, True])
def test_pages_uneven_test_shape(use_starts):
    """The page's own kernel-test case: 17 / 32,768 / 71 gathered rows, starts
    3 / 17 / 5, block 64, entry 576, 1,024 blocks, every table row a full
    permutation of the blocks (rows alias)."""
    wl = workloads.pages_uneven_test(workloads.RAW, use_starts)
    assert wl.cu_seq_lens.tolist() == [0, 17, 17 + 32768, 17 + 32768 + 71]
    assert (wl.block_size, wl.entry, wl.num_blocks) == (64, 576, 1024)
    assert tuple(wl.block_table.shape) == (3, 1024)
    for r in range(3):
        assert sorted(wl.block_table[r].tolist()) == list(range(1024))
    assert (wl.seq_starts.tolist() if use_starts else None) == ([3, 17, 5] if use_starts else None)
    u8 = workloads.pages_uneven_test(workloads.RAW, use_starts, torch.uint8)
    assert u8.cache_base.dtype == torch.uint8 and u8.workspace.dtype == torch.uint8


def test_bench_defaults_name_the_single_request_gathers_and_the_indexer():
    sys.path.insert(0, REPO)
    import bench

    assert bench.DEFAULT_WORKLOAD == "single_300k_fp8_upconvert"
    assert bench.ALSO_WORKLOADS == ("single_60k_raw", "indexer_single_300k_flat")
    assert set(workloads.NAMED) >= {bench.DEFAULT_WORKLOAD, bench.ALSO_WORKLOADS[0]}
    assert bench.ALSO_WORKLOADS[1] in workloads.INDEXER_NAMED


@pytest.mark.parametrize("name,parts", [("indexer_tiny_flat", 4), ("indexer_skew8_tiled", 16)])
def test_threaded_indexer_oracle_matches_oracle(name, parts):
    """The indexer CPU baseline's row-range split (token_to_seq and the
    destinations from r0 on, cu_seqlen shifted by r0) reproduces the oracle's
    output of the whole gather, including rows claiming another batch."""
    from concurrent.futures import ThreadPoolExecutor

    sys.path.insert(0, REPO)
    import bench

    iw = workloads.named(name)
    iw.token_to_seq[::97] = -1
    iw.token_to_seq[1::89] = 0
    want_v, want_s, rows = oracle.run_indexer_workload(iw)
    v, s = iw.fresh_values(), iw.fresh_scales()
    with ThreadPoolExecutor(max_workers=4) as pool:
        got = bench.indexer_oracle_threaded(iw, parts, v, s)(pool)
    assert got == rows
    assert torch.equal(v, want_v) and torch.equal(s.view(torch.uint8), want_s.view(torch.uint8))


def test_indexer_workload_shapes():
    iw = workloads.named("indexer_single_300k_flat")
    assert (iw.num_tokens, iw.block_size, iw.head_dim, iw.block_stride) == (307200, 64, 128, 64 * 132)
    assert iw.num_blocks == 6000 and iw.gathered_rows() == 307200
    assert iw.algorithmic_bytes() == 307200 * (2 * 132 + 4) + 8
    iw = workloads.named("indexer_skew8_tiled")
    assert iw.num_tokens == sum(workloads.SKEW8_LENS) + 8
    assert iw.token_to_seq[-8:].tolist() == [-1] * 8
