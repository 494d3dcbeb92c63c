"""Helpers shared by the GPU parity tests: run a workload through the HIP
library (via the Python binding over the C ABI) and through the CPU oracle, and
compare the whole destination workspace byte for byte."""
from __future__ import annotations

import sys

import torch

import oracle
import paged_kv_cache_device_amd as pkvg
import workloads


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def run_hip(wl_dev: workloads.Workload, ws: torch.Tensor | None = None) -> torch.Tensor:
    """Run the entry point matching ``wl_dev.kind`` into a fresh sentinel workspace
    (or ``ws``) and return that workspace (device)."""
    g = wl_dev
    if ws is None:
        ws = g.fresh_workspace()
    dst = ws[: g.num_tokens, : g.entry]
    if g.kind == workloads.RAW:
        pkvg.gather_cache(g.src_cache(), dst, g.block_table, g.cu_seq_lens, g.num_reqs,
                          g.seq_starts)
    elif g.kind == workloads.DEQUANT_AUTO:
        pkvg.gather_maybe_dequant(g.src_cache(), dst, g.block_table, g.cu_seq_lens, g.num_reqs,
                                  "auto", None, g.seq_starts)
    elif g.kind == workloads.DEQUANT_FP8:
        pkvg.gather_maybe_dequant(g.src_cache(), dst, g.block_table, g.cu_seq_lens, g.num_reqs,
                                  "fp8", g.scale_tensor, g.seq_starts)
    elif g.kind == workloads.UPCONVERT:
        pkvg.gather_upconvert_fp8(g.src_cache(), dst, g.block_table, g.cu_seq_lens, g.num_reqs,
                                  g.scale_tensor, g.seq_starts)
    else:
        raise ValueError(g.kind)
    return ws


def byte_diff(got: torch.Tensor, want: torch.Tensor) -> str:
    a = got.contiguous().view(torch.uint8).view(got.shape[0], -1)
    b = want.contiguous().view(torch.uint8).view(want.shape[0], -1)
    bad = (a != b)
    rows = bad.any(dim=1).nonzero().flatten()
    return f"{int(bad.sum())} bytes differ in {rows.numel()} rows; first rows {rows[:8].tolist()}"


def check_parity(wl: workloads.Workload, device: str = "cuda:0") -> None:
    """HIP result == oracle result, every byte of the workspace (written rows,
    untouched rows, pad columns and the workspace tail)."""
    log(f"[parity] {wl.name} kind={wl.kind} R={wl.num_reqs} T={wl.num_tokens} "
        f"bs={wl.block_size} entry={wl.entry} cache={tuple(wl.cache_base.shape)} "
        f"ws={tuple(wl.workspace.shape)}")
    want, _ = oracle.run_workload(wl)
    g = wl.to(device)
    ws = run_hip(g)
    torch.cuda.synchronize()
    got = ws.cpu()
    same = torch.equal(got.view(torch.uint8), want.view(torch.uint8))
    assert same, f"{wl.name}: " + byte_diff(got, want)


def plan_of(wl_dev: workloads.Workload) -> dict:
    """How the library would run ``wl_dev``'s call (pkvg_plan with the same
    marshalled arguments as the call), so a test can check which path it took."""
    g = wl_dev
    dst = g.workspace[: g.num_tokens, : g.entry]
    common = (g.src_cache(), dst, g.block_table, g.cu_seq_lens, g.num_reqs)
    if g.kind == workloads.RAW:
        a = pkvg.prepare("gather_cache", *common, g.seq_starts)._args
        op, kind, cache, scale = pkvg.PKVG_OP_GATHER_CACHE, a[1], a[2:17], None
    elif g.kind in (workloads.DEQUANT_AUTO, workloads.DEQUANT_FP8):
        fp8 = g.kind == workloads.DEQUANT_FP8
        a = pkvg.prepare("gather_maybe_dequant", *common, "fp8" if fp8 else "auto",
                         scale=g.scale_tensor if fp8 else None, seq_starts=g.seq_starts)._args
        op, kind, cache, scale = pkvg.PKVG_OP_GATHER_MAYBE_DEQUANT, a[1], a[2:17], a[17]
    else:
        a = pkvg.prepare("gather_upconvert_fp8", *common, g.scale_tensor,
                         seq_starts=g.seq_starts)._args
        op, kind, cache, scale = pkvg.PKVG_OP_GATHER_UPCONVERT_FP8, 0, a[1:16], a[16]
    return pkvg.pkvg_plan(op, kind, a[0], *cache, scale)
