"""Seeded synthetic inputs for the paged MLA KV-cache gather.

This module is shared by the tests, the smoke check and the benchmark, and by
both sides of every parity check (the HIP library and the CPU oracle).  It
holds none of the gather's arithmetic: it only draws caches, block tables,
per-request lengths and starts, and allocates sentinel-filled destinations.

Recipe (all draws from one ``torch.Generator('cpu')`` seeded per workload, in
this order: request lengths, seq_starts, physical block permutation, cache
values):

* bf16 caches: ``randn`` in fp32, rounded to bf16 (N(0,1) values).
* fp8 caches: uniform over the 254 non-NaN e4m3fn codes (0x7F and 0xFF are
  the two NaN codes and are never drawn).
* block tables: one ``randperm(num_blocks)`` dealt out request after request,
  ``ceil(context_len / block_size)`` distinct physical blocks per request; the
  unused tail of each row is -1, so a stray read of an unused slot shows up as
  rows left untouched.
* ``cu_seq_lens`` are prefix sums (R + 1 entries, starting at 0) of the rows
  gathered per request; with ``seq_starts`` a request gathers the context
  tokens ``[start, context_len)``.
* destinations are filled with a sentinel byte pattern (0xFF) so rows the
  gather must not touch can be checked.

The five named workloads follow the shapes the pages' scenarios and tests use
(single-request 60K and 300K contexts, a skewed batch with seq_starts, a tiny
uneven batch, a mixed batch with non-vector strides).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

SENTINEL_BYTE = 0xFF

# kind of gather a workload exercises
RAW = "raw"                # gather_cache: bit copy
DEQUANT_AUTO = "dequant_auto"  # gather_maybe_dequant with kv_cache_dtype 'auto' (bit copy of bf16)
DEQUANT_FP8 = "dequant_fp8"    # gather_maybe_dequant with kv_cache_dtype 'fp8'
UPCONVERT = "upconvert"    # gather_upconvert_fp8

FP8_KINDS = (DEQUANT_FP8, UPCONVERT)


@dataclasses.dataclass
class Workload:
    name: str
    kind: str
    block_size: int
    entry: int                      # elements per cache row that are gathered
    cache_base: torch.Tensor        # [num_blocks, block_size, cache_cols] (bf16 or uint8)
    workspace: torch.Tensor         # [workspace_rows, dst_cols] (dst dtype), sentinel filled
    num_tokens: int                 # T: rows of dst = workspace[:T, :entry]
    block_table: torch.Tensor       # int32 [R, W]
    cu_seq_lens: torch.Tensor       # int32 [R + 1]
    seq_starts: Optional[torch.Tensor]  # int32 [R] or None
    context_lens: list
    scale: float = 1.0
    scale_tensor: Optional[torch.Tensor] = None  # fp32 [1] for fp8 kinds
    cu_terminal: bool = True  # False: cu_seq_lens holds R entries, the last request ends at T

    @property
    def num_reqs(self) -> int:
        return self.block_table.shape[0]

    @property
    def num_blocks(self) -> int:
        return self.cache_base.shape[0]

    def src_cache(self) -> torch.Tensor:
        return self.cache_base[..., : self.entry]

    def dst(self) -> torch.Tensor:
        return self.workspace[: self.num_tokens, : self.entry]

    def to(self, device) -> "Workload":
        """A copy whose tensors live on ``device`` (strides of the views are kept)."""
        d = dataclasses.replace(self)
        d.cache_base = self.cache_base.to(device)
        d.workspace = self.workspace.to(device)
        d.block_table = self.block_table.to(device)
        d.cu_seq_lens = self.cu_seq_lens.to(device)
        d.seq_starts = None if self.seq_starts is None else self.seq_starts.to(device)
        d.scale_tensor = None if self.scale_tensor is None else self.scale_tensor.to(device)
        return d

    def fresh_workspace(self) -> torch.Tensor:
        """A new sentinel-filled workspace like this one (same device)."""
        return torch.full_like(self.workspace.view(torch.uint8), SENTINEL_BYTE).view(
            self.workspace.dtype)

    @property
    def src_elem_bytes(self) -> int:
        return self.cache_base.element_size()

    @property
    def dst_elem_bytes(self) -> int:
        return self.workspace.element_size()

    def request_ends(self) -> list:
        """Each request's output end before clamping to num_tokens."""
        cu = self.cu_seq_lens.cpu().tolist()
        R = self.num_reqs
        return [cu[r + 1] if (self.cu_terminal or r + 1 < R) else self.num_tokens
                for r in range(R)]

    def gathered_rows(self) -> int:
        """Rows the request extents cover (before any guard skips)."""
        cu = self.cu_seq_lens.cpu().tolist()
        T = self.num_tokens
        ends = self.request_ends()
        return sum(max(min(ends[r], T) - min(cu[r], T), 0) for r in range(self.num_reqs))

    def open_ended(self) -> "Workload":
        """The same workload with cu_seq_lens in the open-ended convention
        (R entries; the last request runs to num_tokens)."""
        d = dataclasses.replace(self)
        d.cu_seq_lens = self.cu_seq_lens[: self.num_reqs].clone()
        d.cu_terminal = False
        return d

    def algorithmic_bytes(self) -> int:
        """Payload read + payload written + metadata read, for a full (unguarded) gather."""
        rows = self.gathered_rows()
        pay = rows * self.entry * (self.src_elem_bytes + self.dst_elem_bytes)
        meta = 4 * (self.num_reqs + int(self.cu_terminal)) + (
            4 * self.num_reqs if self.seq_starts is not None else 0)
        return pay + meta


# ---------------------------------------------------------------------------
# drawing helpers
# ---------------------------------------------------------------------------

def fp8_nonnan_codes(gen: torch.Generator, shape) -> torch.Tensor:
    """uint8 codes uniform over the 254 e4m3fn codes that are not NaN."""
    idx = torch.randint(0, 254, shape, generator=gen, dtype=torch.uint8)
    # indices 0..126 -> codes 0x00..0x7E, 127..253 -> codes 0x80..0xFE
    return idx + (idx >= 127).to(torch.uint8)


def bf16_normal(gen: torch.Generator, shape) -> torch.Tensor:
    return torch.randn(shape, generator=gen, dtype=torch.float32).to(torch.bfloat16)


def deal_block_table(gen: torch.Generator, context_lens, block_size: int, num_blocks: int,
                     width: Optional[int] = None, allow_alias: bool = False,
                     full_rows: bool = False) -> torch.Tensor:
    """int32 [R, W]: distinct physical blocks from one randperm, -1 in unused slots.

    With ``allow_alias`` each row is an independent ``randperm`` prefix, so rows
    may share physical blocks (legal: the gather only reads the cache).  With
    ``full_rows`` every row is the first W entries of its own
    ``randperm(num_blocks)``: rows alias and no slot is unused.
    """
    pages = [-(-int(n) // block_size) for n in context_lens]
    W = max(pages + [1]) if width is None else width
    assert W >= max(pages + [0])
    bt = torch.full((len(context_lens), W), -1, dtype=torch.int32)
    if full_rows:
        assert W <= num_blocks
        for r in range(len(context_lens)):
            bt[r] = torch.randperm(num_blocks, generator=gen)[:W].to(torch.int32)
        return bt
    if allow_alias:
        for r, p in enumerate(pages):
            assert p <= num_blocks
            bt[r, :p] = torch.randperm(num_blocks, generator=gen)[:p].to(torch.int32)
        return bt
    assert sum(pages) <= num_blocks, (sum(pages), num_blocks)
    perm = torch.randperm(num_blocks, generator=gen).to(torch.int32)
    off = 0
    for r, p in enumerate(pages):
        bt[r, :p] = perm[off: off + p]
        off += p
    return bt


def prefix_sums(rows) -> torch.Tensor:
    cu = [0]
    for n in rows:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def make_workload(name: str, kind: str, context_lens, block_size: int, entry: int,
                  num_blocks: int, seed: int, *, starts=None, width: Optional[int] = None,
                  cache_cols: Optional[int] = None, dst_cols: Optional[int] = None,
                  workspace_rows: Optional[int] = None, num_tokens: Optional[int] = None,
                  scale: float = 1.0, gen: Optional[torch.Generator] = None,
                  allow_alias: bool = False, draw_starts_quarter: bool = False,
                  cache_dtype: torch.dtype = torch.bfloat16, full_rows: bool = False) -> Workload:
    """Build one workload.  ``starts``: explicit list, or None; with
    ``draw_starts_quarter`` each start is drawn uniformly from [0, len // 4].
    ``cache_dtype`` (raw kinds only): bf16 / fp32 values from N(0,1), or uint8
    random bytes; the destination has the same dtype.  fp8 kinds always hold
    e4m3fn codes in a uint8 cache and write bf16."""
    if gen is None:
        gen = torch.Generator("cpu").manual_seed(seed)
    context_lens = [int(x) for x in context_lens]
    R = len(context_lens)
    if draw_starts_quarter:
        starts = [int(torch.randint(0, n // 4 + 1, (1,), generator=gen).item())
                  for n in context_lens]
    bt = deal_block_table(gen, context_lens, block_size, num_blocks, width, allow_alias,
                          full_rows)
    cache_cols = entry if cache_cols is None else cache_cols
    dst_cols = entry if dst_cols is None else dst_cols
    cshape = (num_blocks, block_size, cache_cols)
    if kind in FP8_KINDS:
        cache = fp8_nonnan_codes(gen, cshape)
        dst_dtype = torch.bfloat16
    elif kind == DEQUANT_AUTO or cache_dtype == torch.bfloat16:
        cache = bf16_normal(gen, cshape)
        dst_dtype = torch.bfloat16
    elif cache_dtype == torch.float32:
        cache = torch.randn(cshape, generator=gen, dtype=torch.float32)
        dst_dtype = torch.float32
    elif cache_dtype == torch.uint8:
        cache = torch.randint(0, 256, cshape, generator=gen, dtype=torch.uint8)
        dst_dtype = torch.uint8
    else:
        raise ValueError(f"unsupported cache dtype {cache_dtype}")
    if starts is None:
        rows = context_lens
        seq_starts = None
    else:
        assert len(starts) == R
        rows = [max(n - s, 0) for n, s in zip(context_lens, starts)]
        seq_starts = torch.tensor(starts, dtype=torch.int32)
    cu = prefix_sums(rows)
    T = int(cu[-1]) if num_tokens is None else num_tokens
    ws_rows = T if workspace_rows is None else workspace_rows
    assert ws_rows >= T
    esz = torch.empty(0, dtype=dst_dtype).element_size()
    workspace = torch.full((ws_rows, dst_cols * esz), SENTINEL_BYTE, dtype=torch.uint8).view(
        dst_dtype)
    wl = Workload(name=name, kind=kind, block_size=block_size, entry=entry, cache_base=cache,
                  workspace=workspace, num_tokens=T, block_table=bt, cu_seq_lens=cu,
                  seq_starts=seq_starts, context_lens=context_lens, scale=scale)
    if kind in FP8_KINDS:
        wl.scale_tensor = torch.tensor([scale], dtype=torch.float32)
    return wl


# ---------------------------------------------------------------------------
# the five named workloads
# ---------------------------------------------------------------------------

def _lognormal_lengths(gen, n, median, sigma, lo, hi):
    z = torch.randn(n, generator=gen, dtype=torch.float64)
    lens = torch.exp(z * sigma + math.log(median)).round().clamp(lo, hi)
    return [int(x) for x in lens.tolist()]


def tiny_raw() -> Workload:
    """3 requests of {17, 71, 0} tokens, block 16, entry 576 bf16, 32 blocks, table [3, 8]."""
    return make_workload("tiny_raw", RAW, [17, 71, 0], 16, 576, 32, seed=1001, width=8)


def single_60k_raw() -> Workload:
    """1 request of 61440 tokens (960 pages of 64), entry 576 bf16, 1200 cache blocks."""
    return make_workload("single_60k_raw", RAW, [61440], 64, 576, 1200, seed=1002)


def single_300k_upconvert() -> Workload:
    """1 request of 307200 tokens (4800 pages of 64), 576 fp8 bytes per entry, 6000 blocks,
    per-tensor scale 0.0625, fp8 -> bf16 upconvert."""
    return make_workload("single_300k_fp8_upconvert", UPCONVERT, [307200], 64, 576, 6000,
                         seed=1003, scale=0.0625)


SKEW8_LENS = [131072, 16384, 4096, 1024, 257, 71, 17, 0]


def skew8_raw_starts() -> Workload:
    """8 requests {131072 ... 0}, seq_start uniform in [0, len/4], block 64, entry 576 bf16,
    3000 blocks, table width 2048; dst = workspace[:T] of a sum(len)-row workspace."""
    return make_workload("skew8_raw_seq_starts", RAW, SKEW8_LENS, 64, 576, 3000, seed=1004,
                         width=2048, draw_starts_quarter=True,
                         workspace_rows=sum(SKEW8_LENS))


def skew_raw_starts(k: int, seed: int) -> Workload:
    """The skew-k scenario: the first k lengths of the skew-8 list, with the same
    seq_start rule, block size, entry, cache size and table width as skew-8."""
    lens = SKEW8_LENS[:k]
    return make_workload(f"skew{k}_raw_seq_starts", RAW, lens, 64, 576, 3000, seed=seed,
                         width=2048, draw_starts_quarter=True, workspace_rows=sum(lens))


def skew2_raw_starts() -> Workload:
    """2 requests {131072, 16384} with seq_starts (skew-k reading, k = 2)."""
    return skew_raw_starts(2, 1006)


def skew4_raw_starts() -> Workload:
    """4 requests {131072, 16384, 4096, 1024} with seq_starts (skew-k reading, k = 4)."""
    return skew_raw_starts(4, 1007)


def mixed_dequant_strided() -> Workload:
    """64 requests with log-normal lengths (median 4096, sigma 0.5, clipped to [0, 65536]),
    block 64, fp8 cache rows of 577 bytes using the first 576, scale 0.05, dequantised into
    a bf16 workspace whose rows are 580 elements wide."""
    gen = torch.Generator("cpu").manual_seed(1005)
    lens = _lognormal_lengths(gen, 64, 4096, 0.5, 0, 65536)
    pages = sum(-(-n // 64) for n in lens)
    nb = -(-pages * 5 // 4)
    return make_workload("mixed_fp8_dequant_strided", DEQUANT_FP8, lens, 64, 576, nb, seed=1005,
                         gen=gen, cache_cols=577, dst_cols=580, scale=0.05,
                         workspace_rows=sum(lens) + 16)


# The uneven batch of the page's own kernel test (page 1, "key source
# snippets", test_cp_gather_cache_mla_large_uneven_sequences): 17, 32,768 and
# 71 gathered tokens, starts 3, 17 and 5 when seq_starts are used, block 64,
# entry 576, 1,024 physical blocks, every block-table row its own random
# permutation of all 1,024 blocks.
PAGES_TEST_ROWS = [17, 32768, 71]
PAGES_TEST_STARTS = [3, 17, 5]


def pages_uneven_test(kind: str, use_starts: bool, cache_dtype: torch.dtype = torch.bfloat16,
                      seed: int = 1401) -> Workload:
    """The page's large-uneven-sequences test case for one entry point: ``kind``
    picks the call; for RAW, ``cache_dtype`` bf16 is its 'auto' cache and uint8
    its one-byte fp8 cache copied as bytes."""
    starts = PAGES_TEST_STARTS if use_starts else None
    lens = [n + (s if use_starts else 0) for n, s in zip(PAGES_TEST_ROWS, PAGES_TEST_STARTS)]
    tag = {torch.bfloat16: "bf16", torch.uint8: "u8"}[cache_dtype] if kind == RAW else kind
    return make_workload(f"pages_uneven_{tag}{'_starts' if use_starts else ''}", kind, lens, 64,
                         576, 1024, seed=seed, starts=starts, width=1024, full_rows=True,
                         cache_dtype=cache_dtype, scale=0.0625)


def batch_raw(R: int, bs: int, seed: int, kind: str = RAW) -> Workload:
    """R requests of 12,800 / bs tokens each (800 at bs 16, 400 at bs 32, 200 at
    bs 64: 50, 12.5 and 3.1 pages per request), entry 576, shuffled blocks.  Not a scenario of the pages: batches of many requests
    on small pages, used to choose the workgroup shape by page size."""
    n = 12800 // bs
    name = f"batch{R}_bs{bs}_{'fp8' if kind in FP8_KINDS else 'raw'}"
    return make_workload(name, kind, [n] * R, bs, 576, R * (-(-n // bs)) + 8, seed=seed, scale=0.0625)


def even_batch_60k(R: int, seed: int) -> Workload:
    """R raw requests sharing the single-60K gather's 61,440 tokens evenly (block 64,
    entry 576 bf16, 1200 shuffled blocks, no seq_starts).  Not a scenario of the
    pages: the same bytes as the single-request gather, through the batch task
    lookup (2 and 8 requests: 9 KiB units; 64 requests: whole pages)."""
    return make_workload(f"batch{R}_60k_raw", RAW, [61440 // R] * R, 64, 576, 1200, seed=seed)


def page_size_single(bs: int, tokens: int, seed: int, kind: str = RAW) -> Workload:
    """One request of `tokens` tokens at block size `bs` (entry 576, shuffled
    blocks): the headline single-request gathers with very small or very large
    pages.  Not a scenario of the pages: block size is a runtime argument, and
    these check that one-token pages (moved in groups) and pages of a thousand
    tokens (split into parts) keep the headline rate."""
    tag = "fp8_upconvert" if kind in FP8_KINDS else "raw"
    name = f"single_{tokens // 1024}k_bs{bs}_{tag}"
    return make_workload(name, kind, [tokens], bs, 576, -(-tokens // bs) * 5 // 4 + 8, seed=seed, scale=0.0625)


def short_batch(R: int, n: int, bs: int, seed: int) -> Workload:
    """R raw requests of n tokens each at block size bs (entry 576, shuffled
    blocks): many short requests on one-token pages."""
    return make_workload(f"batch{R}x{n}_bs{bs}_raw", RAW, [n] * R, bs, 576, R * (-(-n // bs)) + 8, seed=seed)


NAMED = {
    "tiny_raw": tiny_raw,
    "single_60k_raw": single_60k_raw,
    "single_300k_fp8_upconvert": single_300k_upconvert,
    "skew8_raw_seq_starts": skew8_raw_starts,
    "skew2_raw_seq_starts": skew2_raw_starts,
    "skew4_raw_seq_starts": skew4_raw_starts,
    "mixed_fp8_dequant_strided": mixed_dequant_strided,
    "batch512_bs16_raw": lambda: batch_raw(512, 16, 1101),
    "batch512_bs16_fp8": lambda: batch_raw(512, 16, 1102, UPCONVERT),
    "batch512_bs32_raw": lambda: batch_raw(512, 32, 1103),
    "batch512_bs64_raw": lambda: batch_raw(512, 64, 1104),
    "batch512_bs64_fp8": lambda: batch_raw(512, 64, 1105, UPCONVERT),
    "single_60k_bs1_raw": lambda: page_size_single(1, 61440, 1201),
    "single_300k_bs1_fp8_upconvert": lambda: page_size_single(1, 307200, 1202, UPCONVERT),
    "single_60k_bs1024_raw": lambda: page_size_single(1024, 61440, 1203),
    "batch512x200_bs1_raw": lambda: short_batch(512, 200, 1, 1204),
    "batch2_60k_raw": lambda: even_batch_60k(2, 1301),
    "batch8_60k_raw": lambda: even_batch_60k(8, 1302),
    "batch64_60k_raw": lambda: even_batch_60k(64, 1303),
}


def named(name: str):
    if name in INDEXER_NAMED:
        return INDEXER_NAMED[name]()
    return NAMED[name]()


# ---------------------------------------------------------------------------
# indexer quant-cache gather (the per-row gather of page 3's
# _cp_gather_indexer_quant_cache_kernel)
# ---------------------------------------------------------------------------

INDEXER_LAYOUT_FLAT = 0
INDEXER_LAYOUT_TILED = 1
INDEXER = "indexer"


@dataclasses.dataclass
class IndexerWorkload:
    """Inputs of one indexer quant-cache gather.  The cache is [num_blocks,
    block_stride] bytes of packed block records whose bytes are drawn uniformly
    (the gather copies bytes, so no byte pattern is special); the generator
    does not place values or scales, it only draws bytes."""
    name: str
    layout: int
    head_dim: int
    block_tile: int
    head_tile: int
    block_size: int
    cache: torch.Tensor          # uint8 [num_blocks, block_stride]
    token_to_seq: torch.Tensor   # int32 [num_tokens]
    cu_seqlen: torch.Tensor      # int32 [num_batches + 1]
    block_table: torch.Tensor    # int32 [num_batches, ld]; columns [0, block_table_width) are read
    block_table_width: int
    num_tokens: int
    values: torch.Tensor         # uint8 [workspace_rows, value_cols], sentinel filled
    scales: torch.Tensor         # float32 [workspace_rows, scale_cols], sentinel bytes
    kind: str = INDEXER

    @property
    def num_blocks(self) -> int:
        return self.cache.shape[0]

    @property
    def block_stride(self) -> int:
        return self.cache.stride(0)

    @property
    def num_batches(self) -> int:
        return self.cu_seqlen.numel() - 1

    def to(self, device) -> "IndexerWorkload":
        d = dataclasses.replace(self)
        for f in ("cache", "token_to_seq", "cu_seqlen", "block_table", "values", "scales"):
            setattr(d, f, getattr(self, f).to(device))
        return d

    def fresh_values(self) -> torch.Tensor:
        return torch.full_like(self.values, SENTINEL_BYTE)

    def fresh_scales(self) -> torch.Tensor:
        return torch.full_like(self.scales.view(torch.uint8), SENTINEL_BYTE).view(torch.float32)

    def dst_values(self, values=None) -> torch.Tensor:
        v = self.values if values is None else values
        return v[: self.num_tokens, : self.head_dim]

    def dst_scales(self, scales=None) -> torch.Tensor:
        s = self.scales if scales is None else scales
        return s[: self.num_tokens, 0]

    def gathered_rows(self) -> int:
        """Rows whose batch id and extent are consistent (before block guards)."""
        t2s = self.token_to_seq[: self.num_tokens].tolist()
        cu = self.cu_seqlen.tolist()
        B = self.num_batches
        return sum(1 for t, b in enumerate(t2s) if 0 <= b < B and cu[b] <= t < cu[b + 1])

    def algorithmic_bytes(self) -> int:
        """Per row: head_dim value bytes and a 4-byte scale read and written, and
        its 4-byte token_to_seq entry; plus cu_seqlen once per batch."""
        rows = self.gathered_rows()
        return rows * 2 * (self.head_dim + 4) + 4 * self.num_tokens + 4 * (self.num_batches + 1)


def make_indexer_workload(name: str, seq_lens, block_size: int, head_dim: int, num_blocks: int,
                          seed: int, *, layout: int = INDEXER_LAYOUT_FLAT, block_tile: int = 16,
                          head_tile: int = 16, record_pad: int = 0, pad_rows: int = 0,
                          value_cols: Optional[int] = None, scale_cols: int = 1,
                          width: Optional[int] = None, allow_alias: bool = False) -> IndexerWorkload:
    """Sequences of ``seq_lens`` tokens gathered into rows cu_seqlen[b] ..
    cu_seqlen[b + 1]; token_to_seq names each row's sequence and is -1 for the
    ``pad_rows`` rows after the last sequence (num_tokens = sum + pad_rows).
    Block records are block_size * (head_dim + 4) + record_pad bytes.  Draw
    order: block permutation, then cache bytes."""
    gen = torch.Generator("cpu").manual_seed(seed)
    seq_lens = [int(x) for x in seq_lens]
    bt = deal_block_table(gen, seq_lens, block_size, num_blocks, width, allow_alias)
    stride = block_size * (head_dim + 4) + record_pad
    cache = torch.randint(0, 256, (num_blocks, stride), generator=gen, dtype=torch.uint8)
    cu = prefix_sums(seq_lens)
    total = int(cu[-1])
    T = total + pad_rows
    t2s = torch.full((T,), -1, dtype=torch.int32)
    for b, n in enumerate(seq_lens):
        t2s[int(cu[b]): int(cu[b]) + n] = b
    value_cols = head_dim if value_cols is None else value_cols
    values = torch.full((T, value_cols), SENTINEL_BYTE, dtype=torch.uint8)
    scales = torch.full((T, 4 * scale_cols), SENTINEL_BYTE, dtype=torch.uint8).view(torch.float32)
    return IndexerWorkload(name=name, layout=layout, head_dim=head_dim, block_tile=block_tile,
                           head_tile=head_tile, block_size=block_size, cache=cache,
                           token_to_seq=t2s, cu_seqlen=cu, block_table=bt,
                           block_table_width=bt.shape[1], num_tokens=T, values=values,
                           scales=scales)


def indexer_single(tokens: int, layout: int, seed: int) -> IndexerWorkload:
    """One sequence of `tokens` tokens, block 64, head_dim 128 fp8 values plus one
    fp32 scale per token, 5/4 of the blocks needed, shuffled."""
    tag = "tiled" if layout == INDEXER_LAYOUT_TILED else "flat"
    pages = -(-tokens // 64)
    return make_indexer_workload(f"indexer_single_{tokens // 1024}k_{tag}", [tokens], 64, 128,
                                 pages * 5 // 4, seed, layout=layout)


def indexer_skew8(layout: int, seed: int) -> IndexerWorkload:
    """The skew-8 lengths as indexer sequences (block 64, head_dim 128), 3000
    shuffled blocks, 8 padding rows (token_to_seq -1) after the last sequence."""
    tag = "tiled" if layout == INDEXER_LAYOUT_TILED else "flat"
    return make_indexer_workload(f"indexer_skew8_{tag}", SKEW8_LENS, 64, 128, 3000, seed,
                                 layout=layout, pad_rows=8)


INDEXER_NAMED = {
    "indexer_tiny_flat": lambda: make_indexer_workload("indexer_tiny_flat", [17, 71, 0], 16, 128,
                                                        32, 1501, pad_rows=5),
    "indexer_tiny_tiled": lambda: make_indexer_workload("indexer_tiny_tiled", [17, 71, 0], 16, 128,
                                                         32, 1502, layout=INDEXER_LAYOUT_TILED,
                                                         pad_rows=5),
    "indexer_single_300k_flat": lambda: indexer_single(307200, INDEXER_LAYOUT_FLAT, 1503),
    "indexer_single_300k_tiled": lambda: indexer_single(307200, INDEXER_LAYOUT_TILED, 1504),
    "indexer_skew8_flat": lambda: indexer_skew8(INDEXER_LAYOUT_FLAT, 1505),
    "indexer_skew8_tiled": lambda: indexer_skew8(INDEXER_LAYOUT_TILED, 1506),
}
