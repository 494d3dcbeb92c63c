"""Pins of the CPU oracle: checks of every oracle function against something
other than itself -- hand-worked cases from the method's definition, the OCP
FP8 specification, torch's own fp8 / bf16 casts (library routines), closed
forms, and a gather built by a different algorithm (the page-task method, and
torch advanced indexing).

Each ``check_*`` takes an ``oracle.Oracle`` and raises AssertionError on a
mismatch.  ``tests/test_oracle_pins.py`` runs them on the real oracle, and
``tests/test_oracle_mutants.py`` runs them on copies of the oracle with planted
mistakes, each of which must fail at least one check.
"""
from __future__ import annotations

import json
import math
import os
import struct

import numpy as np
import torch

import oracle as oracle_mod
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def _bits_f32(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", b & 0xFFFFFFFF))[0]


def _bf16_to_float(b: int) -> float:
    return _bits_f32(b << 16)


# ---------------------------------------------------------------------------
# fp8 decode
# ---------------------------------------------------------------------------

def _spec_value(s: str) -> float:
    if s == "nan":
        return math.nan
    if s == "-0":
        return -0.0
    if s.startswith("2^"):
        return 2.0 ** int(s[2:])
    if "*2^" in s:
        a, e = s.split("*2^")
        return float(a) * 2.0 ** int(e)
    return float(s)


def check_decode_spec_values(o):
    for item in _golden("e4m3fn_spec_values.json")["values"]:
        code = int(item["code"], 16)
        want = _spec_value(item["value"])
        got = _bits_f32(o.e4m3fn_to_f32_bits(code))
        if math.isnan(want):
            assert math.isnan(got), (item, got)
        else:
            assert _f32_bits(got) == _f32_bits(want), (item, got)


def check_decode_matches_torch(o):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).float()
    ref_bits = ref.view(torch.int32).tolist()
    for c in range(256):
        got = o.e4m3fn_to_f32_bits(c)
        if math.isnan(ref[c].item()):
            assert math.isnan(_bits_f32(got)), c
            assert (got >> 31) == (c >> 7), c
        else:
            assert got == (ref_bits[c] & 0xFFFFFFFF), (hex(c), hex(got), hex(ref_bits[c]))


# ---------------------------------------------------------------------------
# bf16 rounding
# ---------------------------------------------------------------------------

# (fp32 bits, bf16 bits), worked by hand from IEEE-754 round-to-nearest-even
BF16_HAND = [
    (0x3F808000, 0x3F80),  # tie, even kept
    (0x3F818000, 0x3F82),  # tie, odd rounds up
    (0x3F808001, 0x3F81),  # above tie
    (0x3F807FFF, 0x3F80),  # below tie
    (0xBF818000, 0xBF82),  # negative tie to even (magnitude up)
    (0x7F7FFFFF, 0x7F80),  # largest finite rounds to +inf
    (0xFF7FFFFF, 0xFF80),  # and to -inf
    (0x7F7F7FFF, 0x7F7F),  # largest finite bf16 stays
    (0x7F800000, 0x7F80),  # +inf
    (0x80000000, 0x8000),  # -0
    (0x00008000, 0x0000),  # subnormal tie to even zero
    (0x00018000, 0x0002),  # subnormal tie, odd up
    (0x3DCCCCCD, 0x3DCD),  # 0.1f
]


def check_bf16_hand(o):
    for bits, want in BF16_HAND:
        assert o.f32_bits_to_bf16_rne(bits) == want, (hex(bits), hex(want))
    for nan_bits in (0x7FC00000, 0x7F800001, 0xFF800001, 0x7FFFFFFF):
        got = o.f32_bits_to_bf16_rne(nan_bits)
        assert (got & 0x7F80) == 0x7F80 and (got & 0x7F) != 0, (hex(nan_bits), hex(got))


def check_bf16_matches_torch(o, n=20000, seed=7):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    ref = torch.from_numpy(bits.view(np.float32).copy()).bfloat16().view(torch.int16)
    ref = ref.numpy().astype(np.uint16)
    for b, r in zip(bits.tolist(), ref.tolist()):
        got = o.f32_bits_to_bf16_rne(b)
        f = _bits_f32(b)
        if math.isnan(f):
            assert math.isnan(_bf16_to_float(got)), hex(b)
        else:
            assert got == r, (hex(b), hex(got), hex(r))


# ---------------------------------------------------------------------------
# dequant chain
# ---------------------------------------------------------------------------

# 9.7 and 0.5395833 (as fp32) are scales where rounding the product to fp32
# first and then to bf16 differs from rounding the exact product to bf16 once
# (28 codes each), so the two-step chain itself is pinned.
SCALES = [0.0625, 0.05, 1.0, 3.0, 1e-3, -0.5, 7.62939453125e-06, 1.7e38, 9.7, 0.5395833253860474]


def torch_dequant(codes_u8: torch.Tensor, scale: float) -> torch.Tensor:
    """fp8 codes -> bf16 bits via torch's own casts (fp8 -> fp32, fp32 multiply, -> bf16)."""
    s = torch.tensor(scale, dtype=torch.float32)
    return (codes_u8.view(torch.float8_e4m3fn).float() * s).bfloat16().view(torch.int16)


def check_dequant_worked(o):
    for case in _golden("dequant_worked_values.json")["cases"]:
        got = o.dequant_e4m3fn_bf16(int(case["code"], 16), case["scale"])
        assert got == int(case["bf16"], 16), (case, hex(got))


def check_dequant_matches_torch(o):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    for scale in SCALES:
        ref = (torch_dequant(codes, scale).numpy().astype(np.uint16)).tolist()
        for c in range(256):
            got = o.dequant_e4m3fn_bf16(c, scale)
            if c in (0x7F, 0xFF):
                assert math.isnan(_bf16_to_float(got)), (c, scale)
            else:
                assert got == ref[c], (hex(c), scale, hex(got), hex(ref[c]))


def check_dequant_power_of_two_exact(o):
    # closed form: with scale 2^-4 the product is exact and has <= 4 significant
    # bits, so bf16(decode(code) * 2^-4) equals decode(code) / 16 exactly.
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    dec = codes.view(torch.float8_e4m3fn).double().tolist()
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        got = _bf16_to_float(o.dequant_e4m3fn_bf16(c, 0.0625))
        assert got == dec[c] / 16.0, (hex(c), got, dec[c])
        assert math.copysign(1.0, got) == math.copysign(1.0, dec[c])


# ---------------------------------------------------------------------------
# the gather: hand-worked cases
# ---------------------------------------------------------------------------

def check_gather_hand_worked(o):
    g = _golden("hand_worked_gather.json")
    nb, bs = 4, 2
    cache = np.array([[10 * pb + s for s in range(bs)] for pb in range(nb)], dtype=np.int16)
    for case in g["cases"]:
        bt = np.array(case["block_table"], dtype=np.int32)
        dst = np.full(4, g["sentinel"], dtype=np.int16)
        R = bt.shape[0]
        rows = o.gather(oracle_mod.MODE_COPY, cache.view(np.uint8).reshape(-1), 2, nb, bs, 1,
                        bs, 1, dst.view(np.uint8), 2, case["num_tokens"], 1, bt.reshape(-1),
                        case["width"], bt.shape[1], case["cu_seq_lens"], case["seq_starts"], R)
        assert dst.tolist() == case["expected"], (case["name"], dst.tolist())
        assert rows == case["rows_written"], (case["name"], rows)


def check_gather_open_end_hand_worked(o):
    g = _golden("hand_worked_gather.json")["open_end_cases"]
    nb, bs = 4, 2
    cache = np.array([[10 * pb + s for s in range(bs)] for pb in range(nb)], dtype=np.int16)
    for case in g["cases"]:
        bt = np.array(case["block_table"], dtype=np.int32)
        dst = np.full(case["rows"], g["sentinel"], dtype=np.int16)
        R = bt.shape[0]
        rows = o.gather(oracle_mod.MODE_COPY, cache.view(np.uint8).reshape(-1), 2, nb, bs, 1,
                        bs, 1, dst.view(np.uint8), 2, case["num_tokens"], 1, bt.reshape(-1),
                        case["width"], bt.shape[1], case["cu_seq_lens"], case["seq_starts"], R,
                        terminal=False)
        assert dst.tolist() == case["expected"], (case["name"], dst.tolist())
        assert rows == case["rows_written"], (case["name"], rows)


def check_gather_fp8_hand_worked(o):
    g = _golden("hand_worked_gather.json")["fp8_case"]
    cache = np.array([[[int(x, 16) for x in row] for row in blk] for blk in g["cache_codes"]],
                     dtype=np.uint8)
    nb, bs, e = cache.shape
    bt = np.array(g["block_table"], dtype=np.int32)
    n_out = len(g["expected"])
    dst = np.full((n_out, e), 0xFFFF, dtype=np.uint16)
    rows = o.gather(oracle_mod.MODE_E4M3FN_TO_BF16, cache.reshape(-1), 1, nb, bs, e, bs * e, e,
                    dst.view(np.uint8).reshape(-1), 2, n_out, e, bt.reshape(-1), bt.shape[1],
                    bt.shape[1], g["cu_seq_lens"], g["seq_starts"], bt.shape[0], g["scale"])
    want = [[int(x, 16) for x in row] for row in g["expected"]]
    assert dst.tolist() == want, dst.tolist()
    assert rows == n_out


# ---------------------------------------------------------------------------
# the gather vs independent formulations, on random small workloads
# ---------------------------------------------------------------------------

def random_small_workloads(seed: int, count: int):
    """Small seeded workloads spanning the cases the method has: partial first and
    last pages, seq_starts on/off, zero-length requests, aliased physical
    blocks, strided cache rows and destination rows, num_tokens clamping, raw
    bf16 / fp32 / byte entries and fp8 dequant, and guard-skipped pages."""
    out = []
    g = torch.Generator("cpu").manual_seed(seed)

    def ri(lo, hi):
        return int(torch.randint(lo, hi + 1, (1,), generator=g).item())

    kinds = [workloads.RAW, workloads.DEQUANT_FP8, workloads.UPCONVERT, workloads.DEQUANT_AUTO]
    for k in range(count):
        R = ri(1, 6)
        bs = [1, 2, 3, 16, 64][ri(0, 4)]
        lens = [0 if ri(0, 4) == 0 else ri(1, 3 * bs + 5) for _ in range(R)]
        use_starts = ri(0, 1) == 1
        starts = [ri(0, n) for n in lens] if use_starts else None
        entry = ri(1, 9)
        kind = kinds[k % 4]
        cache_dtype = [torch.bfloat16, torch.float32, torch.uint8][ri(0, 2)]
        pages = sum(-(-n // bs) for n in lens)
        alias = ri(0, 2) == 0
        nb = max(pages, 1) + ri(0, 4) if not alias else max([-(-n // bs) for n in lens] + [1]) + 1
        wl = workloads.make_workload(
            f"rand{seed}_{k}", kind, lens, bs, entry, nb, seed=seed * 1000 + k,
            starts=starts, cache_cols=entry + ri(0, 3), dst_cols=entry + ri(0, 3),
            workspace_rows=None, scale=[0.0625, 0.05, 3.0][ri(0, 2)], allow_alias=alias,
            cache_dtype=cache_dtype)
        total = int(wl.cu_seq_lens[-1])
        # clamp case: fewer destination rows than requested
        if ri(0, 3) == 0 and total > 0:
            T = ri(0, total)
            wl.num_tokens = T
            wl.workspace = wl.workspace[: max(T, 1)].clone()
        else:
            wl.workspace = torch.cat([wl.workspace, wl.fresh_workspace()[:2]])  # guard rows
        # open-ended cu_seq_lens: drop the terminal entry; the last request then
        # runs to num_tokens, which here is at most its terminal end
        if ri(0, 4) == 0:
            wl = wl.open_ended()
        # guard case: corrupt some table entries (out of range ids, -1)
        if ri(0, 3) == 0 and wl.block_table.numel() > 0:
            flat = wl.block_table.view(-1)
            i = ri(0, flat.numel() - 1)
            flat[i] = [nb, nb + 5, -1, -7][ri(0, 3)]
        out.append(wl)
    return out


def torch_indexing_reference(wl) -> torch.Tensor:
    """The pages' test formulation: per request, index the cache with the
    physical block of every source token (advanced indexing), then place the
    rows; tokens whose logical block or physical id is out of range are left out."""
    ws = wl.fresh_workspace()
    cache = wl.src_cache()
    bt = wl.block_table.long()
    W = bt.shape[1]
    cu = wl.cu_seq_lens.tolist()
    T = wl.num_tokens
    bs = wl.block_size
    R = wl.num_reqs
    for r in range(R):
        end = cu[r + 1] if (wl.cu_terminal or r + 1 < R) else T
        b = min(cu[r], T)
        n = max(min(end, T) - b, 0)
        s = 0 if wl.seq_starts is None else int(wl.seq_starts[r])
        tok = torch.arange(s, s + n)
        lb = tok // bs
        ok = lb < W
        pb = torch.full_like(tok, -1)
        pb[ok] = bt[r, lb[ok]]
        ok &= (pb >= 0) & (pb < wl.num_blocks)
        rows = torch.arange(b, b + n)[ok]
        vals = cache[pb[ok], (tok % bs)[ok]]
        if wl.kind in workloads.FP8_KINDS:
            vals = torch_dequant(vals.contiguous(), wl.scale).view(torch.bfloat16)
        ws[rows, : wl.entry] = vals
    return ws


def page_tasks_by_intersection(wl) -> list:
    """The page decomposition from interval arithmetic, request by request: the
    logical pages a request touches are those from floor(s / bs) up to
    ceil((s + n) / bs) (the page's count), and each page's copied slots are the
    intersection of the request's source interval [s, s + n) with the page's
    token interval [lb * bs, (lb + 1) * bs), computed for all of the request's
    pages at once.  This count yields one empty page for a request with n == 0
    whose start is not page-aligned; it is kept here (the method launches it)."""
    cu = wl.cu_seq_lens.tolist()
    T = wl.num_tokens
    bs = wl.block_size
    R = wl.num_reqs
    starts = [0] * R if wl.seq_starts is None else wl.seq_starts.tolist()
    tasks = []
    for r in range(R):
        b = min(cu[r], T)
        end = cu[r + 1] if (wl.cu_terminal or r + 1 < R) else T
        n = max(min(end, T) - b, 0)
        s = starts[r]
        lbs = np.arange(s // bs, -(-(s + n) // bs), dtype=np.int64)
        page_lo, page_hi = lbs * bs, (lbs + 1) * bs
        lo = np.clip(page_lo, s, s + n)
        hi = np.clip(page_hi, s, s + n)
        for lb, a, z, p0 in zip(lbs.tolist(), lo.tolist(), hi.tolist(), page_lo.tolist()):
            tasks.append((r, lb, a - p0, z - p0, b + (a - s)))
    return tasks


def pages_method_reference(wl) -> tuple[torch.Tensor, list]:
    """The page method: take the page decomposition of
    ``page_tasks_by_intersection`` and copy each page's slot range with one
    slice of the cache, the whole page at once.  A different algorithm from
    the per-token definition; the method claims the two give the same output."""
    ws = wl.fresh_workspace()
    cache = wl.src_cache()
    bt = wl.block_table.tolist()
    W = len(bt[0]) if bt else 0
    tasks = page_tasks_by_intersection(wl)
    for r, logical, pbeg, pend, obeg in tasks:
        if pend > pbeg and logical < W:
            phys = bt[r][logical]
            if 0 <= phys < wl.num_blocks:
                vals = cache[phys, pbeg:pend]
                if wl.kind in workloads.FP8_KINDS:
                    vals = torch_dequant(vals.contiguous(), wl.scale).view(torch.bfloat16)
                ws[obeg: obeg + (pend - pbeg), : wl.entry] = vals
    return ws, tasks


def _oracle_workspace(o, wl):
    ws = wl.fresh_workspace()
    mode = (oracle_mod.MODE_E4M3FN_TO_BF16 if wl.kind in workloads.FP8_KINDS
            else oracle_mod.MODE_COPY)
    rows = o.gather_tensors(mode, wl.src_cache(), ws[: wl.num_tokens, : wl.entry],
                            wl.block_table, wl.cu_seq_lens, wl.seq_starts, wl.num_reqs, wl.scale,
                            wl.cu_terminal)
    return ws, rows


def _same_bytes(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def check_gather_vs_torch_indexing(o, seed=11, count=60):
    for wl in random_small_workloads(seed, count):
        got, _ = _oracle_workspace(o, wl)
        want = torch_indexing_reference(wl)
        assert _same_bytes(got, want), wl.name


def check_gather_vs_page_method(o, seed=12, count=60):
    for wl in random_small_workloads(seed, count):
        got, _ = _oracle_workspace(o, wl)
        want, tasks = pages_method_reference(wl)
        assert _same_bytes(got, want), wl.name
        otasks = o.page_tasks(wl.cu_seq_lens, wl.seq_starts, wl.num_reqs, wl.num_tokens,
                              wl.block_size, wl.cu_terminal)
        # the oracle opens no task for a request without rows; the page count
        # gives such a request one empty page when its start is unaligned
        nonempty = [t for t in tasks if t[3] > t[2]]
        assert [tuple(x) for x in otasks.tolist()] == nonempty, wl.name


def check_self_identifying_invariants(o, seed=13, count=30):
    """Each cache element encodes (physical block, slot, column) in 32 bits; every
    written row must decode to the block the table names for its token, the slot
    t % bs, and columns 0..entry-1 in order; the count of written rows equals the
    requested rows (no guards fire here); rows outside every request extent keep
    the sentinel."""
    g = torch.Generator("cpu").manual_seed(seed)
    for k in range(count):
        R = int(torch.randint(1, 7, (1,), generator=g))
        bs = [1, 2, 16, 64][int(torch.randint(0, 4, (1,), generator=g))]
        lens = torch.randint(0, 4 * bs + 3, (R,), generator=g).tolist()
        starts = [int(torch.randint(0, n + 1, (1,), generator=g)) for n in lens]
        use_starts = k % 2 == 0
        entry = 5
        wl = workloads.make_workload("selfid", workloads.RAW, lens, bs, entry,
                                     max(sum(-(-n // bs) for n in lens), 1) + 2, seed=k,
                                     starts=starts if use_starts else None,
                                     cache_dtype=torch.float32)
        nb = wl.num_blocks
        ids = (torch.arange(nb).view(nb, 1, 1) * 65536 + torch.arange(bs).view(1, bs, 1) * 256
               + torch.arange(entry).view(1, 1, entry)).to(torch.int32)
        wl.cache_base = ids.view(torch.float32).clone()
        ws, rows = _oracle_workspace(o, wl)
        got = ws.view(torch.int32)
        cu = wl.cu_seq_lens.tolist()
        assert rows == cu[-1] == sum(max(n - (s if use_starts else 0), 0)
                                     for n, s in zip(lens, starts))
        touched = torch.zeros(ws.shape[0], dtype=torch.bool)
        for r in range(R):
            s = starts[r] if use_starts else 0
            for i in range(cu[r + 1] - cu[r]):
                t = s + i
                row = got[cu[r] + i].tolist()
                pb, slot = row[0] // 65536, (row[0] // 256) % 256
                assert pb == int(wl.block_table[r, t // bs]), (k, r, i)
                assert slot == t % bs
                assert [x % 256 for x in row] == list(range(entry))
                assert len({x // 256 for x in row}) == 1
                touched[cu[r] + i] = True
        assert bool((ws.view(torch.uint8)[~touched] == workloads.SENTINEL_BYTE).all())


# ---------------------------------------------------------------------------
# the page-task list: closed forms and coverage
# ---------------------------------------------------------------------------

def check_page_task_closed_forms(o):
    # single request of L tokens from 0 with block size bs: ceil(L / bs) tasks
    for L, bs, want in [(61440, 64, 960), (307200, 64, 4800), (17, 16, 2), (71, 16, 5),
                        (0, 16, 0), (1, 64, 1), (64, 64, 1), (65, 64, 2)]:
        n = len(o.page_tasks([0, L], None, 1, L, bs))
        assert n == want, (L, bs, n)
    # tiny uneven batch {17, 71, 0} with block 16: 2 + 5 + 0
    assert len(o.page_tasks([0, 17, 88, 88], None, 3, 88, 16)) == 7
    # seq_starts: [10, 110) over block 64 touches pages 0 and 1; [63, 65) too
    assert o.page_tasks([0, 100], [10], 1, 100, 64).tolist() == [[0, 0, 10, 64, 0],
                                                                [0, 1, 0, 46, 54]]
    assert o.page_tasks([0, 2], [63], 1, 2, 64).tolist() == [[0, 0, 63, 64, 0],
                                                            [0, 1, 0, 1, 1]]
    # a request with no rows opens no task, whether its start sits on a page
    # boundary or inside a page (where the page's count would give one empty task)
    assert len(o.page_tasks([0, 0], [64], 1, 0, 64)) == 0
    assert len(o.page_tasks([0, 0], [65], 1, 0, 64)) == 0
    assert o.page_tasks([0, 0, 3], [65, 2], 2, 3, 64).tolist() == [[1, 0, 2, 5, 0]]
    # clamp to num_tokens: 100 rows asked, 30 available; the second request is cut off
    assert o.page_tasks([0, 20, 100], [60, 0], 2, 30, 16).tolist() == [
        [0, 3, 12, 16, 0], [0, 4, 0, 16, 4], [1, 0, 0, 10, 20]]


def check_page_task_coverage(o, seed=14, count=200):
    """Every (request, source token) pair of every request extent is covered by
    exactly one task; each task stays inside one page; output rows follow."""
    g = torch.Generator("cpu").manual_seed(seed)
    for _ in range(count):
        R = int(torch.randint(1, 17, (1,), generator=g))
        bs = [1, 2, 5, 16, 64][int(torch.randint(0, 5, (1,), generator=g))]
        lens = torch.randint(0, 5 * bs + 2, (R,), generator=g)
        lens[torch.rand(R, generator=g) < 0.2] = 0
        starts = torch.randint(0, 3 * bs, (R,), generator=g)
        use = bool(torch.randint(0, 2, (1,), generator=g))
        cu = [0] + torch.cumsum(lens, 0).tolist()
        T = cu[-1] if torch.rand(1, generator=g) < 0.7 else int(torch.randint(0, cu[-1] + 1, (1,), generator=g))
        tasks = o.page_tasks(cu, starts.tolist() if use else None, R, T, bs)
        seen = set()
        for r, lb, pbeg, pend, obeg in tasks.tolist():
            assert 0 <= pbeg <= pend <= bs
            s = int(starts[r]) if use else 0
            for k in range(pbeg, pend):
                t = lb * bs + k
                key = (r, t)
                assert key not in seen
                seen.add(key)
                assert obeg + (k - pbeg) == min(cu[r], T) + (t - s)
        want = set()
        for r in range(R):
            s = int(starts[r]) if use else 0
            n = max(min(cu[r + 1], T) - min(cu[r], T), 0)
            want |= {(r, s + i) for i in range(n)}
        assert seen == want
        # one task per touched (request, logical page), none empty, in request
        # then page order: with the exact cover above this fixes the list
        keys = [(r, lb) for r, lb, _, _, _ in tasks.tolist()]
        assert keys == sorted(set(keys))
        assert all(pend > pbeg for _, _, pbeg, pend, _ in tasks.tolist())


# ---------------------------------------------------------------------------
# the indexer quant-cache gather
# ---------------------------------------------------------------------------

def check_indexer_hand_worked(o):
    g = _golden("indexer_hand_worked.json")
    nb, bs, hd, stride = g["num_blocks"], g["block_size"], g["head_dim"], g["block_stride"]
    cache = (np.arange(nb * stride) % 256).astype(np.uint8)  # block k byte i = 16k + i
    T = len(g["token_to_seq"])
    vs, ss = g["dst_value_stride"], g["dst_scale_stride_bytes"]
    bt = np.array(g["block_table"], dtype=np.int32)
    for case in g["cases"]:
        vals = np.full(T * vs, g["sentinel"], dtype=np.uint8)
        scal = np.full(T * ss, g["sentinel"], dtype=np.uint8)
        rows = o.indexer_gather(cache, nb, bs, stride, case["layout"], hd, case["block_tile"],
                                case["head_tile"], vals, vs, scal, ss, T, g["token_to_seq"],
                                g["cu_seqlen"], g["num_batches"], bt, case["block_table_width"],
                                bt.shape[1])
        assert rows == sum(v is not None for v in case["values"]), case["why"]
        for t in range(T):
            want_v = case["values"][t] or [g["sentinel"]] * hd
            want_s = case["scales"][t] or [g["sentinel"]] * 4
            assert vals[t * vs: t * vs + hd].tolist() == want_v, (case["why"], t)
            assert scal[t * ss: t * ss + 4].tolist() == want_s, (case["why"], t)
            # the pad byte of each value row and the second scale slot stay untouched
            assert vals[t * vs + hd] == g["sentinel"] and (scal[t * ss + 4:(t + 1) * ss] == 255).all()


def pack_indexer_records(values: np.ndarray, scales: np.ndarray, layout: int, block_tile: int,
                         head_tile: int, pad: int) -> np.ndarray:
    """Pack logical per-token values [NB, bs, D] (bytes) and scales [NB, bs, 4]
    (bytes) into block records: the value area (token-major, or tile after tile
    for the tiled layout, by numpy reshape/transpose), then the scales, then
    `pad` zero bytes."""
    nb, bs, hd = values.shape
    if layout == workloads.INDEXER_LAYOUT_FLAT:
        area = values.reshape(nb, bs * hd)
    else:
        t = values.reshape(nb, bs // block_tile, block_tile, hd // head_tile, head_tile)
        area = t.transpose(0, 1, 3, 2, 4).reshape(nb, bs * hd)
    return np.ascontiguousarray(np.concatenate(
        [area, scales.reshape(nb, bs * 4), np.zeros((nb, pad), dtype=np.uint8)], axis=1))


def check_indexer_vs_logical_tensors(o, seed=21, count=80):
    """Random indexer gathers on caches packed from logical value / scale
    tensors (both layouts, several tile shapes); the expected rows come from
    indexing the logical tensors with masks for the batch id, the row range,
    the table width and the block id, computed over all rows at once."""
    rng = np.random.default_rng(seed)
    for k in range(count):
        B = int(rng.integers(1, 6))
        bs = int(rng.choice([2, 4, 8, 16, 32]))
        hd = int(rng.choice([16, 32, 64]))
        layout = k % 2
        bt_, ht_ = (int(rng.choice([t for t in (1, 2, 4, 8, 16) if bs % t == 0])),
                    int(rng.choice([t for t in (1, 2, 4, 8, 16) if hd % t == 0])))
        lens = rng.integers(0, 4 * bs + 3, size=B)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        T = int(cu[-1]) + int(rng.integers(0, 4))
        t2s = np.full(T, -1, dtype=np.int64)
        for b in range(B):
            t2s[cu[b]:cu[b + 1]] = b
        # corruptions: padding ids, ids past the batch count, rows claiming another batch
        for _ in range(int(rng.integers(0, 4))):
            if T:
                t2s[int(rng.integers(0, T))] = int(rng.choice([-1, -5, B, B + 3, int(rng.integers(0, B))]))
        # a batch's first row claiming the previous batch, just past that batch's rows
        for b in range(1, B):
            if lens[b] and rng.random() < 0.5:
                t2s[cu[b]] = b - 1
        W = max(int(-(-lens.max() // bs)), 1)
        width = W if rng.random() < 0.7 else int(rng.integers(0, W + 1))
        ld = W + int(rng.integers(0, 3))
        nb = int(rng.integers(1, 3 * W + 2))
        # one more batch in the arrays than num_batches: ids >= B must not reach it
        table = rng.integers(-2, nb + 2, size=(B + 1, ld)).astype(np.int32)
        cu_arr = np.concatenate([cu, [cu[-1] + T + 1]])
        vals = rng.integers(0, 256, size=(nb, bs, hd), dtype=np.uint8)
        scl = rng.integers(0, 256, size=(nb, bs, 4), dtype=np.uint8)
        pad = int(rng.choice([0, 4, 16]))
        cache = pack_indexer_records(vals, scl, layout, bt_, ht_, pad)
        stride = cache.shape[1]
        vs, ss = hd + int(rng.integers(0, 3)), 4 * int(rng.integers(1, 3))
        got_v = np.full((T, vs), 0xAB, dtype=np.uint8)
        got_s = np.full((T, ss), 0xCD, dtype=np.uint8)
        rows = o.indexer_gather(cache.reshape(-1), nb, bs, stride, layout, hd, bt_, ht_,
                                got_v.reshape(-1), vs, got_s.reshape(-1), ss, T,
                                t2s.astype(np.int32), cu_arr.astype(np.int32), B, table, width, ld)
        # expected, all rows at once
        tid = np.arange(T)
        ok = (t2s >= 0) & (t2s < B)
        b = np.where(ok, t2s, 0)
        start, end = cu[b], cu[b + 1]
        ok &= (tid >= start) & (tid < end)
        pos = np.where(ok, tid - start, 0)
        col, off = pos // bs, pos % bs
        ok &= col < width
        blk = np.where(ok, table[b, np.minimum(col, ld - 1)], -1)
        ok &= (blk >= 0) & (blk < nb)
        want_v = np.full((T, vs), 0xAB, dtype=np.uint8)
        want_s = np.full((T, ss), 0xCD, dtype=np.uint8)
        want_v[ok, :hd] = vals[blk[ok], off[ok]]
        want_s[ok, :4] = scl[blk[ok], off[ok]]
        assert rows == int(ok.sum()), k
        assert np.array_equal(got_v, want_v), (k, layout, bs, hd, bt_, ht_)
        assert np.array_equal(got_s, want_s), (k, layout, bs, hd)


ALL_CHECKS = [
    check_decode_spec_values, check_decode_matches_torch, check_bf16_hand,
    check_bf16_matches_torch, check_dequant_worked, check_dequant_matches_torch,
    check_dequant_power_of_two_exact, check_gather_hand_worked, check_gather_open_end_hand_worked,
    check_gather_fp8_hand_worked,
    check_gather_vs_torch_indexing, check_gather_vs_page_method,
    check_self_identifying_invariants, check_page_task_closed_forms, check_page_task_coverage,
    check_indexer_hand_worked, check_indexer_vs_logical_tensors,
]
