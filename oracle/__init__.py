"""CPU oracle for the paged MLA KV-cache gather -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (the HIP library under
``paged_kv_cache_device_amd/`` and its binding) never imports, links or calls
it, and it shares no code with that path.

The arithmetic lives in ``oracle.c`` (plain single-threaded C, built with gcc
without fast-math); this module only compiles it and marshals arguments.  Every
function is pinned by ``tests/test_oracle_pins.py``; the header of ``oracle.c``
names the passages of the method each function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

MODE_COPY = 0
MODE_E4M3FN_TO_BF16 = 1


def compile_source(source: str, out: str) -> str:
    """gcc a C oracle source into a shared library (no fast-math, no contraction)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build() -> str:
    """Compile ``oracle.c`` into ``liboracle.so``."""
    return compile_source(SOURCE, LIBRARY)


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _as_i32(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


class Oracle:
    """ctypes marshalling around one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i32, i64, f32, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
        lib.oracle_e4m3fn_to_f32.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3fn_to_f32.restype = f32
        lib.oracle_f32_to_bf16_rne.argtypes = [f32]
        lib.oracle_f32_to_bf16_rne.restype = ctypes.c_uint16
        lib.oracle_dequant_e4m3fn_bf16.argtypes = [ctypes.c_uint8, f32]
        lib.oracle_dequant_e4m3fn_bf16.restype = ctypes.c_uint16
        lib.oracle_gather.argtypes = [i32, vp, i32, i64, i32, i32, i64, i64,
                                      vp, i32, i64, i64, vp, i32, i64, vp, i32, vp, i32, f32]
        lib.oracle_gather.restype = i64
        lib.oracle_page_tasks.argtypes = [vp, i32, vp, i32, i64, i32, vp, i64]
        lib.oracle_page_tasks.restype = i64
        lib.oracle_indexer_gather.argtypes = [vp, i64, i32, i64, i32, i32, i32, i32, vp, i64, vp,
                                              i64, i64, vp, vp, i32, vp, i32, i64]
        lib.oracle_indexer_gather.restype = i64
        self.lib = lib
        self.path = path

    # -- element functions -------------------------------------------------
    def e4m3fn_to_f32_bits(self, code: int) -> int:
        """fp32 bit pattern of the decoded code (keeps -0 and the NaN sign)."""
        v = ctypes.c_float(self.lib.oracle_e4m3fn_to_f32(code))
        return ctypes.c_uint32.from_buffer_copy(v).value

    def f32_bits_to_bf16_rne(self, bits: int) -> int:
        f = ctypes.c_float.from_buffer_copy(ctypes.c_uint32(bits & 0xFFFFFFFF))
        return int(self.lib.oracle_f32_to_bf16_rne(f))

    def dequant_e4m3fn_bf16(self, code: int, scale: float) -> int:
        return int(self.lib.oracle_dequant_e4m3fn_bf16(code, ctypes.c_float(scale)))

    # -- array functions (numpy in place) ------------------------------------
    def gather(self, mode: int, src_bytes: np.ndarray, src_elem_bytes: int, num_blocks: int,
               block_size: int, entry: int, src_block_stride: int, src_token_stride: int,
               dst_bytes: np.ndarray, dst_elem_bytes: int, num_tokens: int, dst_row_stride: int,
               block_table, block_table_width: int, block_table_ld: int,
               cu_seq_lens, seq_starts, num_reqs: int, scale: float = 1.0,
               terminal: bool = True) -> int:
        """Per-token oracle gather into ``dst_bytes`` (in place); returns rows written.

        ``src_bytes`` / ``dst_bytes`` are flat uint8 arrays starting at element
        (0, 0, 0) / (0, 0); strides are in elements of their own array.
        ``terminal``: cu_seq_lens holds num_reqs + 1 entries; otherwise
        num_reqs entries and the last request ends at num_tokens.
        """
        assert src_bytes.dtype == np.uint8 and dst_bytes.dtype == np.uint8
        bt = _as_i32(block_table)
        cu = _as_i32(cu_seq_lens)
        ss = _as_i32(seq_starts)
        assert cu.size >= num_reqs + (1 if terminal else 0)
        assert ss is None or ss.size >= num_reqs
        return int(self.lib.oracle_gather(
            mode, _ptr(src_bytes), src_elem_bytes, num_blocks, block_size, entry,
            src_block_stride, src_token_stride, _ptr(dst_bytes), dst_elem_bytes,
            num_tokens, dst_row_stride, _ptr(bt), block_table_width, block_table_ld,
            _ptr(cu), int(terminal), _ptr(ss), num_reqs, ctypes.c_float(scale)))

    def page_tasks(self, cu_seq_lens, seq_starts, num_reqs: int, num_tokens: int,
                   block_size: int, terminal: bool = True) -> np.ndarray:
        """Page tasks [num_tasks, 5] int32: (req_id, logical_block,
        page_token_begin, page_token_end, output_token_begin)."""
        cu = _as_i32(cu_seq_lens)
        ss = _as_i32(seq_starts)
        count = self.lib.oracle_page_tasks(_ptr(cu), int(terminal), _ptr(ss), num_reqs,
                                           num_tokens, block_size, None, 0)
        out = np.zeros((max(count, 1), 5), dtype=np.int32)
        self.lib.oracle_page_tasks(_ptr(cu), int(terminal), _ptr(ss), num_reqs, num_tokens,
                                   block_size, _ptr(out), count)
        return out[:count]

    def indexer_gather(self, cache: np.ndarray, num_blocks: int, block_size: int,
                       block_stride: int, layout: int, head_dim: int, block_tile: int,
                       head_tile: int, dst_values: np.ndarray, dst_value_stride: int,
                       dst_scales: np.ndarray, dst_scale_stride: int, num_tokens: int,
                       token_to_seq, cu_seqlen, num_batches: int, block_table,
                       block_table_width: int, block_table_ld: int) -> int:
        """Indexer quant-cache gather into ``dst_values`` / ``dst_scales`` (flat
        uint8 arrays, in place); strides in bytes.  Returns rows written."""
        for a in (cache, dst_values, dst_scales):
            assert a.dtype == np.uint8 and a.flags["C_CONTIGUOUS"]
        t2s = _as_i32(token_to_seq)
        cu = _as_i32(cu_seqlen)
        bt = _as_i32(block_table)
        assert t2s.size >= num_tokens
        return int(self.lib.oracle_indexer_gather(
            _ptr(cache), num_blocks, block_size, block_stride, layout, head_dim, block_tile,
            head_tile, _ptr(dst_values), dst_value_stride, _ptr(dst_scales), dst_scale_stride,
            num_tokens, _ptr(t2s), _ptr(cu), num_batches, _ptr(bt), block_table_width,
            block_table_ld))

    def gather_tensors(self, mode: int, src_cache, dst, block_table, cu_seq_lens, seq_starts,
                       num_reqs: int, scale: float = 1.0, terminal: bool = True) -> int:
        """Run the oracle on torch CPU tensors, writing ``dst`` in place.

        ``src_cache``: a (possibly strided) [num_blocks, block_size, entry] view;
        ``dst``: a (possibly strided) [num_tokens, entry] view; both with
        innermost stride 1.  Storage offsets of the views are honoured.
        """
        import torch  # CPU tensors only; used for storage access

        assert src_cache.device.type == "cpu" and dst.device.type == "cpu"
        assert src_cache.dim() == 3 and dst.dim() == 2
        assert src_cache.stride(2) == 1 and dst.stride(1) == 1
        num_blocks, block_size, entry = src_cache.shape
        assert dst.shape[1] == entry

        def flat_bytes(t):
            base = torch.empty(0, dtype=torch.uint8).set_(t.untyped_storage())
            off = t.storage_offset() * t.element_size()
            return base.numpy()[off:]

        bt = block_table.to(torch.int32).contiguous()
        return self.gather(
            mode, flat_bytes(src_cache), src_cache.element_size(), num_blocks, block_size,
            entry, src_cache.stride(0), src_cache.stride(1), flat_bytes(dst),
            dst.element_size(), dst.shape[0], dst.stride(0), bt.numpy(), bt.shape[1],
            bt.shape[1], cu_seq_lens.to(torch.int32).numpy(),
            None if seq_starts is None else seq_starts.to(torch.int32).numpy(),
            num_reqs, scale, terminal)


_default: Oracle | None = None


def load() -> Oracle:
    """The oracle built from ``oracle.c`` (compiled on first use if absent or stale)."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            build()
        _default = Oracle(LIBRARY)
    return _default


def run_workload(wl, ws=None):
    """Oracle gather for a ``workloads.Workload`` on CPU into the workspace ``ws``
    (default: a fresh sentinel-filled one).  Returns (workspace, rows written)."""
    import workloads

    o = load()
    ws = wl.fresh_workspace() if ws is None else ws
    dst_view = ws[: wl.num_tokens, : wl.entry]
    mode = MODE_E4M3FN_TO_BF16 if wl.kind in workloads.FP8_KINDS else MODE_COPY
    rows = o.gather_tensors(mode, wl.src_cache(), dst_view, wl.block_table, wl.cu_seq_lens,
                            wl.seq_starts, wl.num_reqs, wl.scale, wl.cu_terminal)
    return ws, rows


def run_indexer_workload(iw, values=None, scales=None):
    """Oracle indexer gather for a ``workloads.IndexerWorkload`` on CPU into the
    destinations ``values`` / ``scales`` (default: fresh sentinel-filled ones).
    Returns (values, scales, rows written)."""
    import torch

    o = load()
    values = iw.fresh_values() if values is None else values
    scales = iw.fresh_scales() if scales is None else scales
    assert values.is_contiguous() and scales.is_contiguous()
    rows = o.indexer_gather(
        iw.cache.numpy().reshape(-1), iw.num_blocks, iw.block_size, iw.block_stride, iw.layout,
        iw.head_dim, iw.block_tile, iw.head_tile, values.numpy().reshape(-1), values.stride(0),
        scales.view(torch.uint8).numpy().reshape(-1), 4 * scales.stride(0), iw.num_tokens,
        iw.token_to_seq.numpy(), iw.cu_seqlen.numpy(), iw.num_batches,
        iw.block_table.numpy(), iw.block_table_width, iw.block_table.shape[1])
    return values, scales, rows
