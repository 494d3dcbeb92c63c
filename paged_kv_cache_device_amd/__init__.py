"""paged_kv_cache_device_amd -- paged MLA KV-cache gather on AMD Instinct MI355X.

Thin Python binding over ``libpkvg.so`` (C ABI in ``include/pkvg.h``).  This
module only marshals torch tensors into pointers, sizes and strides and passes
the current HIP stream; every step of the gather runs in the library's HIP
kernels.  torch is used for device memory and streams only.  There is no CPU
or PyTorch fallback: if the library is missing or a call fails, an exception
is raised.

Entry points (names as in the C ABI):

* ``gather_cache(src_cache, dst, block_table, cu_seq_lens, batch_size, seq_starts=None)``
* ``gather_maybe_dequant(src_cache, dst, block_table, cu_seq_lens, batch_size,
  kv_cache_dtype, scale=None, seq_starts=None)``
* ``gather_upconvert_fp8(src_cache, dst, block_table, cu_seq_lens, batch_size, scale,
  seq_starts=None)``
* ``gather_page_tasks(cu_seq_lens, seq_starts, batch_size, num_tokens, block_size,
  block_table, num_blocks, capacity=None)``
* ``pkvg_plan(op, kind, ...)``: how a call would run (kernel, shape, task units,
  grid), from plain sizes, strides and addresses; nothing is enqueued
* ``gather_indexer_quant_cache(cache, dst_values, dst_scales, token_to_seq,
  cu_seqlen, block_table, block_size, layout='flat', ...)``: the indexer
  quant-cache gather (per output row, keyed by ``token_to_seq``)

``src_cache`` is a [num_blocks, block_size, entry] view (innermost stride 1;
a view of wider rows is fine), ``dst`` a [num_tokens, entry] view (innermost
stride 1), ``block_table`` int32 [batch, width] (row stride >= width),
``cu_seq_lens`` int32 [batch + 1], ``seq_starts`` int32 [batch] or None.
A ``cu_seq_lens`` of exactly ``batch`` entries (or ``cu_terminal=False``)
means the open-ended convention: the last request ends at ``num_tokens``.
"""
from __future__ import annotations

import ctypes
import os

import torch  # imported first: the library binds to the HIP runtime torch has loaded

from . import build as _build

LIBRARY = _build.LIBRARY

PKVG_OK = 0
PKVG_E_NULL = 1
PKVG_E_SHAPE = 2
PKVG_E_STRIDE = 3
PKVG_E_DTYPE = 4
PKVG_E_LIMIT = 5
PKVG_E_HIP = 6
PKVG_E_SCRATCH = 7
PKVG_NOALLOC_MAX_REQS = 65535
PKVG_NOALLOC_MAX_TASKS = 262144
PKVG_KV_AUTO = 0
PKVG_KV_FP8_E4M3 = 1
PKVG_TASK_INTS = 8
PKVG_OP_GATHER_CACHE = 0
PKVG_OP_GATHER_MAYBE_DEQUANT = 1
PKVG_OP_GATHER_UPCONVERT_FP8 = 2
PKVG_KERNEL_PAGES = 0
PKVG_KERNEL_GROUPS = 1
PKVG_TASKS_WAVE = 0
PKVG_TASKS_LDS = 1
PKVG_TASKS_TABLE = 2
PKVG_TASKS_SINGLE = 3
PKVG_TASKS_WALK = 4
PKVG_INDEXER_FLAT = 0
PKVG_INDEXER_TILED = 1

# the C entry points and their argument types, as declared in include/pkvg.h
_i32, _i64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
_CACHE_ARGS = [_i64, _i32, _i32, _i64, _i64, _vp, _i64, _i64, _vp, _i32, _i64, _vp, _i32, _vp, _i32]
SIGNATURES = {
    "gather_cache": [_vp, _i32] + _CACHE_ARGS + [_vp],
    "gather_maybe_dequant": [_vp, _i32] + _CACHE_ARGS + [_vp, _vp],
    "gather_maybe_dequant_noalloc": [_vp, _i32] + _CACHE_ARGS + [_vp, _vp],
    "gather_upconvert_fp8": [_vp] + _CACHE_ARGS + [_vp, _vp],
    "gather_page_tasks": [_vp, _i32, _vp, _i32, _i64, _i32, _vp, _i32, _i64, _i64, _vp, _i64, _vp,
                          _vp],
    "pkvg_plan": [_i32, _i32, _vp] + _CACHE_ARGS + [_vp, _vp],
    "gather_indexer_quant_cache": [_vp, _i64, _i32, _i64, _i32, _i32, _i32, _i32, _vp, _i64, _vp,
                                   _i64, _i64, _vp, _vp, _i32, _vp, _i32, _i64, _vp],
    "pkvg_status_string": [ctypes.c_int],
    "pkvg_last_hip_error": [],
}


class PlanInfo(ctypes.Structure):
    """pkvg_plan_info of include/pkvg.h."""
    _fields_ = [(n, ctypes.c_int32) for n in (
        "kernel", "threads", "batch_bytes", "task_mode", "convert", "access_width", "flat",
        "src_vector", "task_tokens", "split_shift", "group_shift", "grid_rows")] + [
        ("grid", ctypes.c_int64), ("task_capacity", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}


class PkvgError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {status_string(status)}"
        if status == PKVG_E_HIP:
            msg += f" (hipError {library().pkvg_last_hip_error()})"
        super().__init__(msg)


_lib = None


def library(path: str | None = None) -> ctypes.CDLL:
    """Load ``libpkvg.so`` (built in-tree by ``__graft_entry__.build()`` or
    ``python -m paged_kv_cache_device_amd.build``).  Raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIBRARY
    if not os.path.exists(p):
        raise ImportError(
            f"{p} is not built; run `python -m paged_kv_cache_device_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(p)
    for name, args in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "pkvg_status_string" else ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return library().pkvg_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != PKVG_OK:
        raise PkvgError(status, where)


def _stream_handle() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _device_i32(t: torch.Tensor | None, name: str, dim: int) -> torch.Tensor | None:
    if t is None:
        return None
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != dim:
        raise ValueError(f"{name} must be {dim}-D")
    if dim == 1 and t.stride(0) != 1:
        raise ValueError(f"{name} must be contiguous")
    if dim == 2 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit innermost stride")
    return t


def _same_device(named) -> None:
    """Every tensor on one device, and that device current: the library
    launches on the current device's stream with the tensors' raw pointers."""
    named = [(n, t) for n, t in named if t is not None]
    dev = named[0][1].device
    for n, t in named[1:]:
        if t.device != dev:
            raise ValueError(f"{n} is on {t.device}, {named[0][0]} on {dev}")
    if dev.index is not None and dev.index != torch.cuda.current_device():
        raise ValueError(f"the tensors are on {dev}, the current device is cuda:{torch.cuda.current_device()}")


def _terminal(cu_seq_lens: torch.Tensor, batch_size: int, cu_terminal) -> int:
    """1 when cu_seq_lens carries a terminal entry, 0 when the last request runs
    to num_tokens; by default decided by its length."""
    if cu_terminal is None:
        cu_terminal = cu_seq_lens.numel() != batch_size
    need = batch_size + (1 if cu_terminal else 0)
    if cu_seq_lens.numel() < need:
        raise ValueError(f"cu_seq_lens needs {need} entries")
    return 1 if cu_terminal else 0


def _cache_args(src_cache, dst, block_table, cu_seq_lens, batch_size, seq_starts,
                cu_terminal=None):
    for name, t, d in (("src_cache", src_cache, 3), ("dst", dst, 2)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.dim() != d:
            raise ValueError(f"{name} must be {d}-D")
        if t.stride(-1) != 1:
            raise ValueError(f"{name} must have unit innermost stride")
    _device_i32(block_table, "block_table", 2)
    _device_i32(cu_seq_lens, "cu_seq_lens", 1)
    _device_i32(seq_starts, "seq_starts", 1)
    num_blocks, block_size, entry = src_cache.shape
    if dst.shape[1] != entry:
        raise ValueError(f"dst has {dst.shape[1]} columns, cache rows gather {entry}")
    terminal = _terminal(cu_seq_lens, batch_size, cu_terminal)
    if block_table.shape[0] < batch_size:
        raise ValueError("block_table needs batch_size rows")
    if seq_starts is not None and seq_starts.numel() < batch_size:
        raise ValueError("seq_starts needs batch_size entries")
    _same_device([("dst", dst), ("src_cache", src_cache), ("block_table", block_table),
                  ("cu_seq_lens", cu_seq_lens), ("seq_starts", seq_starts)])
    return [num_blocks, block_size, entry, src_cache.stride(0), src_cache.stride(1),
            _ptr(dst), dst.shape[0], dst.stride(0), _ptr(block_table), block_table.shape[1],
            block_table.stride(0), _ptr(cu_seq_lens), terminal, _ptr(seq_starts), batch_size]


class PreparedCall:
    """A library call with its arguments already marshalled (pointers, sizes,
    strides and the stream), for loops that issue the same gather many times.
    Calling it enqueues the gather; the tensors it was prepared from must stay
    alive and unchanged in shape."""

    def __init__(self, name: str, args: list):
        self._fn = getattr(library(), name)
        self._args = args
        self._name = name

    def __call__(self) -> None:
        status = self._fn(*self._args)
        if status != PKVG_OK:
            raise PkvgError(status, self._name)


def _prepare_cache(src_cache, dst, block_table, cu_seq_lens, batch_size, seq_starts, stream,
                   cu_terminal=None):
    if src_cache.element_size() != dst.element_size():
        raise TypeError("gather_cache copies bits: cache and dst element sizes must match")
    args = _cache_args(src_cache, dst, block_table, cu_seq_lens, batch_size, seq_starts,
                       cu_terminal)
    return PreparedCall("gather_cache", [_ptr(src_cache), src_cache.element_size(), *args,
                                         _stream_handle() if stream is None else stream])


def _fp8_source(src_cache: torch.Tensor) -> None:
    if src_cache.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError(f"an fp8 cache must be uint8 or float8_e4m3fn, got {src_cache.dtype}")


def _scale_tensor(scale, dst: torch.Tensor) -> torch.Tensor:
    if not isinstance(scale, torch.Tensor) or scale.dtype != torch.float32 or not scale.is_cuda:
        raise TypeError("scale must be a float32 device tensor with one element")
    if scale.numel() < 1:
        raise ValueError("scale must hold one element")
    if scale.device != dst.device:
        raise ValueError(f"scale is on {scale.device}, dst on {dst.device}")
    return scale


def _prepare_maybe_dequant(src_cache, dst, block_table, cu_seq_lens, batch_size, kv_cache_dtype,
                           scale, seq_starts, stream, cu_terminal=None,
                           entry_point="gather_maybe_dequant"):
    if dst.dtype != torch.bfloat16:
        raise TypeError("gather_maybe_dequant writes a bf16 destination")
    if kv_cache_dtype == "auto":
        if src_cache.dtype != torch.bfloat16:
            raise TypeError("kv_cache_dtype 'auto' needs a bf16 cache")
        code, sc = PKVG_KV_AUTO, None
    elif kv_cache_dtype in ("fp8", "fp8_e4m3"):
        _fp8_source(src_cache)
        code, sc = PKVG_KV_FP8_E4M3, _scale_tensor(scale, dst)
    else:
        raise ValueError(f"unknown kv_cache_dtype {kv_cache_dtype!r}")
    args = _cache_args(src_cache, dst, block_table, cu_seq_lens, batch_size, seq_starts,
                       cu_terminal)
    return PreparedCall(entry_point, [_ptr(src_cache), code, *args, _ptr(sc),
                                      _stream_handle() if stream is None else stream])


def _prepare_upconvert(src_cache, dst, block_table, cu_seq_lens, batch_size, scale, seq_starts,
                       stream, cu_terminal=None):
    if dst.dtype != torch.bfloat16:
        raise TypeError("gather_upconvert_fp8 writes a bf16 destination")
    _fp8_source(src_cache)
    sc = _scale_tensor(scale, dst)
    args = _cache_args(src_cache, dst, block_table, cu_seq_lens, batch_size, seq_starts,
                       cu_terminal)
    return PreparedCall("gather_upconvert_fp8", [_ptr(src_cache), *args, _ptr(sc),
                                                 _stream_handle() if stream is None else stream])


def gather_cache(src_cache: torch.Tensor, dst: torch.Tensor, block_table: torch.Tensor,
                 cu_seq_lens: torch.Tensor, batch_size: int,
                 seq_starts: torch.Tensor | None = None, *, cu_terminal: bool | None = None) -> None:
    """Raw gather: dst rows = cache rows, bit for bit (same element size)."""
    _prepare_cache(src_cache, dst, block_table, cu_seq_lens, batch_size, seq_starts, None,
                   cu_terminal)()


def gather_maybe_dequant(src_cache: torch.Tensor, dst: torch.Tensor, block_table: torch.Tensor,
                         cu_seq_lens: torch.Tensor, batch_size: int, kv_cache_dtype: str,
                         scale: torch.Tensor | None = None,
                         seq_starts: torch.Tensor | None = None, *,
                         cu_terminal: bool | None = None) -> None:
    """Gather into a bf16 dst; kv_cache_dtype 'auto' copies a bf16 cache,
    'fp8' dequantises e4m3fn codes with the per-tensor fp32 ``scale``."""
    _prepare_maybe_dequant(src_cache, dst, block_table, cu_seq_lens, batch_size, kv_cache_dtype,
                           scale, seq_starts, None, cu_terminal)()


def gather_maybe_dequant_noalloc(src_cache: torch.Tensor, dst: torch.Tensor,
                                 block_table: torch.Tensor, cu_seq_lens: torch.Tensor,
                                 batch_size: int, kv_cache_dtype: str,
                                 scale: torch.Tensor | None = None,
                                 seq_starts: torch.Tensor | None = None, *,
                                 cu_terminal: bool | None = None) -> None:
    """``gather_maybe_dequant`` that allocates nothing: batches of more than
    1,024 requests keep their task table in the library's fixed device array
    (calls that overlap on one device race on it; see include/pkvg.h)."""
    _prepare_maybe_dequant(src_cache, dst, block_table, cu_seq_lens, batch_size, kv_cache_dtype,
                           scale, seq_starts, None, cu_terminal,
                           entry_point="gather_maybe_dequant_noalloc")()


def gather_upconvert_fp8(src_cache: torch.Tensor, dst: torch.Tensor, block_table: torch.Tensor,
                         cu_seq_lens: torch.Tensor, batch_size: int, scale: torch.Tensor,
                         seq_starts: torch.Tensor | None = None, *,
                         cu_terminal: bool | None = None) -> None:
    """fp8 (e4m3fn) cache -> bf16 dst: bf16_rne(fp32(code) * scale)."""
    _prepare_upconvert(src_cache, dst, block_table, cu_seq_lens, batch_size, scale, seq_starts,
                       None, cu_terminal)()


def prepare(entry_point: str, *args, **kwargs) -> PreparedCall:
    """Marshal the arguments of ``gather_cache`` / ``gather_maybe_dequant`` /
    ``gather_maybe_dequant_noalloc`` / ``gather_upconvert_fp8`` once, on the
    current stream (the same arguments as the function of that name); returns
    a callable that enqueues the call."""
    stream = None
    if entry_point == "gather_cache":
        return _prepare_cache(*args, **kwargs, stream=stream)
    if entry_point in ("gather_maybe_dequant", "gather_maybe_dequant_noalloc"):
        kwargs.setdefault("scale", None)
        kwargs.setdefault("seq_starts", None)
        return _prepare_maybe_dequant(*args, **kwargs, stream=stream, entry_point=entry_point)
    if entry_point == "gather_upconvert_fp8":
        kwargs.setdefault("seq_starts", None)
        return _prepare_upconvert(*args, **kwargs, stream=stream)
    raise ValueError(entry_point)


def gather_page_tasks(cu_seq_lens: torch.Tensor, seq_starts: torch.Tensor | None,
                      batch_size: int, num_tokens: int, block_size: int,
                      block_table: torch.Tensor, num_blocks: int,
                      capacity: int | None = None, *, cu_terminal: bool | None = None):
    """Run the page-task builder alone.  Returns (tasks int32 [capacity, 8],
    count int32 [1]), both on the device; rows past count are unspecified."""
    _device_i32(block_table, "block_table", 2)
    _device_i32(cu_seq_lens, "cu_seq_lens", 1)
    _device_i32(seq_starts, "seq_starts", 1)
    _same_device([("cu_seq_lens", cu_seq_lens), ("block_table", block_table), ("seq_starts", seq_starts)])
    if capacity is None:
        capacity = num_tokens // block_size + 2 * batch_size + 1
    dev = cu_seq_lens.device
    tasks = torch.empty((max(capacity, 1), PKVG_TASK_INTS), dtype=torch.int32, device=dev)
    count = torch.empty(1, dtype=torch.int32, device=dev)
    terminal = _terminal(cu_seq_lens, batch_size, cu_terminal)
    _check(library().gather_page_tasks(
        _ptr(cu_seq_lens), terminal, _ptr(seq_starts), batch_size, num_tokens, block_size,
        _ptr(block_table), block_table.shape[1], block_table.stride(0), num_blocks,
        _ptr(tasks), capacity, _ptr(count), _stream_handle()), "gather_page_tasks")
    return tasks[:capacity], count


def pkvg_plan(op: int, kind: int, src: int, num_blocks: int, block_size: int, entry: int,
              src_block_stride: int, src_token_stride: int, dst: int, num_tokens: int,
              dst_row_stride: int, block_table: int | None, block_table_width: int,
              block_table_ld: int, cu_seq_lens: int, cu_terminal: int, seq_starts: int | None,
              num_reqs: int, scale: int | None) -> dict:
    """How a gather call with these arguments would run (``pkvg_plan`` of the C
    ABI): addresses are plain integers, checked for NULL and alignment only and
    never read, so this needs no device.  Raises PkvgError with the status the
    call itself would return."""
    info = PlanInfo()
    _check(library().pkvg_plan(op, kind, src, num_blocks, block_size, entry, src_block_stride,
                               src_token_stride, dst, num_tokens, dst_row_stride, block_table,
                               block_table_width, block_table_ld, cu_seq_lens, cu_terminal,
                               seq_starts, num_reqs, scale, ctypes.byref(info)), "pkvg_plan")
    return info.as_dict()


_INDEXER_LAYOUTS = {"flat": PKVG_INDEXER_FLAT, "tiled": PKVG_INDEXER_TILED}


def prepare_indexer(cache: torch.Tensor, dst_values: torch.Tensor, dst_scales: torch.Tensor,
                    token_to_seq: torch.Tensor, cu_seqlen: torch.Tensor, block_table: torch.Tensor,
                    block_size: int, layout: str = "flat", *, block_tile: int = 16,
                    head_tile: int = 16, num_batches: int | None = None,
                    block_table_width: int | None = None) -> PreparedCall:
    """Marshal one ``gather_indexer_quant_cache`` call on the current stream.

    ``cache``: uint8 [num_blocks, block_stride] (unit inner stride) of packed
    block records; ``dst_values``: uint8 [num_tokens, head_dim] view (unit
    inner stride; head_dim is its column count); ``dst_scales``: float32
    [num_tokens] (any positive stride); ``token_to_seq``: int32 [num_tokens];
    ``cu_seqlen``: int32 [num_batches + 1]; ``block_table``: int32
    [num_batches, >= width]."""
    if cache.dtype != torch.uint8 or cache.dim() != 2 or cache.stride(1) != 1 or not cache.is_cuda:
        raise ValueError("cache must be a uint8 [num_blocks, block_stride] device tensor")
    if (dst_values.dtype != torch.uint8 or dst_values.dim() != 2 or dst_values.stride(1) != 1
            or not dst_values.is_cuda):
        raise ValueError("dst_values must be a uint8 [num_tokens, head_dim] device view")
    if dst_scales.dtype != torch.float32 or dst_scales.dim() != 1 or not dst_scales.is_cuda:
        raise ValueError("dst_scales must be a float32 [num_tokens] device tensor")
    _device_i32(token_to_seq, "token_to_seq", 1)
    _device_i32(cu_seqlen, "cu_seqlen", 1)
    _device_i32(block_table, "block_table", 2)
    T = dst_values.shape[0]
    if dst_scales.shape[0] != T or token_to_seq.numel() < T:
        raise ValueError("dst_scales and token_to_seq need num_tokens entries")
    nb = cu_seqlen.numel() - 1 if num_batches is None else num_batches
    if cu_seqlen.numel() < nb + 1 or block_table.shape[0] < nb:
        raise ValueError("cu_seqlen needs num_batches + 1 entries and block_table num_batches rows")
    if layout not in _INDEXER_LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(_INDEXER_LAYOUTS)}")
    width = block_table.shape[1] if block_table_width is None else block_table_width
    _same_device([("cache", cache), ("dst_values", dst_values), ("dst_scales", dst_scales),
                  ("token_to_seq", token_to_seq), ("cu_seqlen", cu_seqlen),
                  ("block_table", block_table)])
    return PreparedCall("gather_indexer_quant_cache", [
        _ptr(cache), cache.shape[0], block_size, cache.stride(0), _INDEXER_LAYOUTS[layout],
        dst_values.shape[1], block_tile, head_tile, _ptr(dst_values), dst_values.stride(0),
        _ptr(dst_scales), dst_scales.stride(0), T, _ptr(token_to_seq), _ptr(cu_seqlen), nb,
        _ptr(block_table), width, block_table.stride(0), _stream_handle()])


def gather_indexer_quant_cache(cache, dst_values, dst_scales, token_to_seq, cu_seqlen, block_table,
                               block_size: int, layout: str = "flat", **kwargs) -> None:
    """Indexer quant-cache gather: rows of ``dst_values`` / ``dst_scales`` whose
    batch, extent, table column and block are valid take their token's value
    bytes and fp32 scale from the packed cache; other rows are untouched."""
    prepare_indexer(cache, dst_values, dst_scales, token_to_seq, cu_seqlen, block_table,
                    block_size, layout, **kwargs)()
