// pkvg_capi.hip -- host side of libpkvg.so: argument validation, access-width
// and layout selection, launch.  The C ABI is declared in include/pkvg.h.
//
// Every argument check happens before the first HIP call, so a rejected call
// enqueues nothing and touches no device.  Nothing here synchronises with the
// device; launches go to the caller's stream.
#include "pkvg.h"
#include "gather_kernels.hpp"
#include "indexer_kernels.hpp"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

// Scratch of the no-allocation entry point (gather_maybe_dequant_noalloc):
// room for the task table of a batch of up to 65,535 requests and 262,144
// task units (P and count: 260 KiB; records: 8 MiB).  Each device the library
// runs on holds its own copy until the process ends.  In host code `scratch`
// names a host-side stand-in, not a device address: its device address comes
// from hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kNoAllocScratchBytes = (size_t(260) << 10) + (size_t(8) << 20);
static_assert(kNoAllocScratchBytes >= 4 * (size_t(PKVG_NOALLOC_MAX_REQS) + 2) + 255 + 32 * size_t(PKVG_NOALLOC_MAX_TASKS),
              "the scratch holds the header's largest task table");
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

using pkvg::GatherParams;
using pkvg::TaskRecord;

static_assert(pkvg::kFusedMaxReqs == PKVG_FUSED_MAX_REQS, "the fused task paths cover the header's batch limit");
static_assert(pkvg::kIndexerFlat == PKVG_INDEXER_FLAT && pkvg::kIndexerTiled == PKVG_INDEXER_TILED,
              "the header's indexer layout codes are the kernel's");
static_assert(pkvg::kWaveRegs == PKVG_TASKS_WAVE && pkvg::kLdsPrefix == PKVG_TASKS_LDS &&
                  pkvg::kTable == PKVG_TASKS_TABLE && pkvg::kSingle == PKVG_TASKS_SINGLE &&
                  pkvg::kWalk == PKVG_TASKS_WALK,
              "the header's task-mode codes are the kernel's");

thread_local int g_last_hip_error = 0;

// Workgroups launched: one per task up to this cap (32 times the workgroups
// the chip holds at once); any grid is correct because workgroups stride over
// tasks, and beyond the cap they do.
constexpr int64_t kMaxGrid = int64_t(1) << 16;

int hip_fail(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return PKVG_E_HIP;
}

uint32_t magic_for(uint32_t d) {
  if (d <= 1) return 0xFFFFFFFFu;
  return static_cast<uint32_t>(((uint64_t(1) << 32) + d - 1) / d);
}

bool aligned(const void* p, int64_t a) { return (reinterpret_cast<uintptr_t>(p) % static_cast<uint64_t>(a)) == 0; }

// A validated gather, strides in bytes.
struct Plan {
  GatherParams p{};
  int convert = pkvg::kCopy;
  int width = 1;          // bytes per lane access (copy) or codes per lane access (fp8)
  int layout = pkvg::kRows;
  bool src_vec = true;
  int32_t mode = pkvg::kSingle;  // TaskMode
  int32_t rule_reqs = 1;  // the batch size the unit and shape rules see (1 for a table walk)
  int64_t capacity = 0;   // upper bound on the number of page tasks
  int64_t grid = 0;       // workgroups launched along x (per table row for a walk)
  int64_t grid_rows = 1;  // along y: the requests for a walk, else 1
  int shape = 0;          // workgroup shape (ShapeId)
};

enum ShapeId : int { kShapeSmall = 0, kShapeMid = 1, kShapeNarrow = 2, kShapeWide = 3 };

// Checks shared by every gather entry point.  Returns PKVG_OK or an error
// code; `*nothing` is set when there is no work (nothing is launched then).
int check_common(const void* src, int64_t num_blocks, int32_t block_size, int32_t entry,
                 int64_t src_block_stride, int64_t src_token_stride, void* dst,
                 int64_t num_tokens, int64_t dst_row_stride, const int32_t* block_table,
                 int32_t block_table_width, int64_t block_table_ld, const int32_t* cu_seq_lens,
                 int32_t cu_terminal, int32_t num_reqs, bool* nothing) {
  *nothing = false;
  if (num_reqs < 0 || num_tokens < 0 || num_blocks < 0 || block_table_width < 0) return PKVG_E_SHAPE;
  if (cu_terminal != 0 && cu_terminal != 1) return PKVG_E_SHAPE;
  if (block_size <= 0 || entry <= 0) return PKVG_E_SHAPE;
  if (src_block_stride < 0 || src_token_stride < 0 || dst_row_stride < entry ||
      block_table_ld < block_table_width)
    return PKVG_E_STRIDE;
  if (num_reqs == 0 || num_tokens == 0) {
    *nothing = true;
    return PKVG_OK;
  }
  // a table with no columns is never read (every page fails the width guard)
  if (!src || !dst || !cu_seq_lens || (!block_table && block_table_width > 0)) return PKVG_E_NULL;
  // output rows are int32, like the cu_seq_lens entries that address them
  if (num_tokens > INT32_MAX) return PKVG_E_LIMIT;
  // page tasks: at most floor(T / bs) + 2 per request (non-decreasing cu_seq_lens)
  const int64_t capacity = num_tokens / block_size + 2 * int64_t(num_reqs) + 1;
  if (capacity >= (int64_t(1) << 31)) return PKVG_E_LIMIT;
  return PKVG_OK;
}

int64_t max_bytes_stride(int64_t stride, int64_t elem) {
  return stride > INT64_MAX / elem ? -1 : stride * elem;
}

// Workgroup shape by task-unit size and batch (each choice measured; a unit
// is a page, a part of one, or a group of pages, as planned below):
//  * units of at most 20 KiB of output take the small shape, of at most 36 KiB
//    the mid one: sized to the unit, they fit more units per CU (2.0-2.5x on
//    16- and 32-token pages);
//  * larger units take the wide shape when the batch is found in wave
//    registers or is one request (at most 64 requests) and there are at least
//    this many tasks (about four workgroups per CU), or the pages are fp8
//    written as one contiguous span (they take the wide shape's store bursts
//    and write-through stores);
//  * otherwise the narrow shape (fewer tasks, or batches of more than 64
//    requests, whose per-workgroup prefix build hides better behind more,
//    smaller workgroups).
constexpr int64_t kWideMinTasks = 1024;
constexpr int64_t kSmallMaxPageBytes = 20 * 1024;
constexpr int64_t kMidMaxPageBytes = 36 * 1024;

// hipLaunchKernel returns the launch's own status, so the calling thread's
// error state (which other libraries use) is neither read nor cleared.
template <typename... Args>
hipError_t launch(void (*kernel)(Args...), dim3 grid, unsigned block, size_t lds, hipStream_t stream,
                  Args... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, dim3(block), argv, lds, stream);
}

// Where the gather kernel finds its page tasks: a prebuilt table (large
// batches), one request, the block table walked directly (batches with a
// dense table), or a prefix built in wave registers (small batches) or LDS.
int32_t task_mode(int32_t num_reqs, bool walk) {
  if (num_reqs > PKVG_FUSED_MAX_REQS && !walk) return pkvg::kTable;
  if (num_reqs == 1) return pkvg::kSingle;
  if (walk) return pkvg::kWalk;
  return num_reqs <= pkvg::kWaveMaxReqs ? pkvg::kWaveRegs : pkvg::kLdsPrefix;
}

// Each kernel has a build for one request, one for the table walk and one for
// the prefix and table modes (the task mode is then a constant, or known to be
// neither of the others).
template <int BUILD>
constexpr bool build_matches(int32_t mode) {
  return BUILD == pkvg::kBuildSingle ? mode == pkvg::kSingle
                                     : (BUILD == pkvg::kBuildWalk ? mode == pkvg::kWalk
                                                                  : mode != pkvg::kSingle && mode != pkvg::kWalk);
}

template <class SH, int CONVERT, int W, int LAYOUT, bool SRC_VEC, int BUILD>
hipError_t launch_pages_build(const Plan& pl, size_t lds, hipStream_t stream) {
  const GatherParams& p = pl.p;
  return launch(pkvg::gather_pages_kernel<SH, CONVERT, W, LAYOUT, SRC_VEC, BUILD>,
                dim3(static_cast<unsigned>(pl.grid), static_cast<unsigned>(pl.grid_rows)), SH::threads, lds,
                stream, p.cu_seq_lens, p.block_table, p.seq_starts, pl.mode | (p.split_shift << 8), p.num_reqs,
                p.task_tokens, p.task_tokens_magic, p.block_table_width, p.cu_terminal,
                static_cast<int32_t>(p.num_tokens), static_cast<int32_t>(pl.mode == pkvg::kWalk ? p.block_table_ld : 0),
                p);
}

template <class SH, int CONVERT, int W, int LAYOUT, bool SRC_VEC>
hipError_t launch_shape(const Plan& pl, size_t lds, hipStream_t stream) {
  if (pl.mode == pkvg::kSingle)
    return launch_pages_build<SH, CONVERT, W, LAYOUT, SRC_VEC, pkvg::kBuildSingle>(pl, lds, stream);
  if (pl.mode == pkvg::kWalk)
    return launch_pages_build<SH, CONVERT, W, LAYOUT, SRC_VEC, pkvg::kBuildWalk>(pl, lds, stream);
  return launch_pages_build<SH, CONVERT, W, LAYOUT, SRC_VEC, pkvg::kBuildPrefix>(pl, lds, stream);
}

template <class SH, int CONVERT, int W, int LAYOUT, bool SRC_VEC, int BUILD>
hipError_t launch_groups_build(const Plan& pl, size_t lds, hipStream_t stream) {
  const GatherParams& p = pl.p;
  return launch(pkvg::gather_groups_kernel<SH, CONVERT, W, LAYOUT, SRC_VEC, BUILD>,
                dim3(static_cast<unsigned>(pl.grid), static_cast<unsigned>(pl.grid_rows)), SH::threads, lds,
                stream, p.cu_seq_lens, p.block_table, p.seq_starts, pl.mode | (p.group_shift << 8), p.num_reqs,
                p.task_tokens, p.task_tokens_magic, p.block_table_width, p.cu_terminal,
                static_cast<int32_t>(p.num_tokens), static_cast<int32_t>(pl.mode == pkvg::kWalk ? p.block_table_ld : 0),
                p);
}

template <class SH, int CONVERT, int W, int LAYOUT, bool SRC_VEC>
hipError_t launch_groups(const Plan& pl, size_t lds, hipStream_t stream) {
  if (pl.mode == pkvg::kSingle)
    return launch_groups_build<SH, CONVERT, W, LAYOUT, SRC_VEC, pkvg::kBuildSingle>(pl, lds, stream);
  if (pl.mode == pkvg::kWalk)
    return launch_groups_build<SH, CONVERT, W, LAYOUT, SRC_VEC, pkvg::kBuildWalk>(pl, lds, stream);
  return launch_groups_build<SH, CONVERT, W, LAYOUT, SRC_VEC, pkvg::kBuildPrefix>(pl, lds, stream);
}

// The workgroup shape of a plan (the rules above; the group kernel always
// takes the small shape).
int shape_for(const Plan& pl) {
  if (pl.p.group_shift > 0) return kShapeSmall;
  const int64_t page_out = int64_t(pl.p.task_tokens) * pl.p.row_in_bytes * (pl.convert == pkvg::kFp8Bf16 ? 2 : 1);
  if (page_out <= kSmallMaxPageBytes) return kShapeSmall;
  if (page_out <= kMidMaxPageBytes) return kShapeMid;
  if (pl.rule_reqs <= pkvg::kWaveMaxReqs &&
      (pl.grid * pl.grid_rows >= kWideMinTasks || (pl.convert == pkvg::kFp8Bf16 && pl.layout == pkvg::kFlat)))
    return kShapeWide;
  return kShapeNarrow;
}

template <int CONVERT, int W, int LAYOUT, bool SRC_VEC>
hipError_t launch_gather(const Plan& pl, size_t lds, hipStream_t stream) {
  if (pl.p.group_shift > 0) return launch_groups<pkvg::Small, CONVERT, W, LAYOUT, SRC_VEC>(pl, lds, stream);
  switch (pl.shape) {
    case kShapeSmall: return launch_shape<pkvg::Small, CONVERT, W, LAYOUT, SRC_VEC>(pl, lds, stream);
    case kShapeMid: return launch_shape<pkvg::Mid, CONVERT, W, LAYOUT, SRC_VEC>(pl, lds, stream);
    case kShapeWide: return launch_shape<pkvg::Wide, CONVERT, W, LAYOUT, SRC_VEC>(pl, lds, stream);
    default: return launch_shape<pkvg::Narrow, CONVERT, W, LAYOUT, SRC_VEC>(pl, lds, stream);
  }
}

template <int CONVERT, int W, bool SRC_VEC>
hipError_t launch_layout(const Plan& pl, size_t lds, hipStream_t stream) {
  if (pl.layout == pkvg::kFlat) return launch_gather<CONVERT, W, pkvg::kFlat, SRC_VEC>(pl, lds, stream);
  return launch_gather<CONVERT, W, pkvg::kRows, SRC_VEC>(pl, lds, stream);
}

hipError_t dispatch(const Plan& pl, size_t lds, hipStream_t stream) {
  if (pl.convert == pkvg::kCopy) {
    switch (pl.width) {
      case 16: return launch_layout<pkvg::kCopy, 16, true>(pl, lds, stream);
      case 8: return launch_layout<pkvg::kCopy, 8, true>(pl, lds, stream);
      case 4: return launch_layout<pkvg::kCopy, 4, true>(pl, lds, stream);
      case 2: return launch_layout<pkvg::kCopy, 2, true>(pl, lds, stream);
      default: return launch_layout<pkvg::kCopy, 1, true>(pl, lds, stream);
    }
  }
  if (pl.src_vec) {
    switch (pl.width) {
      case 8: return launch_layout<pkvg::kFp8Bf16, 8, true>(pl, lds, stream);
      case 4: return launch_layout<pkvg::kFp8Bf16, 4, true>(pl, lds, stream);
      case 2: return launch_layout<pkvg::kFp8Bf16, 2, true>(pl, lds, stream);
      default: return launch_layout<pkvg::kFp8Bf16, 1, true>(pl, lds, stream);
    }
  }
  switch (pl.width) {
    case 8: return launch_layout<pkvg::kFp8Bf16, 8, false>(pl, lds, stream);
    case 4: return launch_layout<pkvg::kFp8Bf16, 4, false>(pl, lds, stream);
    case 2: return launch_layout<pkvg::kFp8Bf16, 2, false>(pl, lds, stream);
    default: return launch_layout<pkvg::kFp8Bf16, 1, true>(pl, lds, stream);  // one code: any alignment
  }
}

// Builder for large batches and for gather_page_tasks: P scan, then records.
hipError_t build_tasks(const GatherParams& p, int32_t* P, int32_t* count, TaskRecord* out,
                       int64_t capacity, hipStream_t stream) {
  hipError_t e = launch(pkvg::scan_page_counts_kernel, dim3(1), pkvg::kScanThreads, 0, stream, p, P, count);
  if (e != hipSuccess || capacity == 0) return e;
  const int64_t blocks = (capacity + 255) / 256;
  const unsigned grid = static_cast<unsigned>(blocks < 4096 ? blocks : 4096);
  return launch(pkvg::expand_tasks_kernel, dim3(grid), 256, 0, stream, p, const_cast<const int32_t*>(P), out,
                static_cast<int32_t>(capacity));
}

// Task units in one block-table row for a walk: the row's columns split into
// 2^split_shift parts each, or grouped 2^group_shift at a time.
int64_t walk_units_per_row(const Plan& pl) {
  const int64_t w = pl.p.block_table_width;
  if (pl.p.group_shift > 0) return (w + (int64_t(1) << pl.p.group_shift) - 1) >> pl.p.group_shift;
  return w << pl.p.split_shift;
}

// Grid and workgroup shape, once the task units are fixed.
void finish_plan(Plan& pl) {
  if (pl.mode == pkvg::kWalk) {
    pl.grid = walk_units_per_row(pl);
    pl.grid_rows = pl.p.num_reqs;
  } else {
    pl.grid = pl.capacity < kMaxGrid ? pl.capacity : kMaxGrid;
    pl.grid_rows = 1;
  }
  pl.shape = shape_for(pl);
}

// Task-table scratch of a large batch: P[R+1] | count | (256-byte aligned) records[capacity].
size_t table_records_offset(int32_t R) { return (sizeof(int32_t) * (size_t(R) + 2) + 255) / 256 * 256; }

size_t table_scratch_bytes(const Plan& pl) {
  return table_records_offset(pl.p.num_reqs) + sizeof(TaskRecord) * size_t(pl.capacity);
}

// A large batch: the builder writes its task table into `table_mem` (every field
// the gather reads is written first, so nothing needs clearing), then the
// gather reads it.
hipError_t run_tabled(Plan& pl, void* table_mem, hipStream_t stream) {
  const int32_t R = pl.p.num_reqs;
  int32_t* P = static_cast<int32_t*>(table_mem);
  int32_t* count = P + R + 1;
  TaskRecord* rec = reinterpret_cast<TaskRecord*>(static_cast<char*>(table_mem) + table_records_offset(R));
  hipError_t e = build_tasks(pl.p, P, count, rec, pl.capacity, stream);
  if (e != hipSuccess) return e;
  pl.p.tasks = rec;
  pl.p.task_count = count;
  pl.p.task_capacity = static_cast<int32_t>(pl.capacity);
  return dispatch(pl, 0, stream);
}

// Runs a prepared plan.  Batches of at most PKVG_FUSED_MAX_REQS requests need
// no scratch; larger ones use `fixed_scratch` when given (at least
// table_scratch_bytes(pl) bytes), else a stream-ordered allocation.
int run_plan(Plan& pl, hipStream_t stream, void* fixed_scratch = nullptr) {
  const int32_t R = pl.p.num_reqs;
  if (pl.mode != pkvg::kTable) {
    const size_t lds = pl.mode == pkvg::kLdsPrefix ? sizeof(int32_t) * (3 * size_t(R) + 3) : 0;
    hipError_t e = dispatch(pl, lds, stream);
    return e == hipSuccess ? PKVG_OK : hip_fail(e);
  }
  if (fixed_scratch) {
    const hipError_t e = run_tabled(pl, fixed_scratch, stream);
    return e == hipSuccess ? PKVG_OK : hip_fail(e);
  }
  void* table_mem = nullptr;
  hipError_t e = hipMallocAsync(&table_mem, table_scratch_bytes(pl), stream);
  if (e != hipSuccess) return hip_fail(e);
  e = run_tabled(pl, table_mem, stream);
  const hipError_t ef = hipFreeAsync(table_mem, stream);
  if (e != hipSuccess) return hip_fail(e);
  if (ef != hipSuccess) return hip_fail(ef);
  return PKVG_OK;
}

// ---------------------------------------------------------------------------
// the no-allocation entry point's scratch: a fixed device array
// ---------------------------------------------------------------------------

// The fixed array `scratch` (above the anonymous namespace) holds the table.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch`.  Calls no allocating routine.
int scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return PKVG_E_LIMIT;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e);
      if (!p) return hip_fail(hipErrorInvalidSymbol);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PKVG_OK;
}

void fill_common(Plan& pl, const void* src, void* dst, const int32_t* block_table,
                 int32_t block_table_width, int64_t block_table_ld, const int32_t* cu_seq_lens,
                 int32_t cu_terminal, const int32_t* seq_starts, int32_t num_reqs, int64_t num_blocks,
                 int32_t block_size, int64_t num_tokens) {
  pl.p.src = static_cast<const uint8_t*>(src);
  pl.p.dst = static_cast<uint8_t*>(dst);
  pl.p.block_table = block_table;
  pl.p.cu_seq_lens = cu_seq_lens;
  pl.p.cu_terminal = cu_terminal;
  pl.p.seq_starts = seq_starts;
  pl.p.block_table_ld = block_table_ld;
  pl.p.block_table_width = block_table_width;
  pl.p.num_reqs = num_reqs;
  pl.p.num_blocks = num_blocks;
  pl.p.task_tokens = block_size;
  pl.p.task_tokens_magic = magic_for(static_cast<uint32_t>(block_size));
  pl.p.split_shift = 0;
  pl.p.group_shift = 0;
  pl.p.num_tokens = num_tokens;
  pl.capacity = num_tokens / block_size + 2 * int64_t(num_reqs) + 1;
}

// Pages of more than one narrow batch of output (256 lanes x 288 bytes) are
// split into 2^k equal task units, halving while the unit is an even number of
// tokens and still larger than that batch: a few large pages then spread over
// the whole chip instead of leaving most CUs idle (240 pages of 256 tokens
// would fill 240 of 256 CUs with one workgroup each).  Splitting only when the
// task count stays within int32.
constexpr int64_t kSplitAboveBytes = int64_t(pkvg::Narrow::threads) * pkvg::Narrow::lane_bytes;

// One request's raw pages are split further, into units of at most 9 KiB
// (8 tokens of 1152-byte rows), which take the small shape.  Measured: the
// 61,440-token gather on 64-token pages 26.6 -> 25.4 us, the 307,200-token
// one 120.4 -> 118.9 us, 1,024-token pages 26.0 -> 25.3 us; 18 KiB and 36 KiB
// units gain less or lose.  So are the raw pages of batches of at most 64
// requests (wave-register prefix) with fewer whole-page tasks than the wide
// shape takes: 2, 8 and 64 requests over 61,440 tokens 27.2-27.4 -> 26.7-26.8
// us.  With more tasks they lose (skew-2/4/8 +0.5-1.5%), and so do larger
// batches (512 requests +15%) and fp8 pages (the 307,200-token upconvert +14%).
constexpr int64_t kSplitSingleRawBytes = 9 * 1024;

// Pages of batches of more than 64 requests (the LDS-prefix and task-table
// paths) are split into units of at most 18 KiB of output (small shape).
// Raw, on 64-token pages, 36 KiB units against whole pages: 65 x 2000 tokens
// -6%, 128 x 800 -1.6%, 300 x 3000 -5.5%, 512 x 200 -5%, 1024 x 200 -1.6%,
// 2048 x 100 -6%; 18 KiB units against 36 KiB (since the LDS prefix costs
// one round trip): 300 x 3000 -2.7%, 128 x 2000 -1.6%, 512 x 200 -0.5%, and
// 9 KiB units lose 2-7%.  fp8 to bf16, 18 KiB units against whole pages:
// 128 x 2000 tokens -4.1%, 512 x 200 -2.8% (9 KiB units lose up to 38%).
// Batches of at most 64 requests lose with 18 KiB fp8 units (8 x 38,400
// tokens +2.6%) or 36 KiB raw ones (skew-8 +5%).
constexpr int64_t kSplitBatchBytes = 18 * 1024;

// Small pages go to the group kernel, whose task is G = 2^k consecutive pages
// of one request (always the small shape).  Which pages, measured on one
// request of 61,440 (raw) or 307,200 (fp8) tokens with 1152-byte output rows:
// as groups, 1-token pages are 2.9x (raw) and 4.3x (fp8) faster, 2-token raw
// pages 1.6x, 4-token raw pages the same; 8-token raw pages are 8% faster one
// per workgroup, 8-token fp8 pages 7% slower.  Batches of many short requests
// gain 1.1-5.9x from 8- down to 1-token pages (the page kernel's workgroups
// each build the task prefix for one small page).  So: pages of at most
// 4.5 KiB of output always, of at most 9 KiB for batches and fp8.
// How many: the largest G <= 64 whose pages hold at most 9 KiB of output (one
// request, raw), 20 KiB (one request, fp8) or 18 KiB (batches).  Against 20 KiB
// groups, one request's raw 1- and 2-token pages take 1.8% less time in 9 KiB
// groups (its fp8 pages 4% more).  Batches against 36 KiB groups: 512 x 200
// one-token pages -5.7% (fp8 -2%), 8 x 7,680 and 64 x 960 one-token pages
// -4%, 128 x 2000 four-token pages -5%; 9 KiB groups lose 1-40%.
constexpr int64_t kGroupMaxPageBytes = 4608;
constexpr int64_t kGroupMaxPageBytesBatchOrFp8 = 9216;
constexpr int64_t kGroupBatchBytes = 18 * 1024;
constexpr int32_t kMaxGroupShift = 6;

void plan_group(Plan& pl, int64_t row_out_bytes) {
  if (pl.p.split_shift > 0) return;  // units are already parts of a page
  const int32_t bs = pl.p.task_tokens;
  const int64_t page_out = int64_t(bs) * row_out_bytes;
  const bool batch_or_fp8 = pl.rule_reqs > 1 || pl.convert == pkvg::kFp8Bf16;
  if (page_out > (batch_or_fp8 ? kGroupMaxPageBytesBatchOrFp8 : kGroupMaxPageBytes)) return;
  const int64_t max_group_bytes =
      pl.rule_reqs > 1 ? kGroupBatchBytes : (pl.convert == pkvg::kFp8Bf16 ? kSmallMaxPageBytes : kSplitSingleRawBytes);
  int32_t k = 0;
  while (k < kMaxGroupShift && (page_out << (k + 1)) <= max_group_bytes) ++k;
  if (k == 0) return;
  pl.p.page_tokens = bs;
  pl.p.page_tokens_magic = magic_for(static_cast<uint32_t>(bs));
  pl.p.task_tokens = bs << k;
  pl.p.task_tokens_magic = magic_for(static_cast<uint32_t>(bs << k));
  pl.p.group_shift = k;
  pl.capacity = pl.p.num_tokens / (int64_t(bs) << k) + 2 * int64_t(pl.p.num_reqs) + 1;
}

void plan_split(Plan& pl, int64_t row_out_bytes, int64_t max_unit_bytes) {
  int32_t tt = pl.p.task_tokens;
  int32_t k = 0;
  while ((tt & 1) == 0 && int64_t(tt) * row_out_bytes > max_unit_bytes) {
    tt >>= 1;
    ++k;
  }
  const int64_t capacity = pl.p.num_tokens / tt + 2 * int64_t(pl.p.num_reqs) + 1;
  if (k == 0 || capacity >= (int64_t(1) << 31)) return;
  pl.p.task_tokens = tt;
  pl.p.task_tokens_magic = magic_for(static_cast<uint32_t>(tt));
  pl.p.split_shift = k;
  pl.capacity = capacity;
}

// Raw copy plan: pick the widest access that every row, stride and base allows.
int plan_copy(Plan& pl, const void* src, void* dst, int64_t elem, int32_t entry, int64_t sbs,
              int64_t sts, int64_t drs, int32_t block_size) {
  const int64_t row = int64_t(entry) * elem;
  const int64_t sb = max_bytes_stride(sbs, elem), st = max_bytes_stride(sts, elem),
                dr = max_bytes_stride(drs, elem);
  if (sb < 0 || st < 0 || dr < 0) return PKVG_E_LIMIT;
  // in-page offsets are 32-bit: a page's source and destination rows span < 2^31 bytes
  if (int64_t(block_size) * row >= (int64_t(1) << 31)) return PKVG_E_LIMIT;
  if (int64_t(block_size - 1) * st + row >= (int64_t(1) << 31)) return PKVG_E_LIMIT;
  // 16- and 8-byte chunks need rows of that many bytes and dword-aligned
  // strides and bases; narrower chunks need their own alignment
  auto fits = [&](int64_t a) {
    return sb % a == 0 && st % a == 0 && dr % a == 0 && aligned(src, a) && aligned(dst, a);
  };
  int w = 16;
  while (w > 1 && (row % w || !fits(w < 4 ? w : 4))) w >>= 1;
  pl.convert = pkvg::kCopy;
  pl.width = w;
  pl.layout = (st == row && dr == row) ? pkvg::kFlat : pkvg::kRows;
  pl.p.src_block_stride = sb;
  pl.p.src_token_stride = st;
  pl.p.dst_row_stride = dr;
  pl.p.chunks_per_row = static_cast<int32_t>(row / w);
  pl.p.chunks_magic = magic_for(static_cast<uint32_t>(row / w));
  pl.p.row_in_bytes = static_cast<int32_t>(row);
  return PKVG_OK;
}

// fp8 -> bf16 plan: K codes per lane, limited by the row length and the bf16
// rows' alignment; code rows that are not dword-aligned are read as shifted
// dword windows (K >= 4) or byte by byte (shorter rows, K < 4).
int plan_fp8(Plan& pl, const void* src, void* dst, int32_t entry, int64_t sbs, int64_t sts,
             int64_t drs_elems, int32_t block_size) {
  const int64_t dr = max_bytes_stride(drs_elems, 2);
  if (dr < 0) return PKVG_E_LIMIT;
  if (int64_t(block_size) * entry * 2 >= (int64_t(1) << 31)) return PKVG_E_LIMIT;
  // k codes per lane store 2k bytes of bf16: dword-aligned rows suffice for
  // k >= 2 (multi-dword stores need only dword alignment), 2-byte rows for k = 1;
  // their loads are k-byte words when the code rows are dword-aligned (k >= 4)
  // or k-aligned (k < 4)
  int k = 8;
  while (k > 1 && (entry % k || dr % 4 || !aligned(dst, 4))) k >>= 1;
  pl.convert = pkvg::kFp8Bf16;
  const int64_t src_align = k < 4 ? k : 4;
  pl.src_vec = (sbs % src_align == 0) && (sts % src_align == 0) && aligned(src, src_align);
  // unaligned code rows are read as shifted dword windows, which need rows of
  // at least 16 codes; shorter unaligned rows use one code per lane
  if (!pl.src_vec && k >= 4 && entry < 16) k = 1;
  pl.width = k;
  pl.layout = (sts == entry && dr == 2 * int64_t(entry)) ? pkvg::kFlat : pkvg::kRows;
  pl.p.src_block_stride = sbs;
  pl.p.src_token_stride = sts;
  pl.p.dst_row_stride = dr;
  pl.p.chunks_per_row = entry / k;
  pl.p.chunks_magic = magic_for(static_cast<uint32_t>(entry / k));
  pl.p.row_in_bytes = entry;
  // in-page source offsets are 32-bit (the unaligned path also reads up to 3
  // bytes around a chunk)
  if (int64_t(block_size - 1) * sts + entry + 8 >= (int64_t(1) << 31)) return PKVG_E_LIMIT;
  return PKVG_OK;
}


// The arguments every gather call shares (strides in elements, as passed).
struct GatherArgs {
  const void* src;
  int64_t num_blocks;
  int32_t block_size;
  int32_t entry;
  int64_t src_block_stride;
  int64_t src_token_stride;
  void* dst;
  int64_t num_tokens;
  int64_t dst_row_stride;
  const int32_t* block_table;
  int32_t block_table_width;
  int64_t block_table_ld;
  const int32_t* cu_seq_lens;
  int32_t cu_terminal;
  const int32_t* seq_starts;
  int32_t num_reqs;
};

// Batches whose block table is dense are walked directly (kWalk, one
// workgroup per unit of each table row): dense when the table's pages are at
// most 5/4 of the most pages the call's rows can fill, so the workgroups that
// find no rows stay few.  The y extent of the grid bounds the batch; the table
// pitch travels as a 32-bit kernel argument.
constexpr int32_t kMaxWalkReqs = 65535;

bool walk_fits(const GatherArgs& a) {
  if (a.num_reqs < 2 || a.num_reqs > kMaxWalkReqs || a.block_table_width < 1 || a.block_table_ld > INT32_MAX)
    return false;
  const int64_t table_pages = int64_t(a.num_reqs) * a.block_table_width;
  const int64_t row_pages = a.num_tokens / a.block_size + 2 * int64_t(a.num_reqs) + 1;
  return table_pages * 4 <= row_pages * 5;
}

int plan_units(int32_t elem_bytes, const GatherArgs& a, const float* scale, bool walk, Plan& pl);

// Validates a call and plans it (access width, task units, grid, shape);
// touches no device.  `kind`: elem_bytes (gather_cache) or kv_cache_dtype
// (gather_maybe_dequant); unused for the upconvert.  `*nothing` is set when
// the call has no work.
int prepare(int32_t op, int32_t kind, const GatherArgs& a, const float* scale, Plan& pl, bool* nothing) {
  *nothing = false;
  int32_t elem_bytes = 0;  // raw copy element size; 0: fp8
  if (op == PKVG_OP_GATHER_CACHE) {
    if (kind != 1 && kind != 2 && kind != 4 && kind != 8) return PKVG_E_DTYPE;
    elem_bytes = kind;
  } else if (op == PKVG_OP_GATHER_MAYBE_DEQUANT) {
    if (kind == PKVG_KV_AUTO) elem_bytes = 2;
    else if (kind != PKVG_KV_FP8_E4M3) return PKVG_E_DTYPE;
  } else if (op != PKVG_OP_GATHER_UPCONVERT_FP8) {
    return PKVG_E_SHAPE;
  }
  int st = check_common(a.src, a.num_blocks, a.block_size, a.entry, a.src_block_stride, a.src_token_stride, a.dst,
                        a.num_tokens, a.dst_row_stride, a.block_table, a.block_table_width, a.block_table_ld,
                        a.cu_seq_lens, a.cu_terminal, a.num_reqs, nothing);
  if (st != PKVG_OK || *nothing) return st;
  if (elem_bytes == 0 && !scale) return PKVG_E_NULL;
  st = plan_units(elem_bytes, a, scale, walk_fits(a), pl);
  if (st == PKVG_OK && pl.mode == pkvg::kWalk && walk_units_per_row(pl) > kMaxGrid)
    st = plan_units(elem_bytes, a, scale, false, pl);  // rows of too many units: not walked
  if (st != PKVG_OK) return st;
  finish_plan(pl);
  return PKVG_OK;
}

// Fills the plan of a checked call: task mode, access width, task units.
int plan_units(int32_t elem_bytes, const GatherArgs& a, const float* scale, bool walk, Plan& pl) {
  pl = Plan{};
  pl.mode = task_mode(a.num_reqs, walk);
  pl.rule_reqs = pl.mode == pkvg::kWalk ? 1 : a.num_reqs;
  int st = PKVG_OK;
  fill_common(pl, a.src, a.dst, a.block_table, a.block_table_width, a.block_table_ld, a.cu_seq_lens,
              a.cu_terminal, a.seq_starts, a.num_reqs, a.num_blocks, a.block_size, a.num_tokens);
  if (elem_bytes > 0) {
    st = plan_copy(pl, a.src, a.dst, elem_bytes, a.entry, a.src_block_stride, a.src_token_stride,
                   a.dst_row_stride, a.block_size);
    if (st != PKVG_OK) return st;
    const int64_t row = int64_t(a.entry) * elem_bytes;
    // pl.capacity still counts whole pages here
    const int32_t rr = pl.rule_reqs;
    const bool small_unit = rr == 1 || (rr <= pkvg::kWaveMaxReqs && pl.capacity < kWideMinTasks);
    plan_split(pl, row,
               small_unit ? kSplitSingleRawBytes : (rr > pkvg::kWaveMaxReqs ? kSplitBatchBytes : kSplitAboveBytes));
    plan_group(pl, row);
  } else {
    pl.p.scale = scale;
    st = plan_fp8(pl, a.src, a.dst, a.entry, a.src_block_stride, a.src_token_stride, a.dst_row_stride,
                  a.block_size);
    if (st != PKVG_OK) return st;
    plan_split(pl, 2 * int64_t(a.entry), pl.rule_reqs > pkvg::kWaveMaxReqs ? kSplitBatchBytes : kSplitAboveBytes);
    plan_group(pl, 2 * int64_t(a.entry));
  }
  return PKVG_OK;
}

int run_call(int32_t op, int32_t kind, const GatherArgs& a, const float* scale, void* stream) {
  Plan pl;
  bool nothing;
  const int st = prepare(op, kind, a, scale, pl, &nothing);
  if (st != PKVG_OK || nothing) return st;
  return run_plan(pl, static_cast<hipStream_t>(stream));
}

int32_t shape_threads(int shape) {
  switch (shape) {
    case kShapeSmall: return pkvg::Small::threads;
    case kShapeMid: return pkvg::Mid::threads;
    case kShapeWide: return pkvg::Wide::threads;
    default: return pkvg::Narrow::threads;
  }
}

int32_t shape_lane_bytes(int shape) {
  switch (shape) {
    case kShapeSmall: return pkvg::Small::lane_bytes;
    case kShapeMid: return pkvg::Mid::lane_bytes;
    case kShapeWide: return pkvg::Wide::lane_bytes;
    default: return pkvg::Narrow::lane_bytes;
  }
}

// ---------------------------------------------------------------------------
// indexer quant-cache gather
// ---------------------------------------------------------------------------

// Structural constants (template parameters): the record layout, the head
// dimension and the tile sizes; every other size is a runtime argument.
bool indexer_structure_supported(int32_t layout, int32_t head_dim, int32_t block_tile, int32_t head_tile) {
  const bool dim = head_dim == 64 || head_dim == 128 || head_dim == 256;
  if (layout == PKVG_INDEXER_FLAT) return dim;
  if (layout == PKVG_INDEXER_TILED) return dim && block_tile == 16 && head_tile == 16;
  return false;
}

template <int LAYOUT, int HEAD_DIM, int BT, int HT, int W>
hipError_t launch_indexer_cu(const pkvg::IndexerParams& p, unsigned grid, hipStream_t stream) {
  const int32_t ncu = p.num_batches + 1;
  auto kernel = ncu <= 64 ? pkvg::indexer_gather_kernel<LAYOUT, HEAD_DIM, BT, HT, W, pkvg::kCuWave>
                          : pkvg::indexer_gather_kernel<LAYOUT, HEAD_DIM, BT, HT, W, pkvg::kCuGlobal>;
  return launch(kernel, grid, pkvg::kIndexerThreads, 0, stream, p.token_to_seq, p.cu_seqlen, p.num_tokens,
                p.num_batches, p.block_table, p.block_table_ld, p.block_table_width, p.block_size,
                p.block_size_magic, p);
}

template <int LAYOUT, int HEAD_DIM, int BT, int HT>
hipError_t launch_indexer_w(const pkvg::IndexerParams& p, bool vec, unsigned grid, hipStream_t stream) {
  if (vec) return launch_indexer_cu<LAYOUT, HEAD_DIM, BT, HT, 16>(p, grid, stream);
  return launch_indexer_cu<LAYOUT, HEAD_DIM, BT, HT, 1>(p, grid, stream);
}

template <int LAYOUT, int BT, int HT>
hipError_t launch_indexer_dim(const pkvg::IndexerParams& p, int32_t head_dim, bool vec, unsigned grid,
                              hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_indexer_w<LAYOUT, 64, BT, HT>(p, vec, grid, stream);
    case 128: return launch_indexer_w<LAYOUT, 128, BT, HT>(p, vec, grid, stream);
    default: return launch_indexer_w<LAYOUT, 256, BT, HT>(p, vec, grid, stream);
  }
}

// Rows per workgroup (one wave of 64 rows); the grid covers every row once,
// up to this many workgroups (far more than the chip holds at once; more
// rows, past 4,194,304, are taken by striding).
constexpr int64_t kIndexerMaxGrid = int64_t(1) << 16;

// Validates an indexer gather and fills its parameters; touches no device.
int prepare_indexer(const void* cache, int64_t num_blocks, int32_t block_size, int64_t block_stride,
                    int32_t layout, int32_t head_dim, int32_t block_tile, int32_t head_tile, void* dst_values,
                    int64_t dst_value_stride, float* dst_scales, int64_t dst_scale_stride, int64_t num_tokens,
                    const int32_t* token_to_seq, const int32_t* cu_seqlen, int32_t num_batches,
                    const int32_t* block_table, int32_t block_table_width, int64_t block_table_ld,
                    pkvg::IndexerParams* out, bool* vec, bool* nothing) {
  *nothing = false;
  if (num_tokens < 0 || num_batches < 0 || num_blocks < 0 || block_table_width < 0 || block_size <= 0)
    return PKVG_E_SHAPE;
  if (!indexer_structure_supported(layout, head_dim, block_tile, head_tile)) return PKVG_E_DTYPE;
  if (layout == PKVG_INDEXER_TILED && block_size % block_tile != 0) return PKVG_E_SHAPE;
  const int64_t record_bytes = int64_t(block_size) * (head_dim + 4);
  if (block_stride < record_bytes || dst_value_stride < head_dim || dst_scale_stride < 1 ||
      block_table_ld < block_table_width)
    return PKVG_E_STRIDE;
  // no row can pass the masks: nothing to enqueue (a launched kernel relies on
  // record 0 existing, as the address masked rows keep, and on row 0 of the
  // table having a column, which its speculative entry reads)
  if (num_tokens == 0 || num_batches == 0 || num_blocks == 0 || block_table_width == 0) {
    *nothing = true;
    return PKVG_OK;
  }
  if (!cache || !dst_values || !dst_scales || !token_to_seq || !cu_seqlen ||
      (!block_table && block_table_width > 0))
    return PKVG_E_NULL;
  // the records hold fp32 scales: dword-aligned records; fp32 destination scales
  if (!aligned(cache, 4) || block_stride % 4 != 0 || !aligned(dst_scales, 4)) return PKVG_E_STRIDE;
  // rows are int32 (a wave's 64 rows stay below 2^31); in-record offsets are 32-bit
  if (num_tokens > INT32_MAX - 64 || block_stride >= (int64_t(1) << 31)) return PKVG_E_LIMIT;
  if (dst_scale_stride > INT64_MAX / 4) return PKVG_E_LIMIT;
  pkvg::IndexerParams& p = *out;
  p = pkvg::IndexerParams{};
  p.cache = static_cast<const uint8_t*>(cache);
  p.dst_values = static_cast<uint8_t*>(dst_values);
  p.dst_scales = reinterpret_cast<uint8_t*>(dst_scales);
  p.token_to_seq = token_to_seq;
  p.cu_seqlen = cu_seqlen;
  p.block_table = block_table;
  p.block_stride = block_stride;
  p.dst_value_stride = dst_value_stride;
  p.dst_scale_stride = dst_scale_stride * 4;
  p.block_table_ld = block_table_ld;
  p.num_blocks = num_blocks;
  p.num_tokens = static_cast<int32_t>(num_tokens);
  p.num_batches = num_batches;
  p.block_table_width = block_table_width;
  p.block_size = block_size;
  p.block_size_magic = magic_for(static_cast<uint32_t>(block_size));
  p.scale_area = static_cast<uint32_t>(int64_t(block_size) * head_dim);
  // 16-byte chunks need dword-aligned destination rows (the source rows are),
  // and a wave's 64 rows within the 2^31-byte range of its store resource
  *vec = aligned(dst_values, 4) && dst_value_stride % 4 == 0 && dst_value_stride < (int64_t(1) << 25);
  return PKVG_OK;
}

int64_t indexer_grid(int64_t num_tokens) {
  const int64_t rows_per_wg = int64_t(pkvg::kIndexerThreads / 64) * pkvg::kIndexerRowsPerWave;
  const int64_t g = (num_tokens + rows_per_wg - 1) / rows_per_wg;
  return g < kIndexerMaxGrid ? g : kIndexerMaxGrid;
}

}  // namespace

extern "C" {

int gather_indexer_quant_cache(const void* cache, int64_t num_blocks, int32_t block_size, int64_t block_stride,
                               int32_t layout, int32_t head_dim, int32_t block_tile, int32_t head_tile,
                               void* dst_values, int64_t dst_value_stride, float* dst_scales,
                               int64_t dst_scale_stride, int64_t num_tokens, const int32_t* token_to_seq,
                               const int32_t* cu_seqlen, int32_t num_batches, const int32_t* block_table,
                               int32_t block_table_width, int64_t block_table_ld, void* stream) {
  pkvg::IndexerParams p;
  bool vec = false, nothing = false;
  const int st = prepare_indexer(cache, num_blocks, block_size, block_stride, layout, head_dim, block_tile,
                                 head_tile, dst_values, dst_value_stride, dst_scales, dst_scale_stride, num_tokens,
                                 token_to_seq, cu_seqlen, num_batches, block_table, block_table_width,
                                 block_table_ld, &p, &vec, &nothing);
  if (st != PKVG_OK || nothing) return st;
  const unsigned grid = static_cast<unsigned>(indexer_grid(num_tokens));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = layout == PKVG_INDEXER_FLAT
                           ? launch_indexer_dim<pkvg::kIndexerFlat, 1, 16>(p, head_dim, vec, grid, s)
                           : launch_indexer_dim<pkvg::kIndexerTiled, 16, 16>(p, head_dim, vec, grid, s);
  return e == hipSuccess ? PKVG_OK : hip_fail(e);
}

int gather_cache(const void* src_cache, int32_t elem_bytes, int64_t num_blocks, int32_t block_size,
                 int32_t entry, int64_t src_block_stride, int64_t src_token_stride, void* dst,
                 int64_t num_tokens, int64_t dst_row_stride, const int32_t* block_table,
                 int32_t block_table_width, int64_t block_table_ld, const int32_t* cu_seq_lens,
                 int32_t cu_terminal, const int32_t* seq_starts, int32_t num_reqs, void* stream) {
  const GatherArgs a{src_cache, num_blocks, block_size, entry, src_block_stride, src_token_stride, dst,
                     num_tokens, dst_row_stride, block_table, block_table_width, block_table_ld,
                     cu_seq_lens, cu_terminal, seq_starts, num_reqs};
  return run_call(PKVG_OP_GATHER_CACHE, elem_bytes, a, nullptr, stream);
}

int gather_maybe_dequant(const void* src_cache, int32_t kv_cache_dtype, int64_t num_blocks,
                         int32_t block_size, int32_t entry, int64_t src_block_stride,
                         int64_t src_token_stride, void* dst, int64_t num_tokens, int64_t dst_row_stride,
                         const int32_t* block_table, int32_t block_table_width, int64_t block_table_ld,
                         const int32_t* cu_seq_lens, int32_t cu_terminal, const int32_t* seq_starts,
                         int32_t num_reqs, const float* scale, void* stream) {
  const GatherArgs a{src_cache, num_blocks, block_size, entry, src_block_stride, src_token_stride, dst,
                     num_tokens, dst_row_stride, block_table, block_table_width, block_table_ld,
                     cu_seq_lens, cu_terminal, seq_starts, num_reqs};
  return run_call(PKVG_OP_GATHER_MAYBE_DEQUANT, kv_cache_dtype, a, scale, stream);
}

int gather_maybe_dequant_noalloc(const void* src_cache, int32_t kv_cache_dtype, int64_t num_blocks,
                                 int32_t block_size, int32_t entry, int64_t src_block_stride,
                                 int64_t src_token_stride, void* dst, int64_t num_tokens,
                                 int64_t dst_row_stride, const int32_t* block_table, int32_t block_table_width,
                                 int64_t block_table_ld, const int32_t* cu_seq_lens, int32_t cu_terminal,
                                 const int32_t* seq_starts, int32_t num_reqs, const float* scale, void* stream) {
  const GatherArgs a{src_cache, num_blocks, block_size, entry, src_block_stride, src_token_stride, dst,
                     num_tokens, dst_row_stride, block_table, block_table_width, block_table_ld,
                     cu_seq_lens, cu_terminal, seq_starts, num_reqs};
  Plan pl;
  bool nothing;
  int st = prepare(PKVG_OP_GATHER_MAYBE_DEQUANT, kv_cache_dtype, a, scale, pl, &nothing);
  if (st != PKVG_OK || nothing) return st;
  void* sp = nullptr;
  if (pl.mode == pkvg::kTable) {
    if (num_reqs > PKVG_NOALLOC_MAX_REQS || pl.capacity > PKVG_NOALLOC_MAX_TASKS) return PKVG_E_SCRATCH;
    st = scratch_for_current_device(&sp);
    if (st != PKVG_OK) return st;
  }
  return run_plan(pl, static_cast<hipStream_t>(stream), sp);
}

int gather_upconvert_fp8(const void* src_cache, int64_t num_blocks, int32_t block_size, int32_t entry,
                         int64_t src_block_stride, int64_t src_token_stride, void* dst, int64_t num_tokens,
                         int64_t dst_row_stride, const int32_t* block_table, int32_t block_table_width,
                         int64_t block_table_ld, const int32_t* cu_seq_lens, int32_t cu_terminal,
                         const int32_t* seq_starts, int32_t num_reqs, const float* scale, void* stream) {
  const GatherArgs a{src_cache, num_blocks, block_size, entry, src_block_stride, src_token_stride, dst,
                     num_tokens, dst_row_stride, block_table, block_table_width, block_table_ld,
                     cu_seq_lens, cu_terminal, seq_starts, num_reqs};
  return run_call(PKVG_OP_GATHER_UPCONVERT_FP8, 0, a, scale, stream);
}

int pkvg_plan(int32_t op, int32_t kind, const void* src_cache, int64_t num_blocks, int32_t block_size,
              int32_t entry, int64_t src_block_stride, int64_t src_token_stride, void* dst, int64_t num_tokens,
              int64_t dst_row_stride, const int32_t* block_table, int32_t block_table_width,
              int64_t block_table_ld, const int32_t* cu_seq_lens, int32_t cu_terminal, const int32_t* seq_starts,
              int32_t num_reqs, const float* scale, pkvg_plan_info* info) {
  if (!info) return PKVG_E_NULL;
  *info = pkvg_plan_info{};
  const GatherArgs a{src_cache, num_blocks, block_size, entry, src_block_stride, src_token_stride, dst,
                     num_tokens, dst_row_stride, block_table, block_table_width, block_table_ld,
                     cu_seq_lens, cu_terminal, seq_starts, num_reqs};
  Plan pl;
  bool nothing;
  const int st = prepare(op, kind, a, scale, pl, &nothing);
  if (st != PKVG_OK || nothing) return st;
  info->kernel = pl.p.group_shift > 0 ? PKVG_KERNEL_GROUPS : PKVG_KERNEL_PAGES;
  info->threads = shape_threads(pl.shape);
  info->batch_bytes = shape_threads(pl.shape) * shape_lane_bytes(pl.shape);
  info->task_mode = pl.mode;
  info->grid_rows = static_cast<int32_t>(pl.grid_rows);
  info->convert = pl.convert;
  info->access_width = pl.width;
  info->flat = pl.layout == pkvg::kFlat ? 1 : 0;
  info->src_vector = pl.src_vec ? 1 : 0;
  info->task_tokens = pl.p.task_tokens;
  info->split_shift = pl.p.split_shift;
  info->group_shift = pl.p.group_shift;
  info->grid = pl.grid;
  info->task_capacity = pl.capacity;
  return PKVG_OK;
}

int gather_page_tasks(const int32_t* cu_seq_lens, int32_t cu_terminal, const int32_t* seq_starts,
                      int32_t num_reqs, int64_t num_tokens, int32_t block_size, const int32_t* block_table,
                      int32_t block_table_width, int64_t block_table_ld, int64_t num_blocks, int32_t* tasks,
                      int64_t capacity, int32_t* num_tasks, void* stream) {
  if (num_reqs < 0 || num_tokens < 0 || block_size <= 0 || block_table_width < 0 || num_blocks < 0 ||
      capacity < 0 || (cu_terminal != 0 && cu_terminal != 1))
    return PKVG_E_SHAPE;
  if (block_table_ld < block_table_width) return PKVG_E_STRIDE;
  if (!num_tasks || (num_reqs > 0 && (!cu_seq_lens || (!block_table && block_table_width > 0))) ||
      (capacity > 0 && !tasks))
    return PKVG_E_NULL;
  if (capacity >= (int64_t(1) << 31) || num_tokens > INT32_MAX) return PKVG_E_LIMIT;
  if (num_tokens / block_size + 2 * int64_t(num_reqs) + 1 >= (int64_t(1) << 31)) return PKVG_E_LIMIT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  GatherParams p{};
  p.block_table = block_table;
  p.cu_seq_lens = cu_seq_lens;
  p.cu_terminal = cu_terminal;
  p.seq_starts = seq_starts;
  p.block_table_ld = block_table_ld;
  p.block_table_width = block_table_width;
  p.num_reqs = num_reqs;
  p.num_blocks = num_blocks;
  p.task_tokens = block_size;  // one task per page
  p.task_tokens_magic = magic_for(static_cast<uint32_t>(block_size));
  p.split_shift = 0;
  p.num_tokens = num_tokens;
  void* prefix_mem = nullptr;
  hipError_t e = hipMallocAsync(&prefix_mem, sizeof(int32_t) * (size_t(num_reqs) + 1), s);
  if (e != hipSuccess) return hip_fail(e);
  e = build_tasks(p, static_cast<int32_t*>(prefix_mem), num_tasks, reinterpret_cast<TaskRecord*>(tasks),
                  capacity, s);
  const hipError_t ef = hipFreeAsync(prefix_mem, s);
  if (e != hipSuccess) return hip_fail(e);
  if (ef != hipSuccess) return hip_fail(ef);
  return PKVG_OK;
}

const char* pkvg_status_string(int status) {
  switch (status) {
    case PKVG_OK: return "PKVG_OK";
    case PKVG_E_NULL: return "PKVG_E_NULL: a required pointer is NULL";
    case PKVG_E_SHAPE: return "PKVG_E_SHAPE: a count or size is out of range";
    case PKVG_E_STRIDE: return "PKVG_E_STRIDE: a stride is negative or rows overlap";
    case PKVG_E_DTYPE: return "PKVG_E_DTYPE: unsupported element size, kv_cache_dtype or record layout";
    case PKVG_E_LIMIT: return "PKVG_E_LIMIT: beyond an implementation limit";
    case PKVG_E_HIP: return "PKVG_E_HIP: a HIP runtime call failed";
    case PKVG_E_SCRATCH:
      return "PKVG_E_SCRATCH: the batch's task table exceeds the no-allocation entry point's fixed scratch";
    default: return "unknown pkvg status";
  }
}

int pkvg_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
