// gather_kernels.hpp -- HIP device code of the paged MLA KV-cache gather for
// gfx950 (CDNA4, wave64).
//
// Method: the prhub.com.cn summary of vLLM pull request 51739, "MLA cache
// gather scheduled by logical page; raw copy up to 331x faster", section
// "implementation breakdown" step 1: every workgroup gathers one logical
// page, looks the block table up once per page, and moves the page's valid
// rows (partial first/last pages included) with wide vector accesses; the
// fp8 variants convert to bf16 and write coalesced rows.  The page's task
// fields (section "key source snippets": request, logical block, slot range
// inside the page, first output row) are produced here from an exclusive scan
// of per-request page counts, instead of the page's linear scan over requests.
//
// Design for gfx950:
//  * how a workgroup finds its page depends on the batch: one request needs
//    no scan (its first block-table entry is fetched with the request extent),
//    and neither does a batch whose block table is dense (workgroup (x, y)
//    takes unit x of request y's table row); otherwise up to 64 requests are
//    scanned in wave registers and found with a ballot, up to 1024 in LDS
//    with a binary search, and more use a task table built by two small
//    kernels.  Task fields live in SGPRs (readfirstlane), so no barrier
//    follows the lookup;
//  * the hot loop moves 16-byte (dwordx4) chunks, consecutive lanes on
//    consecutive chunks, so one wave instruction covers 1 KiB of a row span;
//    a whole page's loads are in flight before the matching stores, with the
//    nontemporal cache policy (each byte is touched once);
//  * flat pages that convert, or take the wide shape, store through a buffer
//    resource over the page's output, and a chunk past the unit's end takes
//    an offset beyond its range, which the hardware drops: the stores need no
//    branch, so the compiler keeps each load ahead of them and each store
//    waits only for its own load;
//  * all addressing that can exceed 2^31 bytes (page bases, output row bases)
//    is int64; in-page offsets are 32-bit (the host guarantees that a page's
//    rows span < 2^31 bytes);
//  * fp8 pages: each lane reads 8 codes (8 bytes) and writes 8 bf16 (16
//    bytes): v_cvt_pk_f32_fp8 (OCP e4m3fn on gfx950), one v_mul_f32 by the
//    scale, v_cvt_pk_bf16_f32 (round to nearest even);
//  * a task is normally one logical page; pages far larger than one
//    workgroup batch are split into 2^k equal parts (each its own task), and
//    pages of one to a few tokens are moved by a second kernel whose task is
//    a group of 2^k consecutive pages, so page sizes from 1 to thousands of
//    tokens all keep the chip busy;
//  * every shape is a runtime argument; templates cover only the workgroup
//    shape, the access width, and whether a page's rows are one contiguous
//    span;
//  * the fields the task lookup needs first are leading scalar kernel
//    arguments, preloaded into SGPRs at wave start, so the metadata loads
//    leave without waiting for a kernel-argument fetch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace pkvg {

// Workgroup shapes: threads per workgroup and output bytes per lane per batch.
// A narrow batch (256 lanes x 288 bytes = 72 KiB of output) holds a whole
// 64-token page of 1152-byte rows, so all of a page's loads are in flight at
// once; the wide shape (1024 x 80 bytes) does the same with four times the
// waves per workgroup.  Smaller pages take shapes sized to them (mid: 36 KiB,
// small: 20 KiB), so more of them fit on a CU at once and each workgroup's
// metadata round trip hides behind other pages' data.  Chunks per lane per
// batch follow from the chunk's output size (see unroll_of).
template <int NT, int LANE_BYTES>
struct Shape {
  static constexpr int threads = NT;
  static constexpr int lane_bytes = LANE_BYTES;
  static constexpr int waves = NT / 64;
};
using Narrow = Shape<256, 288>;
using Wide = Shape<1024, 80>;
using Mid = Shape<256, 144>;
using Small = Shape<256, 80>;

constexpr int kScanThreads = 1024;

// how a page's rows sit in memory
enum Layout : int {
  kFlat = 0,  // source token stride == destination row stride == row bytes: one contiguous span each
  kRows = 1,  // general strides: (row, chunk) addressing
};

// element conversion
enum Convert : int {
  kCopy = 0,     // bit copy
  kFp8Bf16 = 1,  // e4m3fn code -> fp32 * scale -> bf16 (RNE)
};

// One page task as the standalone builder writes it (8 int32).
struct TaskRecord {
  int32_t req;
  int32_t logical;
  int32_t page_begin;
  int32_t page_end;
  int32_t out_begin;
  int32_t phys;  // -1: skipped by the guards
  int32_t pad0;
  int32_t pad1;
};
static_assert(sizeof(TaskRecord) == 32, "task record is 32 bytes");

struct GatherParams {
  const uint8_t* src;            // element (0,0,0) of the cache
  uint8_t* dst;                  // element (0,0) of the destination
  const int32_t* block_table;
  const int32_t* cu_seq_lens;
  const int32_t* seq_starts;     // nullptr: every request starts at token 0
  const float* scale;            // fp8 only
  const TaskRecord* tasks;       // nullptr: tasks are found in the kernel (no prebuilt table)
  const int32_t* task_count;     // with tasks: device count of valid records
  int64_t src_block_stride;      // bytes
  int64_t src_token_stride;      // bytes
  int64_t dst_row_stride;        // bytes
  int64_t block_table_ld;        // int32 elements
  int64_t num_blocks;
  int64_t num_tokens;
  int32_t num_reqs;
  int32_t cu_terminal;           // 1: cu_seq_lens has num_reqs + 1 entries; 0: the last request ends at num_tokens
  int32_t task_tokens;           // tokens per task: block_size >> split_shift
  int32_t split_shift;           // a page is 2^split_shift tasks (large pages); 0: one task per page
  int32_t block_table_width;
  int32_t chunks_per_row;        // row chunks (kRows), or chunks per row of the flat span (kFlat)
  int32_t row_in_bytes;          // bytes of a source row that are gathered
  uint32_t chunks_magic;         // ceil(2^32 / chunks_per_row), or 0xFFFFFFFF for 1
  uint32_t task_tokens_magic;    // ceil(2^32 / task_tokens), or 0xFFFFFFFF for 1
  int32_t task_capacity;         // with tasks: records available
  int32_t group_shift;           // group kernel: a task is 2^group_shift consecutive pages (small pages)
  int32_t page_tokens;           // group kernel: block_size
  uint32_t page_tokens_magic;    // group kernel: ceil(2^32 / block_size), or 0xFFFFFFFF for 1
};

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ int32_t uniform(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// n / d for n < 2^32 and 1 <= d < 2^31, with a precomputed magic =
// ceil(2^32 / d) (d >= 2) or 0xFFFFFFFF (d == 1).  The multiply-high is off by
// at most one (too high for d >= 2, too low for d == 1); one step corrects it.
__device__ __forceinline__ uint32_t div_magic(uint32_t n, uint32_t d, uint32_t magic) {
  uint32_t q = __umulhi(n, magic);
  const int32_t r = static_cast<int32_t>(n - q * d);
  if (r < 0) --q;
  else if (static_cast<uint32_t>(r) >= d) ++q;
  return q;
}

// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data format;
// no swizzle, no index stride).
constexpr int32_t kBufferWord3 = 0x00020000;

// Native vector types: they stay in VGPRs through every transformation (the
// HIP uint4/uint2 wrapper structs can end up in scratch memory).  Declared with
// 4-byte alignment: CDNA's multi-dword global accesses need only dword
// alignment, so 16-byte chunks also serve rows whose pitch is a multiple of 4
// (a 1160-byte bf16 row, say).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2), aligned(4)));

// Page data is touched exactly once: nontemporal loads and stores (the "nt"
// cache policy) stream it through the caches without displacing other lines.
template <typename V>
__device__ __forceinline__ V load_stream(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
}

template <typename V>
__device__ __forceinline__ void store_stream(uint8_t* p, V v) {
  __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
}

// Cache-policy operand of the buffer store builtins on gfx950: bit 1 = nt,
// bit 4 = sc1.  sc1 alone is device scope, so the store is written through
// the XCD's L2 instead of waiting there as a dirty line; nt streams it.
constexpr int32_t kPolicyDeviceStream = 0x12;

typedef uint32_t u32x4_plain __attribute__((ext_vector_type(4)));

// Plain streaming (nt) policy of the buffer store builtins.
constexpr int32_t kPolicyStream = 0x02;

// A 16-byte device-scope streaming store at byte `off` of a buffer resource.
__device__ __forceinline__ void store_write_through(__amdgpu_buffer_rsrc_t r, uint32_t off, const u32x4_plain& v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kPolicyDeviceStream);
}

typedef uint32_t u32x2_plain __attribute__((ext_vector_type(2)));

// A chunk of 1 to 16 bytes stored at byte `off` of a buffer resource with the
// cache policy POLICY.  The hardware drops a store whose offset lies at or
// past the resource's range: a lane whose chunk is out of range passes
// kMaskedOffset (every resource here spans fewer than 2^31 bytes) and is
// masked without a branch.  Without a branch around the stores the compiler
// keeps each load ahead of them and waits for each load only before its own
// store; with one, it can move a load whose only use is the guarded store
// under the guard, and wait for every load (even every store already issued)
// before the first.
constexpr uint32_t kMaskedOffset = 0x80000000u;

template <int32_t POLICY, class T>
__device__ __forceinline__ void store_buffer(__amdgpu_buffer_rsrc_t r, uint32_t off, T v) {
  if constexpr (sizeof(T) == 16) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_plain, v), r, off, 0, POLICY);
  else if constexpr (sizeof(T) == 8) __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_plain, v), r, off, 0, POLICY);
  else if constexpr (sizeof(T) == 4) __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, POLICY);
  else if constexpr (sizeof(T) == 2) __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, v), r, off, 0, POLICY);
  else __builtin_amdgcn_raw_buffer_store_b8(__builtin_bit_cast(uint8_t, v), r, off, 0, POLICY);
}

// An empty asm statement that uses the first word of a loaded value: the load
// stays where it is issued (ahead of the guarded stores that follow) instead
// of being moved under its own store's guard.
template <class T>
__device__ __forceinline__ void keep_load_ahead(const T& x) {
  if constexpr (sizeof(T) >= 4) {
    uint32_t w;
    __builtin_memcpy(&w, &x, 4);
    asm volatile("" ::"v"(w));
  } else {
    asm volatile("" ::"v"(static_cast<uint32_t>(x)));
  }
}

template <int BYTES> struct VecOf;
template <> struct VecOf<16> { using T = u32x4; };
template <> struct VecOf<8> { using T = u32x2; };
template <> struct VecOf<4> { using T = uint32_t; };
template <> struct VecOf<2> { using T = uint16_t; };
template <> struct VecOf<1> { using T = uint8_t; };

// Token index -> task unit: floor(t / task_tokens) for 0 <= t < 2^32, a
// multiply-high instead of a 64-bit division.  Token indices stay below 2^32:
// a request starts below 2^31 and gathers fewer than 2^31 rows.  A task unit
// is a logical page, or with split_shift > 0 one of the 2^split_shift equal
// parts of a page, so that a few very large pages still spread over many
// workgroups.
__device__ __forceinline__ uint32_t page_of(const GatherParams& p, int64_t t) {
  return div_magic(static_cast<uint32_t>(t), static_cast<uint32_t>(p.task_tokens), p.task_tokens_magic);
}

// Task counts of one request: rows [b, e) of the output, source tokens from s,
// i.e. the task units holding tokens s .. s + (e - b) - 1.  A request with no
// rows has no tasks.
__device__ __forceinline__ int32_t page_count(const GatherParams& p, int64_t b, int64_t e, int64_t s) {
  const int64_t n = e - b;
  if (n <= 0) return 0;
  return static_cast<int32_t>(page_of(p, s + n - 1) - page_of(p, s) + 1);
}

__device__ __forceinline__ int64_t clamp_rows(int64_t cu, int64_t T) { return cu < T ? cu : T; }

// Unclamped output end of request r: the next cu_seq_lens entry, or num_tokens
// for the last request when cu_seq_lens has no terminal entry.
__device__ __forceinline__ int64_t request_end(const GatherParams& p, int32_t r) {
  if (p.cu_terminal || r + 1 < p.num_reqs) return p.cu_seq_lens[r + 1];
  return p.num_tokens;
}

// Inclusive prefix sum over the 64 lanes of a wave, in registers (DPP): four
// row shifts (row_shr 1, 2, 4, 8; a lane whose source lies before its row of
// 16 adds 0) give each row's own prefix, then lane 15 of rows 0 and 2 is added
// into rows 1 and 3 (row_bcast:15) and lane 31 into rows 2 and 3
// (row_bcast:31).  No LDS round trip, unlike a shuffle.
__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// Exclusive scan over the workgroup; `tmp` holds NWAVES ints of LDS.
template <int NTHREADS>
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t x, int32_t* tmp, int32_t& total) {
  constexpr int NW = NTHREADS / 64;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int32_t incl = wave_inclusive_scan(x);
  if (lane == 63) tmp[wid] = incl;
  __syncthreads();
  int32_t before = 0;
  int32_t sum = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int32_t v = tmp[w];
    before += (w < wid) ? v : 0;
    sum += v;
  }
  __syncthreads();  // tmp may be reused by the caller
  total = sum;
  return before + incl - x;
}

// ---------------------------------------------------------------------------
// task resolution
// ---------------------------------------------------------------------------

// A resolved page, all fields wave-uniform.
struct Page {
  int64_t src_off;   // byte offset of the first copied source row
  int64_t dst_off;   // byte offset of the first written destination row
  int32_t rows;      // rows to copy (<= 0: nothing)
};

// Batches of at most this many requests find their tasks inside the gather
// kernel (wave registers or an LDS prefix); larger ones use a prebuilt table.
constexpr int kFusedMaxReqs = 1024;

// Fill the LDS task prefix for the fused path: P[0..R] exclusive prefix of page
// counts, B[0..R] clamped output begins (B[R] = clamped end of the last
// request), S[0..R) source starts.  Every thread of the workgroup takes part:
// thread t owns requests [t * PER, t * PER + PER) and issues all its loads
// (PER + 1 cu_seq_lens entries, PER starts) before using any of them, so the
// prefix costs one memory round trip.  Requires R <= NT * PER.
template <int NT, int PER>
__device__ __forceinline__ void build_prefix_lds(const GatherParams& p, int32_t* P, int32_t* B,
                                                 int32_t* S, int32_t* scan_tmp) {
  const int32_t R = p.num_reqs;
  const int32_t ncu = R + p.cu_terminal;  // entries of cu_seq_lens
  const int32_t lo = static_cast<int32_t>(threadIdx.x) * PER;
  // Every load is unconditional, at an index clamped into its array (cu has
  // ncu >= R >= 1 entries, seq_starts R; without seq_starts the cu array
  // stands in), so all of them are in flight before the first wait; the
  // values past an array's end are replaced afterwards.
  const int32_t* starts = p.seq_starts != nullptr ? p.seq_starts : p.cu_seq_lens;
  int32_t cu_raw[PER + 1];
  int32_t st_raw[PER];
#pragma unroll
  for (int k = 0; k <= PER; ++k) cu_raw[k] = p.cu_seq_lens[min(lo + k, ncu - 1)];
#pragma unroll
  for (int k = 0; k < PER; ++k) st_raw[k] = starts[min(lo + k, R - 1)];
  // used here, before any branch, so no load is sunk behind another's wait
#pragma unroll
  for (int k = 0; k <= PER; ++k) asm volatile("" ::"v"(cu_raw[k]));
#pragma unroll
  for (int k = 0; k < PER; ++k) asm volatile("" ::"v"(st_raw[k]));
  // cu[lo + k], or num_tokens past the array: request r ends at entry r + 1
  int64_t cuv[PER + 1];
  int32_t st[PER];
#pragma unroll
  for (int k = 0; k <= PER; ++k) cuv[k] = lo + k < ncu ? static_cast<int64_t>(cu_raw[k]) : p.num_tokens;
#pragma unroll
  for (int k = 0; k < PER; ++k) st[k] = (p.seq_starts != nullptr && lo + k < R) ? st_raw[k] : 0;
  int32_t cnt[PER];
  int32_t sum = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    cnt[k] = 0;
    if (lo + k < R) {
      const int64_t b = clamp_rows(cuv[k], p.num_tokens);
      const int64_t e = clamp_rows(cuv[k + 1], p.num_tokens);
      cnt[k] = page_count(p, b, e, st[k]);
      B[lo + k] = static_cast<int32_t>(b);
      S[lo + k] = st[k];
      sum += cnt[k];
      if (lo + k == R - 1) B[R] = static_cast<int32_t>(e);  // the last request's clamped end
    }
  }
  int32_t total;
  int32_t off = block_exclusive_scan<NT>(sum, scan_tmp, total);
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if (lo + k < R) {
      P[lo + k] = off;
      off += cnt[k];
    }
  }
  if (threadIdx.x == 0) P[R] = total;
  __syncthreads();
}

// The LDS prefix with the smallest share of requests per thread that covers
// the batch: each thread's loads, page counts and serial scan grow with its
// share, whatever the batch size.  Against one share for every batch size (4
// requests per thread of a 256-lane workgroup), measured: 512 x 200 tokens on
// 64-token pages 46.5 -> 44.2 us (fp8 38.1 -> 36.4 us), on one-token pages
// 47.2 -> 45.0 us, on 16-token pages -1.1%; 128 x 2000 fp8 tokens 80.6 -> 78.2
// us; 300 x 3000 tokens +1.3%; 1,024 requests (the full share) unchanged.
template <int NT>
__device__ __forceinline__ void build_prefix_lds_for(const GatherParams& p, int32_t* P, int32_t* B,
                                                     int32_t* S, int32_t* scan_tmp) {
  constexpr int MAX_PER = (kFusedMaxReqs + NT - 1) / NT;
  if constexpr (MAX_PER >= 4) {
    if (p.num_reqs <= NT) return build_prefix_lds<NT, 1>(p, P, B, S, scan_tmp);
    if (p.num_reqs <= 2 * NT) return build_prefix_lds<NT, 2>(p, P, B, S, scan_tmp);
  }
  build_prefix_lds<NT, MAX_PER>(p, P, B, S, scan_tmp);
}

// Batches of at most 64 requests: every wave holds the whole task prefix in
// registers (lane r <-> request r), built without LDS or a barrier.
constexpr int kWaveMaxReqs = 64;

struct WavePrefix {
  int32_t incl;   // inclusive prefix of page counts up to this lane's request
  int32_t count;  // this lane's page count
  int32_t b;      // clamped output begin of this lane's request
  int32_t e;      // clamped output end
  int32_t s;      // source start
  int32_t total;  // all tasks (uniform)
};

// The wave prefix's metadata: this lane's cu_seq_lens entry, the next one and
// its seq_start.  The three loads are unconditional, at indices clamped into
// their arrays (cu_seq_lens has ncu >= R >= 1 entries, seq_starts R; without
// seq_starts the cu array stands in), so they share one memory round trip;
// build_prefix_wave replaces the values of lanes past the arrays' ends.  The
// batch builds issue them first thing, ahead of the task-mode branches: where
// the other modes' code joins the path in front of them, the compiler waits
// for every outstanding scalar load (the parameter struct's fetch among them)
// before they go out.  Measured: 8 x 7,680 one-token pages 27.84 -> 27.49 us;
// the page kernel's batches unchanged.
struct WaveLoads {
  int32_t c0, c1, sv;
};

__device__ __forceinline__ WaveLoads issue_wave_loads(const GatherParams& p) {
  const int lane = threadIdx.x & 63;
  const int32_t R = p.num_reqs;
  const int32_t ncu = R + p.cu_terminal;
  const int32_t* starts = p.seq_starts ? p.seq_starts : p.cu_seq_lens;
  WaveLoads l;
  l.c0 = p.cu_seq_lens[min(lane, ncu - 1)];
  l.c1 = p.cu_seq_lens[min(lane + 1, ncu - 1)];
  l.sv = starts[min(lane, R - 1)];
  // used here, so the compiler cannot sink a load into a later branch (behind
  // the wait for the others)
  asm volatile("" ::"v"(l.c0), "v"(l.c1), "v"(l.sv));
  return l;
}

// Request r ends at entry r + 1, or at num_tokens when that entry does not exist.

__device__ __forceinline__ WavePrefix build_prefix_wave(const GatherParams& p, const WaveLoads& l) {
  const int lane = threadIdx.x & 63;
  const int32_t R = p.num_reqs;
  WavePrefix w;
  // lanes past the arrays' ends replace the loaded values
  const int32_t ncu = R + p.cu_terminal;
  const int32_t c0 = l.c0, c1 = l.c1, sv = l.sv;
  const int64_t cb = lane < R ? c0 : 0;
  const int64_t ce = lane < R ? (lane + 1 < ncu ? static_cast<int64_t>(c1) : p.num_tokens) : 0;
  w.b = static_cast<int32_t>(clamp_rows(cb, p.num_tokens));
  w.e = static_cast<int32_t>(clamp_rows(ce, p.num_tokens));
  w.s = (lane < R && p.seq_starts) ? sv : 0;
  w.count = lane < R ? page_count(p, w.b, w.e, w.s) : 0;
  const int32_t incl = wave_inclusive_scan(w.count);
  w.incl = incl;
  w.total = uniform(__builtin_amdgcn_readlane(incl, 63));
  return w;
}

// Largest r in [0, R) with P[r] <= task (P non-decreasing, P[0] = 0).
__device__ __forceinline__ int32_t find_request(const int32_t* P, int32_t R, int32_t task) {
  int32_t lo = 0, hi = R;  // answer in [lo, hi)
  while (hi - lo > 1) {
    const int32_t mid = (lo + hi) >> 1;
    if (P[mid] <= task) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Geometry of task `task` of request r: copies slots [pbeg, pend) of logical
// page `logical` into output rows from `out_begin`.
struct TaskGeom {
  int32_t logical;
  int32_t pbeg;
  int32_t pend;
  int64_t out_begin;
};

__device__ __forceinline__ TaskGeom task_geometry(const GatherParams& p, int32_t j, int64_t b, int64_t e,
                                                  int64_t s) {
  const int32_t tt = p.task_tokens;
  const int64_t n = e - b > 0 ? e - b : 0;
  const int64_t unit = static_cast<int64_t>(page_of(p, s)) + j;
  const int64_t unit0 = unit * tt;
  const int64_t cb = s > unit0 ? s : unit0;
  const int64_t ce = (s + n) < (unit0 + tt) ? (s + n) : (unit0 + tt);
  // the unit's first slot inside its page
  const int32_t sub = static_cast<int32_t>(unit & ((int64_t(1) << p.split_shift) - 1)) * tt;
  TaskGeom g;
  g.logical = static_cast<int32_t>(unit >> p.split_shift);
  g.pbeg = static_cast<int32_t>(cb - unit0) + sub;
  g.pend = static_cast<int32_t>(ce - unit0) + sub;
  g.out_begin = b + (cb - s);
  return g;
}

// Physical block of (r, logical), or -1 if a guard skips the page.
__device__ __forceinline__ int64_t lookup_block(const GatherParams& p, int32_t r, int32_t logical) {
  if (logical < 0 || logical >= p.block_table_width) return -1;
  const int64_t pb = p.block_table[static_cast<int64_t>(r) * p.block_table_ld + logical];
  if (pb < 0 || pb >= p.num_blocks) return -1;
  return pb;
}

__device__ __forceinline__ Page page_from(const GatherParams& p, int64_t phys, int32_t pbeg, int32_t pend,
                                          int64_t out_begin) {
  Page pg;
  pg.rows = phys < 0 ? 0 : pend - pbeg;
  pg.src_off = phys * p.src_block_stride + static_cast<int64_t>(pbeg) * p.src_token_stride;
  pg.dst_off = out_begin * p.dst_row_stride;
  return pg;
}

// ---------------------------------------------------------------------------
// page bodies
// ---------------------------------------------------------------------------

// K fp8 codes held in registers: 8 codes in two dwords, fewer in one.
template <int K> struct CodesOf { using T = uint32_t; };
template <> struct CodesOf<8> { using T = u32x2; };

// K fp8 codes, read as one K-byte word when SRC_VEC (code rows dword-aligned
// for K >= 4, K-aligned below) else byte by byte.
template <int K, bool SRC_VEC>
__device__ __forceinline__ typename CodesOf<K>::T load_codes(const uint8_t* q) {
  if constexpr (SRC_VEC && K == 8) {
    return load_stream<u32x2>(q);
  } else if constexpr (SRC_VEC && K == 4) {
    return load_stream<uint32_t>(q);
  } else if constexpr (SRC_VEC && K == 2) {
    return load_stream<uint16_t>(q);
  } else if constexpr (K == 8) {
    u32x2 w = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w.x |= static_cast<uint32_t>(q[i]) << (8 * i);
      w.y |= static_cast<uint32_t>(q[4 + i]) << (8 * i);
    }
    return w;
  } else {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < K; ++i) w |= static_cast<uint32_t>(q[i]) << (8 * i);
    return w;
  }
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two codes (bytes 0-1 or 2-3 of w) -> two bf16 packed in one dword:
// v_cvt_pk_f32_fp8 (exact), v_mul_f32 by the scale, v_cvt_pk_bf16_f32 (RNE).
__device__ __forceinline__ uint32_t dequant_pair(uint32_t w, bool high, float scale) {
  f32x2 f = high ? __builtin_amdgcn_cvt_pk_f32_fp8(w, true) : __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  f.x = f.x * scale;
  f.y = f.y * scale;
  const bf16x2 h = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

template <int K>
struct OutOf {
  using T = typename VecOf<2 * K>::T;
};

template <int K>
__device__ __forceinline__ typename OutOf<K>::T dequant_codes(typename CodesOf<K>::T w, float scale) {
  if constexpr (K == 8) {
    u32x4 o;
    o.x = dequant_pair(w.x, false, scale);
    o.y = dequant_pair(w.x, true, scale);
    o.z = dequant_pair(w.y, false, scale);
    o.w = dequant_pair(w.y, true, scale);
    return o;
  } else if constexpr (K == 4) {
    u32x2 o;
    o.x = dequant_pair(w, false, scale);
    o.y = dequant_pair(w, true, scale);
    return o;
  } else if constexpr (K == 2) {
    return dequant_pair(w, false, scale);
  } else {
    return static_cast<uint16_t>(dequant_pair(w, false, scale) & 0xFFFFu);
  }
}

// Where a page's source rows are read from.  fp8 code rows that are not
// dword-aligned (a 577-byte row pitch, say) are read as dword-aligned windows
// around each lane's K codes, then shifted into place: one 12- or 8-byte load
// instead of K byte loads.  A window is clamped to end at `lim`, the page's
// used bytes rounded up to a whole dword, so no load touches a dword that
// holds none of the page's codes.
struct PageSrc {
  const uint8_t* ptr;    // first copied row of the page
  const uint8_t* base4;  // windowed mode: ptr rounded down to 4 bytes
  uint32_t delta;        // windowed mode: ptr - base4
  uint32_t lim;          // windowed mode: used bytes from base4, rounded up to 4
};

__device__ __forceinline__ PageSrc page_src(const uint8_t* ptr, uint32_t used_bytes) {
  PageSrc ps;
  ps.ptr = ptr;
  ps.delta = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ptr) & 3u);
  ps.base4 = ptr - ps.delta;
  ps.lim = (used_bytes + ps.delta + 3u) & ~3u;
  return ps;
}

// K (4 or 8) codes at byte `off` from base4, any alignment.  The window starts
// at the dword holding byte `off`, or earlier when that would pass `lim`; the
// codes then sit 0..4 bytes into it.  Needs lim >= 12 (K = 8) or 8 (K = 4).
template <int K>
__device__ __forceinline__ typename CodesOf<K>::T load_codes_window(const uint8_t* base4, uint32_t off,
                                                                   uint32_t lim) {
  constexpr uint32_t kWin = K == 8 ? 12u : 8u;
  const uint32_t a = min(off & ~3u, lim - kWin);
  const uint32_t sh = off - a;
  if constexpr (K == 8) {
    const u32x2 lo = load_stream<u32x2>(base4 + a);
    const uint32_t hi = load_stream<uint32_t>(base4 + a + 8);
    u32x2 w;
    w.x = sh == 4 ? lo.y : __builtin_amdgcn_alignbyte(lo.y, lo.x, sh);
    w.y = sh == 4 ? hi : __builtin_amdgcn_alignbyte(hi, lo.y, sh);
    return w;
  } else {
    static_assert(K == 4, "windowed code loads take 4 or 8 codes");
    const u32x2 d = load_stream<u32x2>(base4 + a);
    return sh == 4 ? d.y : __builtin_amdgcn_alignbyte(d.y, d.x, sh);
  }
}

// What one chunk stores: W raw bytes, or the 2W bytes of bf16 for W codes.
template <int CONVERT, int W> struct ChunkOut { using T = typename VecOf<W>::T; };
template <int W> struct ChunkOut<kFp8Bf16, W> { using T = typename OutOf<W>::T; };

// Where a page's rows are written: the first output row, and a buffer resource
// over the page's output span (used by write-through stores, which address it
// with 32-bit offsets).
struct PageDst {
  uint8_t* ptr;
  __amdgpu_buffer_rsrc_t rsrc;
};

__device__ __forceinline__ PageDst page_dst(uint8_t* ptr, uint32_t span_bytes) {
  PageDst pd;
  pd.ptr = ptr;
  pd.rsrc = __builtin_amdgcn_make_buffer_rsrc(ptr, 0, static_cast<int32_t>(span_bytes), kBufferWord3);
  return pd;
}

// How one chunk of a page moves: a raw chunk is W bytes; an fp8 chunk is W
// codes in, 2W bytes of bf16 out.  Chunk c of a page lies at byte c * in_bytes
// (kFlat) or at row c / chunks_per_row, column c % chunks_per_row (kRows).
template <int CONVERT, int W, int LAYOUT, bool SRC_VEC>
struct Mover {
  static constexpr int in_bytes = W;
  static constexpr int out_bytes = CONVERT == kCopy ? W : 2 * W;
  static constexpr int layout = LAYOUT;
  static constexpr bool is_copy = CONVERT == kCopy;
  // unaligned fp8 code rows of 4 or 8 codes per lane are read as shifted windows
  static constexpr bool windowed = CONVERT == kFp8Bf16 && !SRC_VEC && (W == 4 || W == 8);
  using Reg = typename std::conditional<CONVERT == kCopy, typename VecOf<W>::T, typename CodesOf<W>::T>::type;

  __device__ static __forceinline__ void load(const GatherParams& p, const PageSrc& src, uint32_t c, Reg& r) {
    uint32_t off;  // byte offset of chunk c from the page's first row
    if constexpr (LAYOUT == kFlat) {
      off = c * in_bytes;
    } else {
      const uint32_t cpr = static_cast<uint32_t>(p.chunks_per_row);
      const uint32_t row = div_magic(c, cpr, p.chunks_magic);
      off = row * static_cast<uint32_t>(p.src_token_stride) + (c - row * cpr) * in_bytes;
    }
    if constexpr (windowed) r = load_codes_window<W>(src.base4, off + src.delta, src.lim);
    else if constexpr (CONVERT == kCopy) r = load_stream<Reg>(src.ptr + off);
    else r = load_codes<W, SRC_VEC>(src.ptr + off);
  }

  // what a chunk stores: the loaded bytes, or the bf16 values of its codes
  using Out = typename ChunkOut<CONVERT, W>::T;

  __device__ static __forceinline__ Out convert(const Reg& r, float scale) {
    if constexpr (CONVERT == kCopy) return r;
    else return dequant_codes<W>(r, scale);
  }

  // WRITE_THROUGH (16-byte chunks of a flat page only): a device-scope
  // streaming store through the page's buffer resource; otherwise a plain
  // nontemporal store.
  template <bool WRITE_THROUGH>
  __device__ static __forceinline__ void store(const GatherParams& p, const PageDst& dst, uint32_t c,
                                               const Out& o) {
    if constexpr (WRITE_THROUGH) {
      static_assert(LAYOUT == kFlat && out_bytes == 16, "write-through stores take 16-byte chunks of flat pages");
      store_write_through(dst.rsrc, c * out_bytes, __builtin_bit_cast(u32x4_plain, o));
    } else {
      uint8_t* q;
      if constexpr (LAYOUT == kFlat) {
        q = dst.ptr + c * out_bytes;
      } else {
        const uint32_t cpr = static_cast<uint32_t>(p.chunks_per_row);
        const uint32_t row = div_magic(c, cpr, p.chunks_magic);
        q = dst.ptr + row * p.dst_row_stride + (c - row * cpr) * out_bytes;
      }
      store_stream(q, o);
    }
  }
};

// Chunks per lane per batch: the shape's output bytes per lane over one
// chunk's output bytes, at most 18 (16-byte chunks: 18 narrow, 5 wide).
template <class SH, class M>
constexpr int unroll_of() {
  constexpr int u = SH::lane_bytes / M::out_bytes;
  return u < 1 ? 1 : (u > 18 ? 18 : u);
}

// A batch is U = unroll_of<SH, M>() chunks per lane: chunks c0 + u * SH::threads.  Every
// lane issues its loads back to back; a lane whose chunk runs past the end
// (n chunks) loads the last chunk again (in bounds, one cache line) and later
// skips its store, so the loads carry no branch.  The page pointers are
// deliberately not __restrict__: that keeps the compiler from moving a load
// below an earlier store (which would interleave load, wait, store).
template <class SH, class M>
__device__ __forceinline__ void load_batch(const GatherParams& p, const PageSrc& s, uint32_t n, uint32_t c0,
                                           typename M::Reg (&r)[unroll_of<SH, M>()]) {
#pragma unroll
  for (int u = 0; u < unroll_of<SH, M>(); ++u) M::load(p, s, min(c0 + u * SH::threads, n - 1), r[u]);
}

// Stores of one batch.  Each chunk past the unit's end is masked: by an
// out-of-range buffer offset (flat pages that convert or take the wide shape,
// no branch) or by its lane's guard (the rest).  On flat pages with the wide
// shape, a wave whose lanes all have their first U - 1 chunks in range (every
// wave of a full page: a page's chunk count is a multiple of 64, so the
// wave's lanes agree on each chunk but the last) waits for all its loads,
// converts every chunk, and issues those U - 1 stores back to back, then the
// last one masked (the 300K fp8 gather -4%, skew-8 raw -1.5%; slower on the
// narrow-shape and strided gathers).  16-byte chunks of flat pages go out as
// device-scope (write-through) streaming stores, in every shape: nothing is
// left dirty in the XCD's L2 for the end of the launch to write back (a
// single cold call of the 60K raw gather 28.1 -> 27.1 us, back to back
// 24.83 -> 24.67 us).  Row-layout pages keep nontemporal stores: their rows'
// partial lines would reach memory as separate masked writes.
template <class SH, class M>
__device__ __forceinline__ void store_batch(const GatherParams& p, const PageDst& d, uint32_t n, uint32_t c0,
                                            const typename M::Reg (&r)[unroll_of<SH, M>()], float scale) {
  constexpr int U = unroll_of<SH, M>();
  constexpr bool burst = SH::threads == Wide::threads && M::layout == kFlat && U >= 2;
  // device-scope write-through stores for every 16-byte chunk of a flat page
  constexpr bool write_through = M::layout == kFlat && M::out_bytes == 16;
  // masked buffer stores for flat pages that convert or take the wide shape; raw
  // copies in the narrower shapes keep lane-guarded stores, where a batch's
  // slots past the unit's end (a 9 KiB unit fills 2.25 of the small shape's 5)
  // would otherwise all issue dropped stores
  constexpr bool buffer_stores = M::layout == kFlat && (!M::is_copy || SH::threads == Wide::threads);
  if constexpr (burst) {
    // chunk c0 of the wave's last lane (wave-uniform): in range means every lane is
    const uint32_t wave_last = static_cast<uint32_t>(uniform(static_cast<int32_t>(c0 - (threadIdx.x & 63u)))) + 63u;
    if (wave_last + (U - 2) * SH::threads < n) {
      typename M::Out o[U];
#pragma unroll
      for (int u = 0; u < U; ++u) o[u] = M::convert(r[u], scale);
      // a copy has no conversion to wait on: wait for all its loads here
      if constexpr (M::is_copy) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
      for (int u = 0; u < U - 1; ++u) M::template store<write_through>(p, d, c0 + u * SH::threads, o[u]);
      const uint32_t c = c0 + (U - 1) * SH::threads;
      if (c < n) M::template store<write_through>(p, d, c, o[U - 1]);
      return;
    }
  }
  if constexpr (buffer_stores) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t c = c0 + u * SH::threads;
      store_buffer<write_through ? kPolicyDeviceStream : kPolicyStream>(d.rsrc, c < n ? c * M::out_bytes : kMaskedOffset,
                                                                        M::convert(r[u], scale));
    }
  } else {
    if constexpr (M::layout == kFlat) keep_load_ahead(r[0]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t c = c0 + u * SH::threads;
      if (c < n) M::template store<write_through>(p, d, c, M::convert(r[u], scale));
    }
  }
}

// A page of any size: batch after batch.
template <class SH, class M>
__device__ __forceinline__ void move_page(const GatherParams& p, const PageSrc& s, const PageDst& d, uint32_t n,
                                          float scale) {
  constexpr int U = unroll_of<SH, M>();
  for (uint32_t c0 = threadIdx.x; c0 - threadIdx.x < n; c0 += SH::threads * U) {
    typename M::Reg r[U];
    load_batch<SH, M>(p, s, n, c0, r);
    store_batch<SH, M>(p, d, n, c0, r, scale);
  }
}

// ---------------------------------------------------------------------------
// the gather kernel
// ---------------------------------------------------------------------------

// Task lookup for one workgroup: in-wave registers (small batches), an LDS
// prefix, a prebuilt task table (large batches), or one request.
// kWalk: the table is walked directly -- workgroup (x, y) takes task unit x of
// request y's block-table row (unit x of the row's columns, whether or not the
// request's rows reach it), so its table entry and its request's extent are
// known before any load, as for one request.  Chosen for batches whose table
// is dense (rows about as wide as their requests' pages), where the units
// past a request's pages that find nothing to do are few.
enum TaskMode : int { kWaveRegs = 0, kLdsPrefix = 1, kTable = 2, kSingle = 3, kWalk = 4 };

struct TaskSource {
  int mode;
  WavePrefix wp;
  const int32_t* P;
  const int32_t* B;
  const int32_t* S;
  int32_t r;               // kSingle, kWalk: the request
  int32_t b, e, s;         // kSingle, kWalk: the request's clamped extent and source start
  int32_t first_phys_raw;  // kSingle, kWalk: table entry of this workgroup's first task (-1 past the row)
};

// Resolve `task` (the same for every lane) to its page, all fields wave-uniform.
__device__ __forceinline__ Page resolve_task(const GatherParams& p, const TaskSource& ts, int32_t task) {
  if (ts.mode == kSingle) {
    const TaskGeom g = task_geometry(p, task, ts.b, ts.e, ts.s);
    int64_t phys;
    if (task == static_cast<int32_t>(blockIdx.x)) {
      phys = g.logical < p.block_table_width ? ts.first_phys_raw : -1;
      if (phys >= p.num_blocks) phys = -1;
    } else {
      phys = lookup_block(p, 0, g.logical);
    }
    return page_from(p, uniform64(phys < 0 ? -1 : phys), g.pbeg, g.pend, g.out_begin);
  }
  if (ts.mode == kWalk) {
    // task = the unit's index in its table row; j = its index among the request's units
    const int32_t j = task - static_cast<int32_t>(page_of(p, ts.s));
    if (j < 0 || j >= page_count(p, ts.b, ts.e, ts.s)) return Page{0, 0, 0};
    const TaskGeom g = task_geometry(p, j, ts.b, ts.e, ts.s);
    int64_t phys;
    if (task == static_cast<int32_t>(blockIdx.x)) {
      phys = ts.first_phys_raw;
      if (phys >= p.num_blocks) phys = -1;
    } else {
      phys = lookup_block(p, ts.r, g.logical);
    }
    return page_from(p, uniform64(phys < 0 ? -1 : phys), g.pbeg, g.pend, g.out_begin);
  }
  if (ts.mode == kWaveRegs) {
    // the task's request: the number of requests whose inclusive prefix is <= task
    // (at most R - 1 while task < total; the min keeps every table row in range regardless)
    const int32_t r = min(uniform(static_cast<int32_t>(__popcll(__ballot(ts.wp.incl <= task)))), p.num_reqs - 1);
    const int32_t b = uniform(__builtin_amdgcn_readlane(ts.wp.b, r));
    const int32_t e = uniform(__builtin_amdgcn_readlane(ts.wp.e, r));
    const int32_t s = uniform(__builtin_amdgcn_readlane(ts.wp.s, r));
    const int32_t first = uniform(__builtin_amdgcn_readlane(ts.wp.incl - ts.wp.count, r));
    const TaskGeom g = task_geometry(p, task - first, b, e, s);
    return page_from(p, uniform64(lookup_block(p, r, g.logical)), g.pbeg, g.pend, g.out_begin);
  }
  if (ts.mode == kLdsPrefix) {
    const int32_t r = uniform(find_request(ts.P, p.num_reqs, task));
    const TaskGeom g = task_geometry(p, task - uniform(ts.P[r]), uniform(ts.B[r]), uniform(ts.B[r + 1]),
                                     uniform(ts.S[r]));
    return page_from(p, uniform64(lookup_block(p, r, g.logical)), g.pbeg, g.pend, g.out_begin);
  }
  const TaskRecord t = p.tasks[task];
  return page_from(p, uniform(t.phys), uniform(t.page_begin), uniform(t.page_end),
                   static_cast<int64_t>(uniform(t.out_begin)));
}

// One int32 read through the vector memory path.  Its wait (vmcnt) leaves the
// scalar loads in flight alone: scalar loads complete in any order, so waiting
// for one scalar load waits for all of them, kernel arguments included.
__device__ __forceinline__ int32_t load_i32_vector_path(const int32_t* q) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(q), 0, 4, kBufferWord3);
  return uniform(__builtin_amdgcn_raw_buffer_load_b32(r, 0, 0, 0));
}

// The task mode of a launch (low byte of the mode argument).  Each kernel is
// built three times: for one request, where the mode is the constant kSingle
// and the other modes' code drops out; for the table walk, where it is the
// constant kWalk; and for batches found through a prefix or a task table,
// where the compiler is told it is neither.  Measured on one request against
// a single build for all modes: 61,440 tokens on 64-token pages 25.2 -> 25.05
// us, on 1,024-token pages 25.14 -> 24.92 us.
enum Build : int { kBuildSingle = 0, kBuildWalk = 1, kBuildPrefix = 2 };

template <int BUILD>
__device__ __forceinline__ int task_mode_of(int32_t mode_arg) {
  if constexpr (BUILD == kBuildSingle) return kSingle;
  if constexpr (BUILD == kBuildWalk) return kWalk;
  const int mode = mode_arg & 0xFF;
  __builtin_assume(mode != kSingle && mode != kWalk);
  return mode;
}

// The walk's prologue: this workgroup's request is blockIdx.y and its first
// unit blockIdx.x; the block-table entry at column `lb0` of the request's row
// (per lane in the group kernel, where lanes without a page of the group pass
// lane_reads = false), the extent and the start are all requested at once.
// Every load is unconditional: an always-valid address stands in for an
// absent one.  Returns the entry read, or -1 past the row.
__device__ __forceinline__ int32_t walk_prologue(const GatherParams& p, int32_t table_ld, int64_t lb0,
                                                 bool lane_reads, TaskSource& ts) {
  const int32_t r = static_cast<int32_t>(blockIdx.y);
  const bool in_row = lane_reads && lb0 < p.block_table_width;
  const int32_t* entry_at = in_row ? p.block_table + int64_t(r) * table_ld + lb0 : p.cu_seq_lens;
  const bool has_end = p.cu_terminal || r + 1 < p.num_reqs;  // else the request ends at num_tokens
  const int32_t* end_at = p.cu_seq_lens + (has_end ? r + 1 : r);
  // the table entry does not depend on the start, so it goes out first
  const int32_t raw = *entry_at;
  const int32_t cb = uniform(p.cu_seq_lens[r]);
  const int32_t ce = uniform(*end_at);
  ts.s = p.seq_starts ? load_i32_vector_path(p.seq_starts + r) : 0;
  ts.r = r;
  ts.b = static_cast<int32_t>(clamp_rows(cb, p.num_tokens));
  ts.e = static_cast<int32_t>(clamp_rows(has_end ? ce : p.num_tokens, p.num_tokens));
  return in_row ? raw : -1;
}


// CONVERT == kCopy: W = bytes per lane access.  CONVERT == kFp8Bf16: W = codes
// per lane access.  Grid: any size along x (the host launches one workgroup
// per task); workgroup w takes tasks w, w + gridDim.x, ...; along y, the
// requests of a table walk (1 otherwise).  Dynamic LDS (LDS-prefix mode, 64 <
// num_reqs): (3 * num_reqs + 2) int32.
//
// The leading scalar arguments repeat the fields of `params` that the task
// lookup needs first (num_tokens as 32 bits, which the host guarantees, and
// the table pitch, used by the walk); `mode_and_split` holds the TaskMode the
// host chose (low byte) and split_shift (the byte above it).  These 14 dwords
// are preloaded into SGPRs when a wave starts (gfx950 kernarg preloading, at
// most 14 argument dwords), so the metadata loads go out without waiting for
// a kernel argument fetch; the struct arrives while they are in flight.
template <class SH, int CONVERT, int W, int LAYOUT, bool SRC_VEC, int BUILD>
__global__ __launch_bounds__(SH::threads) void gather_pages_kernel(
    const int32_t* cu_seq_lens, const int32_t* block_table, const int32_t* seq_starts,
    int32_t mode_and_split, int32_t num_reqs, int32_t task_tokens, uint32_t task_tokens_magic,
    int32_t block_table_width, int32_t cu_terminal, int32_t num_tokens, int32_t table_ld,
    GatherParams params) {
  using M = Mover<CONVERT, W, LAYOUT, SRC_VEC>;
  GatherParams p = params;
  p.cu_seq_lens = cu_seq_lens;
  p.block_table = block_table;
  p.seq_starts = seq_starts;
  p.num_reqs = num_reqs;
  p.task_tokens = task_tokens;
  p.task_tokens_magic = task_tokens_magic;
  p.split_shift = mode_and_split >> 8;
  p.block_table_width = block_table_width;
  p.cu_terminal = cu_terminal;
  p.num_tokens = num_tokens;
  extern __shared__ int32_t lds[];
  __shared__ int32_t scan_tmp[SH::waves];

  const int32_t R = p.num_reqs;
  TaskSource ts;
  ts.mode = task_mode_of<BUILD>(mode_and_split);
  WaveLoads wave_loads{};
  if constexpr (BUILD == kBuildPrefix) {
    if (ts.mode == kWaveRegs) wave_loads = issue_wave_loads(p);
  }
  int32_t* P = lds;
  int32_t* B = lds + (R + 1);
  int32_t* S = lds + 2 * (R + 1);
  ts.P = P;
  ts.B = B;
  ts.S = S;

  int32_t num_tasks;
  if (ts.mode == kWalk) {
    // one workgroup per unit of each table row (grid x by num_reqs): this
    // workgroup takes exactly its own unit
    ts.first_phys_raw = uniform(walk_prologue(p, table_ld, blockIdx.x >> p.split_shift, true, ts));
    num_tasks = static_cast<int32_t>(blockIdx.x) + 1;
  } else if (ts.mode == kSingle) {
    // The first task's logical block is (seq_start / task_tokens + blockIdx.x)
    // >> split_shift: its block-table entry is requested together with the
    // request extent instead of after it (one dependent memory round trip
    // less).  Every load here is unconditional (an always-valid address stands
    // in for an absent one) and the start goes through the vector path, so
    // without seq_starts nothing waits before the entry and the extent are
    // requested.
    ts.s = p.seq_starts ? load_i32_vector_path(p.seq_starts) : 0;
    const uint32_t lb0 = (page_of(p, ts.s) + blockIdx.x) >> p.split_shift;
    const bool in_row = lb0 < static_cast<uint32_t>(p.block_table_width);
    const int32_t* entry_at = in_row ? p.block_table + lb0 : p.cu_seq_lens;
    const int32_t* end_at = p.cu_seq_lens + p.cu_terminal;  // cu_terminal is 0 or 1
    const int32_t raw = uniform(*entry_at);
    const int32_t cb = uniform(p.cu_seq_lens[0]);
    const int32_t ce = uniform(*end_at);
    // The page copy's kernel arguments are fetched while those loads are in
    // flight: the empty asm needs them in SGPRs before the loaded values are
    // used, so the compiler cannot leave their fetch for after that wait.
    asm volatile("" ::"s"(p.src), "s"(p.dst), "s"(p.src_block_stride), "s"(p.src_token_stride),
                 "s"(p.dst_row_stride), "s"(p.num_blocks), "s"(p.row_in_bytes), "s"(p.chunks_per_row));
    ts.first_phys_raw = in_row ? raw : -1;
    ts.b = static_cast<int32_t>(clamp_rows(cb, p.num_tokens));
    ts.e = static_cast<int32_t>(clamp_rows(p.cu_terminal ? ce : p.num_tokens, p.num_tokens));
    num_tasks = page_count(p, ts.b, ts.e, ts.s);
  } else if (ts.mode == kWaveRegs) {
    ts.wp = build_prefix_wave(p, wave_loads);
    num_tasks = ts.wp.total;
  } else if (ts.mode == kLdsPrefix) {
    build_prefix_lds_for<SH::threads>(p, P, B, S, scan_tmp);
    num_tasks = P[R];
  } else {
    num_tasks = min(*p.task_count, p.task_capacity);
  }
  num_tasks = uniform(num_tasks);
  float scale = 1.0f;
  if constexpr (CONVERT == kFp8Bf16)
    scale = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(*p.scale)));

  const uint32_t cpr = static_cast<uint32_t>(p.chunks_per_row);
  for (int32_t task = blockIdx.x; task < num_tasks; task += gridDim.x) {
    const Page pg = resolve_task(p, ts, task);
    if (pg.rows <= 0) continue;
    const uint32_t used = static_cast<uint32_t>(pg.rows - 1) * static_cast<uint32_t>(p.src_token_stride) +
                          static_cast<uint32_t>(p.row_in_bytes);
    const uint32_t n = static_cast<uint32_t>(pg.rows) * cpr;
    move_page<SH, M>(p, page_src(p.src + uniform64(pg.src_off), used),
                     page_dst(p.dst + uniform64(pg.dst_off), n * M::out_bytes), n, scale);
  }
}

// ---------------------------------------------------------------------------
// page groups: pages of a few tokens
// ---------------------------------------------------------------------------

// A page of one to a few rows is too little work for a workgroup of its own:
// the metadata round trips, not the data, would set the pace.  The group
// kernel's task is instead G = 2^group_shift consecutive logical pages of one
// request (task_tokens = G * block_size), whose rows are contiguous in the
// output but scattered in the cache.  Each wave looks the group's G pages up
// once (lane i holds page i's physical block, -1 when a guard skips it), and
// every chunk fetches its row's block from that lane with a cross-lane read.

struct GroupTask {
  int32_t req;
  int32_t unit;       // group index within the request's logical pages
  int32_t gbeg;       // first token copied, relative to the group's first token
  int32_t gend;
  int64_t out_begin;  // first output row
};

__device__ __forceinline__ GroupTask group_from(int32_t r, const TaskGeom& g) {
  GroupTask t;
  t.req = r;
  t.unit = g.logical;
  t.gbeg = g.pbeg;
  t.gend = g.pend;
  t.out_begin = g.out_begin;
  return t;
}

// `task` -> its group, all fields wave-uniform (task geometry with split_shift 0
// and task_tokens = G * block_size gives group-relative token ranges).
__device__ __forceinline__ GroupTask resolve_group(const GatherParams& p, const TaskSource& ts, int32_t task) {
  if (ts.mode == kSingle) return group_from(0, task_geometry(p, task, ts.b, ts.e, ts.s));
  if (ts.mode == kWalk) {
    // task = the group's index in its table row; j = its index among the request's groups
    const int32_t j = task - static_cast<int32_t>(page_of(p, ts.s));
    if (j < 0 || j >= page_count(p, ts.b, ts.e, ts.s)) {
      GroupTask none{};
      return none;  // gbeg == gend: nothing to move
    }
    return group_from(ts.r, task_geometry(p, j, ts.b, ts.e, ts.s));
  }
  if (ts.mode == kWaveRegs) {
    // (at most R - 1 while task < total; the min keeps every table row in range regardless)
    const int32_t r = min(uniform(static_cast<int32_t>(__popcll(__ballot(ts.wp.incl <= task)))), p.num_reqs - 1);
    const int32_t b = uniform(__builtin_amdgcn_readlane(ts.wp.b, r));
    const int32_t e = uniform(__builtin_amdgcn_readlane(ts.wp.e, r));
    const int32_t s = uniform(__builtin_amdgcn_readlane(ts.wp.s, r));
    const int32_t first = uniform(__builtin_amdgcn_readlane(ts.wp.incl - ts.wp.count, r));
    return group_from(r, task_geometry(p, task - first, b, e, s));
  }
  if (ts.mode == kLdsPrefix) {
    const int32_t r = uniform(find_request(ts.P, p.num_reqs, task));
    return group_from(r, task_geometry(p, task - uniform(ts.P[r]), uniform(ts.B[r]), uniform(ts.B[r + 1]),
                                       uniform(ts.S[r])));
  }
  const TaskRecord rec = p.tasks[task];
  GroupTask t;
  t.req = uniform(rec.req);
  t.unit = uniform(rec.logical);
  t.gbeg = uniform(rec.page_begin);
  t.gend = uniform(rec.page_end);
  t.out_begin = uniform(rec.out_begin);
  return t;
}

// Moves a group's n chunks in batches of U per lane: chunk c is column c % cpr
// of the group's row c / cpr, which holds token gbeg + c / cpr counted from the
// group's first token.  `lane_phys` is the physical block of this lane's page
// of the group (lane < G), -1 when a guard skips it.  In a batch every chunk
// first finds its row and page, then all chunks fetch their page's block with
// cross-lane reads, then all loads go out: the phases keep the cross-lane
// reads from serialising the loads.  As in the page kernel, a lane past the end re-reads the last chunk
// and skips its store, and rows of skipped pages read block 0 (it exists
// whenever some page of the group is valid) and store nothing.
template <class SH, class M, int LAYOUT>
__device__ __forceinline__ void move_group(const GatherParams& p, int32_t lane_phys, uint32_t gbeg, uint32_t n,
                                           uint8_t* dst_first, float scale) {
  constexpr int U = unroll_of<SH, M>();
  const uint32_t cpr = static_cast<uint32_t>(p.chunks_per_row);
  const uint32_t bs = static_cast<uint32_t>(p.page_tokens);
  // a flat group's output: n chunks from dst_first (fewer than 2^31 bytes)
  const __amdgpu_buffer_rsrc_t group_out =
      __builtin_amdgcn_make_buffer_rsrc(dst_first, 0, static_cast<int32_t>(n * M::out_bytes), kBufferWord3);
  for (uint32_t c0 = threadIdx.x; c0 - threadIdx.x < n; c0 += SH::threads * U) {
    uint32_t row[U], col[U], k[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t c = min(c0 + u * SH::threads, n - 1);
      row[u] = div_magic(c, cpr, p.chunks_magic);
      col[u] = c - row[u] * cpr;
      k[u] = div_magic(gbeg + row[u], bs, p.page_tokens_magic);
    }
    int32_t phys[U];
#pragma unroll
    for (int u = 0; u < U; ++u) phys[u] = __shfl(lane_phys, static_cast<int>(k[u]), 64);
    typename M::Reg r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t slot = gbeg + row[u] - k[u] * bs;
      const int64_t base = static_cast<int64_t>(phys[u] < 0 ? 0 : phys[u]) * p.src_block_stride;
      const uint8_t* rowp = p.src + base + slot * static_cast<uint32_t>(p.src_token_stride);
      M::load(p, page_src(rowp, static_cast<uint32_t>(p.row_in_bytes)), col[u], r[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t c = c0 + u * SH::threads;
      if (phys[u] < 0 || c >= n) continue;
      if constexpr (LAYOUT == kFlat && M::out_bytes == 16) {
        // device-scope write-through, as the page kernel's flat 16-byte chunks
        store_write_through(group_out, c * M::out_bytes, __builtin_bit_cast(u32x4_plain, M::convert(r[u], scale)));
        continue;
      }
      uint8_t* q;
      if constexpr (LAYOUT == kFlat) {
        q = dst_first + c * M::out_bytes;
      } else {
        q = dst_first + row[u] * p.dst_row_stride + col[u] * M::out_bytes;
      }
      store_stream(q, M::convert(r[u], scale));
    }
  }
}

// The group kernel: the page kernel's task lookup with task_tokens = G *
// block_size, then per-lane page lookups and move_group.  Same leading
// arguments; `mode_and_group` holds the TaskMode (low byte) and group_shift
// (the byte above it).  Loads always use flat (row-relative) chunk addressing:
// each row is addressed on its own.
template <class SH, int CONVERT, int W, int LAYOUT, bool SRC_VEC, int BUILD>
__global__ __launch_bounds__(SH::threads) void gather_groups_kernel(
    const int32_t* cu_seq_lens, const int32_t* block_table, const int32_t* seq_starts,
    int32_t mode_and_group, int32_t num_reqs, int32_t task_tokens, uint32_t task_tokens_magic,
    int32_t block_table_width, int32_t cu_terminal, int32_t num_tokens, int32_t table_ld,
    GatherParams params) {
  using M = Mover<CONVERT, W, kFlat, SRC_VEC>;
  GatherParams p = params;
  p.cu_seq_lens = cu_seq_lens;
  p.block_table = block_table;
  p.seq_starts = seq_starts;
  p.num_reqs = num_reqs;
  p.task_tokens = task_tokens;
  p.task_tokens_magic = task_tokens_magic;
  p.block_table_width = block_table_width;
  p.cu_terminal = cu_terminal;
  p.num_tokens = num_tokens;
  p.split_shift = 0;
  p.group_shift = mode_and_group >> 8;
  extern __shared__ int32_t lds[];
  __shared__ int32_t scan_tmp[SH::waves];

  const int lane = threadIdx.x & 63;
  const int32_t G = 1 << p.group_shift;
  const int32_t R = p.num_reqs;
  const int32_t first_task = static_cast<int32_t>(blockIdx.x);
  TaskSource ts;
  ts.mode = task_mode_of<BUILD>(mode_and_group);
  WaveLoads wave_loads{};
  if constexpr (BUILD == kBuildPrefix) {
    if (ts.mode == kWaveRegs) wave_loads = issue_wave_loads(p);
  }
  int32_t* P = lds;
  int32_t* B = lds + (R + 1);
  int32_t* S = lds + 2 * (R + 1);
  ts.P = P;
  ts.B = B;
  ts.S = S;

  int32_t num_tasks;
  if (ts.mode == kWalk) {
    // this workgroup's first group: columns (blockIdx.x << group_shift) + lane of its request's row
    ts.first_phys_raw = walk_prologue(p, table_ld, (int64_t(blockIdx.x) << p.group_shift) + lane, lane < G, ts);
    num_tasks = static_cast<int32_t>(blockIdx.x) + 1;  // exactly its own group
  } else if (ts.mode == kSingle) {
    // as in the page kernel: this workgroup's first group's table entries
    // (one per lane) are requested together with the request extent
    ts.s = p.seq_starts ? load_i32_vector_path(p.seq_starts) : 0;
    const int64_t lp = (static_cast<int64_t>(page_of(p, ts.s) + first_task) << p.group_shift) + lane;
    const bool in_row = lane < G && lp < p.block_table_width;
    const int32_t* entry_at = in_row ? p.block_table + lp : p.cu_seq_lens;
    const int32_t* end_at = p.cu_seq_lens + p.cu_terminal;
    const int32_t raw = *entry_at;
    const int32_t cb = uniform(p.cu_seq_lens[0]);
    const int32_t ce = uniform(*end_at);
    ts.first_phys_raw = in_row ? raw : -1;
    ts.b = static_cast<int32_t>(clamp_rows(cb, p.num_tokens));
    ts.e = static_cast<int32_t>(clamp_rows(p.cu_terminal ? ce : p.num_tokens, p.num_tokens));
    num_tasks = page_count(p, ts.b, ts.e, ts.s);
  } else if (ts.mode == kWaveRegs) {
    ts.wp = build_prefix_wave(p, wave_loads);
    num_tasks = ts.wp.total;
  } else if (ts.mode == kLdsPrefix) {
    build_prefix_lds_for<SH::threads>(p, P, B, S, scan_tmp);
    num_tasks = P[R];
  } else {
    num_tasks = min(*p.task_count, p.task_capacity);
  }
  num_tasks = uniform(num_tasks);
  float scale = 1.0f;
  if constexpr (CONVERT == kFp8Bf16)
    scale = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(*p.scale)));

  const uint32_t cpr = static_cast<uint32_t>(p.chunks_per_row);
  for (int32_t task = first_task; task < num_tasks; task += gridDim.x) {
    const GroupTask t = resolve_group(p, ts, task);
    const int32_t rows = t.gend - t.gbeg;
    if (rows <= 0) continue;
    int64_t phys = -1;
    if (lane < G) {
      const int64_t lp = (static_cast<int64_t>(t.unit) << p.group_shift) + lane;
      if ((ts.mode == kSingle || ts.mode == kWalk) && task == first_task) {
        phys = ts.first_phys_raw;
      } else if (lp < p.block_table_width) {
        phys = p.block_table[static_cast<int64_t>(t.req) * p.block_table_ld + lp];
      }
      if (phys >= p.num_blocks) phys = -1;
    }
    if (phys < 0) phys = -1;
    if (__ballot(phys >= 0) == 0) continue;  // every page of the group skipped
    move_group<SH, M, LAYOUT>(p, static_cast<int32_t>(phys), static_cast<uint32_t>(t.gbeg),
                              static_cast<uint32_t>(rows) * cpr, p.dst + t.out_begin * p.dst_row_stride, scale);
  }
}

// ---------------------------------------------------------------------------
// standalone builder (large batches, and the gather_page_tasks entry point)
// ---------------------------------------------------------------------------

// One workgroup of kScanThreads: P[0..R] = exclusive prefix of page counts,
// *count = P[R].  A round covers kScanPer * kScanThreads requests.  Their
// extents and starts are loaded in coalesced slices (lane t of slice k on
// request base + k * kScanThreads + t), all requested, at clamped indices,
// before any is used; the page counts go through LDS so that each thread
// takes kScanPer consecutive requests, sums them, and one block scan orders
// the round; the prefixes go back through LDS and out in coalesced slices.
// One memory round trip and one block scan per round, where a round of one
// slice cost both per kScanThreads requests (60,000 requests 56.5 us).
constexpr int kScanPer = 8;

__global__ __launch_bounds__(kScanThreads) void scan_page_counts_kernel(GatherParams p, int32_t* P,
                                                                        int32_t* count) {
  __shared__ int32_t scan_tmp[kScanThreads / 64];
  __shared__ int32_t round_lds[kScanPer * kScanThreads];  // the round's counts, then its prefixes
  const int32_t R = p.num_reqs;
  const int32_t ncu = R + p.cu_terminal;  // cu_seq_lens entries
  const int32_t t = static_cast<int32_t>(threadIdx.x);
  int32_t carry = 0;
  for (int32_t base = 0; base < R; base += kScanThreads * kScanPer) {
    int32_t cb[kScanPer], ce[kScanPer], st[kScanPer];
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
      const int32_t r = base + k * kScanThreads + t;
      cb[k] = p.cu_seq_lens[min(r, ncu - 1)];
      ce[k] = p.cu_seq_lens[min(r + 1, ncu - 1)];
      st[k] = p.seq_starts ? p.seq_starts[min(r, R - 1)] : 0;
    }
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
      const int32_t r = base + k * kScanThreads + t;
      int32_t c = 0;
      if (r < R) {
        // request_end: the next entry, or num_tokens for the last request
        // when cu_seq_lens has no terminal entry
        const int64_t e_raw = (p.cu_terminal || r + 1 < R) ? ce[k] : p.num_tokens;
        c = page_count(p, clamp_rows(cb[k], p.num_tokens), clamp_rows(e_raw, p.num_tokens), st[k]);
      }
      round_lds[k * kScanThreads + t] = c;
    }
    __syncthreads();
    // thread t: requests base + t * kScanPer .. + kScanPer - 1 (0 past R)
    int32_t v[kScanPer];
    int32_t sum = 0;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      v[j] = round_lds[t * kScanPer + j];
      sum += v[j];
    }
    int32_t total;
    int32_t off = carry + block_exclusive_scan<kScanThreads>(sum, scan_tmp, total);  // ends with a barrier
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      round_lds[t * kScanPer + j] = off;
      off += v[j];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
      const int32_t r = base + k * kScanThreads + t;
      if (r < R) P[r] = round_lds[k * kScanThreads + t];
    }
    carry += total;
    __syncthreads();  // the next round rewrites round_lds
  }
  if (threadIdx.x == 0) {
    P[R] = carry;
    *count = carry;
  }
}

// One thread per task (grid-stride): binary search of P in global memory,
// task geometry, block lookup with guards, one 32-byte record.
__global__ __launch_bounds__(256) void expand_tasks_kernel(GatherParams p, const int32_t* __restrict__ P,
                                                           TaskRecord* __restrict__ out, int32_t capacity) {
  const int32_t R = p.num_reqs;
  const int32_t n = min(P[R], capacity);
  for (int32_t task = blockIdx.x * blockDim.x + threadIdx.x; task < n; task += gridDim.x * blockDim.x) {
    const int32_t r = find_request(P, R, task);
    const int64_t b = clamp_rows(p.cu_seq_lens[r], p.num_tokens);
    const int64_t e = clamp_rows(request_end(p, r), p.num_tokens);
    const int64_t s = p.seq_starts ? p.seq_starts[r] : 0;
    const TaskGeom g = task_geometry(p, task - P[r], b, e, s);
    TaskRecord t;
    t.req = r;
    t.logical = g.logical;
    t.page_begin = g.pbeg;
    t.page_end = g.pend;
    t.out_begin = static_cast<int32_t>(g.out_begin);
    // group tasks look their pages up in the gather kernel
    t.phys = p.group_shift > 0 ? -1 : static_cast<int32_t>(lookup_block(p, r, g.logical));
    t.pad0 = 0;
    t.pad1 = 0;
    out[task] = t;
  }
}

}  // namespace pkvg
