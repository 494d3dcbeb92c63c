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
// inside the page, first output row) are produced here by an exclusive scan
// of per-request page counts and a binary search, instead of the page's
// linear scan over requests.
//
// Design for gfx950:
//  * the scan lives in LDS once per workgroup; each wave then resolves its
//    page itself (binary search over LDS) and holds the task and physical
//    block in SGPRs (readfirstlane), so no second barrier is needed;
//  * the hot loop moves 16-byte (dwordx4) chunks, consecutive lanes on
//    consecutive chunks, so one wave instruction covers 1 KiB of a row span;
//    kUnroll loads are in flight per lane before the matching stores;
//  * all addressing that can exceed 2^31 bytes (page bases, output row bases)
//    is int64; in-page offsets are 32-bit (the host guarantees that a page's
//    rows span < 2^31 bytes);
//  * fp8 pages: each lane reads 8 codes (8 bytes) and writes 8 bf16 (16
//    bytes): v_cvt_pk_f32_fp8 (OCP e4m3fn on gfx950), one v_mul_f32 by the
//    scale, v_cvt_pk_bf16_f32 (round to nearest even);
//  * every shape is a runtime argument; templates cover only the access
//    width and whether a page's rows are one contiguous span.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkvg {

#ifndef PKVG_THREADS
#define PKVG_THREADS 256
#endif
#ifndef PKVG_UNROLL
#define PKVG_UNROLL 8
#endif

constexpr int kThreads = PKVG_THREADS;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = PKVG_UNROLL;
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
  const TaskRecord* tasks;       // nullptr: tasks are built in the kernel (LDS scan)
  const int32_t* task_count;     // with tasks: device count of valid records
  int64_t src_block_stride;      // bytes
  int64_t src_token_stride;      // bytes
  int64_t dst_row_stride;        // bytes
  int64_t block_table_ld;        // int32 elements
  int64_t num_blocks;
  int64_t num_tokens;
  int32_t num_reqs;
  int32_t block_size;
  int32_t block_table_width;
  int32_t chunks_per_row;        // row chunks (kRows), or chunks per row of the flat span (kFlat)
  uint32_t chunks_magic;         // ceil(2^32 / chunks_per_row), or 0xFFFFFFFF for 1
  int32_t task_capacity;         // with tasks: records available
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

// n / d for n, d < 2^31 with a precomputed magic = ceil(2^32 / d) (d >= 2) or
// 0xFFFFFFFF (d == 1): the multiply-high is off by at most one either way.
__device__ __forceinline__ uint32_t div_magic(uint32_t n, uint32_t d, uint32_t magic) {
  uint32_t q = __umulhi(n, magic);
  const int32_t r = static_cast<int32_t>(n - q * d);
  if (r < 0) --q;
  else if (static_cast<uint32_t>(r) >= d) ++q;
  return q;
}

// Keeps the compiler from sinking a batch of loads down to their stores (it
// otherwise interleaves load, wait, store and leaves one load in flight).  The
// page pointers are deliberately not __restrict__: with them the compiler may
// move the loads across this fence.
__device__ __forceinline__ void loads_before_stores() { asm volatile("" ::: "memory"); }

template <int BYTES> struct VecOf;
template <> struct VecOf<16> { using T = uint4; };
template <> struct VecOf<8> { using T = uint2; };
template <> struct VecOf<4> { using T = uint32_t; };
template <> struct VecOf<2> { using T = uint16_t; };
template <> struct VecOf<1> { using T = uint8_t; };

// Page counts of one request: rows [b, e) of the output, source tokens from s.
// A request with no rows has no pages.
__device__ __forceinline__ int32_t page_count(int64_t b, int64_t e, int64_t s, int32_t bs) {
  const int64_t n = e - b;
  if (n <= 0) return 0;
  return static_cast<int32_t>((s + n + bs - 1) / bs - s / bs);
}

__device__ __forceinline__ int64_t clamp_rows(int32_t cu, int64_t T) {
  return cu < T ? static_cast<int64_t>(cu) : T;
}

// Exclusive scan over the workgroup; `tmp` holds NWAVES ints of LDS.
template <int NTHREADS>
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t x, int32_t* tmp, int32_t& total) {
  constexpr int NW = NTHREADS / 64;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  int32_t incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
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

// Fill the LDS task prefix for the fused path: P[0..R] exclusive prefix of page
// counts, B[0..R] clamped output begins (B[R] = clamped end of the last
// request), S[0..R) source starts.  Every thread of the workgroup takes part.
__device__ __forceinline__ void build_prefix_lds(const GatherParams& p, int32_t* P, int32_t* B,
                                                 int32_t* S, int32_t* scan_tmp) {
  const int32_t R = p.num_reqs;
  const int32_t per = (R + kThreads - 1) / kThreads;
  const int32_t lo = min(static_cast<int32_t>(threadIdx.x) * per, R);
  const int32_t hi = min(lo + per, R);
  int32_t sum = 0;
  for (int32_t r = lo; r < hi; ++r) {
    const int64_t b = clamp_rows(p.cu_seq_lens[r], p.num_tokens);
    const int64_t e = clamp_rows(p.cu_seq_lens[r + 1], p.num_tokens);
    const int32_t s = p.seq_starts ? p.seq_starts[r] : 0;
    const int32_t c = page_count(b, e, s, p.block_size);
    B[r] = static_cast<int32_t>(b);
    S[r] = s;
    P[r] = c;
    sum += c;
  }
  int32_t total;
  int32_t off = block_exclusive_scan<kThreads>(sum, scan_tmp, total);
  for (int32_t r = lo; r < hi; ++r) {
    const int32_t c = P[r];
    P[r] = off;
    off += c;
  }
  if (threadIdx.x == 0) {
    P[R] = total;
    B[R] = static_cast<int32_t>(clamp_rows(p.cu_seq_lens[R], p.num_tokens));
  }
  __syncthreads();
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

__device__ __forceinline__ TaskGeom task_geometry(int32_t j, int64_t b, int64_t e, int64_t s, int32_t bs) {
  const int64_t n = e - b > 0 ? e - b : 0;
  const int64_t logical = s / bs + j;
  const int64_t page0 = logical * bs;
  const int64_t cb = s > page0 ? s : page0;
  const int64_t ce = (s + n) < (page0 + bs) ? (s + n) : (page0 + bs);
  TaskGeom g;
  g.logical = static_cast<int32_t>(logical);
  g.pbeg = static_cast<int32_t>(cb - page0);
  g.pend = static_cast<int32_t>(ce - page0);
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

// Raw copy of `rows` rows.  VW: bytes per lane access.  Every lane issues its
// kUnroll loads back to back before the first store.  A lane whose chunk index
// runs past the end works on the last chunk instead: it loads it and stores
// the same bytes to the same place as that chunk's own lane, so no access
// needs a branch and all loads stay in flight together.
template <int VW, int LAYOUT>
__device__ __forceinline__ void copy_rows_raw(const GatherParams& p, const uint8_t* s, uint8_t* d,
                                              int32_t rows) {
  using V = typename VecOf<VW>::T;
  const uint32_t cpr = static_cast<uint32_t>(p.chunks_per_row);
  const uint32_t n = static_cast<uint32_t>(rows) * cpr;
  const uint32_t last = n - 1;
  for (uint32_t c0 = threadIdx.x; c0 - threadIdx.x < n; c0 += kThreads * kUnroll) {
    V v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t c = min(c0 + u * kThreads, last);
      if constexpr (LAYOUT == kFlat) {
        v[u] = *reinterpret_cast<const V*>(s + c * VW);
      } else {
        const uint32_t row = div_magic(c, cpr, p.chunks_magic);
        const uint32_t col = c - row * cpr;
        v[u] = *reinterpret_cast<const V*>(s + row * p.src_token_stride + col * VW);
      }
    }
    loads_before_stores();
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t c = min(c0 + u * kThreads, last);
      if constexpr (LAYOUT == kFlat) {
        *reinterpret_cast<V*>(d + c * VW) = v[u];
      } else {
        const uint32_t row = div_magic(c, cpr, p.chunks_magic);
        const uint32_t col = c - row * cpr;
        *reinterpret_cast<V*>(d + row * p.dst_row_stride + col * VW) = v[u];
      }
    }
  }
}

// K fp8 codes, read as one K-byte word when SRC_VEC (aligned) else byte by byte.
template <int K, bool SRC_VEC>
__device__ __forceinline__ void load_codes(const uint8_t* q, uint32_t (&w)[(K + 3) / 4]) {
  if constexpr (SRC_VEC && K == 8) {
    const uint2 x = *reinterpret_cast<const uint2*>(q);
    w[0] = x.x;
    w[1] = x.y;
  } else if constexpr (SRC_VEC && K == 4) {
    w[0] = *reinterpret_cast<const uint32_t*>(q);
  } else if constexpr (SRC_VEC && K == 2) {
    w[0] = *reinterpret_cast<const uint16_t*>(q);
  } else {
#pragma unroll
    for (int i = 0; i < (K + 3) / 4; ++i) w[i] = 0;
#pragma unroll
    for (int i = 0; i < K; ++i) w[i / 4] |= static_cast<uint32_t>(q[i]) << (8 * (i % 4));
  }
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two codes (bytes 0-1 or 2-3 of w) -> two bf16 packed in one dword.
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
__device__ __forceinline__ typename OutOf<K>::T dequant_codes(const uint32_t (&w)[(K + 3) / 4], float scale) {
  if constexpr (K == 8) {
    uint4 o;
    o.x = dequant_pair(w[0], false, scale);
    o.y = dequant_pair(w[0], true, scale);
    o.z = dequant_pair(w[1], false, scale);
    o.w = dequant_pair(w[1], true, scale);
    return o;
  } else if constexpr (K == 4) {
    uint2 o;
    o.x = dequant_pair(w[0], false, scale);
    o.y = dequant_pair(w[0], true, scale);
    return o;
  } else if constexpr (K == 2) {
    return dequant_pair(w[0], false, scale);
  } else {
    return static_cast<uint16_t>(dequant_pair(w[0], false, scale) & 0xFFFFu);
  }
}

// fp8 -> bf16 of `rows` rows; K codes per lane access.  Chunk indices are
// clamped to the last chunk as in copy_rows_raw (a clamped lane writes the
// same bf16 values as the chunk's own lane), so all loads are in flight
// together.
template <int K, int LAYOUT, bool SRC_VEC>
__device__ __forceinline__ void copy_rows_fp8(const GatherParams& p, const uint8_t* s, uint8_t* d,
                                              int32_t rows, float scale) {
  using O = typename OutOf<K>::T;
  constexpr int NW = (K + 3) / 4;
  const uint32_t cpr = static_cast<uint32_t>(p.chunks_per_row);
  const uint32_t n = static_cast<uint32_t>(rows) * cpr;
  const uint32_t last = n - 1;
  for (uint32_t c0 = threadIdx.x; c0 - threadIdx.x < n; c0 += kThreads * kUnroll) {
    uint32_t w[kUnroll][NW];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t c = min(c0 + u * kThreads, last);
      if constexpr (LAYOUT == kFlat) {
        load_codes<K, SRC_VEC>(s + c * K, w[u]);
      } else {
        const uint32_t row = div_magic(c, cpr, p.chunks_magic);
        const uint32_t col = c - row * cpr;
        load_codes<K, SRC_VEC>(s + row * p.src_token_stride + col * K, w[u]);
      }
    }
    loads_before_stores();
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t c = min(c0 + u * kThreads, last);
      const O o = dequant_codes<K>(w[u], scale);
      if constexpr (LAYOUT == kFlat) {
        *reinterpret_cast<O*>(d + c * (2 * K)) = o;
      } else {
        const uint32_t row = div_magic(c, cpr, p.chunks_magic);
        const uint32_t col = c - row * cpr;
        *reinterpret_cast<O*>(d + row * p.dst_row_stride + col * (2 * K)) = o;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// the gather kernel
// ---------------------------------------------------------------------------

// CONVERT == kCopy: W = bytes per lane access.  CONVERT == kFp8Bf16: W = codes
// per lane access.  Grid: any size; workgroup w takes tasks w, w + gridDim.x, ...
// Dynamic LDS (fused path): (3 * num_reqs + 2) int32.
template <int CONVERT, int W, int LAYOUT, bool SRC_VEC>
__global__ __launch_bounds__(kThreads) void gather_pages_kernel(GatherParams p) {
  extern __shared__ int32_t lds[];
  __shared__ int32_t scan_tmp[kWaves];

  const bool fused = p.tasks == nullptr;
  const int32_t R = p.num_reqs;
  int32_t* P = lds;
  int32_t* B = lds + (R + 1);
  int32_t* S = lds + 2 * (R + 1);
  float scale = 1.0f;
  if constexpr (CONVERT == kFp8Bf16)
    scale = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(*p.scale)));

  int32_t num_tasks;
  if (fused) {
    build_prefix_lds(p, P, B, S, scan_tmp);
    num_tasks = P[R];
  } else {
    num_tasks = min(*p.task_count, p.task_capacity);
  }
  num_tasks = uniform(num_tasks);

  for (int32_t task = blockIdx.x; task < num_tasks; task += gridDim.x) {
    Page pg;
    if (fused) {
      const int32_t r = uniform(find_request(P, R, task));
      const int64_t b = uniform(B[r]);
      const int64_t e = uniform(B[r + 1]);
      const int64_t s = uniform(S[r]);
      const TaskGeom g = task_geometry(task - uniform(P[r]), b, e, s, p.block_size);
      const int64_t phys = uniform64(lookup_block(p, r, g.logical));
      pg = page_from(p, phys, g.pbeg, g.pend, g.out_begin);
    } else {
      const TaskRecord t = p.tasks[task];
      pg = page_from(p, uniform(t.phys), uniform(t.page_begin), uniform(t.page_end),
                     static_cast<int64_t>(uniform(t.out_begin)));
    }
    if (pg.rows <= 0) continue;
    const uint8_t* s = p.src + uniform64(pg.src_off);
    uint8_t* d = p.dst + uniform64(pg.dst_off);
    if constexpr (CONVERT == kCopy) {
      copy_rows_raw<W, LAYOUT>(p, s, d, pg.rows);
    } else {
      copy_rows_fp8<W, LAYOUT, SRC_VEC>(p, s, d, pg.rows, scale);
    }
  }
}

// ---------------------------------------------------------------------------
// standalone builder (large batches, and the gather_page_tasks entry point)
// ---------------------------------------------------------------------------

// One workgroup of kScanThreads: P[0..R] = exclusive prefix of page counts,
// *count = P[R].
__global__ __launch_bounds__(kScanThreads) void scan_page_counts_kernel(GatherParams p, int32_t* P,
                                                                        int32_t* count) {
  __shared__ int32_t scan_tmp[kScanThreads / 64];
  const int32_t R = p.num_reqs;
  int32_t carry = 0;
  for (int32_t base = 0; base < R; base += kScanThreads) {
    const int32_t r = base + static_cast<int32_t>(threadIdx.x);
    int32_t c = 0;
    if (r < R) {
      const int64_t b = clamp_rows(p.cu_seq_lens[r], p.num_tokens);
      const int64_t e = clamp_rows(p.cu_seq_lens[r + 1], p.num_tokens);
      const int32_t s = p.seq_starts ? p.seq_starts[r] : 0;
      c = page_count(b, e, s, p.block_size);
    }
    int32_t total;
    const int32_t off = block_exclusive_scan<kScanThreads>(c, scan_tmp, total);
    if (r < R) P[r] = carry + off;
    carry += total;
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
    const int64_t e = clamp_rows(p.cu_seq_lens[r + 1], p.num_tokens);
    const int64_t s = p.seq_starts ? p.seq_starts[r] : 0;
    const TaskGeom g = task_geometry(task - P[r], b, e, s, p.block_size);
    TaskRecord t;
    t.req = r;
    t.logical = g.logical;
    t.page_begin = g.pbeg;
    t.page_end = g.pend;
    t.out_begin = static_cast<int32_t>(g.out_begin);
    t.phys = static_cast<int32_t>(lookup_block(p, r, g.logical));
    t.pad0 = 0;
    t.pad1 = 0;
    out[task] = t;
  }
}

}  // namespace pkvg
