/*
 * pkvg.h -- paged MLA KV-cache gather for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpkvg.so.  The gather copies each request's cached context,
 * scattered over physical pages of a paged KV cache and addressed through an
 * int32 block table, into one contiguous destination of num_tokens rows, as
 * chunked prefill needs it.  Method: the prhub.com.cn summary of vLLM pull
 * request 51739, "MLA cache gather scheduled by logical page; raw copy up to
 * 331x faster" -- its sections "implementation breakdown" (step 1: one
 * workgroup per logical page, partial first/last pages, vector and scalar
 * stride paths; step 2: the destination is sliced to exactly num_tokens rows)
 * and "key source snippets" (the page-task fields and the per-token
 * reference the kernels must match).  gather_indexer_quant_cache is the
 * per-row indexer gather of the summary of pull request 56153 and keeps its
 * own argument conventions, given with its declaration; the conventions below
 * are those of the paged gathers.
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 *  - Every array pointer is a DEVICE pointer on the calling thread's current
 *    HIP device.  The caller owns all memory; the library keeps no pointer
 *    after a call returns.
 *  - Strides are in ELEMENTS of their own array (like torch.Tensor.stride());
 *    the innermost stride of the cache and of the destination is 1.
 *  - The cache is [num_blocks, block_size, >= entry] with strides
 *    (src_block_stride, src_token_stride, 1); the first `entry` elements of
 *    each cache row are gathered.
 *  - The destination is [num_tokens, >= entry] with strides
 *    (dst_row_stride, 1); only columns [0, entry) of rows in [0, num_tokens)
 *    may be written.
 *  - block_table is int32 [num_reqs, >= block_table_width] with row pitch
 *    block_table_ld; entry [r][l] is the physical block holding logical page
 *    l of request r.  With block_table_width == 0 it is never read and may be
 *    NULL (every page then fails the width guard).
 *  - cu_seq_lens is int32 [num_reqs + 1] with cu_terminal = 1: request r
 *    writes output rows [min(cu[r], T), min(cu[r+1], T)) with T = num_tokens
 *    (the clamps of the page-task map).  With cu_terminal = 0 it holds only
 *    the num_reqs starts and the last request ends at T (the map's
 *    has_terminal_start switch).  cu_terminal must be 0 or 1 (else
 *    PKVG_E_SHAPE).  seq_starts is int32 [num_reqs] or NULL: request r reads
 *    its context from token seq_starts[r] on (0 when NULL); output row
 *    min(cu[r],T) + i takes token t = seq_starts[r] + i, i.e. slot
 *    t % block_size of physical block block_table[r][t / block_size].
 *  - Guards: a page whose logical block is >= block_table_width, or whose
 *    physical id lies outside [0, num_blocks), is skipped and its output rows
 *    are left untouched (the bound check the page's review section asks for).
 *    Bad device-side data is therefore not an error and is never reported.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL is the null
 *    stream) and is asynchronous: nothing synchronises with the host.  The
 *    caller keeps every buffer alive until the stream has passed the work.
 *  - Calls are thread-safe and re-entrant.  Batches of more than
 *    PKVG_FUSED_MAX_REQS requests allocate a stream-ordered scratch buffer
 *    (hipMallocAsync / hipFreeAsync on `stream`) unless their block table is
 *    dense (then the table is walked directly, see PKVG_TASKS_WALK); other
 *    calls allocate nothing.
 *    A call enqueues kernel launches only (plus that allocation and its free)
 *    and no memset, so it can be captured into a HIP graph; each replay reads
 *    the buffers' contents at replay time.
 *  - Preconditions (not checked, out of contract): cu_seq_lens is
 *    non-decreasing with cu[0] >= 0; seq_starts >= 0; the source and
 *    destination do not overlap.
 *  - Return value: PKVG_OK (0) on success.  Argument errors return a nonzero
 *    PKVG_E_* code BEFORE anything is enqueued.  num_reqs == 0 or
 *    num_tokens == 0 returns PKVG_OK without enqueueing anything.
 */
#ifndef PKVG_H
#define PKVG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define PKVG_OK 0
#define PKVG_E_NULL 1   /* a required pointer is NULL while there is work to do */
#define PKVG_E_SHAPE 2  /* a count or size is out of range (negative, zero where positive is required) */
#define PKVG_E_STRIDE 3 /* a stride is negative, or the destination rows overlap (dst_row_stride < entry),
                           or block_table_ld < block_table_width */
#define PKVG_E_DTYPE 4  /* unsupported element size, kv_cache_dtype or indexer record layout */
#define PKVG_E_LIMIT 5  /* beyond an implementation limit: num_tokens >= 2^31; one page's rows
                           span >= 2^31 bytes (block_size * row bytes, or (block_size - 1) *
                           token stride + row bytes); or num_tokens / block_size + 2 * num_reqs
                           >= 2^31 */
#define PKVG_E_HIP 6    /* a HIP runtime call failed (launch or allocation); see pkvg_last_hip_error */
#define PKVG_E_SCRATCH 7 /* gather_maybe_dequant_noalloc: the batch needs more task-table scratch than
                            its fixed array holds (PKVG_NOALLOC_MAX_* below) */

/* kv_cache_dtype values for gather_maybe_dequant */
#define PKVG_KV_AUTO 0     /* cache holds bf16 entries: bit copy into the bf16 destination */
#define PKVG_KV_FP8_E4M3 1 /* cache holds OCP e4m3fn codes: dequantise into the bf16 destination */

/* requests up to this count build their page tasks inside the gather kernel
 * (no scratch); larger batches use a separate builder and a scratch buffer */
#define PKVG_FUSED_MAX_REQS 1024

/* one page task as written by gather_page_tasks: 8 int32 (32 bytes) */
#define PKVG_TASK_INTS 8

/*
 * gather_cache -- raw copy gather (the page's cp_gather_cache).
 *
 * Copies `entry` elements of `elem_bytes` bytes each (1, 2, 4 or 8) from the
 * cache rows described above into the destination rows, bit for bit.
 *
 *   src_cache         device, [num_blocks, block_size, >=entry] elements of elem_bytes
 *   elem_bytes        1, 2, 4 or 8 (the same for source and destination)
 *   num_blocks        >= 0: physical blocks in the cache (the guard bound)
 *   block_size        > 0: tokens per page
 *   entry             > 0: elements gathered per token
 *   src_block_stride  >= 0, src_token_stride >= 0: cache strides, in elements
 *   dst               device, [num_tokens, >=entry]; dst_row_stride >= entry
 *   num_tokens        >= 0: T, rows of dst
 *   block_table       device int32; block_table_width >= 0; block_table_ld >= width
 *   cu_seq_lens       device int32 [num_reqs + cu_terminal]
 *   cu_terminal       1: cu_seq_lens ends with a terminal entry; 0: the last
 *                     request ends at num_tokens
 *   seq_starts        device int32 [num_reqs] or NULL
 *   num_reqs          >= 0
 *   stream            hipStream_t or NULL
 *
 * Errors: PKVG_E_NULL (src_cache, dst or cu_seq_lens NULL, or block_table
 * NULL with block_table_width > 0, while there is work to do), PKVG_E_SHAPE,
 * PKVG_E_STRIDE, PKVG_E_DTYPE (elem_bytes), PKVG_E_LIMIT, PKVG_E_HIP.
 */
int gather_cache(const void *src_cache, int32_t elem_bytes,
                 int64_t num_blocks, int32_t block_size, int32_t entry,
                 int64_t src_block_stride, int64_t src_token_stride,
                 void *dst, int64_t num_tokens, int64_t dst_row_stride,
                 const int32_t *block_table, int32_t block_table_width,
                 int64_t block_table_ld,
                 const int32_t *cu_seq_lens, int32_t cu_terminal, const int32_t *seq_starts,
                 int32_t num_reqs, void *stream);

/*
 * gather_maybe_dequant -- gather into a bf16 destination, dequantising when
 * the cache is fp8 (the page's gather_and_maybe_dequant_cache).
 *
 *   kv_cache_dtype == PKVG_KV_AUTO: the cache holds bf16 elements (strides in
 *     bf16 elements); each element is copied bit for bit; `scale` is ignored
 *     and may be NULL.
 *   kv_cache_dtype == PKVG_KV_FP8_E4M3: the cache holds one-byte OCP e4m3fn
 *     codes (strides in bytes); each element becomes
 *     bf16_rne(fp32(decode(code)) * scale[0]), one fp32 multiply rounded to
 *     nearest-even, then rounded to bf16 nearest-even.  `scale` is a device
 *     pointer to one fp32 (per-tensor scale), read on the device.
 *
 * dst is bf16 (2-byte elements) with row stride dst_row_stride elements.  The
 * other arguments are as for gather_cache.  Errors: as gather_cache, plus
 * PKVG_E_DTYPE for an unknown kv_cache_dtype and PKVG_E_NULL for a NULL scale
 * with PKVG_KV_FP8_E4M3.
 */
int gather_maybe_dequant(const void *src_cache, int32_t kv_cache_dtype,
                         int64_t num_blocks, int32_t block_size, int32_t entry,
                         int64_t src_block_stride, int64_t src_token_stride,
                         void *dst, int64_t num_tokens, int64_t dst_row_stride,
                         const int32_t *block_table, int32_t block_table_width,
                         int64_t block_table_ld,
                         const int32_t *cu_seq_lens, int32_t cu_terminal,
                         const int32_t *seq_starts,
                         int32_t num_reqs, const float *scale, void *stream);

/*
 * gather_maybe_dequant_noalloc -- gather_maybe_dequant for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, results and errors
 * as gather_maybe_dequant, and it calls no hipMalloc, hipFree, stream-ordered
 * allocator or other allocating routine.
 *
 * Batches of at most PKVG_FUSED_MAX_REQS requests use no scratch (as in
 * gather_maybe_dequant).  Larger batches keep their page-task table (the
 * exclusive page-count prefix, a task count and one 32-byte record per task
 * unit) in a fixed array inside the library's device code instead of a
 * stream-ordered allocation: room for at most PKVG_NOALLOC_MAX_REQS requests
 * and PKVG_NOALLOC_MAX_TASKS task units (8.25 MiB in all; a task unit holds up to 16
 * tokens of 1152-byte bf16 rows in such batches, so about four million such
 * tokens).  A batch beyond that returns PKVG_E_SCRATCH before anything is
 * enqueued.  Each device the library runs on holds its own copy of the array
 * until the process ends; its address is looked up on the first call on that
 * device (hipGetSymbolAddress, not an allocation).
 *
 * All calls on one device share that array, which keeps the last call's
 * contents (every entry a call reads, it has written first).  Calls that can
 * overlap on one device -- on different streams, or from different threads
 * without ordering -- race on it and must not be issued; calls ordered on one
 * stream are safe.
 */
#define PKVG_NOALLOC_MAX_REQS 65535
#define PKVG_NOALLOC_MAX_TASKS 262144

int gather_maybe_dequant_noalloc(const void *src_cache, int32_t kv_cache_dtype,
                                 int64_t num_blocks, int32_t block_size, int32_t entry,
                                 int64_t src_block_stride, int64_t src_token_stride,
                                 void *dst, int64_t num_tokens, int64_t dst_row_stride,
                                 const int32_t *block_table, int32_t block_table_width,
                                 int64_t block_table_ld,
                                 const int32_t *cu_seq_lens, int32_t cu_terminal,
                                 const int32_t *seq_starts,
                                 int32_t num_reqs, const float *scale, void *stream);

/*
 * gather_upconvert_fp8 -- fp8 (OCP e4m3fn) cache to bf16 destination (the
 * page's cp_gather_and_upconvert_fp8_kv_cache, with coalesced bf16 writes).
 * Same arithmetic as gather_maybe_dequant with PKVG_KV_FP8_E4M3; `scale`
 * (device, one fp32) is required.  Cache strides are in bytes, destination
 * strides in bf16 elements.
 */
int gather_upconvert_fp8(const void *src_cache,
                         int64_t num_blocks, int32_t block_size, int32_t entry,
                         int64_t src_block_stride, int64_t src_token_stride,
                         void *dst, int64_t num_tokens, int64_t dst_row_stride,
                         const int32_t *block_table, int32_t block_table_width,
                         int64_t block_table_ld,
                         const int32_t *cu_seq_lens, int32_t cu_terminal,
                         const int32_t *seq_starts,
                         int32_t num_reqs, const float *scale, void *stream);

/*
 * gather_page_tasks -- the page-task builder on its own (the page's
 * GatherPageTask / map_gather_page_task, built as an exclusive scan of
 * per-request page counts plus a binary search instead of a linear scan).
 *
 * Writes, for task k < min(count, capacity), PKVG_TASK_INTS int32 at
 * tasks[k * PKVG_TASK_INTS]: req_id, logical_block, page_token_begin,
 * page_token_end (exclusive), output_token_begin, physical_block (-1 when the
 * guards skip the page), 0, 0; and writes count to num_tasks[0] (device).
 * Tasks are ordered by request, then logical page.  A request that gathers no
 * rows contributes no task.
 *
 *   cu_seq_lens, cu_terminal, seq_starts, num_reqs, num_tokens, block_size: as above
 *   block_table, block_table_width, block_table_ld, num_blocks: as above
 *   tasks      device int32 [capacity * PKVG_TASK_INTS]
 *   capacity   >= 0 task records available
 *   num_tasks  device int32 [1]
 *
 * Errors: PKVG_E_NULL, PKVG_E_SHAPE, PKVG_E_STRIDE, PKVG_E_LIMIT, PKVG_E_HIP.
 * num_reqs == 0 still writes num_tasks[0] = 0.
 */
int gather_page_tasks(const int32_t *cu_seq_lens, int32_t cu_terminal, const int32_t *seq_starts,
                      int32_t num_reqs, int64_t num_tokens, int32_t block_size,
                      const int32_t *block_table, int32_t block_table_width,
                      int64_t block_table_ld, int64_t num_blocks,
                      int32_t *tasks, int64_t capacity, int32_t *num_tasks,
                      void *stream);

/*
 * gather_indexer_quant_cache -- the indexer quant-cache gather: the per-row
 * kernel of the prhub.com.cn summary of vLLM pull request 56153, "indexer
 * kernel takes runtime arguments; no per-shape recompiles" (section "key
 * source snippets": the masks and the clamp-then-widen block addressing;
 * section "implementation breakdown", steps 2-4: layout, head dimension and
 * tile sizes are structural, every shape-derived value is a runtime argument).
 *
 * Output row tid (0 <= tid < num_tokens) belongs to batch
 * b = token_to_seq[tid]; it is written only if 0 <= b < num_batches,
 * cu_seqlen[b] <= tid < cu_seqlen[b + 1], the block-table column
 * pos / block_size (pos = tid - cu_seqlen[b]) is below block_table_width, and
 * the physical block block_table[b * block_table_ld + column] lies in
 * [0, num_blocks).  Any other row is left untouched (padding rows carry -1).
 * A written row receives slot pos % block_size of that block: its head_dim
 * value bytes into dst_values[tid][0 .. head_dim) and its 4-byte fp32 scale
 * into dst_scales[tid * dst_scale_stride], both copied bit for bit.
 *
 * The cache is [num_blocks] packed block records of block_stride bytes (the
 * page elides the record; the reading taken): the values of the block's
 * block_size tokens first, head_dim bytes per token, then one fp32 scale per
 * token in token order at byte block_size * head_dim.  The value bytes are
 *   PKVG_INDEXER_FLAT:  token o, byte d at o * head_dim + d;
 *   PKVG_INDEXER_TILED: in block_tile x head_tile tiles stored tile after
 *     tile, tile rows outermost: at ((o / bt) * (head_dim / ht) + d / ht) *
 *     bt * ht + (o % bt) * ht + d % ht.
 *
 *   cache             device, dword-aligned; block_stride bytes per record,
 *                     a multiple of 4, >= block_size * (head_dim + 4), < 2^31
 *   num_blocks        >= 0 (the block-id bound); block_size > 0
 *   layout, head_dim, block_tile, head_tile
 *                     structural: FLAT with head_dim 64, 128 or 256 (tiles
 *                     ignored), or TILED with head_dim 64, 128 or 256 and
 *                     16 x 16 tiles (block_size a multiple of 16); else
 *                     PKVG_E_DTYPE
 *   dst_values        device bytes [num_tokens, >= head_dim], row stride
 *                     dst_value_stride bytes (>= head_dim)
 *   dst_scales        device fp32 [num_tokens], stride dst_scale_stride
 *                     elements (>= 1), dword-aligned
 *   num_tokens        >= 0, <= 2^31 - 65
 *   token_to_seq      device int32 [num_tokens]
 *   cu_seqlen         device int32 [num_batches + 1] (entries past it are never read)
 *   block_table       device int32 rows of pitch block_table_ld >= block_table_width;
 *                     may be NULL when block_table_width == 0
 *   stream            hipStream_t or NULL
 *
 * Nothing is allocated; one kernel is enqueued.  num_tokens == 0,
 * num_batches == 0, num_blocks == 0 or block_table_width == 0 (no row can
 * pass the masks) returns PKVG_OK without enqueueing anything.  Errors
 * (before anything is enqueued): PKVG_E_NULL, PKVG_E_SHAPE, PKVG_E_STRIDE
 * (also a misaligned cache, record stride or dst_scales), PKVG_E_DTYPE,
 * PKVG_E_LIMIT, PKVG_E_HIP.
 */
#define PKVG_INDEXER_FLAT 0
#define PKVG_INDEXER_TILED 1

int gather_indexer_quant_cache(const void *cache, int64_t num_blocks, int32_t block_size,
                               int64_t block_stride, int32_t layout, int32_t head_dim,
                               int32_t block_tile, int32_t head_tile,
                               void *dst_values, int64_t dst_value_stride,
                               float *dst_scales, int64_t dst_scale_stride,
                               int64_t num_tokens, const int32_t *token_to_seq,
                               const int32_t *cu_seqlen, int32_t num_batches,
                               const int32_t *block_table, int32_t block_table_width,
                               int64_t block_table_ld, void *stream);

/*
 * pkvg_plan -- how a gather call with these arguments would run, worked out
 * by the same host code as the call itself, without enqueueing anything or
 * touching a device: pointers are checked for NULL and alignment only and are
 * never read.  For tests of the host's choices, and for tuning.
 *
 *   op     PKVG_OP_GATHER_CACHE, PKVG_OP_GATHER_MAYBE_DEQUANT or
 *          PKVG_OP_GATHER_UPCONVERT_FP8
 *   kind   the call's elem_bytes (gather_cache) or kv_cache_dtype
 *          (gather_maybe_dequant); ignored for the upconvert
 *   scale  as for the fp8 calls (checked for NULL only)
 *   the other arguments as for the call (no stream)
 *   info   host pointer, filled on PKVG_OK (all zero when the call has no work)
 *
 * Returns what the call would return from its argument checks (never
 * PKVG_E_HIP), PKVG_E_SHAPE for an unknown op, PKVG_E_NULL for a NULL info.
 */
#define PKVG_OP_GATHER_CACHE 0
#define PKVG_OP_GATHER_MAYBE_DEQUANT 1
#define PKVG_OP_GATHER_UPCONVERT_FP8 2

#define PKVG_KERNEL_PAGES 0   /* one task = one logical page, or one of 2^split_shift equal parts of it */
#define PKVG_KERNEL_GROUPS 1  /* one task = 2^group_shift consecutive logical pages of one request */

#define PKVG_TASKS_WAVE 0     /* task prefix built in wave registers (2..64 requests) */
#define PKVG_TASKS_LDS 1      /* task prefix built in LDS (65..PKVG_FUSED_MAX_REQS requests) */
#define PKVG_TASKS_TABLE 2    /* task table built by two kernels first (more requests) */
#define PKVG_TASKS_SINGLE 3   /* one request: no prefix */
#define PKVG_TASKS_WALK 4     /* the block table walked directly: one workgroup per task unit of each
                                 table row (batches whose table is about as wide as their pages) */

typedef struct pkvg_plan_info {
  int32_t kernel;        /* PKVG_KERNEL_* */
  int32_t threads;       /* workgroup size */
  int32_t batch_bytes;   /* output bytes one workgroup moves per batch of loads */
  int32_t task_mode;     /* PKVG_TASKS_* */
  int32_t convert;       /* 0: bit copy; 1: fp8 e4m3fn -> bf16 */
  int32_t access_width;  /* bytes (copy) or codes (fp8) per lane access */
  int32_t flat;          /* 1: source token stride and destination row stride equal the row bytes */
  int32_t src_vector;    /* fp8: 1 when code rows are read as aligned words */
  int32_t task_tokens;   /* tokens per task unit */
  int32_t split_shift;   /* a page is 2^split_shift task units */
  int32_t group_shift;   /* a task unit is 2^group_shift pages */
  int32_t grid_rows;     /* workgroups along y: the requests for PKVG_TASKS_WALK, else 1 */
  int64_t grid;          /* workgroups launched along x */
  int64_t task_capacity; /* upper bound on the number of task units */
} pkvg_plan_info;

int pkvg_plan(int32_t op, int32_t kind, const void *src_cache,
              int64_t num_blocks, int32_t block_size, int32_t entry,
              int64_t src_block_stride, int64_t src_token_stride,
              void *dst, int64_t num_tokens, int64_t dst_row_stride,
              const int32_t *block_table, int32_t block_table_width,
              int64_t block_table_ld,
              const int32_t *cu_seq_lens, int32_t cu_terminal,
              const int32_t *seq_starts,
              int32_t num_reqs, const float *scale, pkvg_plan_info *info);

/* Human-readable name of a status code (static storage; never NULL). */
const char *pkvg_status_string(int status);

/* The hipError_t of the calling thread's last PKVG_E_HIP, or 0. */
int pkvg_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PKVG_H */
