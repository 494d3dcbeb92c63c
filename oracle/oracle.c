/*
 * oracle.c -- plain, slow, single-threaded CPU oracle for the paged MLA
 * KV-cache gather.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library and its
 * Python binding) may include, link, load or call this file.  Only the test
 * suite, the smoke check and the CPU-baseline leg of the benchmark use it.
 * It shares no code, header, table or constant with the HIP path.
 *
 * Source of the method: the prhub.com.cn summary of vLLM pull request 51739,
 * "MLA cache gather scheduled by logical page; raw copy up to 331x faster"
 * (page 1 of the reference pages), and for the indexer quant-cache gather at
 * the end of this file the summary of pull request 56153, "indexer kernel
 * takes runtime arguments; no per-shape recompiles" (page 3).  Every function
 * cites the passage it follows.  Where a page is silent the readings taken
 * are stated inline.
 *
 * Every function here is pinned by a CPU test against something other than
 * itself (a hand-worked case, a library cast, a closed form, or an
 * independently formulated gather); no function is "parity unpinned".
 *
 * Build: gcc -O2 -fPIC -shared -std=c11 (no -ffast-math: the fp32 multiply
 * must be one IEEE-754 round-to-nearest-even operation).
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

/* ------------------------------------------------------------------------
 * Element arithmetic
 * ------------------------------------------------------------------------ */

/*
 * OCP 8-bit floating point, E4M3 "fn" variant (bias 7, no infinities, the
 * single NaN pattern S.1111.111, max finite 448, signed zero).  The page only
 * says "FP8"; this is the format that vLLM's fp8 KV cache and torch's
 * float8_e4m3fn use.  Decoding is exact in fp32.
 *
 *   e == 0             : value = m * 2^-9           (subnormal, 2^(1-7) * m/8)
 *   e == 15 && m == 7  : NaN
 *   otherwise          : value = (8 + m) * 2^(e-10) (1.m * 2^(e-7))
 */
float oracle_e4m3fn_to_f32(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7)
        return sign ? -NAN : NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 10);
    return (float)(sign ? -v : v);
}

/*
 * fp32 -> bf16 with IEEE-754 round-to-nearest, ties-to-even: keep the upper
 * 16 bits of the fp32 pattern, rounding on the lower 16.  A NaN stays a NaN
 * (quiet bit forced).  Overflow of the rounding carries into the exponent,
 * which gives +-inf exactly as IEEE rounding of a too-large value does.
 */
uint16_t oracle_f32_to_bf16_rne(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lower = u & 0xFFFFu;
    uint32_t upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u;
    return (uint16_t)upper;
}

/*
 * One dequantised element: decode the fp8 code exactly to fp32, multiply by
 * the per-tensor fp32 scale in fp32 (one rounding), round the product to bf16
 * (second rounding).  The page names the FP8 -> BF16 conversion without
 * its arithmetic; this chain (fp8 -> fp32, times scale, -> bf16 RNE) is the
 * reading taken for both the dequant and the upconvert variants.
 */
uint16_t oracle_dequant_e4m3fn_bf16(uint8_t code, float scale)
{
    /* volatile: the product is stored as an fp32 value (one rounding) even if
     * the host compiler were to keep intermediates in wider registers. */
    volatile float product = oracle_e4m3fn_to_f32(code) * scale;
    return oracle_f32_to_bf16_rne(product);
}

/* ------------------------------------------------------------------------
 * The gather
 * ------------------------------------------------------------------------ */

enum { ORACLE_MODE_COPY = 0, ORACLE_MODE_E4M3FN_TO_BF16 = 1 };

static int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
static int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

/*
 * End of request r's output extent before clamping: cu_seq_lens[r + 1] when
 * the array holds num_reqs + 1 entries (terminal); otherwise the last request
 * ends at num_tokens (the page-task map's has_terminal_start switch, section
 * "key source snippets").
 */
static int64_t request_end(const int32_t *cu_seq_lens, int32_t r, int32_t num_reqs,
                           int64_t num_tokens, int32_t terminal)
{
    if (terminal || r + 1 < num_reqs)
        return cu_seq_lens[r + 1];
    return num_tokens;
}

/*
 * The per-token gather: the definition the page's own tests compare every
 * kernel against (section "key source snippets", the reference built token
 * by token in test_cp_gather_cache_mla_large_uneven_sequences).  For request
 * r the output rows are [b, b+n), with b and the row count n read from
 * consecutive cu_seq_lens entries and both clamped to num_tokens (the clamps
 * of the page-task mapping in the same section).  Output row b+i takes source
 * token t = s + i of that request, where s = seq_starts[r] (0 when
 * seq_starts is NULL), i.e. slot t % block_size of the physical block
 * block_table[r][t / block_size].
 *
 * Guards (readings of the review section's out-of-bounds finding): a token
 * whose logical block is at or beyond block_table_width, or whose physical
 * block id lies outside [0, num_blocks), is skipped and its output row is
 * left untouched.
 *
 * Strides are in elements of their own array; element sizes in bytes.
 * COPY mode copies src_elem_bytes == dst_elem_bytes bytes per element
 * unchanged; E4M3FN_TO_BF16 reads 1-byte codes and writes 2-byte bf16 via
 * oracle_dequant_e4m3fn_bf16.  Returns the number of rows written.
 */
int64_t oracle_gather(int32_t mode,
                      const uint8_t *src, int32_t src_elem_bytes,
                      int64_t num_blocks, int32_t block_size, int32_t entry,
                      int64_t src_block_stride, int64_t src_token_stride,
                      uint8_t *dst, int32_t dst_elem_bytes,
                      int64_t num_tokens, int64_t dst_row_stride,
                      const int32_t *block_table, int32_t block_table_width,
                      int64_t block_table_ld,
                      const int32_t *cu_seq_lens, int32_t terminal, const int32_t *seq_starts,
                      int32_t num_reqs, float scale)
{
    int64_t rows_written = 0;
    for (int32_t r = 0; r < num_reqs; ++r) {
        int64_t b = min64(cu_seq_lens[r], num_tokens);
        int64_t e = min64(request_end(cu_seq_lens, r, num_reqs, num_tokens, terminal), num_tokens);
        int64_t n = max64(e - b, 0);
        int64_t s = seq_starts ? seq_starts[r] : 0;
        for (int64_t i = 0; i < n; ++i) {
            int64_t t = s + i;
            int64_t logical = t / block_size;
            int64_t slot = t % block_size;
            if (logical >= block_table_width)
                continue;
            int64_t phys = block_table[(int64_t)r * block_table_ld + logical];
            if (phys < 0 || phys >= num_blocks)
                continue;
            const uint8_t *src_row =
                src + (phys * src_block_stride + slot * src_token_stride) * src_elem_bytes;
            uint8_t *dst_row = dst + (b + i) * dst_row_stride * dst_elem_bytes;
            for (int32_t c = 0; c < entry; ++c) {
                if (mode == ORACLE_MODE_COPY) {
                    memcpy(dst_row + (int64_t)c * dst_elem_bytes,
                           src_row + (int64_t)c * src_elem_bytes,
                           (size_t)src_elem_bytes);
                } else {
                    uint16_t y = oracle_dequant_e4m3fn_bf16(src_row[c], scale);
                    memcpy(dst_row + (int64_t)c * 2, &y, 2);
                }
            }
            ++rows_written;
        }
    }
    return rows_written;
}

/* ------------------------------------------------------------------------
 * The page-task decomposition
 * ------------------------------------------------------------------------ */

/*
 * The page-task decomposition (section "implementation breakdown", step 1, and
 * the GatherPageTask fields of section "key source snippets"): a task is one
 * logical page of one request together with the run of that request's
 * gathered tokens that lie on it.
 *
 * Defined here straight from the per-token gather above.  The tokens of each
 * request are visited in output order, as oracle_gather visits them: output
 * row b + i takes source token t = s + i, which lies in slot t % block_size of
 * logical page t / block_size.  Consecutive tokens of one request that share
 * a logical page belong to one task; a token whose (request, logical page)
 * pair differs from the previous token's opens the next task.  A task
 * records (req_id, logical_block, page_token_begin, page_token_end,
 * output_token_begin): the slot of its first token, one past the slot of its
 * last token, and the output row of its first token.  Tasks are numbered in
 * the order they open (request by request, page by page).
 *
 * A request that gathers no rows has no tokens and therefore no task.  The
 * page's own count of pages per request gives such a request one task with an
 * empty slot range when its start is not a multiple of block_size; that task
 * copies nothing, so both readings give the same gather.
 *
 * Tasks are written five int32 at a time into out (room for cap tasks); the
 * return value is the total number of tasks, which may exceed cap (then only
 * the first cap are written).
 */
int64_t oracle_page_tasks(const int32_t *cu_seq_lens, int32_t terminal, const int32_t *seq_starts,
                          int32_t num_reqs, int64_t num_tokens, int32_t block_size,
                          int32_t *out, int64_t cap)
{
    int64_t count = 0;
    for (int32_t r = 0; r < num_reqs; ++r) {
        int64_t b = min64(cu_seq_lens[r], num_tokens);
        int64_t e = min64(request_end(cu_seq_lens, r, num_reqs, num_tokens, terminal), num_tokens);
        int64_t n = max64(e - b, 0);
        int64_t s = seq_starts ? seq_starts[r] : 0;
        int64_t open_page = -1; /* logical page of the task the previous token joined */
        for (int64_t i = 0; i < n; ++i) {
            int64_t t = s + i;
            int64_t page = t / block_size;
            int64_t slot = t % block_size;
            if (page != open_page) {
                open_page = page;
                if (count < cap) {
                    int32_t *task = out + 5 * count;
                    task[0] = r;
                    task[1] = (int32_t)page;
                    task[2] = (int32_t)slot;
                    task[3] = (int32_t)(slot + 1);
                    task[4] = (int32_t)(b + i);
                }
                ++count;
            } else if (count <= cap) {
                out[5 * (count - 1) + 3] = (int32_t)(slot + 1);
            }
        }
    }
    return count;
}

/* ------------------------------------------------------------------------
 * The indexer quant-cache gather
 * ------------------------------------------------------------------------ */

/*
 * Source: the prhub.com.cn summary of vLLM pull request 56153, "indexer
 * kernel takes runtime arguments; no per-shape recompiles" (page 3 of the
 * reference pages), section "key source snippets" (the masks and the
 * clamp-then-widen block addressing of _cp_gather_indexer_quant_cache_kernel)
 * and section "implementation breakdown", steps 2-4 (which values are
 * structural constants and which are runtime bounds, used only in the masks).
 *
 * One program per output row tid: the row belongs to batch (sequence)
 * token_to_seq[tid]; the batch's rows are [cu_seqlen[b], cu_seqlen[b + 1]).
 * The snippet shows the masks on tid, on the batch id, on the block-table
 * column and the in-block offset, and on the physical block id, then the
 * block id clamped to 0 when invalid and only then widened to 64 bits.  It
 * elides the index arithmetic in between and the packed cache layout; the
 * readings taken here:
 *
 *  - valid_token: the batch is valid and batch_start <= tid < batch_end; the
 *    row's position in its sequence is pos = tid - batch_start.
 *  - block_table_id = pos / block_size, block_offset = pos % block_size,
 *    block_table_offset = b * block_table_ld + block_table_id.
 *  - Packed block record (block_stride bytes per physical block): the values
 *    of the block's block_size tokens (head_dim fp8 bytes each) first, then
 *    one fp32 scale per token (4 bytes each, token order) at byte
 *    block_size * head_dim.  LAYOUT picks how the value bytes are ordered:
 *      0 (flat):  token o, byte d at o * head_dim + d;
 *      1 (tiled): the value area is cut into tiles of block_tile tokens by
 *                 head_tile bytes, stored tile after tile: tile rows
 *                 (o / block_tile) outermost, then tile columns
 *                 (d / head_tile), and inside a tile token-major, i.e.
 *                 ((o / bt) * (head_dim / ht) + d / ht) * bt * ht
 *                   + (o % bt) * ht + d % ht.
 *  - A row whose mask is false is left untouched (masked stores); a valid
 *    row gets the token's head_dim value bytes in dst_values[tid] and its 4
 *    scale bytes in dst_scales[tid], both copied bit for bit.
 *
 * Strides: block_stride and dst_value_stride in bytes, dst_scale_stride in
 * bytes too (the HIP boundary takes it in fp32 elements).  Returns the number
 * of rows written.
 */
int64_t oracle_indexer_gather(const uint8_t *cache, int64_t num_blocks, int32_t block_size,
                              int64_t block_stride, int32_t layout, int32_t head_dim,
                              int32_t block_tile, int32_t head_tile,
                              uint8_t *dst_values, int64_t dst_value_stride,
                              uint8_t *dst_scales, int64_t dst_scale_stride,
                              int64_t num_tokens, const int32_t *token_to_seq,
                              const int32_t *cu_seqlen, int32_t num_batches,
                              const int32_t *block_table, int32_t block_table_width,
                              int64_t block_table_ld)
{
    int64_t rows_written = 0;
    for (int64_t tid = 0; tid < num_tokens; ++tid) {
        /* the batch of this row, and its rows [batch_start, batch_end) */
        int64_t batch = token_to_seq[tid];
        if (batch < 0 || batch >= num_batches)
            continue;
        int64_t batch_start = cu_seqlen[batch];
        int64_t batch_end = cu_seqlen[batch + 1];
        if (tid < batch_start || tid >= batch_end)
            continue;
        /* position in the sequence -> block-table column and slot */
        int64_t pos = tid - batch_start;
        int64_t block_table_id = pos / block_size;
        int64_t block_offset = pos % block_size;
        if (block_table_id < 0 || block_table_id >= block_table_width ||
            block_offset < 0 || block_offset >= block_size)
            continue;
        int64_t block_id = block_table[batch * block_table_ld + block_table_id];
        if (block_id < 0 || block_id >= num_blocks)
            continue;
        /* the block id is valid here, so clamping is a no-op; widen before the multiply */
        const uint8_t *record = cache + block_id * block_stride;
        uint8_t *out = dst_values + tid * dst_value_stride;
        for (int32_t d = 0; d < head_dim; ++d) {
            int64_t at;
            if (layout == 0) {
                at = block_offset * head_dim + d;
            } else {
                int64_t tile = (block_offset / block_tile) * (head_dim / head_tile) + d / head_tile;
                at = tile * block_tile * head_tile + (block_offset % block_tile) * head_tile +
                     d % head_tile;
            }
            out[d] = record[at];
        }
        const uint8_t *scale = record + (int64_t)block_size * head_dim + block_offset * 4;
        memcpy(dst_scales + tid * dst_scale_stride, scale, 4);
        ++rows_written;
    }
    return rows_written;
}
