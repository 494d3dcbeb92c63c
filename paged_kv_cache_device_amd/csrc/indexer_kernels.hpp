// indexer_kernels.hpp -- HIP device code of the indexer quant-cache gather for
// gfx950 (CDNA4, wave64).
//
// Method: the prhub.com.cn summary of vLLM pull request 56153, "indexer kernel
// takes runtime arguments; no per-shape recompiles", section "key source
// snippets": each output row tid belongs to the batch token_to_seq[tid], whose
// rows are [cu_seqlen[b], cu_seqlen[b + 1]); the row's position in its
// sequence picks a block-table column and an in-block slot; masks on the batch
// id, the row range, the column, the slot and the physical block id leave a
// row untouched when any fails; the block id is clamped before it is widened
// to 64 bits for the packed record's large stride.  Section "implementation
// breakdown", steps 2-4: the record layout, the head dimension and the tile
// sizes are structural (template parameters here); the token count, batch
// count, table width and block count are runtime values used only in the
// masks.
//
// The packed block record (the page elides it; the reading taken): the
// block's block_size tokens' value bytes (HEAD_DIM each) first, token-major
// (flat) or in BT x HT tiles stored tile after tile, tile rows outermost; then
// one 4-byte fp32 scale per token, in token order, at byte block_size *
// HEAD_DIM of the record.
//
// Design for gfx950: the work unit is the output row (token_to_seq may send
// any row to any batch, and padding rows carry -1), so a wave owns 64
// consecutive rows, and is a workgroup of its own.  Lane r resolves row r (token_to_seq, the batch's extent,
// the block-table entry: dependent loads, the entry of a row of the first
// batch requested ahead, speculatively) to a source address; then
// the wave moves the 64 rows' value bytes in W-byte chunks, consecutive lanes
// on consecutive chunks of consecutive rows (a 16-byte chunk per lane puts
// 1 KiB of contiguous rows under one wave instruction), taking each row's
// address from its owner lane with a cross-lane read; each lane also moves its
// own row's 4-byte scale.  A lane's scale and chunk loads all go out before
// its stores, with the nontemporal policy (each byte is touched once).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkvg {

enum IndexerLayout : int {
  kIndexerFlat = 0,   // token o, byte d of the value area at o * HEAD_DIM + d
  kIndexerTiled = 1,  // BT x HT tiles, tile rows outermost, token-major inside a tile
};

struct IndexerParams {
  const uint8_t* cache;           // record 0, byte 0
  uint8_t* dst_values;            // row 0, byte 0
  uint8_t* dst_scales;            // row 0's fp32 scale
  const int32_t* token_to_seq;    // [num_tokens]
  const int32_t* cu_seqlen;       // [num_batches + 1]
  const int32_t* block_table;     // [num_batches, ld]; NULL when block_table_width == 0
  int64_t block_stride;           // bytes per record
  int64_t dst_value_stride;       // bytes
  int64_t dst_scale_stride;       // bytes
  int64_t block_table_ld;         // int32 elements
  int64_t num_blocks;
  int32_t num_tokens;
  int32_t num_batches;
  int32_t block_table_width;
  int32_t block_size;
  uint32_t block_size_magic;      // ceil(2^32 / block_size), or 0xFFFFFFFF for 1
  uint32_t scale_area;            // block_size * HEAD_DIM: byte of the first scale in a record
};

// One wave per workgroup: the dispatcher then spreads the waves evenly over
// the CUs, where workgroups of four waves left some CUs a third more rows than
// others (single sequences of 76,800 rows 6.5 -> 5.8 us, skew-8 10.3 -> 9.5
// us, 300K rows 16.1 -> 16.0 us; 128-thread workgroups in between, 512 and
// 1024 slower still).
constexpr int kIndexerThreads = 64;
constexpr int kIndexerRowsPerWave = 64;

// Where a row's batch extent cu_seqlen[b], cu_seqlen[b + 1] comes from.  When
// the array fits in a wave's lanes it is loaded together with token_to_seq
// (one round trip); larger ones are read per row after its batch id (a second
// round trip, but measured faster than copying the array into LDS first:
// 64 to 4,095 batches over 300,000 rows 16.6-17.1 -> 15.8-16.2 us).
enum IndexerCuSource : int {
  kCuWave = 0,    // num_batches + 1 <= 64: lane i of every wave holds cu_seqlen[i]
  kCuGlobal = 1,  // larger: each row loads its two entries after its batch id
};

// Byte offset of chunk j (bytes j*W .. j*W+W-1 of a token) from the token's
// first value byte (indexer_row_base): consecutive in the flat layout; in the
// tiled one, HT bytes per tile and BT * HT bytes between a row's tiles.  A
// chunk never crosses a tile (W divides HT).
template <int LAYOUT, int HEAD_DIM, int BT, int HT, int W>
__device__ __forceinline__ uint32_t indexer_chunk_offset(uint32_t j) {
  const uint32_t d = j * W;
  if constexpr (LAYOUT == kIndexerFlat) {
    return d;
  } else {
    static_assert(HT % W == 0, "a chunk stays inside one tile");
    return (d / HT) * (BT * HT) + d % HT;
  }
}

// Byte offset of a token's first value byte inside its record: slot * HEAD_DIM
// (flat), or the start of its tile row plus its row inside the first tile.
template <int LAYOUT, int HEAD_DIM, int BT, int HT>
__device__ __forceinline__ uint32_t indexer_row_base(uint32_t slot) {
  if constexpr (LAYOUT == kIndexerFlat) return slot * HEAD_DIM;
  else return (slot / BT) * (HEAD_DIM * BT) + (slot % BT) * HT;
}

template <int W> struct IndexerChunk;
template <> struct IndexerChunk<16> { using T = u32x4; };
template <> struct IndexerChunk<1> { using T = uint8_t; };

// The cache through a global (address space 1) pointer.  A row's address is
// rebuilt from halves another lane holds; as a generic pointer its load would
// be a flat load, which the hardware counts with the LDS operations, so the
// wait before the next cross-lane read would also wait for that load to
// return and the wave's loads would go out one round trip at a time.
typedef const __attribute__((address_space(1))) uint8_t* IndexerCache;

template <typename V>
__device__ __forceinline__ V load_cache(IndexerCache base, uint64_t off) {
  return __builtin_nontemporal_load(reinterpret_cast<const __attribute__((address_space(1))) V*>(base + off));
}

// 16-byte chunks are stored through a buffer resource over the wave's own
// destination rows (fewer than 2^31 bytes: the host checks the row stride),
// masked chunks with an out-of-range offset (store_buffer): no branch.  They
// are device-scope write-through stores, as the gather's flat 16-byte chunks:
// a single call leaves nothing dirty in L2 for its end to write back (the
// 300K flat gather's cold call 19.2 -> 18.7 us; back to back unchanged).

// Grid: any size; wave w of workgroup g takes rows from (g * WAVES + w) * 64
// on, striding by the grid's rows.  Source rows are dword-aligned (the host
// checks the cache base and the record stride; value rows start at multiples
// of 16 bytes inside a record), so bit 0 of a row's offset carries its mask
// when the offset crosses lanes.  The host launches only with num_tokens,
// num_batches, num_blocks and block_table_width all >= 1 (otherwise every row
// is masked): a masked row keeps an offset inside record 0, and the
// speculative table entry lies in row 0 below the width, so every load is in
// bounds and goes out without a branch, and only the stores are masked.
// W == 16 needs dword-aligned destination rows and 64 * dst_value_stride <
// 2^31 (the host picks W == 1 otherwise).  No LDS.
//
// The fields the first two dependent loads need (batch ids, batch extents,
// their counts, the block table and its geometry) are leading scalar
// arguments, preloaded into SGPRs at wave start; read from the parameter
// struct instead, each wave would first wait for two scalar-load round trips
// before its first batch-id load could leave.  The struct's copies of those
// fields are ignored.
template <int LAYOUT, int HEAD_DIM, int BT, int HT, int W, int CU>
__global__ __launch_bounds__(kIndexerThreads) void indexer_gather_kernel(
    const int32_t* token_to_seq, const int32_t* cu_seqlen, int32_t num_tokens, int32_t num_batches,
    const int32_t* block_table, int64_t block_table_ld, int32_t block_table_width, int32_t block_size,
    uint32_t block_size_magic, IndexerParams params) {
  IndexerParams p = params;
  p.token_to_seq = token_to_seq;
  p.cu_seqlen = cu_seqlen;
  p.num_tokens = num_tokens;
  p.num_batches = num_batches;
  p.block_table = block_table;
  p.block_table_ld = block_table_ld;
  p.block_table_width = block_table_width;
  p.block_size = block_size;
  p.block_size_magic = block_size_magic;
  using V = typename IndexerChunk<W>::T;
  constexpr int CPR = HEAD_DIM / W;  // chunks per row
  constexpr int WAVES = kIndexerThreads / 64;
  static_assert(HEAD_DIM % W == 0 && HEAD_DIM % 16 == 0, "rows are whole chunks, 16-byte multiples");
  // the wave's 64 rows are 64 * CPR chunks: CPR per lane, moved in batches of
  // at most 16 loads in flight per lane (all of them for 16-byte chunks of
  // rows up to 256 bytes)
  constexpr int PER_LANE = CPR;
  constexpr int BATCH = PER_LANE < 16 ? PER_LANE : 16;
  static_assert(PER_LANE % BATCH == 0, "whole batches");
  const int lane = threadIdx.x & 63;
  // wave-uniform, so a wave's row range and its destination resource sit in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t first_row0 = (int64_t(blockIdx.x) * WAVES + wave) * kIndexerRowsPerWave;
  const int32_t ncu = p.num_batches + 1;

  // The first rows' batch ids and the batch extents leave first thing, from
  // preloaded arguments only: the loop below needs fields of the parameter
  // struct, and the compiler waits for their scalar loads before its body.
  // (A wave past the last row reads row num_tokens - 1 and skips the loop.)
  const int32_t first_row = static_cast<int32_t>(first_row0) + lane;
  const int32_t first_batch = p.token_to_seq[first_row < p.num_tokens ? first_row : p.num_tokens - 1];
  int32_t cu_lane = 0;
  if constexpr (CU == kCuWave) cu_lane = p.cu_seqlen[lane < ncu ? lane : ncu - 1];
  // A speculative block-table entry, requested with the batch ids: row 0's
  // column first_row / block_size, the column of a row of batch 0 when
  // cu_seqlen[0] == 0.  A first-round row whose batch turns out to be 0 and
  // whose column is that one would load this same entry, so it takes it
  // instead; a wave whose rows all do skips the dependent table load (one
  // memory round trip fewer for the first batch's rows).
  const uint32_t spec_col = div_magic(static_cast<uint32_t>(min(first_row, p.num_tokens - 1)),
                                      static_cast<uint32_t>(p.block_size), p.block_size_magic);
  const int32_t spec_block = p.block_table[min(spec_col, static_cast<uint32_t>(p.block_table_width - 1))];
  const int64_t stride_rows = int64_t(gridDim.x) * WAVES * kIndexerRowsPerWave;

  for (int64_t row0 = first_row0; row0 < p.num_tokens; row0 += stride_rows) {
    // --- this lane's row: its batch, position, block and source ------------
    const int32_t row = static_cast<int32_t>(row0) + lane;
    bool ok = row < p.num_tokens;
    const int32_t batch = row0 == first_row0 ? first_batch : p.token_to_seq[ok ? row : p.num_tokens - 1];
    ok = ok && batch >= 0 && batch < p.num_batches;
    const int32_t b = ok ? batch : 0;
    int32_t start, end;
    if constexpr (CU == kCuWave) {
      start = __shfl(cu_lane, b, 64);
      end = __shfl(cu_lane, b + 1, 64);
    } else {
      start = p.cu_seqlen[b];
      end = p.cu_seqlen[b + 1];
    }
    ok = ok && row >= start && row < end;
    const uint32_t pos = ok ? static_cast<uint32_t>(row - start) : 0u;
    const uint32_t col = div_magic(pos, static_cast<uint32_t>(p.block_size), p.block_size_magic);
    const uint32_t slot = pos - col * static_cast<uint32_t>(p.block_size);
    ok = ok && col < static_cast<uint32_t>(p.block_table_width);
    int32_t block = -1;
    if (ok) {
      const bool same_entry = row0 == first_row0 && b == 0 && col == spec_col;
      block = same_entry ? spec_block : p.block_table[int64_t(b) * p.block_table_ld + col];
    }
    ok = ok && block >= 0 && block < p.num_blocks;
    // clamped to block 0 when invalid, then widened: the record stride is large
    const IndexerCache cache = (IndexerCache)p.cache;  // an address-space cast: the cache is global memory
    const uint64_t record = static_cast<uint64_t>(int64_t(ok ? block : 0) * p.block_stride);
    const uint64_t src_off = record + indexer_row_base<LAYOUT, HEAD_DIM, BT, HT>(slot);
    const uint32_t off_lo = static_cast<uint32_t>(src_off) | (ok ? 1u : 0u);
    const uint32_t off_hi = static_cast<uint32_t>(src_off >> 32);
    uint32_t scale = 0;
    // this wave's destination rows (16-byte chunks): row0 .. row0 + 63, cut at num_tokens
    const int64_t wave_rows = p.num_tokens - row0 < 64 ? p.num_tokens - row0 : 64;
    const __amdgpu_buffer_rsrc_t dst_rows = __builtin_amdgcn_make_buffer_rsrc(
        p.dst_values + row0 * p.dst_value_stride, 0, static_cast<int32_t>(wave_rows * p.dst_value_stride),
        kBufferWord3);

    // --- value bytes: chunk c = lane + 64k is chunk c % CPR of row c / CPR ---
#pragma unroll
    for (int k0 = 0; k0 < PER_LANE; k0 += BATCH) {
      // every chunk's row offset first (cross-lane reads), then every load
      uint64_t off[BATCH];
      bool take[BATCH];
#pragma unroll
      for (int k = 0; k < BATCH; ++k) {
        const uint32_t c = static_cast<uint32_t>(lane + 64 * (k0 + k));
        const int r = static_cast<int>(c / CPR);
        const uint32_t lo = static_cast<uint32_t>(__shfl(static_cast<int>(off_lo), r, 64));
        const uint32_t hi = static_cast<uint32_t>(__shfl(static_cast<int>(off_hi), r, 64));
        take[k] = (lo & 1u) != 0u;
        off[k] = ((static_cast<uint64_t>(hi) << 32) | (lo & ~1u)) +
                 indexer_chunk_offset<LAYOUT, HEAD_DIM, BT, HT, W>(c % CPR);
      }
      V v[BATCH];
#pragma unroll
      for (int k = 0; k < BATCH; ++k) v[k] = load_cache<V>(cache, off[k]);
      // the scale of this lane's own row goes out with the first batch's loads
      if (k0 == 0) scale = load_cache<uint32_t>(cache, record + p.scale_area + slot * 4u);
      if constexpr (W == 16) {
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
          const uint32_t c = static_cast<uint32_t>(lane + 64 * (k0 + k));
          const uint32_t o = take[k] ? (c / CPR) * static_cast<uint32_t>(p.dst_value_stride) + (c % CPR) * W
                                     : kMaskedOffset;
          store_buffer<kPolicyDeviceStream>(dst_rows, o, v[k]);
        }
      } else {
        // lane-guarded stores: keep the first chunk's load ahead of them
        keep_load_ahead(v[0]);
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
          const uint32_t c = static_cast<uint32_t>(lane + 64 * (k0 + k));
          const int64_t r = row0 + static_cast<int64_t>(c / CPR);
          if (take[k]) store_stream(p.dst_values + r * p.dst_value_stride + (c % CPR) * W, v[k]);
        }
      }
    }
    if (ok) store_stream(p.dst_scales + int64_t(row) * p.dst_scale_stride, scale);
  }
}

}  // namespace pkvg
