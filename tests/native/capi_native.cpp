// A native caller of the C ABI (include/pkvg.h): no Python, no torch.  Device
// memory from hipMalloc, inputs from a seeded generator, one call of each of
// gather_cache, gather_upconvert_fp8 and gather_indexer_quant_cache on the
// default stream, and every output byte compared with the CPU oracle (the
// plain C definitions in oracle/oracle.c, test infrastructure, linked here only
// as the checker).  Prints one line per case; exits 0 when all match.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "pkvg.h"

extern "C" {
int64_t oracle_gather(int32_t mode, const uint8_t* src, int32_t src_elem_bytes, int64_t num_blocks,
                      int32_t block_size, int32_t entry, int64_t src_block_stride, int64_t src_token_stride,
                      uint8_t* dst, int32_t dst_elem_bytes, int64_t num_tokens, int64_t dst_row_stride,
                      const int32_t* block_table, int32_t block_table_width, int64_t block_table_ld,
                      const int32_t* cu_seq_lens, int32_t terminal, const int32_t* seq_starts,
                      int32_t num_reqs, float scale);
int64_t oracle_indexer_gather(const uint8_t* cache, int64_t num_blocks, int32_t block_size,
                              int64_t block_stride, int32_t layout, int32_t head_dim, int32_t block_tile,
                              int32_t head_tile, uint8_t* dst_values, int64_t dst_value_stride,
                              uint8_t* dst_scales, int64_t dst_scale_stride, int64_t num_tokens,
                              const int32_t* token_to_seq, const int32_t* cu_seqlen, int32_t num_batches,
                              const int32_t* block_table, int32_t block_table_width,
                              int64_t block_table_ld);
}

namespace {

constexpr int32_t kOracleCopy = 0;
constexpr int32_t kOracleE4m3fnToBf16 = 1;

#define HIP_OK(x)                                                                        \
  do {                                                                                   \
    hipError_t e_ = (x);                                                                 \
    if (e_ != hipSuccess) {                                                              \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);         \
      return false;                                                                      \
    }                                                                                    \
  } while (0)

// A seeded 64-bit linear congruential generator (Knuth's MMIX constants).
struct Lcg {
  uint64_t s;
  uint32_t next() {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return static_cast<uint32_t>(s >> 33);
  }
};

template <class T>
bool to_device(const std::vector<T>& h, T** d) {
  HIP_OK(hipMalloc(reinterpret_cast<void**>(d), h.size() * sizeof(T) + 16));
  HIP_OK(hipMemcpy(*d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice));
  return true;
}

// A shuffled table: request r gets pages[r] distinct physical blocks out of num_blocks;
// unused slots are -1.
std::vector<int32_t> deal_table(Lcg& g, const std::vector<int32_t>& pages, int32_t width, int64_t num_blocks) {
  std::vector<int32_t> perm(static_cast<size_t>(num_blocks));
  for (int64_t i = 0; i < num_blocks; ++i) perm[i] = static_cast<int32_t>(i);
  for (int64_t i = num_blocks - 1; i > 0; --i) std::swap(perm[i], perm[g.next() % (i + 1)]);
  std::vector<int32_t> table(pages.size() * width, -1);
  size_t k = 0;
  for (size_t r = 0; r < pages.size(); ++r)
    for (int32_t j = 0; j < pages[r]; ++j) table[r * width + j] = perm[k++];
  return table;
}

// One paged gather (raw bf16 or fp8 -> bf16) through the C ABI against oracle_gather.
bool gather_case(bool fp8) {
  Lcg g{fp8 ? 202u : 101u};
  const int32_t bs = 16, entry = 576, R = 4;
  const std::vector<int32_t> lens = {17, 130, 0, 64};     // context lengths
  const std::vector<int32_t> starts = {3, 5, 0, 16};      // tokens skipped at each context's start
  std::vector<int32_t> cu(R + 1, 0), pages(R);
  for (int32_t r = 0; r < R; ++r) {
    cu[r + 1] = cu[r] + (lens[r] - starts[r]);
    pages[r] = (lens[r] + bs - 1) / bs;
  }
  const int64_t T = cu[R], rows = T + 5;                  // workspace tail of 5 untouched rows
  const int32_t width = 12;
  const int64_t nb = 40;
  std::vector<int32_t> table = deal_table(g, pages, width, nb);
  table[1 * width + 2] = static_cast<int32_t>(nb) + 3;    // a guard-failing entry: its rows stay untouched
  const int32_t src_elem = fp8 ? 1 : 2;
  std::vector<uint8_t> cache(static_cast<size_t>(nb) * bs * entry * src_elem);
  for (auto& b : cache) {
    b = static_cast<uint8_t>(g.next());
    if (fp8 && (b & 0x7f) == 0x7f) b &= 0xfe;            // no NaN codes
  }
  std::vector<uint8_t> want(static_cast<size_t>(rows) * entry * 2, 0xff);
  std::vector<uint8_t> got(want.size(), 0);
  const float scale = 0.0625f;
  const int64_t written = oracle_gather(fp8 ? kOracleE4m3fnToBf16 : kOracleCopy, cache.data(), src_elem, nb, bs,
                                        entry, int64_t(bs) * entry, entry, want.data(), 2, T, entry, table.data(),
                                        width, width, cu.data(), 1, starts.data(), R, scale);

  uint8_t* d_cache; uint8_t* d_dst; int32_t* d_table; int32_t* d_cu; int32_t* d_starts; float* d_scale;
  if (!to_device(cache, &d_cache) || !to_device(table, &d_table) || !to_device(cu, &d_cu) ||
      !to_device(starts, &d_starts))
    return false;
  std::vector<float> hscale = {scale};
  if (!to_device(hscale, &d_scale)) return false;
  HIP_OK(hipMalloc(reinterpret_cast<void**>(&d_dst), want.size()));
  HIP_OK(hipMemset(d_dst, 0xff, want.size()));
  const int st = fp8 ? gather_upconvert_fp8(d_cache, nb, bs, entry, int64_t(bs) * entry, entry, d_dst, T, entry,
                                            d_table, width, width, d_cu, 1, d_starts, R, d_scale, nullptr)
                     : gather_cache(d_cache, 2, nb, bs, entry, int64_t(bs) * entry, entry, d_dst, T, entry,
                                    d_table, width, width, d_cu, 1, d_starts, R, nullptr);
  if (st != PKVG_OK) {
    std::printf("%s returned %d (%s)\n", fp8 ? "gather_upconvert_fp8" : "gather_cache", st, pkvg_status_string(st));
    return false;
  }
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(got.data(), d_dst, got.size(), hipMemcpyDeviceToHost));
  for (void* p : {static_cast<void*>(d_cache), static_cast<void*>(d_dst), static_cast<void*>(d_table),
                  static_cast<void*>(d_cu), static_cast<void*>(d_starts), static_cast<void*>(d_scale)})
    HIP_OK(hipFree(p));
  const bool ok = got == want && written > 0 && written < T;
  std::printf("native %s: %lld of %lld rows written by the oracle, workspace %s\n",
              fp8 ? "gather_upconvert_fp8" : "gather_cache", static_cast<long long>(written),
              static_cast<long long>(T), ok ? "identical" : "DIFFERS");
  return ok;
}

// The indexer quant-cache gather (flat records) through the C ABI against oracle_indexer_gather.
bool indexer_case() {
  Lcg g{303u};
  const int32_t bs = 64, hd = 128, B = 3;
  const std::vector<int32_t> lens = {200, 0, 70};
  std::vector<int32_t> cu(B + 1, 0), pages(B);
  for (int32_t b = 0; b < B; ++b) {
    cu[b + 1] = cu[b] + lens[b];
    pages[b] = (lens[b] + bs - 1) / bs;
  }
  const int64_t T = cu[B] + 6;                             // 6 padding rows (batch id -1)
  std::vector<int32_t> t2s(static_cast<size_t>(T), -1);
  for (int32_t b = 0; b < B; ++b)
    for (int32_t i = cu[b]; i < cu[b + 1]; ++i) t2s[i] = b;
  t2s[5] = 7;                                              // a batch id past the batch count: masked
  const int32_t width = 5;
  const int64_t nb = 9, stride = int64_t(bs) * (hd + 4);
  std::vector<int32_t> table = deal_table(g, pages, width, nb);
  std::vector<uint8_t> cache(static_cast<size_t>(nb * stride));
  for (auto& b : cache) b = static_cast<uint8_t>(g.next());
  std::vector<uint8_t> want_v(static_cast<size_t>(T) * hd, 0xff), got_v(want_v.size(), 0);
  std::vector<uint8_t> want_s(static_cast<size_t>(T) * 4, 0xff), got_s(want_s.size(), 0);
  const int64_t written = oracle_indexer_gather(cache.data(), nb, bs, stride, PKVG_INDEXER_FLAT, hd, 16, 16,
                                                want_v.data(), hd, want_s.data(), 4, T, t2s.data(), cu.data(), B,
                                                table.data(), width, width);

  uint8_t* d_cache; uint8_t* d_v; float* d_s; int32_t* d_t2s; int32_t* d_cu; int32_t* d_table;
  if (!to_device(cache, &d_cache) || !to_device(t2s, &d_t2s) || !to_device(cu, &d_cu) ||
      !to_device(table, &d_table))
    return false;
  HIP_OK(hipMalloc(reinterpret_cast<void**>(&d_v), want_v.size()));
  HIP_OK(hipMalloc(reinterpret_cast<void**>(&d_s), want_s.size()));
  HIP_OK(hipMemset(d_v, 0xff, want_v.size()));
  HIP_OK(hipMemset(d_s, 0xff, want_s.size()));
  const int st = gather_indexer_quant_cache(d_cache, nb, bs, stride, PKVG_INDEXER_FLAT, hd, 16, 16, d_v, hd, d_s, 1,
                                            T, d_t2s, d_cu, B, d_table, width, width, nullptr);
  if (st != PKVG_OK) {
    std::printf("gather_indexer_quant_cache returned %d (%s)\n", st, pkvg_status_string(st));
    return false;
  }
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(got_v.data(), d_v, got_v.size(), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(got_s.data(), d_s, got_s.size(), hipMemcpyDeviceToHost));
  for (void* p : {static_cast<void*>(d_cache), static_cast<void*>(d_v), static_cast<void*>(d_s),
                  static_cast<void*>(d_t2s), static_cast<void*>(d_cu), static_cast<void*>(d_table)})
    HIP_OK(hipFree(p));
  const bool ok = got_v == want_v && got_s == want_s && written == cu[B] - 1;
  std::printf("native gather_indexer_quant_cache: %lld of %lld rows written by the oracle, outputs %s\n",
              static_cast<long long>(written), static_cast<long long>(T), ok ? "identical" : "DIFFER");
  return ok;
}

}  // namespace

int main() {
  int devices = 0;
  if (hipGetDeviceCount(&devices) != hipSuccess || devices < 1) {
    std::printf("no GPU\n");
    return 2;
  }
  bool ok = gather_case(false);
  ok = gather_case(true) && ok;
  ok = indexer_case() && ok;
  std::printf("%s\n", ok ? "native C-ABI parity ok" : "native C-ABI parity FAILED");
  return ok ? 0 : 1;
}
