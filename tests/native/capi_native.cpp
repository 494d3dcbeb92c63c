// A native caller of the C ABI (include/pkvg.h): no Python, no torch.  Device
// memory from hipMalloc, inputs from a seeded generator, every compute entry
// point called on the default stream (the four paged gathers on a small batch
// and on 1,500 short requests, which build a task table first; the page-task
// builder; the indexer gather), and every output byte compared with the CPU
// oracle (the plain C definitions in oracle/oracle.c, test infrastructure,
// linked here only as the checker).  Prints one line per case; exits 0 when
// all match.
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
int64_t oracle_page_tasks(const int32_t* cu_seq_lens, int32_t terminal, const int32_t* seq_starts, int32_t num_reqs,
                          int64_t num_tokens, int32_t block_size, int32_t* out, int64_t cap);
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

// Which entry point a paged case calls.
enum class Call { kCache, kUpconvert, kDequantAuto, kDequantFp8, kNoallocAuto, kNoallocFp8 };

const char* call_name(Call c) {
  switch (c) {
    case Call::kCache: return "gather_cache";
    case Call::kUpconvert: return "gather_upconvert_fp8";
    case Call::kDequantAuto: return "gather_maybe_dequant(auto)";
    case Call::kDequantFp8: return "gather_maybe_dequant(fp8)";
    case Call::kNoallocAuto: return "gather_maybe_dequant_noalloc(auto)";
    default: return "gather_maybe_dequant_noalloc(fp8)";
  }
}

bool is_fp8(Call c) { return c == Call::kUpconvert || c == Call::kDequantFp8 || c == Call::kNoallocFp8; }

// A batch of paged requests: context lengths, the tokens skipped at each
// context's start, the page size and the table width.
struct Batch {
  std::vector<int32_t> lens, starts;
  int32_t bs, width;
};

// A small batch with partial first and last pages, an empty request and a
// guard-failing table entry; or `requests` random short contexts (more than
// the fused task paths take, so the task table is built first).
Batch make_batch(Lcg& g, int32_t requests) {
  Batch b;
  if (requests == 0) {
    b.lens = {17, 130, 0, 64};
    b.starts = {3, 5, 0, 16};
    b.bs = 16;
    b.width = 12;
    return b;
  }
  b.bs = 16;
  b.width = 6;
  for (int32_t r = 0; r < requests; ++r) {
    const int32_t n = g.next() % 8 == 0 ? 0 : static_cast<int32_t>(g.next() % 80);
    b.lens.push_back(n);
    b.starts.push_back(n ? static_cast<int32_t>(g.next() % (n + 1)) : 0);
  }
  return b;
}

// One paged gather through the C ABI against oracle_gather, every byte of the
// workspace compared (5 rows past num_tokens and the pad columns included).
bool gather_case(Call call, int32_t requests) {
  Lcg g{101u + 7u * static_cast<uint32_t>(call) + static_cast<uint32_t>(requests)};
  const bool fp8 = is_fp8(call);
  const Batch bt = make_batch(g, requests);
  const int32_t bs = bt.bs, entry = 576, R = static_cast<int32_t>(bt.lens.size()), width = bt.width;
  std::vector<int32_t> cu(R + 1, 0), pages(R);
  int64_t total_pages = 0;
  for (int32_t r = 0; r < R; ++r) {
    cu[r + 1] = cu[r] + (bt.lens[r] - bt.starts[r]);
    pages[r] = (bt.lens[r] + bs - 1) / bs;
    total_pages += pages[r];
  }
  const int64_t T = cu[R], rows = T + 5;                  // workspace tail of 5 untouched rows
  const int64_t nb = total_pages + 8;
  std::vector<int32_t> table = deal_table(g, pages, width, nb);
  if (pages[1] > 2) table[1 * width + 2] = static_cast<int32_t>(nb) + 3;  // guard fails: rows untouched
  const int32_t src_elem = fp8 ? 1 : 2;
  const int32_t dst_cols = entry + 2;                     // two pad columns per row, never written
  std::vector<uint8_t> cache(static_cast<size_t>(nb) * bs * entry * src_elem);
  for (auto& b : cache) {
    b = static_cast<uint8_t>(g.next());
    if (fp8 && (b & 0x7f) == 0x7f) b &= 0xfe;            // no NaN codes
  }
  std::vector<uint8_t> want(static_cast<size_t>(rows) * dst_cols * 2, 0xff);
  std::vector<uint8_t> got(want.size(), 0);
  const float scale = 0.0625f;
  const int64_t written = oracle_gather(fp8 ? kOracleE4m3fnToBf16 : kOracleCopy, cache.data(), src_elem, nb, bs,
                                        entry, int64_t(bs) * entry, entry, want.data(), 2, T, dst_cols, table.data(),
                                        width, width, cu.data(), 1, bt.starts.data(), R, scale);

  uint8_t* d_cache; uint8_t* d_dst; int32_t* d_table; int32_t* d_cu; int32_t* d_starts; float* d_scale;
  if (!to_device(cache, &d_cache) || !to_device(table, &d_table) || !to_device(cu, &d_cu) ||
      !to_device(bt.starts, &d_starts))
    return false;
  std::vector<float> hscale = {scale};
  if (!to_device(hscale, &d_scale)) return false;
  HIP_OK(hipMalloc(reinterpret_cast<void**>(&d_dst), want.size()));
  HIP_OK(hipMemset(d_dst, 0xff, want.size()));
  const int64_t sbs = int64_t(bs) * entry;
  int st = PKVG_OK;
  switch (call) {
    case Call::kCache:
      st = gather_cache(d_cache, 2, nb, bs, entry, sbs, entry, d_dst, T, dst_cols, d_table, width, width, d_cu, 1,
                        d_starts, R, nullptr);
      break;
    case Call::kUpconvert:
      st = gather_upconvert_fp8(d_cache, nb, bs, entry, sbs, entry, d_dst, T, dst_cols, d_table, width, width, d_cu,
                                1, d_starts, R, d_scale, nullptr);
      break;
    case Call::kDequantAuto:
    case Call::kDequantFp8:
      st = gather_maybe_dequant(d_cache, fp8 ? PKVG_KV_FP8_E4M3 : PKVG_KV_AUTO, nb, bs, entry, sbs, entry, d_dst, T,
                                dst_cols, d_table, width, width, d_cu, 1, d_starts, R, fp8 ? d_scale : nullptr,
                                nullptr);
      break;
    default:
      st = gather_maybe_dequant_noalloc(d_cache, fp8 ? PKVG_KV_FP8_E4M3 : PKVG_KV_AUTO, nb, bs, entry, sbs, entry,
                                        d_dst, T, dst_cols, d_table, width, width, d_cu, 1, d_starts, R,
                                        fp8 ? d_scale : nullptr, nullptr);
  }
  if (st != PKVG_OK) {
    std::printf("%s returned %d (%s)\n", call_name(call), st, pkvg_status_string(st));
    return false;
  }
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(got.data(), d_dst, got.size(), hipMemcpyDeviceToHost));
  for (void* p : {static_cast<void*>(d_cache), static_cast<void*>(d_dst), static_cast<void*>(d_table),
                  static_cast<void*>(d_cu), static_cast<void*>(d_starts), static_cast<void*>(d_scale)})
    HIP_OK(hipFree(p));
  const bool ok = got == want && written > 0 && written <= T;
  std::printf("native %s, %d requests: %lld of %lld rows written by the oracle, workspace %s\n", call_name(call), R,
              static_cast<long long>(written), static_cast<long long>(T), ok ? "identical" : "DIFFERS");
  return ok;
}

// The page-task builder on its own (gather_page_tasks) against oracle_page_tasks:
// the five task fields, and each task's physical block against the table and
// its guards.
bool page_tasks_case(int32_t requests) {
  Lcg g{505u + static_cast<uint32_t>(requests)};
  const Batch bt = make_batch(g, requests);
  const int32_t bs = bt.bs, R = static_cast<int32_t>(bt.lens.size()), width = bt.width;
  std::vector<int32_t> cu(R + 1, 0), pages(R);
  int64_t total_pages = 0;
  for (int32_t r = 0; r < R; ++r) {
    cu[r + 1] = cu[r] + (bt.lens[r] - bt.starts[r]);
    pages[r] = (bt.lens[r] + bs - 1) / bs;
    total_pages += pages[r];
  }
  const int64_t T = cu[R], nb = total_pages + 8;
  std::vector<int32_t> table = deal_table(g, pages, width, nb);
  if (pages[1] > 2) table[1 * width + 2] = -1;            // a guard-failing entry: phys -1
  const int64_t count = oracle_page_tasks(cu.data(), 1, bt.starts.data(), R, T, bs, nullptr, 0);
  std::vector<int32_t> want(static_cast<size_t>(count) * 5);
  oracle_page_tasks(cu.data(), 1, bt.starts.data(), R, T, bs, want.data(), count);

  int32_t* d_cu; int32_t* d_starts; int32_t* d_table; int32_t* d_tasks; int32_t* d_count;
  if (!to_device(cu, &d_cu) || !to_device(bt.starts, &d_starts) || !to_device(table, &d_table)) return false;
  const int64_t cap = count + 4;
  HIP_OK(hipMalloc(reinterpret_cast<void**>(&d_tasks), cap * PKVG_TASK_INTS * sizeof(int32_t)));
  HIP_OK(hipMalloc(reinterpret_cast<void**>(&d_count), sizeof(int32_t)));
  const int st = gather_page_tasks(d_cu, 1, d_starts, R, T, bs, d_table, width, width, nb, d_tasks, cap, d_count,
                                   nullptr);
  if (st != PKVG_OK) {
    std::printf("gather_page_tasks returned %d (%s)\n", st, pkvg_status_string(st));
    return false;
  }
  HIP_OK(hipDeviceSynchronize());
  int32_t got_count = -1;
  std::vector<int32_t> got(static_cast<size_t>(count) * PKVG_TASK_INTS);
  HIP_OK(hipMemcpy(&got_count, d_count, sizeof(int32_t), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(got.data(), d_tasks, got.size() * sizeof(int32_t), hipMemcpyDeviceToHost));
  for (void* p : {static_cast<void*>(d_cu), static_cast<void*>(d_starts), static_cast<void*>(d_table),
                  static_cast<void*>(d_tasks), static_cast<void*>(d_count)})
    HIP_OK(hipFree(p));
  bool ok = got_count == count;
  for (int64_t k = 0; ok && k < count; ++k) {
    const int32_t* t = &got[k * PKVG_TASK_INTS];
    for (int f = 0; f < 5; ++f) ok = ok && t[f] == want[k * 5 + f];
    const int32_t r = t[0], l = t[1];
    const int32_t e = l < width ? table[static_cast<size_t>(r) * width + l] : -1;
    ok = ok && t[5] == (e >= 0 && e < nb ? e : -1) && t[6] == 0 && t[7] == 0;
  }
  std::printf("native gather_page_tasks, %d requests: %d tasks (oracle %lld), records %s\n", R, got_count,
              static_cast<long long>(count), ok ? "identical" : "DIFFER");
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
  bool ok = true;
  for (Call c : {Call::kCache, Call::kUpconvert, Call::kDequantAuto, Call::kDequantFp8, Call::kNoallocAuto,
                 Call::kNoallocFp8})
    for (int32_t requests : {0, 1500}) ok = gather_case(c, requests) && ok;
  for (int32_t requests : {0, 1500}) ok = page_tasks_case(requests) && ok;
  ok = indexer_case() && ok;
  std::printf("%s\n", ok ? "native C-ABI parity ok" : "native C-ABI parity FAILED");
  return ok ? 0 : 1;
}
