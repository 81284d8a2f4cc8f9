// plan_check.cpp -- CPU checks of the planner (csrc/plan.h, csrc/plan.cpp) that the
// kernels rely on, built with the host compiler and run by tests/test_plan_native.py.
//
//  1. The chunk grid the kernels derive from a sequence's table entry (chunk_count,
//     chunk_start, next_cut, boundary_ordinal) equals the host enumeration chunk_grid
//     (cuts at every multiple of 64 and of the block strictly inside the sequence, plus
//     both ends) for every start, length and block tried.
//  2. plan_call lays out units, pages and the staged table consistently: unit0 / page0
//     prefix sums, the unit -> sequence map, the inline / staged decision and the
//     workspace offsets (factorize and scan stages agree).
//  3. join_address widens both halves as unsigned (bit 31 of the low half set).
// Prints "ok" and exits 0, or prints the first mismatch and exits 1.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../gated_deltanet_recurrent_chunk_amd/csrc/plan.h"

using namespace gdn;

static int fails = 0;
#define CHECK(cond, ...)                      \
  do {                                        \
    if (!(cond)) {                            \
      if (fails < 20) {                       \
        std::printf("FAIL %s: ", #cond);      \
        std::printf(__VA_ARGS__);             \
        std::printf("\n");                    \
      }                                       \
      ++fails;                                \
    }                                         \
  } while (0)

static void check_grid(int64_t p0, int64_t len, int32_t block) {
  std::vector<int64_t> cuts;
  chunk_grid(p0, len, block, &cuts);
  const uint32_t lcm = grid_lcm((uint32_t)block);
  const uint32_t n = chunk_count((uint32_t)p0, (uint32_t)len, (uint32_t)block, lcm);
  const uint32_t want = cuts.empty() ? 0 : (uint32_t)cuts.size() - 1;
  CHECK(n == want, "p0=%lld len=%lld block=%d: %u chunks, grid has %u", (long long)p0, (long long)len, block, n, want);
  if (n != want) return;
  uint32_t ord = 0;
  for (uint32_t j = 0; j < n; ++j) {
    const uint32_t st = chunk_start((uint32_t)p0, j, (uint32_t)block, lcm);
    CHECK(st == (uint32_t)cuts[j], "p0=%lld len=%lld block=%d j=%u: start %u, grid %lld", (long long)p0,
          (long long)len, block, j, st, (long long)cuts[j]);
    const uint32_t nx = next_cut(st, (uint32_t)(p0 + len), (uint32_t)block);
    CHECK(nx == (uint32_t)cuts[j + 1], "p0=%lld len=%lld block=%d j=%u: next %u, grid %lld", (long long)p0,
          (long long)len, block, j, nx, (long long)cuts[j + 1]);
    if (block > 0 && cuts[j + 1] % block == 0) {
      CHECK(boundary_ordinal((uint32_t)p0, (uint32_t)cuts[j + 1], (uint32_t)block) == ord,
            "p0=%lld block=%d boundary %lld: ordinal", (long long)p0, block, (long long)cuts[j + 1]);
      ++ord;
    }
  }
  CHECK((int64_t)ord == count_boundaries(p0, len, block), "p0=%lld len=%lld block=%d: boundary count",
        (long long)p0, (long long)len, block);
}

static void check_plan() {
  LayerInfo L;
  gdn_layer layer{2, 4, 128, 4, GDN_BF16, GDN_ACT_SILU, 1.0f};
  CHECK(check_layer(&layer, &L) == GDN_OK, "layer");
  // a batch of n sequences: lengths and starts that mix empty, ragged and boundary cases
  for (int n : {1, 3, 8, 9, 40}) {
    std::vector<SeqSpan> spans;
    int64_t row = 0;
    for (int i = 0; i < n; ++i) {
      const int64_t len = (i * 37) % 211, p0 = (i % 3) * 784 + (i % 2) * 5;
      spans.push_back({row, len, p0});
      row += len;
    }
    for (int32_t block : {0, 64, 784, 896, 80}) {
      std::vector<int32_t> pages, begin;
      int64_t nb = 0;
      for (auto& sp : spans) {
        begin.push_back((int32_t)nb);
        nb += count_boundaries(sp.p0, sp.len, block);
      }
      for (int64_t i = 0; i < nb; ++i) pages.push_back((int32_t)(i % 7) - 1);
      CallPlan scan, fact, conv;
      CHECK(plan_call(L, spans, block, &pages, &begin, true, &scan) == GDN_OK, "plan scan");
      CHECK(plan_call(L, spans, block, nullptr, nullptr, true, &fact) == GDN_OK, "plan factorize");
      CHECK(plan_call(L, spans, block, &pages, &begin, false, &conv) == GDN_OK, "plan conv");
      CHECK(scan.off_factors == fact.off_factors && scan.total_bytes == fact.total_bytes,
            "n=%d block=%d: the two prefill stages lay out the workspace differently", n, block);
      const bool staged = n > kInlineSeqs || nb > kInlinePages;
      CHECK(scan.staged == staged && fact.staged == staged && conv.staged == staged, "n=%d block=%d staged", n, block);
      int64_t units = 0;
      for (int i = 0; i < n; ++i) {
        const SeqEntry& e = scan.seqs[i];
        std::vector<int64_t> cuts;
        chunk_grid(spans[i].p0, spans[i].len, block, &cuts);
        CHECK(e.unit0 == units && e.n_units == (int32_t)(cuts.empty() ? 0 : cuts.size() - 1), "units %d", i);
        CHECK(e.page0 == begin[i] && fact.seqs[i].page0 == begin[i], "page0 %d", i);
        CHECK(e.row0 == spans[i].row0 && e.p0 == spans[i].p0 && e.len == spans[i].len, "entry %d", i);
        units += e.n_units;
        CHECK(conv.seqs[i].n_units == (spans[i].len ? (spans[i].len + 15) / 16 : 1), "tiles %d", i);
      }
      CHECK(scan.n_units == units, "total units");
      if (staged) {
        std::vector<uint8_t> img(scan.table_bytes);
        staged_table(scan, img.data());
        const SeqEntry* se = reinterpret_cast<const SeqEntry*>(img.data());
        const int32_t* pg = reinterpret_cast<const int32_t*>(img.data() + scan.off_pages);
        const int32_t* us = reinterpret_cast<const int32_t*>(img.data() + scan.off_unit_seq);
        for (int i = 0; i < n; ++i) {
          CHECK(se[i].unit0 == scan.seqs[i].unit0, "staged entry %d", i);
          for (int u = 0; u < se[i].n_units; ++u) CHECK(us[se[i].unit0 + u] == i, "unit map %d", i);
        }
        for (int64_t i = 0; i < nb; ++i) CHECK(pg[i] == pages[i], "staged page %lld", (long long)i);
        CHECK(scan.off_unit_seq + (size_t)units * 4 <= scan.table_bytes && scan.table_bytes <= scan.off_factors,
              "staged table bounds");
        CallTable t;
        fill_call_table(scan, reinterpret_cast<void*>(0x1000), &t);
        CHECK(t.seqs == reinterpret_cast<const SeqEntry*>(0x1000) && t.unit_seq != nullptr, "staged pointers");
      } else {
        CallTable t;
        fill_call_table(scan, nullptr, &t);
        CHECK(t.seqs == nullptr && t.pages == nullptr && t.unit_seq == nullptr, "inline pointers");
        for (int i = 0; i < n; ++i) CHECK(t.inl_seqs[i].unit0 == scan.seqs[i].unit0, "inline entry %d", i);
        for (int64_t i = 0; i < nb; ++i) CHECK(t.inl_pages[i] == pages[i], "inline page");
        CHECK(t.n_seqs == n && t.n_pages == nb && t.n_units == units && t.block == block, "inline counts");
      }
    }
  }
  // positions at or past 2^30 are refused
  std::vector<SeqSpan> big{{0, 10, kMaxPosition - 5}};
  CallPlan p;
  CHECK(plan_call(L, big, 64, nullptr, nullptr, true, &p) == GDN_ERR_CAPACITY, "position limit");
}

int main() {
  for (int32_t block : {0, 16, 48, 64, 80, 128, 784, 896, 1000, 4096})
    for (int64_t p0 : {0, 1, 15, 63, 64, 65, 783, 784, 1792, 3136, 5000})
      for (int64_t len : {0, 1, 2, 63, 64, 65, 100, 777, 1792, 3000, 7000}) check_grid(p0, len, block);
  // the long workload's grid
  check_grid(0, 229376, 896);
  check_grid(0, 229376, 784);
  check_plan();
  // bit 31 of the low half set: the address must keep its zero high bits
  CHECK(join_address(0x80001000u, 0x00007f12u) == 0x00007f1280001000ull, "join_address");
  CHECK(join_address(0xFFFFFFF0u, 0u) == 0x00000000FFFFFFF0ull, "join_address low");
  CHECK(join_address((uint32_t)(int32_t)-16, 1u) == 0x00000001FFFFFFF0ull, "join_address signed input");
  if (fails) {
    std::printf("%d failures\n", fails);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
