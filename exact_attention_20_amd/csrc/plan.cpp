// Decode plan: split each request's pages into chunks and order the work.
//
// "FIA / FlashAttention" Q&A, section 2: a plan stage preprocesses the ragged
// lengths and balances load so that requests of different lengths do not
// leave GPU threads idle; the run stage then executes the batch. The
// Flash-Decoding section of "Flash Attention & Paged Attention" splits the KV
// sequence into blocks that different compute units process in parallel.
//
// Pure host code (no HIP call): it is unit-tested on the CPU.
#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <vector>

#include "fa_internal.h"

namespace fa {

namespace {

// Work items per CU the auto mode aims for. Several resident workgroups per
// CU and a few rounds of them keep the tail of near-equal items short.
int items_per_cu() {
  static int v = [] {
    const char* e = std::getenv("FA_DECODE_ITEMS_PER_CU");
    int x = e ? std::atoi(e) : 0;
    return x > 0 ? x : 12;
  }();
  return v;
}

// Smallest chunk in pages: below this the per-item fixed cost (query load,
// epilogue merge, partial write) stops being small next to the page traffic.
constexpr int kMinChunkPages = 4;

}  // namespace

int plan_decode_host(const int32_t* seqlens, int B, int stride, int Hkv, int num_splits_request,
                     int num_cus, WorkItem* items, int capacity, int32_t* splits,
                     PlanResult* res) {
  if (!seqlens || B < 1 || stride < 1 || Hkv < 1 || Hkv > kMaxHeads || num_cus < 1 ||
      num_splits_request < 0 || !res)
    return -1;
  int64_t total_units = 0;  // page-head units
  std::vector<int> pages(B);
  for (int b = 0; b < B; ++b) {
    if (seqlens[b] < 0) return -1;
    int n = (int)(((int64_t)seqlens[b] + kPage - 1) / kPage);
    if (n > stride) return -1;
    pages[b] = n;
    total_units += (int64_t)n * Hkv;
  }
  int chunk = 0;
  if (num_splits_request == 0) {
    int64_t target = (int64_t)num_cus * items_per_cu();
    int64_t c = (total_units + target - 1) / std::max<int64_t>(target, 1);
    chunk = (int)std::max<int64_t>(kMinChunkPages, c);
  }
  // Split counts and near-equal page ranges per request.
  std::vector<WorkItem> list;
  int max_splits = 0;
  for (int b = 0; b < B; ++b) {
    int n = pages[b];
    int ns = 0;
    if (n > 0) ns = num_splits_request > 0 ? std::min(num_splits_request, n) : (n + chunk - 1) / chunk;
    if (ns > (1 << 22)) return -1;
    if (splits) splits[b] = ns;
    max_splits = std::max(max_splits, ns);
    for (int s = 0; s < ns; ++s) {
      int p0 = (int)((int64_t)n * s / ns);
      int p1 = (int)((int64_t)n * (s + 1) / ns);
      for (int g = 0; g < Hkv; ++g) list.push_back(WorkItem{b, g | (s << 8), p0, p1});
    }
  }
  // Longest items first, so the short ones fill the tail.
  std::stable_sort(list.begin(), list.end(), [](const WorkItem& x, const WorkItem& y) {
    return (x.page_end - x.page_begin) > (y.page_end - y.page_begin);
  });
  res->num_splits = max_splits;
  res->chunk_pages = chunk;
  res->n_items = (int)list.size();
  if (items) {
    int n = std::min<int>(capacity, (int)list.size());
    std::copy(list.begin(), list.begin() + n, items);
  }
  return 0;
}

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

WorkspaceLayout workspace_layout(int n_items, int B, int Hq, int D, int num_splits) {
  WorkspaceLayout w;
  w.items_off = 0;
  w.splits_off = align_up(w.items_off + sizeof(WorkItem) * (size_t)std::max(n_items, 1), 256);
  w.part_o_off = align_up(w.splits_off + sizeof(int32_t) * (size_t)B, 256);
  size_t rows = (size_t)B * Hq * (size_t)std::max(num_splits, 1);
  w.part_lse_off = align_up(w.part_o_off + sizeof(float) * rows * D, 256);
  w.total = align_up(w.part_lse_off + sizeof(float) * rows, 256);
  return w;
}

}  // namespace fa
