// Host plans: decode split chunks, and the ragged prefill work order.
//
// "FIA / FlashAttention" Q&A, section 2: a plan stage preprocesses the ragged
// lengths and balances load so that requests of different lengths do not
// leave GPU threads idle; the run stage then executes the batch. The
// Flash-Decoding section of "Flash Attention & Paged Attention" splits the KV
// sequence into blocks that different compute units process in parallel.
//
// Pure host code (no HIP call): it is unit-tested on the CPU.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstdlib>
#include <functional>
#include <queue>
#include <vector>

#include "fa_internal.h"

namespace fa {

namespace {

// Smallest chunk in pages: below this the per-item fixed cost (query load,
// epilogue merge, partial write) stops being small next to the page traffic.
constexpr int kMinChunkPages = 4;

// Split-kernel workgroups resident on one CU at a time (the register and LDS
// use of the split kernels allows two), i.e. work items processed in parallel
// per CU.
constexpr int kResidentPerCU = 2;

// Fixed cost of one work item in page-equivalents (query load, first-page
// latency, epilogue and partial write), used to compare chunk sizes.
constexpr double kItemCost = 2.0;

// The same cost for a segment of a balanced window (a workgroup's second
// item starts only after its first has finished).
constexpr int64_t kWindowItemCost = 2;

// Number of work items for a given chunk size.
int64_t count_items(const std::vector<int>& pages, int Hkv, int chunk) {
  int64_t n = 0;
  for (int p : pages) n += (p + chunk - 1) / chunk;
  return n * Hkv;
}

// Estimated duration, in page-equivalents, of the work list for chunk size
// `chunk` on `slots` workgroups that take items in list order (longest
// first) as slots free up -- how the dispatcher runs the grid.
double makespan(const std::vector<int>& pages, int Hkv, int chunk, int slots) {
  std::vector<int> lens;
  for (int p : pages) {
    const int ns = (p + chunk - 1) / chunk;
    for (int s = 0; s < ns; ++s) {
      const int len = (int)((int64_t)p * (s + 1) / ns - (int64_t)p * s / ns);
      for (int g = 0; g < Hkv; ++g) lens.push_back(len);
    }
  }
  std::sort(lens.begin(), lens.end(), std::greater<int>());
  std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
  for (int i = 0; i < slots; ++i) free_at.push(0.0);
  double end = 0.0;
  for (int len : lens) {
    const double t = free_at.top() + kItemCost + len;
    free_at.pop();
    free_at.push(t);
    end = std::max(end, t);
  }
  return end;
}

// Auto chunk size: for k = 1..10 rounds of the resident workgroups, the
// smallest chunk whose item count fits k full rounds; the candidate with the
// shortest estimated duration wins (ties: the larger chunk, fewer items).
// Item counts just over a multiple of the resident slots leave a nearly empty
// last round, which is what this avoids.
int auto_chunk(const std::vector<int>& pages, int Hkv, int num_cus) {
  int max_pages = kMinChunkPages;
  for (int p : pages) max_pages = std::max(max_pages, p);
  const int slots = std::max(1, num_cus * kResidentPerCU);
  std::vector<int> cands;
  for (int k = 1; k <= 10; ++k) {
    const int64_t limit = (int64_t)k * slots;
    if (count_items(pages, Hkv, max_pages) > limit) continue;  // even one item per request is too many
    int lo = kMinChunkPages, hi = max_pages;                     // count_items is non-increasing in chunk
    while (lo < hi) {
      const int mid = lo + (hi - lo) / 2;
      if (count_items(pages, Hkv, mid) <= limit) hi = mid; else lo = mid + 1;
    }
    cands.push_back(lo);
  }
  if (cands.empty()) return max_pages;
  int best = cands[0];
  double best_t = makespan(pages, Hkv, best, slots);
  for (size_t i = 1; i < cands.size(); ++i) {
    const double t = makespan(pages, Hkv, cands[i], slots);
    if (t < best_t - 1e-9 || (t <= best_t + 1e-9 && cands[i] > best)) {
      best = cands[i];
      best_t = t;
    }
  }
  return best;
}

// Balanced windows for a single round of workgroups. The pages of all
// requests, concatenated in request order (the same for every KV head), are
// cut into at most `per_head` windows of cost at most C, where a window's cost
// is its pages plus kItemCost for each of its segments (its parts inside one
// request). Returns the number of windows needed for bound C (a huge number
// if some window could take no page).
int64_t count_windows(const std::vector<int>& pages, int64_t C) {
  int64_t windows = 0;
  size_t b = 0;
  int64_t rem = 0;
  auto next = [&] {
    while (b < pages.size() && pages[b] == 0) ++b;
    rem = b < pages.size() ? pages[b] : 0;
  };
  next();
  while (rem > 0) {
    ++windows;
    int64_t cost = 0;
    while (rem > 0) {
      const int64_t avail = C - cost - kWindowItemCost;
      if (avail < 1) {
        if (cost == 0) return INT64_MAX;
        break;
      }
      const int64_t take = std::min(avail, rem);
      cost += kWindowItemCost + take;
      rem -= take;
      if (rem == 0) {
        ++b;
        next();
      } else {
        break;
      }
    }
  }
  return windows;
}

}  // namespace

int plan_decode_host(const int32_t* seqlens, int B, int stride, int Hkv, int num_splits_request,
                     int num_cus, WorkItem* items, int capacity, int32_t* splits,
                     PlanResult* res, bool windows) {
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
  if (num_splits_request == 0 && total_units > 0) chunk = auto_chunk(pages, Hkv, num_cus);
  if (num_splits_request == 0 && chunk < 1) chunk = kMinChunkPages;

  // A chunk plan that fits one round of the resident workgroups is bounded by
  // its largest item, so near-equal splits per request leave slots idle at
  // the end. Cost-balanced windows over all requests fill every slot evenly
  // at the price of a second segment (item) where a window crosses a request
  // boundary; they are used when their estimated duration is shorter.
  const int slots = std::max(1, num_cus * kResidentPerCU);
  const int per_head = slots / Hkv;
  if (windows && num_splits_request == 0 && total_units > 0 && per_head >= 1 &&
      count_items(pages, Hkv, chunk) <= slots) {
    int64_t P = 0, maxp = 0;
    for (int n : pages) {
      P += n;
      maxp = std::max<int64_t>(maxp, n);
    }
    int64_t lo = 1 + kWindowItemCost, hi = maxp + 2 * kWindowItemCost;  // hi: one window per request
    if (count_windows(pages, hi) > per_head) hi = P + kWindowItemCost * B + 1;
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo) / 2;
      if (count_windows(pages, mid) <= per_head) hi = mid; else lo = mid + 1;
    }
    const double chunk_t = makespan(pages, Hkv, chunk, slots);
    if (count_windows(pages, lo) <= per_head && (double)lo < chunk_t - 0.5) {
      // Window w of head g runs on workgroup g * n_win + w; its r-th segment
      // is item r * grid + (g * n_win + w); missing segments are padding.
      struct Seg {
        int b, p0, p1;
      };
      std::vector<std::vector<Seg>> win;
      std::vector<int> nseg(B, 0);
      size_t b = 0;
      int64_t pos = 0;  // pages of request b already placed
      while (b < pages.size() && pages[b] == 0) ++b;
      while (b < pages.size()) {
        win.emplace_back();
        int64_t cost = 0;
        while (b < pages.size()) {
          const int64_t avail = lo - cost - kWindowItemCost;
          if (avail < 1) break;
          const int64_t take = std::min<int64_t>(avail, pages[b] - pos);
          win.back().push_back(Seg{(int)b, (int)pos, (int)(pos + take)});
          cost += kWindowItemCost + take;
          pos += take;
          if (pos == pages[b]) {
            ++b;
            pos = 0;
            while (b < pages.size() && pages[b] == 0) ++b;
          } else {
            break;
          }
        }
      }
      const int n_win = (int)win.size();
      const int grid = n_win * Hkv;
      size_t rounds = 0;
      for (const auto& w : win) rounds = std::max(rounds, w.size());
      std::vector<WorkItem> list(rounds * (size_t)grid, WorkItem{-1, 0, 0, 0});
      for (int w = 0; w < n_win; ++w)
        for (size_t r = 0; r < win[w].size(); ++r) {
          const Seg& sg = win[w][r];
          const int split = nseg[sg.b]++;
          for (int g = 0; g < Hkv; ++g)
            list[r * grid + (size_t)g * n_win + w] = WorkItem{sg.b, g | (split << 8), sg.p0, sg.p1};
        }
      int max_splits = 0;
      for (int bb = 0; bb < B; ++bb) {
        if (splits) splits[bb] = nseg[bb];
        max_splits = std::max(max_splits, nseg[bb]);
      }
      res->num_splits = max_splits;
      res->chunk_pages = (int)lo;
      res->n_items = (int)list.size();
      res->grid = grid;
      if (items) std::copy(list.begin(), list.begin() + std::min<int>(capacity, (int)list.size()), items);
      return 0;
    }
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
  res->grid = (int)list.size();
  if (items) {
    int n = std::min<int>(capacity, (int)list.size());
    std::copy(list.begin(), list.begin() + n, items);
  }
  return 0;
}

// Ragged prefill: one item per (request, tile of kPrefillRows new tokens).
// Every item runs on one workgroup per query head, all of equal cost, so the
// longest-first order over items is the longest-processing-time order over
// workgroups. An item's cost is its number of 64-key tiles: the last query
// row of tile qt is new token min(n, 256 (qt+1)) - 1 at position
// L - n + that index, and it sees every key up to its own position.
int plan_prefill_host(const int32_t* seqlens, const int32_t* cu_q, int B, int32_t* items,
                      int capacity) {
  if (!seqlens || !cu_q || B < 1 || cu_q[0] != 0) return -1;
  struct Item {
    int64_t cost;
    int32_t b, qt;
  };
  std::vector<Item> list;
  for (int b = 0; b < B; ++b) {
    const int64_t n = (int64_t)cu_q[b + 1] - cu_q[b];
    const int64_t L = seqlens[b];
    if (n < 0 || L < n) return -1;
    const int64_t ntiles = (n + kPrefillRows - 1) / kPrefillRows;
    if ((int64_t)list.size() + ntiles > (1 << 26)) return -1;
    for (int64_t qt = 0; qt < ntiles; ++qt) {
      const int64_t last = std::min(n, kPrefillRows * (qt + 1)) - 1;
      const int64_t keys = L - n + last + 1;
      list.push_back({(keys + kPage - 1) / kPage, b, (int32_t)qt});
    }
  }
  std::stable_sort(list.begin(), list.end(), [](const Item& x, const Item& y) { return x.cost > y.cost; });
  if (items) {
    const int n = std::min<int>(capacity, (int)list.size());
    for (int i = 0; i < n; ++i) {
      items[2 * i] = list[i].b;
      items[2 * i + 1] = list[i].qt;
    }
  }
  return (int)list.size();
}

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

WorkspaceLayout workspace_layout(int n_items, int B, int Hq, int D, int num_splits,
                                 int n_prefix_items, int n_group_reqs) {
  WorkspaceLayout w;
  w.items_off = 0;
  w.splits_off = align_up(w.items_off + sizeof(WorkItem) * (size_t)std::max(n_items, 1), 256);
  w.part_o_off = align_up(w.splits_off + sizeof(int32_t) * (size_t)B, 256);
  size_t rows = (size_t)B * Hq * (size_t)std::max(num_splits, 1);
  w.part_lse_off = align_up(w.part_o_off + sizeof(float) * rows * D, 256);
  w.prefix_items_off = align_up(w.part_lse_off + sizeof(float) * rows, 256);
  w.group_reqs_off = align_up(w.prefix_items_off + sizeof(PrefixItem) * (size_t)n_prefix_items, 256);
  w.total = align_up(w.group_reqs_off + sizeof(int32_t) * (size_t)n_group_reqs, 256);
  return w;
}

// Shared-prefix (cascade) decode plan.
//
// The prefix of a group is attended once for all of the group's decode
// queries: G query heads of each request fold into the rows of one dense
// tile per KV head (up to kPrefillRows rows per workgroup), and the prefix
// pages are cut into chunks so that there are about as many prefix
// workgroups as CUs (at least kMinPrefixChunk pages each, which keeps the
// per-workgroup start-up small next to its work). Each chunk is one partial
// slot of every request of the group. The suffixes (the tokens after the
// prefix) are planned like ordinary decode requests; their page ranges are
// shifted past the prefix and their slots past the prefix slots, so the LSE
// merge combines prefix and suffix partials of a request in one pass.
constexpr int kMinPrefixChunk = 4;

int plan_cascade_host(const int32_t* seqlens, int B, int stride, int Hq, int Hkv,
                      const int32_t* group, const int32_t* prefix_pages, int n_groups, int num_cus,
                      CascadePlan* out) {
  if (!seqlens || !group || B < 1 || stride < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 ||
      n_groups < 0 || (n_groups > 0 && !prefix_pages) || num_cus < 1 || !out)
    return -1;
  const int G = Hq / Hkv;
  std::vector<int32_t> pre_pages(B, 0), suffix(B, 0);
  std::vector<std::vector<int32_t>> members(n_groups);
  for (int b = 0; b < B; ++b) {
    const int j = group[b];
    if (j < -1 || j >= n_groups || seqlens[b] < 0) return -1;
    if (j >= 0) {
      if (prefix_pages[j] < 0 || prefix_pages[j] > stride) return -1;
      const int64_t pt = (int64_t)kPage * prefix_pages[j];
      if (seqlens[b] < pt) return -1;  // the prefix must lie inside the cache
      pre_pages[b] = prefix_pages[j];
      suffix[b] = (int32_t)(seqlens[b] - pt);
      members[j].push_back(b);
    } else {
      suffix[b] = seqlens[b];
    }
    if (((int64_t)seqlens[b] + kPage - 1) / kPage > stride) return -1;
  }
  // Prefix chunk size from the total prefix work (page x KV head x row block).
  int64_t work = 0;
  for (int j = 0; j < n_groups; ++j) {
    const int64_t rows = (int64_t)members[j].size() * G;
    work += (int64_t)prefix_pages[j] * Hkv * ((rows + kPrefillRows - 1) / kPrefillRows);
  }
  int chunk = (int)std::max<int64_t>(kMinPrefixChunk, (work + num_cus - 1) / std::max(num_cus, 1));
  out->prefix_chunk_pages = work > 0 ? chunk : 0;
  out->group_reqs.clear();
  out->prefix_items.clear();
  std::vector<int32_t> pre_slots(B, 0);
  for (int j = 0; j < n_groups; ++j) {
    const int req_off = (int)out->group_reqs.size();
    out->group_reqs.insert(out->group_reqs.end(), members[j].begin(), members[j].end());
    const int np = prefix_pages[j];
    const int rows = (int)members[j].size() * G;
    if (np == 0 || rows == 0) continue;
    const int nc = (np + chunk - 1) / chunk;
    for (int b : members[j]) pre_slots[b] = nc;
    for (int r0 = 0; r0 < rows; r0 += kPrefillRows)
      for (int c = 0; c < nc; ++c)
        for (int g = 0; g < Hkv; ++g)
          out->prefix_items.push_back(PrefixItem{req_off, g, r0, std::min(kPrefillRows, rows - r0),
                                                 (int)((int64_t)np * c / nc), (int)((int64_t)np * (c + 1) / nc),
                                                 c, members[j][0]});
  }
  std::stable_sort(out->prefix_items.begin(), out->prefix_items.end(), [](const PrefixItem& x, const PrefixItem& y) {
    return (int64_t)(x.page_end - x.page_begin) * x.nrows > (int64_t)(y.page_end - y.page_begin) * y.nrows;
  });
  // Suffixes: an ordinary decode plan on the suffix lengths, then shifted.
  PlanResult r;
  if (plan_decode_host(suffix.data(), B, stride, Hkv, 0, num_cus, nullptr, 0, nullptr, &r, false) != 0) return -1;
  out->items.assign(std::max(r.n_items, 1), WorkItem{});
  out->splits.assign(B, 0);
  plan_decode_host(suffix.data(), B, stride, Hkv, 0, num_cus, out->items.data(), r.n_items, out->splits.data(), &r,
                   false);
  out->items.resize(r.n_items);
  for (WorkItem& it : out->items) {
    const int b = it.b;
    const int g = it.g_split & 255, s = it.g_split >> 8;
    it.page_begin += pre_pages[b];
    it.page_end += pre_pages[b];
    it.g_split = g | ((s + pre_slots[b]) << 8);
  }
  out->num_splits = 0;
  for (int b = 0; b < B; ++b) {
    out->splits[b] += pre_slots[b];
    out->num_splits = std::max(out->num_splits, (int)out->splits[b]);
  }
  return 0;
}

}  // namespace fa
