// Internal declarations shared by the host ABI (abi.cpp) and the kernel
// launchers (*.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

namespace fa {

constexpr int kPage = 64;         // tokens per KV page
constexpr int kMaxHeads = 256;    // limit on Hq and Hkv (head map travels in kernel args)

// ---------------------------------------------------------------- prefill
struct PrefillArgs {
  const void* q;
  const void* k;      // contiguous [B, Hkv, Sk, D], or the K page pool (ragged)
  const void* v;
  void* out;
  float* lse;
  int B, Hq, Hkv, Sq, Sk, D;
  int causal;
  float scale;        // score multiplier (already defaulted)
  int has_map;        // 0: contiguous groups h / (Hq/Hkv)
  // Ragged paged prefill only (the per-request Sq, Sk come from cu_q, seqlens):
  const int32_t* items;       // [n_items][2] (request, query tile), heaviest first
  const int32_t* page_table;  // [B, stride]
  const int32_t* seqlens;     // [B]
  const int32_t* cu_q;        // [B + 1]
  int stride;
  int num_pages;
  // Shared-prefix pass only: folded (request, head) rows, partial results.
  const int32_t* group_reqs;  // requests of every group, concatenated
  const int32_t* splits;      // [B] partial slots per request
  float* part_o;              // [B, Hq, num_splits, D]
  float* part_lse;            // [B, Hq, num_splits]
  int num_splits;
  unsigned* status;           // device status word (paged modes report bad page ids)
  uint8_t kv_map[kMaxHeads];
};

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s);

hipError_t launch_prefill_fp8(const void* q, const void* k, const void* v, const float* q_scale,
                              const float* k_scale, const float* v_scale, void* out, float* lse, int B,
                              int Hq, int Hkv, int Sq, int Sk, int causal, float scale, hipStream_t s);

// Attention backward (bf16, D = 128): delta, dQ and dK/dV kernels.
struct BwdLaunch {
  const void *q, *k, *v, *o, *dO;
  const float* lse;
  float* delta;   // [B, Hq, Sq] workspace
  float* lse2;    // [B, Hq, Sq] workspace: LSE in log2 units, +inf for a row without keys
  void *dq, *dk, *dv;
  int B, Hq, Hkv, Sq, Sk, causal;
  float scale;
};
hipError_t launch_attention_bwd(const BwdLaunch& l, hipStream_t s);

// Static device scratch that stands in for the backward's workspace in the
// entry point for callers that cannot allocate: its size, and its address
// on the current device (looked up once per device).
constexpr size_t kBwdScratchBytes = size_t(32) << 20;
hipError_t bwd_scratch(void** ptr);

// ---------------------------------------------------------------- device status
// One word per device that kernels OR bits into when they meet bad device
// metadata and skip it (status.hip). The bits are those of fa.h's
// fa_device_status.
constexpr unsigned kStatusBadPage = 1u;      // a page-table entry outside [0, num_pages)
constexpr unsigned kStatusBadPosition = 2u;  // an appended token past its page-table row
// Device address of the current device's status word.
hipError_t device_status_ptr(unsigned** ptr);

// Query rows per work item of the bf16 prefill kernel (ragged plan unit).
constexpr int kPrefillRows = 256;
hipError_t launch_prefill_paged_bf16(const PrefillArgs& a, int n_items, hipStream_t s);

// One workgroup of the shared-prefix pass: the decode queries of the
// requests group_reqs[req_off + r / G] (query heads g*G + r % G), rows
// row0 .. row0 + nrows - 1 of that folding, against prefix pages
// [page_begin, page_end) of first_req's page-table row; the result goes to
// partial slot `slot` of each of those (request, head) pairs.
struct PrefixItem {
  int32_t req_off;
  int32_t g;
  int32_t row0;
  int32_t nrows;
  int32_t page_begin;
  int32_t page_end;
  int32_t slot;
  int32_t first_req;
};
static_assert(sizeof(PrefixItem) == 32, "PrefixItem is exported as 8 int32");
hipError_t launch_prefix_bf16(const PrefillArgs& a, int n_items, hipStream_t s);

struct AppendArgs {
  const void* k_new;          // [T, Hkv, D] bf16
  const void* v_new;
  void* k_pages;              // [P, Hkv, 64, D] bf16
  void* v_pages;
  const int32_t* page_table;  // [B, stride]
  const int32_t* seqlens;     // [B]
  const int32_t* cu_q;        // [B + 1]
  int B, T, stride, num_pages, Hkv, D;
  unsigned* status;           // device status word
};
hipError_t launch_kv_append(const AppendArgs& a, hipStream_t s);

// ---------------------------------------------------------------- decode
// One work item of the split-KV decode: pages [page_begin, page_end) of
// request b, KV head g, partial-result slot `split`.
struct WorkItem {
  int32_t b;
  int32_t g_split;   // g | (split << 8)
  int32_t page_begin;
  int32_t page_end;
};

struct DecodeArgs {
  const WorkItem* items;
  int n_items;
  int grid;                       // workgroups; workgroup w runs items w, w + grid, ... (b < 0: padding)
  const int32_t* splits_per_req;  // [B]
  const void* q;                  // [B, Hq, D] bf16
  const void* k_pages;            // [P, Hkv, 64, D]
  const void* v_pages;
  const float* k_scale;           // [P, Hkv] (fp8)
  const float* v_scale;
  const int32_t* page_table;      // [B, stride]
  const int32_t* seqlens;         // [B]
  int stride;                     // page-table row stride
  int num_pages;
  int B, Hq, Hkv, D;
  int num_splits;                 // partial-buffer stride
  float scale;
  float* part_o;                  // [B, Hq, num_splits, D]
  float* part_lse;                // [B, Hq, num_splits]
  void* out;                      // [B, Hq, D] bf16
  float* lse;                     // [B, Hq]
  unsigned* status;               // device status word
};

hipError_t launch_decode_split(const DecodeArgs& a, int group, int fp8, hipStream_t s);
// Split kernel on MFMA for groups of 4, 8 or 16 query heads per KV head.
hipError_t launch_decode_split_mfma(const DecodeArgs& a, int group, int fp8, hipStream_t s);
hipError_t launch_lse_merge(const DecodeArgs& a, hipStream_t s);
hipError_t launch_gather_kv(const void* pages, int elem_bytes, const int32_t* page_table,
                            int stride, int num_pages, int Hkv, int D, int b, int L, int g,
                            void* dst, hipStream_t s);

// ---------------------------------------------------------------- plan (pure host)
struct PlanResult {
  int num_splits = 0;   // max split count over requests
  int chunk_pages = 0;  // target pages per work item (auto mode)
  int n_items = 0;      // including padding items (b = -1)
  int grid = 0;         // workgroups to launch (each runs items w, w + grid, ...)
};

// Returns 0 or a negative fa_status. `items` (capacity entries) and
// `splits` (B entries) may be null to only count. With `windows` (auto mode
// only) the plan may instead cut every KV head's pages into cost-balanced
// windows, one per workgroup of a single round.
int plan_decode_host(const int32_t* seqlens, int B, int stride, int Hkv, int num_splits_request,
                     int num_cus, WorkItem* items, int capacity, int32_t* splits,
                     PlanResult* res, bool windows = true);

// Ragged prefill work list: (request, query tile) pairs of kPrefillRows new
// tokens, sorted by decreasing key count. Returns the item count, or a
// negative fa_status for inconsistent lengths. `items` may be null.
int plan_prefill_host(const int32_t* seqlens, const int32_t* cu_q, int B, int32_t* items,
                      int capacity);

// Shared-prefix (cascade) decode plan: prefix-pass items, the suffix
// split-KV items (page ranges after the prefix, slots after the prefix
// slots), per-request slot counts and the concatenated group members.
struct CascadePlan {
  std::vector<WorkItem> items;
  std::vector<PrefixItem> prefix_items;
  std::vector<int32_t> splits;      // [B]
  std::vector<int32_t> group_reqs;  // requests of group 0, then group 1, ...
  int num_splits = 0;
  int prefix_chunk_pages = 0;
};
// Returns 0 or -1 (invalid lengths or groups). Validation of the page table
// (shared prefix pages) is the caller's.
int plan_cascade_host(const int32_t* seqlens, int B, int stride, int Hq, int Hkv,
                      const int32_t* group, const int32_t* prefix_pages, int n_groups, int num_cus,
                      CascadePlan* out);

// Workspace layout for a plan: work items, per-request split counts,
// partials, and (cascade plans) prefix items and group members.
struct WorkspaceLayout {
  size_t items_off, splits_off, part_o_off, part_lse_off, prefix_items_off, group_reqs_off, total;
};
WorkspaceLayout workspace_layout(int n_items, int B, int Hq, int D, int num_splits,
                                 int n_prefix_items = 0, int n_group_reqs = 0);

}  // namespace fa
