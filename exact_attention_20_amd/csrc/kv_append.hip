// Append of the new tokens' K/V to their requests' paged caches.
//
// "Flash Attention & Paged Attention" blog, "FA and the prefill phase": the
// prefill leaves the K and V it computed in device memory as the KV cache
// that decode reuses; "2. PagedAttention": that cache is kept in fixed-size
// pages reached through a per-request page table. New token i of request b
// (n_b new tokens, L_b tokens in total) is logical position
// t = L_b - n_b + i, stored in slot t % 64 of page page_table[b][t / 64].
//
// Pure data movement, bound by HBM: every byte of K_new and V_new is read
// once and written once. One thread moves one 16-byte unit of K and the
// matching unit of V; the 16 threads of a (token, KV head) cover its 256-byte
// row, so reads are fully coalesced and each page row is written as one
// contiguous 256-byte run. The source unit is the thread's index, so its
// loads are issued before the destination lookup. For batches of up to
// kStagedReqs requests each workgroup stages cu_seqlens_q and the lengths in
// LDS with one coalesced read and searches there, so a thread waits for two
// memory round trips (metadata with its data, then its page id) instead of
// one per step of the search.
#include "fa_internal.h"
#include "hip_common.h"

namespace fa {

namespace {

constexpr int kUnitsPerRow = 128 * 2 / 16;  // 16-byte units in one bf16 row of D = 128
constexpr int kStagedReqs = 1024;           // largest batch whose metadata is staged in LDS

template <bool STAGED>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  __shared__ int s_cu[STAGED ? kStagedReqs + 1 : 1];
  __shared__ int s_len[STAGED ? kStagedReqs + 1 : 1];  // entry B repeats entry B - 1
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t units_per_tok = (int64_t)a.Hkv * kUnitsPerRow;
  const bool live = u < (int64_t)a.T * units_per_tok;
  // Source unit u is ((tk * Hkv + g) * 16 + c) of the packed [T, Hkv, D] rows.
  u32x4_t kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
  if (live) {
    kv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(a.k_new) + u);
    vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(a.v_new) + u);
  }
  if constexpr (STAGED) {
    for (int i = threadIdx.x; i <= a.B; i += 256) {
      const int x = a.cu_q[i], y = a.seqlens[min(i, a.B - 1)];  // both loads in flight together
      s_cu[i] = x;
      s_len[i] = y;
    }
    __syncthreads();
  }
  if (!live) return;
  const int tk = (int)(u / units_per_tok);
  const int rem = (int)(u % units_per_tok);
  const int g = rem / kUnitsPerRow, c = rem % kUnitsPerRow;
  auto cu = [&](int i) { return STAGED ? s_cu[i] : a.cu_q[i]; };

  // Request of packed token tk: the last b with cu[b] <= tk (empty requests
  // share their offset with the next one and are skipped by "last").
  int lo = 0, hi = a.B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu(mid) <= tk) lo = mid;
    else hi = mid;
  }
  const int b = lo;
  const int c0 = cu(b), n = cu(b + 1) - c0;
  const int i = tk - c0;
  if (i < 0 || i >= n) return;
  const int pos = (STAGED ? s_len[b] : a.seqlens[b]) - n + i;
  if (pos < 0) return;
  const int pg = pos / kPage;
  if (pg >= a.stride) return;
  const int pid = a.page_table[(size_t)b * a.stride + pg];
  if ((unsigned)pid >= (unsigned)a.num_pages) return;

  const size_t dst = (((size_t)pid * a.Hkv + g) * kPage + pos % kPage) * kUnitsPerRow + c;
  reinterpret_cast<u32x4_t*>(a.k_pages)[dst] = kv;
  reinterpret_cast<u32x4_t*>(a.v_pages)[dst] = vv;
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t s) {
  const int64_t units = (int64_t)a.T * a.Hkv * kUnitsPerRow;
  if (units == 0) return hipSuccess;
  const int64_t blocks = (units + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.B <= kStagedReqs)
    hipLaunchKernelGGL(kv_append_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(kv_append_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace fa
