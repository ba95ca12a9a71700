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
// contiguous 256-byte run.
#include "fa_internal.h"
#include "hip_common.h"

namespace fa {

namespace {

constexpr int kUnitsPerRow = 128 * 2 / 16;  // 16-byte units in one bf16 row of D = 128

__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t units_per_tok = (int64_t)a.Hkv * kUnitsPerRow;
  if (u >= (int64_t)a.T * units_per_tok) return;
  const int tk = (int)(u / units_per_tok);
  const int rem = (int)(u % units_per_tok);
  const int g = rem / kUnitsPerRow, c = rem % kUnitsPerRow;

  // Request of packed token tk: the last b with cu[b] <= tk (empty requests
  // share their offset with the next one and are skipped by "last").
  int lo = 0, hi = a.B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.cu_q[mid] <= tk) lo = mid;
    else hi = mid;
  }
  const int b = lo;
  const int c0 = a.cu_q[b], n = a.cu_q[b + 1] - c0;
  const int i = tk - c0;
  if (i < 0 || i >= n) return;
  const int pos = a.seqlens[b] - n + i;
  if (pos < 0) return;
  const int pg = pos / kPage;
  if (pg >= a.stride) return;
  const int pid = a.page_table[(size_t)b * a.stride + pg];
  if ((unsigned)pid >= (unsigned)a.num_pages) return;

  const size_t src = ((size_t)tk * a.Hkv + g) * kUnitsPerRow + c;
  const size_t dst = (((size_t)pid * a.Hkv + g) * kPage + pos % kPage) * kUnitsPerRow + c;
  const u32x4_t kv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(a.k_new) + src);
  const u32x4_t vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(a.v_new) + src);
  reinterpret_cast<u32x4_t*>(a.k_pages)[dst] = kv;
  reinterpret_cast<u32x4_t*>(a.v_pages)[dst] = vv;
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t s) {
  const int64_t units = (int64_t)a.T * a.Hkv * kUnitsPerRow;
  if (units == 0) return hipSuccess;
  const int64_t blocks = (units + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace fa
