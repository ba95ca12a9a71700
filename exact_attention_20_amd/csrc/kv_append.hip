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
// once and written once. One wavefront moves one new token: its lanes take
// the token's Hkv 256-byte rows in 16-byte units (consecutive lanes,
// consecutive units: reads and the page-row writes are contiguous runs).
// The token's request, position and page are the same for every lane, so
// they are found with scalar loads (binary search over cu_seqlens_q, then
// one page-table entry) while the lanes' data loads are in flight.
#include "fa_internal.h"
#include "hip_common.h"

namespace fa {

namespace {

constexpr int kUnitsPerRow = 128 * 2 / 16;  // 16-byte units in one bf16 row of D = 128
typedef __attribute__((address_space(4))) const int32_t cint;

// P: 16-byte units per lane at a time (the token's Hkv * 16 units go over
// the 64 lanes in chunks of 64 * P). The first chunk's loads are issued
// before the lookup; with more than one chunk the rest follow it.
template <int P>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int tk = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (tk >= a.T) return;
  const int units = a.Hkv * kUnitsPerRow;
  const size_t src0 = (size_t)tk * units;
  u32x4_t kv[P], vv[P];
  auto load = [&](int base) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int u = base + lane + 64 * p;
      if (u < units) {
        kv[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(a.k_new) + src0 + u);
        vv[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(a.v_new) + src0 + u);
      }
    }
  };
  load(0);
  // Request of packed token tk: the last b with cu[b] <= tk (empty requests
  // share their offset with the next one and are skipped by "last").
  const cint* cu = (const cint*)a.cu_q;
  int lo = 0, hi = a.B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= tk) lo = mid;
    else hi = mid;
  }
  const int b = lo;
  const int c0 = cu[b], n = cu[b + 1] - c0;
  const int i = tk - c0;
  if (i < 0 || i >= n) return;
  const int pos = ((const cint*)a.seqlens)[b] - n + i;
  if (pos < 0) {  // more new tokens than the request's length: not written, reported
    if (lane == 0) report_status(a.status, kStatusBadPosition);
    return;
  }
  const int pg = pos / kPage;
  // Tokens past their page-table row, or whose page id lies outside the
  // pool, are not written; either is reported in the device status word.
  if (pg >= a.stride) {
    if (lane == 0) report_status(a.status, kStatusBadPosition);
    return;
  }
  const int pid = ((const cint*)a.page_table)[(size_t)b * a.stride + pg];
  if ((unsigned)pid >= (unsigned)a.num_pages) {
    if (lane == 0) report_status(a.status, kStatusBadPage);
    return;
  }
  const int slot = pos % kPage;
  for (int base = 0; base < units; base += 64 * P) {
    if (base > 0) load(base);
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int u = base + lane + 64 * p;
      if (u < units) {
        const int g = u / kUnitsPerRow, c = u % kUnitsPerRow;
        const size_t dst = (((size_t)pid * a.Hkv + g) * kPage + slot) * kUnitsPerRow + c;
        reinterpret_cast<u32x4_t*>(a.k_pages)[dst] = kv[p];
        reinterpret_cast<u32x4_t*>(a.v_pages)[dst] = vv[p];
      }
    }
  }
}

template <int P>
hipError_t launch_p(const AppendArgs& a, hipStream_t s) {
  const int64_t blocks = ((int64_t)a.T + 3) / 4;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kv_append_kernel<P>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t s) {
  if ((int64_t)a.T * a.Hkv == 0) return hipSuccess;
  const int per = (a.Hkv * kUnitsPerRow + 63) / 64;
  if (per <= 1) return launch_p<1>(a, s);
  if (per <= 2) return launch_p<2>(a, s);
  return launch_p<4>(a, s);
}

}  // namespace fa
