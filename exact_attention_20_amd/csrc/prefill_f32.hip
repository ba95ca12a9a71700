// fp32 exact-attention prefill (VALU). The small fp32 workload's path: four
// lanes per query row, each holding a quarter of the row's dims (dims
// part + 4i), K/V tiles of 32 keys staged in LDS and read as broadcasts,
// online softmax per row in fp32 with the natural exponential.
//
// The loop is the one in "FasterTransformer vs FlashAttention", section 3:
// load the Q block once, stream K/V blocks, update the running max and
// normaliser, accumulate the output, write it once at the end.
#include <cmath>

#include "fa_internal.h"
#include "hip_common.h"

namespace fa {

namespace {

constexpr int kRows = 64;  // query rows per workgroup
constexpr int kLanes = 4;  // lanes per row; lane `part` holds dims part + 4i
constexpr int kKeys = 32;  // keys per LDS tile

template <int D>
__global__ __launch_bounds__(kRows * kLanes) void prefill_f32_kernel(PrefillArgs a) {
  constexpr int DL = D / kLanes;  // dims per lane
  // Row j of a tile is read by all rows at once: the four lanes of a row read
  // four consecutive words (distinct banks), and lanes of equal part the same
  // word (a broadcast).
  __shared__ float ks[kKeys][D];
  __shared__ float vs[kKeys][D];
  const int b = blockIdx.z, h = blockIdx.y;
  const int g = a.has_map ? a.kv_map[h] : h / (a.Hq / a.Hkv);
  const int r0 = blockIdx.x * kRows;
  const int part = threadIdx.x % kLanes;
  const int row = r0 + threadIdx.x / kLanes;
  const int off = a.Sk - a.Sq;  // causal diagonal offset (bottom-right alignment)
  const float* Q = reinterpret_cast<const float*>(a.q) + ((size_t)b * a.Hq + h) * a.Sq * D;
  const float* K = reinterpret_cast<const float*>(a.k) + ((size_t)b * a.Hkv + g) * a.Sk * D;
  const float* V = reinterpret_cast<const float*>(a.v) + ((size_t)b * a.Hkv + g) * a.Sk * D;

  float q[DL], acc[DL];
  const bool live = row < a.Sq;
#pragma unroll
  for (int i = 0; i < DL; ++i) {
    q[i] = live ? Q[(size_t)row * D + part + kLanes * i] : 0.f;
    acc[i] = 0.f;
  }
  float m = kNegInf, l = 0.f;
  // Keys any row of this block can see.
  int kend = a.Sk;
  if (a.causal) kend = min(a.Sk, r0 + kRows - 1 + off + 1);
  for (int k0 = 0; k0 < kend; k0 += kKeys) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < kKeys * D; idx += kRows * kLanes) {
      const int j = idx / D, d = idx % D;
      const bool in = k0 + j < a.Sk;
      ks[j][d] = in ? K[(size_t)(k0 + j) * D + d] : 0.f;
      vs[j][d] = in ? V[(size_t)(k0 + j) * D + d] : 0.f;
    }
    __syncthreads();
    // Keys of the tile in chunks of 8: scores (a quarter of each dot product
    // per lane, summed over the row's four lanes), then one online-softmax
    // step, which the four lanes take alike.
#pragma unroll 1
    for (int j0 = 0; j0 < kKeys; j0 += 8) {
      float s[8];
      float tmax = kNegInf;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < DL; ++i) dot = fmaf(q[i], ks[j0 + j][part + kLanes * i], dot);
        dot += __shfl_xor(dot, 1);
        dot += __shfl_xor(dot, 2);
        const int key = k0 + j0 + j;
        const bool vis = key < a.Sk && (!a.causal || key <= row + off);
        s[j] = vis ? dot * a.scale : kNegInf;
        tmax = fmaxf(tmax, s[j]);
      }
      const float mn = fmaxf(m, tmax);
      if (mn == kNegInf) continue;  // nothing visible yet for this row
      const float alpha = expf(m - mn);
      l *= alpha;
#pragma unroll
      for (int i = 0; i < DL; ++i) acc[i] *= alpha;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = expf(s[j] - mn);
        l += p;
#pragma unroll
        for (int i = 0; i < DL; ++i) acc[i] = fmaf(p, vs[j0 + j][part + kLanes * i], acc[i]);
      }
      m = mn;
    }
  }
  if (!live) return;
  float* O = reinterpret_cast<float*>(a.out) + ((size_t)b * a.Hq + h) * a.Sq * D + (size_t)row * D;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int i = 0; i < DL; ++i) O[part + kLanes * i] = acc[i] * inv;
  if (part == 0) a.lse[((size_t)b * a.Hq + h) * a.Sq + row] = l > 0.f ? m + logf(l) : kNegInf;
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s) {
  dim3 grid((a.Sq + kRows - 1) / kRows, a.Hq, a.B);
  if (a.D == 64)
    hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, dim3(kRows * kLanes), 0, s, a);
  else
    hipLaunchKernelGGL(prefill_f32_kernel<128>, grid, dim3(kRows * kLanes), 0, s, a);
  return hipGetLastError();
}

}  // namespace fa
