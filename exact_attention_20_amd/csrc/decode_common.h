// Device code shared by the split-KV decode kernels: the end of a work item,
// where the four wavefronts' partial softmax states are combined and the
// splits of a request are merged by their LogSumExp.
//
// Flash-Decoding ("Flash Attention & Paged Attention" blog, "FA and the
// decode phase"): each split of the KV sequence yields a partial output and
// its LogSumExp; a light reduction combines them into the exact result:
//   L* = M + ln sum_s exp(lse_s - M),   O = sum_s exp(lse_s - L*) O_s,
// with M the largest partial LSE (the LSE merge kernel). A request with a
// single split needs no reduction: its work item writes the result itself.
#pragma once

#include "fa_internal.h"
#include "hip_common.h"

namespace fa {

constexpr int kDecD = 128;

// Finishes work item (b, KV head g, split) whose four wavefronts left their
// state for the G query heads in LDS (log2 units):
//   s_m[16 w + h], s_l[16 w + h]   running max and normaliser of wavefront w,
//   s_o[(w G + h) kDecD + d]       its unnormalised output.
// Writes the request's output and LSE when it has a single split, else this
// split's normalised partial output and LSE for the merge. Must be called by
// all 256 threads after a barrier that publishes the LDS.
template <int G>
__device__ __forceinline__ void finish_work_item(const DecodeArgs& a, int b, int g, int split, const float* s_m,
                                                 const float* s_l, const float* s_o) {
  const int ns = a.splits_per_req[b];
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  for (int idx = threadIdx.x; idx < G * kDecD; idx += 256) {
    const int h = idx / kDecD, d = idx % kDecD;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[16 * w + h]);
    float Lsum = 0.f, o = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = fast_exp2(s_m[16 * w + h] - M);
        Lsum += s_l[16 * w + h] * f;
        o += s_o[(w * G + h) * kDecD + d] * f;
      }
    }
    const float val = Lsum > 0.f ? o / Lsum : 0.f;
    const float lse = Lsum > 0.f ? (M + __log2f(Lsum)) * kLn2 : kNegInf;
    const size_t row = (size_t)b * a.Hq + g * G + h;
    if (ns == 1) {
      out[row * kDecD + d] = __builtin_bit_cast(uint16_t, (__bf16)val);
      if (d == 0) a.lse[row] = lse;
    } else {
      const size_t slot = row * a.num_splits + split;
      a.part_o[slot * kDecD + d] = val;
      if (d == 0) a.part_lse[slot] = lse;
    }
  }
}

}  // namespace fa
