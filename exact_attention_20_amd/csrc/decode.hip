// Paged Flash-Decoding on gfx950: split-KV kernel, LSE merge kernel, and a
// debug gather through the page table.
//
// Method ("Flash Attention & Paged Attention" blog, "FA and the decode
// phase"): the single query row cannot be split, so the KV sequence is; each
// split produces a partial output and its LogSumExp, and a light second
// kernel reduces the splits into the exact result. The KV cache is paged
// ("2. PagedAttention": fixed-size pages, logical page table onto
// non-contiguous physical pages; 64-token pages per the "FlashAttention
// breakthrough architecture" article).
//
// gfx950 design: decode is an HBM stream (each cached byte is used once per
// query group), so there is no MFMA here. A workgroup of 4 wavefronts owns
// one work item (request b, KV head g, a range of pages). Each 64-token page
// of one KV head is a contiguous [64, 128] block; wavefront w takes tokens
// 16w..16w+15 of every page of the item, 16 lanes per token (one 16-byte
// bf16 load per lane per token), so every load instruction reads 1 KB of
// contiguous memory. Scores for the G query heads that share the KV head use
// v_dot2_f32_bf16 on the bf16 pairs as loaded (no unpacking), are summed over
// the 16 lanes of a DPP row, and the P*V update uses the same dot2
// instruction over token pairs (p packed to bf16, V repacked by byte
// permutes). The running max is wave-uniform and only moves when a score
// exceeds it by more than kTau (log2 units): the result stays exact, the
// O/l rescale disappears from the steady state. fp8 (OCP e4m3fn) pages are
// converted to bf16 pairs with the gfx950 scaled convert (exact), the K scale
// is folded into the score multiplier and the V scale into p.
#include "fa_internal.h"
#include "hip_common.h"

namespace fa {

namespace {

constexpr int kD = 128;
constexpr float kTau = 8.0f;  // lazy max threshold, log2 units (p <= 2^kTau)

template <bool FP8>
struct KvSlot;
template <>
struct KvSlot<false> {  // 8 bf16 (dims 8*dc .. 8*dc+7)
  uint4 v;
};
template <>
struct KvSlot<true> {  // 8 fp8 codes
  uint2 v;
};

template <bool FP8>
__device__ __forceinline__ void load_slot(KvSlot<FP8>& s, const char* base, size_t off_elems) {
  if constexpr (FP8) {
    s.v = *reinterpret_cast<const uint2*>(base + off_elems);
  } else {
    s.v = *reinterpret_cast<const uint4*>(base + 2 * off_elems);
  }
}

template <bool FP8>
__device__ __forceinline__ void zero_slot(KvSlot<FP8>& s) {
  if constexpr (FP8) {
    s.v = make_uint2(0, 0);
  } else {
    s.v = make_uint4(0, 0, 0, 0);
  }
}

// The 8 elements of a slot as 4 bf16 pairs (dims 2j, 2j+1).
template <bool FP8>
__device__ __forceinline__ void slot_pairs(const KvSlot<FP8>& s, uint32_t out[4]) {
  if constexpr (FP8) {
    out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(s.v.x, 1.0f, false));
    out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(s.v.x, 1.0f, true));
    out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(s.v.y, 1.0f, false));
    out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(s.v.y, 1.0f, true));
  } else {
    out[0] = s.v.x;
    out[1] = s.v.y;
    out[2] = s.v.z;
    out[3] = s.v.w;
  }
}

// Token-pair repacking for P*V: from the slots of tokens t0 and t1, the bf16
// pairs (v_t0[d], v_t1[d]) for the slot's 8 dims d, in dim order.
template <bool FP8>
__device__ __forceinline__ void token_pairs(const KvSlot<FP8>& a, const KvSlot<FP8>& b,
                                            uint32_t out[8]) {
  if constexpr (FP8) {
    // bytes (a0,b0,a1,b1) and (a2,b2,a3,b3), then fp8 pairs -> bf16 pairs
    uint32_t lo0 = perm_b32(b.v.x, a.v.x, 0x05010400u);
    uint32_t hi0 = perm_b32(b.v.x, a.v.x, 0x07030602u);
    uint32_t lo1 = perm_b32(b.v.y, a.v.y, 0x05010400u);
    uint32_t hi1 = perm_b32(b.v.y, a.v.y, 0x07030602u);
    out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo0, 1.0f, false));
    out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo0, 1.0f, true));
    out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi0, 1.0f, false));
    out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi0, 1.0f, true));
    out[4] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo1, 1.0f, false));
    out[5] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo1, 1.0f, true));
    out[6] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi1, 1.0f, false));
    out[7] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi1, 1.0f, true));
  } else {
    const uint32_t av[4] = {a.v.x, a.v.y, a.v.z, a.v.w};
    const uint32_t bv[4] = {b.v.x, b.v.y, b.v.z, b.v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      out[2 * j] = perm_b32(bv[j], av[j], 0x05040100u);      // low halves
      out[2 * j + 1] = perm_b32(bv[j], av[j], 0x07060302u);  // high halves
    }
  }
}

template <int G, bool FP8>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  constexpr int kElem = FP8 ? 1 : 2;
  const WorkItem it = a.items[blockIdx.x];
  const int b = it.b;
  const int g = it.g_split & 255;
  const int split = it.g_split >> 8;
  const int p0 = it.page_begin, p1 = it.page_end;
  const int L = a.seqlens[b];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int row = lane >> 4, dc = lane & 15;

  // Query rows of the G heads of this KV group: 8 bf16 (4 pairs) per lane.
  uint32_t qd[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 v = *reinterpret_cast<const uint4*>(
        reinterpret_cast<const uint16_t*>(a.q) + ((size_t)b * a.Hq + g * G + h) * kD + dc * 8);
    qd[h][0] = v.x; qd[h][1] = v.y; qd[h][2] = v.z; qd[h][3] = v.w;
  }
  const float c_base = a.scale * kLog2e;

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[h][j] = 0.f;
  }

  const size_t page_elems = (size_t)64 * kD;            // one (page, head) block
  const size_t head_stride = page_elems;                // between heads of a page
  const size_t pid_stride = (size_t)a.Hkv * page_elems; // between pages
  const char* kpool = reinterpret_cast<const char*>(a.k_pages);
  const char* vpool = reinterpret_cast<const char*>(a.v_pages);
  const int32_t* table = a.page_table + (size_t)b * a.stride;
  // Element offset of this lane's slot i inside a (page, head) block.
  const int lane_off = (wave * 16 + row) * kD + dc * 8;

  auto page_base = [&](int pid) -> size_t { return (size_t)pid * pid_stride + (size_t)g * head_stride; };

  KvSlot<FP8> kc[4], vc[4];
  int pid_c = 0;
  {
    int pid = table[p0];
    pid_c = pid;
    const size_t base = page_base(((unsigned)pid < (unsigned)a.num_pages) ? pid : 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      load_slot<FP8>(kc[i], kpool, base + lane_off + i * 4 * kD);
      load_slot<FP8>(vc[i], vpool, base + lane_off + i * 4 * kD);
    }
  }

  for (int p = p0; p < p1; ++p) {
    KvSlot<FP8> kn[4], vn[4];
    int pid_n = 0;
    if (p + 1 < p1) {
      pid_n = table[p + 1];
      const size_t base = page_base(((unsigned)pid_n < (unsigned)a.num_pages) ? pid_n : 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        load_slot<FP8>(kn[i], kpool, base + lane_off + i * 4 * kD);
        load_slot<FP8>(vn[i], vpool, base + lane_off + i * 4 * kD);
      }
    }

    // Tokens of this page that belong to the request (all 64 except on the
    // last page); an out-of-range page id contributes nothing.
    int nvalid = min(64, L - p * 64);
    if ((unsigned)pid_c >= (unsigned)a.num_pages) nvalid = 0;
    float c = c_base;
    float vsc = 1.f;
    if constexpr (FP8) {
      if (nvalid > 0) {
        c = c_base * a.k_scale[(size_t)pid_c * a.Hkv + g];
        vsc = a.v_scale[(size_t)pid_c * a.Hkv + g];
      }
    }
    const bool partial = nvalid < 64;
    bool tok_ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tok_ok[i] = (wave * 16 + 4 * i + row) < nvalid;
      if (partial && !tok_ok[i]) {  // tail slots may hold anything (NaN): never use them
        zero_slot<FP8>(kc[i]);
        zero_slot<FP8>(vc[i]);
      }
    }

    // Scores s[i][h] (log2 units) for this lane's 4 tokens.
    float s[4][G];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t kp[4];
      slot_pairs<FP8>(kc[i], kp);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = dot2_bf16(qd[h][0], kp[0], 0.f);
        d = dot2_bf16(qd[h][1], kp[1], d);
        d = dot2_bf16(qd[h][2], kp[2], d);
        d = dot2_bf16(qd[h][3], kp[3], d);
        s[i][h] = d;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = row16_sum(s[i][h]) * c;
        s[i][h] = tok_ok[i] ? d : kNegInf;
      }

    // Lazy running max: move it only when some score exceeds it by > kTau.
    bool need = false;
    float smax[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      smax[h] = fmaxf(fmaxf(s[0][h], s[1][h]), fmaxf(s[2][h], s[3][h]));
      need |= smax[h] > m[h] + kTau;
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float x = fmaxf(smax[h], shfl_xor_f32(smax[h], 16));
        x = fmaxf(x, shfl_xor_f32(x, 32));
        const float mn = fmaxf(m[h], x);
        const float alpha = (mn == kNegInf) ? 1.f : fast_exp2(m[h] - mn);
        l[h] *= alpha;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] *= alpha;
        m[h] = mn;
      }
    }

    uint32_t pp01[G], pp23[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mu = (m[h] == kNegInf) ? 0.f : m[h];
      const float e0 = fast_exp2(s[0][h] - mu), e1 = fast_exp2(s[1][h] - mu);
      const float e2 = fast_exp2(s[2][h] - mu), e3 = fast_exp2(s[3][h] - mu);
      l[h] += (e0 + e1) + (e2 + e3);
      pp01[h] = pack_bf16x2(e0 * vsc, e1 * vsc);
      pp23[h] = pack_bf16x2(e2 * vsc, e3 * vsc);
    }

    uint32_t v01[8], v23[8];
    token_pairs<FP8>(vc[0], vc[1], v01);
    token_pairs<FP8>(vc[2], vc[3], v23);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc[h][j] = dot2_bf16(pp01[h], v01[j], acc[h][j]);
        acc[h][j] = dot2_bf16(pp23[h], v23[j], acc[h][j]);
      }

    if (p + 1 < p1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kc[i] = kn[i];
        vc[i] = vn[i];
      }
      pid_c = pid_n;
    }
  }

  // Combine the 4 token rows of the wave (same running max), then the 4
  // waves through LDS, into this split's normalised partial output and LSE.
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] += shfl_xor_f32(l[h], 16);
    l[h] += shfl_xor_f32(l[h], 32);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[h][j] += shfl_xor_f32(acc[h][j], 16);
      acc[h][j] += shfl_xor_f32(acc[h][j], 32);
    }
  }
  __shared__ float s_acc[4][G][kD];
  __shared__ float s_m[4][G], s_l[4][G];
  if (row == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      *reinterpret_cast<float4*>(&s_acc[wave][h][dc * 8]) = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      *reinterpret_cast<float4*>(&s_acc[wave][h][dc * 8 + 4]) = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
    }
    if (dc == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        s_m[wave][h] = m[h];
        s_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * kD; idx += 256) {
    const int h = idx / kD, d = idx % kD;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][h]);
    float Lsum = 0.f, o = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = fast_exp2(s_m[w][h] - M);
        Lsum += s_l[w][h] * f;
        o += s_acc[w][h][d] * f;
      }
    }
    const size_t slot = ((size_t)b * a.Hq + g * G + h) * a.num_splits + split;
    a.part_o[slot * kD + d] = Lsum > 0.f ? o / Lsum : 0.f;
    if (d == 0) a.part_lse[slot] = Lsum > 0.f ? (M + __log2f(Lsum)) * kLn2 : kNegInf;
  }
}

// One wavefront per (request, query head): merge that request's splits by
// their LSE into the bf16 output and the fp32 LSE.
__global__ __launch_bounds__(256) void lse_merge_kernel(DecodeArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + wave;
  if (bh >= a.B * a.Hq) return;
  const int b = bh / a.Hq;
  const int n = a.splits_per_req[b];
  const float* plse = a.part_lse + (size_t)bh * a.num_splits;
  const float* po = a.part_o + (size_t)bh * a.num_splits * kD;
  float M = kNegInf;
  for (int s = 0; s < n; ++s) M = fmaxf(M, plse[s]);
  float tot = 0.f, o0 = 0.f, o1 = 0.f;
  if (M != kNegInf) {
    for (int s = 0; s < n; ++s) {
      const float w = fast_exp2((plse[s] - M) * kLog2e);
      const float2 x = *reinterpret_cast<const float2*>(po + (size_t)s * kD + 2 * lane);
      tot += w;
      o0 += w * x.x;
      o1 += w * x.y;
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  reinterpret_cast<uint32_t*>(a.out)[(size_t)bh * (kD / 2) + lane] = pack_bf16x2(o0 * inv, o1 * inv);
  if (lane == 0) a.lse[bh] = tot > 0.f ? M + __logf(tot) : kNegInf;
}

// dst[t, :] = pool[page_table[b, t / 64], g, t % 64, :] for t < L.
__global__ void gather_kv_kernel(const char* pages, int elem_bytes, const int32_t* table,
                                 int stride, int num_pages, int Hkv, int D, int b, int L, int g,
                                 char* dst) {
  const int row_bytes = D * elem_bytes;
  const int chunks = row_bytes / 16;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)L * chunks) return;
  const int t = (int)(idx / chunks), cidx = (int)(idx % chunks);
  const int pid = table[(size_t)b * stride + t / 64];
  if ((unsigned)pid >= (unsigned)num_pages) return;
  const size_t src = (((size_t)pid * Hkv + g) * 64 + (t % 64)) * row_bytes + (size_t)cidx * 16;
  *reinterpret_cast<uint4*>(dst + (size_t)t * row_bytes + (size_t)cidx * 16) =
      *reinterpret_cast<const uint4*>(pages + src);
}

template <int G>
hipError_t launch_split_g(const DecodeArgs& a, int fp8, hipStream_t s) {
  if (fp8)
    hipLaunchKernelGGL((decode_split_kernel<G, true>), dim3(a.n_items), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<G, false>), dim3(a.n_items), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_split(const DecodeArgs& a, int group, int fp8, hipStream_t s) {
  switch (group) {
    case 1: return launch_split_g<1>(a, fp8, s);
    case 2: return launch_split_g<2>(a, fp8, s);
    case 4: return launch_split_g<4>(a, fp8, s);
    case 8: return launch_split_g<8>(a, fp8, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_lse_merge(const DecodeArgs& a, hipStream_t s) {
  const int rows = a.B * a.Hq;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gather_kv(const void* pages, int elem_bytes, const int32_t* page_table,
                            int stride, int num_pages, int Hkv, int D, int b, int L, int g,
                            void* dst, hipStream_t s) {
  const int64_t n = (int64_t)L * (D * elem_bytes / 16);
  const int blocks = (int)((n + 255) / 256);
  hipLaunchKernelGGL(gather_kv_kernel, dim3(blocks), dim3(256), 0, s,
                     reinterpret_cast<const char*>(pages), elem_bytes, page_table, stride,
                     num_pages, Hkv, D, b, L, g, reinterpret_cast<char*>(dst));
  return hipGetLastError();
}

}  // namespace fa
