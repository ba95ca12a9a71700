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
#include "decode_common.h"
#include "fa_internal.h"
#include "hip_common.h"

namespace fa {

namespace {

constexpr int kD = 128;
constexpr float kTau = 8.0f;  // lazy max threshold, log2 units (p <= 2^kTau)
// Page buffers per wavefront (pages in flight + 1), by KV element type.
constexpr int kRingBf16 = 3;
constexpr int kRingFp8 = 2;

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

// KV bytes are read exactly once per step, so the loads are nontemporal
// (cache policy nt): they stream past the caches instead of evicting lines
// that are reused. The resource covers one (page, KV head) block.
template <bool FP8>
__device__ __forceinline__ void load_slot(KvSlot<FP8>& s, __amdgpu_buffer_rsrc_t r, int byte_off) {
  constexpr int kNT = 2;
  if constexpr (FP8) {
    const u32x2_t t = __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, kNT);
    s.v = make_uint2(t.x, t.y);
  } else {
    const u32x4_t t = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kNT);
    s.v = make_uint4(t.x, t.y, t.z, t.w);
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

// One page of one KV head as this lane holds it, with its page id and the
// score / probability multipliers (the fp8 scales folded in).
template <bool FP8>
struct PageBuf {
  KvSlot<FP8> k[4], v[4];
  int pid;
  float c, vsc;
};

template <int G, bool FP8, int NB>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  constexpr int kElem = FP8 ? 1 : 2;
  // Workgroup w runs items w, w + grid, ... (one item unless the plan
  // packed several segments per workgroup).
  for (int ii = blockIdx.x; ii < a.n_items; ii += gridDim.x) {
    const WorkItem it = a.items[ii];
    if (it.b < 0) continue;  // padding of a balanced plan
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

    const int blk_bytes = 64 * kD * kElem;  // one (page, KV head) block
    const char* kpool = reinterpret_cast<const char*>(a.k_pages);
    const char* vpool = reinterpret_cast<const char*>(a.v_pages);
    const int32_t* table = a.page_table + (size_t)b * a.stride;
    // Byte offset of this lane's slot i inside a block: token wave*16 + 4i + row,
    // dims dc*8 .. dc*8+7.
    int slot_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) slot_off[i] = ((wave * 16 + 4 * i + row) * kD + dc * 8) * kElem;

    // Page ids of the item, 64 pages per window: lane i holds the id of page
    // w0 + i (and for fp8 that page's K and V scales), read with one vector
    // load each, so no page waits on a dependent page-table or scale load.
    int w0 = p0;
    int tbl = -1;
    float kscl = 0.f, vscl = 0.f;
    int bad_page = 0;  // per lane (a vector register: the scalar ones are all in use)
    auto load_window = [&]() {
      const int pp = w0 + lane;
      tbl = pp < p1 ? table[pp] : -1;
      // A page id outside the pool reads as zeros (below); that it happened is
      // noted here and reported once the item is done (no memory atomic in
      // the page loop).
      bad_page |= pp < p1 && (unsigned)tbl >= (unsigned)a.num_pages;
      if constexpr (FP8) {
        const bool ok = (unsigned)tbl < (unsigned)a.num_pages;
        kscl = ok ? a.k_scale[(size_t)tbl * a.Hkv + g] : 0.f;
        vscl = ok ? a.v_scale[(size_t)tbl * a.Hkv + g] : 0.f;
      }
    };
    load_window();

    // Ring of NB page buffers: page p lives in buf[(p - p0) % NB], and its
    // loads are issued NB-1 pages ahead of its use, so each wavefront keeps
    // NB-1 pages of K and V in flight while it computes on the current one.
    // The page's block address is wave-uniform (scalar registers), so the
    // per-page address work is scalar and the lane offsets are fixed.
    PageBuf<FP8> buf[NB];
    auto issue = [&](PageBuf<FP8>& d, int p) {
      if (p - w0 == 64) {
        w0 += 64;
        load_window();
      }
      const int pid = __builtin_amdgcn_readlane(tbl, p - w0);
      d.pid = pid;
      if constexpr (FP8) {
        d.c = c_base * __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, kscl), p - w0));
        d.vsc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, vscl), p - w0));
      } else {
        d.c = c_base;
        d.vsc = 1.f;
      }
      // The block offset is uniform; readfirstlane makes that visible to the
      // compiler, which otherwise wraps each buffer load in a waterfall loop.
      const size_t off_v = ((size_t)(((unsigned)pid < (unsigned)a.num_pages) ? pid : 0) * a.Hkv + g) * blk_bytes;
      const size_t off = ((size_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(off_v >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)off_v);
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kpool + off), (short)0, blk_bytes, 0x00020000);
      const __amdgpu_buffer_rsrc_t rv =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vpool + off), (short)0, blk_bytes, 0x00020000);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        load_slot<FP8>(d.k[i], rk, slot_off[i]);
        load_slot<FP8>(d.v[i], rv, slot_off[i]);
      }
    };

    auto consume = [&](PageBuf<FP8>& cur, int p) {
      // Tokens of this page that belong to the request: all 64 except on the
      // request's last page; an out-of-range page id contributes nothing. Only
      // such a partial page takes the masking path (a wave-uniform branch).
      const int nvalid = ((unsigned)cur.pid < (unsigned)a.num_pages) ? min(64, L - p * 64) : 0;
      const bool partial = nvalid < 64;
      bool tok_ok[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) tok_ok[i] = (wave * 16 + 4 * i + row) < nvalid;
      if (partial) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!tok_ok[i]) {  // tail slots may hold anything (NaN): never use them
            zero_slot<FP8>(cur.k[i]);
            zero_slot<FP8>(cur.v[i]);
          }
      }

      // Raw dot products q.k for this lane's 4 tokens, summed over the 16 lanes
      // that share a token.
      float s[4][G];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t kp[4];
        slot_pairs<FP8>(cur.k[i], kp);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float d = dot2_bf16(qd[h][0], kp[0], 0.f);
          d = dot2_bf16(qd[h][1], kp[1], d);
          d = dot2_bf16(qd[h][2], kp[2], d);
          d = dot2_bf16(qd[h][3], kp[3], d);
          s[i][h] = row16_sum(d);
        }
      }
      if (partial) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int h = 0; h < G; ++h) s[i][h] = tok_ok[i] ? s[i][h] : kNegInf;
      }

      // Lazy running max in log2 units: the score is c*s with c >= 0, so the
      // tile max is c * max(s). It moves only when some score exceeds it by
      // more than kTau; after the first full page it is finite.
      const float c = cur.c;
      bool need = false;
      float smax[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        smax[h] = fmaxf(fmaxf(s[0][h], s[1][h]), fmaxf(s[2][h], s[3][h]));
        need |= smax[h] * c > m[h] + kTau;
      }
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float x = fmaxf(smax[h], shfl_xor_f32(smax[h], 16));
          x = fmaxf(x, shfl_xor_f32(x, 32));
          const float mn = fmaxf(m[h], x * c);
          const float alpha = fast_exp2(m[h] - mn);  // 0 when m was -inf
          l[h] *= alpha;
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[h][j] *= alpha;
          m[h] = mn;
        }
      }

      // p = 2^(c*s - m); the fp8 V scale is folded into the weights that
      // multiply V, not into the normaliser.
      float e[4][G];
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i][h] = fast_exp2(__builtin_fmaf(s[i][h], c, -m[h]));
      if (partial) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int h = 0; h < G; ++h) e[i][h] = tok_ok[i] ? e[i][h] : 0.f;
      }
      uint32_t pp01[G], pp23[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        l[h] += (e[0][h] + e[1][h]) + (e[2][h] + e[3][h]);
        if constexpr (FP8) {
          const float vsc = cur.vsc;
          pp01[h] = pack_bf16x2(e[0][h] * vsc, e[1][h] * vsc);
          pp23[h] = pack_bf16x2(e[2][h] * vsc, e[3][h] * vsc);
        } else {
          pp01[h] = pack_bf16x2(e[0][h], e[1][h]);
          pp23[h] = pack_bf16x2(e[2][h], e[3][h]);
        }
      }

      uint32_t v01[8], v23[8];
      token_pairs<FP8>(cur.v[0], cur.v[1], v01);
      token_pairs<FP8>(cur.v[2], cur.v[3], v23);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          acc[h][j] = dot2_bf16(pp01[h], v01[j], acc[h][j]);
          acc[h][j] = dot2_bf16(pp23[h], v23[j], acc[h][j]);
        }
    };

#pragma unroll
    for (int j = 0; j < NB - 1; ++j)
      if (p0 + j < p1) issue(buf[j], p0 + j);
    // Unrolled by NB so that every buffer index is a compile-time constant.
    for (int p = p0; p < p1; p += NB) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if (p + j < p1) {
          if (p + j + NB - 1 < p1) issue(buf[(j + NB - 1) % NB], p + j + NB - 1);
          consume(buf[j], p + j);
        }
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
    __shared__ float s_o[4 * G * kD];
    __shared__ float s_m[64], s_l[64];
    if (row == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        *reinterpret_cast<float4*>(&s_o[(wave * G + h) * kD + dc * 8]) = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
        *reinterpret_cast<float4*>(&s_o[(wave * G + h) * kD + dc * 8 + 4]) =
            make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
      }
      if (dc == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          s_m[16 * wave + h] = m[h];
          s_l[16 * wave + h] = l[h];
        }
      }
    }
    __syncthreads();
    finish_work_item<G>(a, b, g, split, s_m, s_l, s_o);
    if (__builtin_amdgcn_ballot_w64(bad_page != 0) != 0 && lane == 0) report_status(a.status, kStatusBadPage);
    __syncthreads();  // the next item reuses this workgroup's LDS
  }
}

// One workgroup of 4 wavefronts per (request, query head) merges that
// request's splits by their LSE into the bf16 output and the fp32 LSE:
// L* = M + ln sum_s exp(lse_s - M), O = sum_s exp(lse_s - L*) O_s, where M is
// the largest partial LSE. Each wavefront takes a contiguous quarter of the
// splits and streams it 8 splits at a time (8 independent 512-byte loads in
// flight); the quarters are combined through LDS. An empty split has
// lse_s = -inf and weight 0; a request with no token gets O = 0, LSE = -inf.
// A request with a single split was written by its work item.
__global__ __launch_bounds__(256) void lse_merge_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = bh / a.Hq;
  // The split count is loaded together with the partials (not before them):
  // the quarters below are cut from the slot capacity num_splits, every slot
  // position is in bounds, and slots past the count are dropped by selection
  // once it arrives, so the merge waits for one memory round trip, not two.
  const int n = a.splits_per_req[b];
  const float* plse = a.part_lse + (size_t)bh * a.num_splits;
  const float* po = a.part_o + (size_t)bh * a.num_splits * kD;
  __shared__ float s_max[4], s_tot[4];
  __shared__ float2 s_o[4][kD / 2];

  // Each wavefront merges a contiguous quarter of the splits on its own,
  // loading the LSEs and partial outputs of up to 8 splits together (one
  // memory round trip per 8 splits) and keeping a running max M, weight
  // sum and weighted output; the four states are then merged the same way.
  const int cap = a.num_splits;
  const int per = (cap + 3) / 4;
  const int s0 = min(cap, wave * per), s1 = min(cap, s0 + per);
  float M = kNegInf, tot = 0.f, o0 = 0.f, o1 = 0.f;
  for (int i = s0; i < s1; i += 8) {
    float w[8];
    float2 x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sj = i + j < s1 ? i + j : s0;  // past the range: a slot whose weight is dropped below
      w[j] = plse[sj];
      x[j] = *reinterpret_cast<const float2*>(po + (size_t)sj * kD + 2 * lane);
    }
    if (n == 1) break;  // written by its work item (uniform across the workgroup)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool ok = i + j < s1 && i + j < n;
      w[j] = ok ? w[j] : kNegInf;  // unused slots may hold anything, NaN included
      x[j].x = ok ? x[j].x : 0.f;
      x[j].y = ok ? x[j].y : 0.f;
    }
    float mc = M;
#pragma unroll
    for (int j = 0; j < 8; ++j) mc = fmaxf(mc, w[j]);
    if (mc == kNegInf) continue;  // only empty splits so far (uniform)
    const float r = fast_exp2((M - mc) * kLog2e);  // 0 when M = -inf
    tot *= r;
    o0 *= r;
    o1 *= r;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float wj = fast_exp2((w[j] - mc) * kLog2e);
      tot += wj;
      o0 += wj * x[j].x;
      o1 += wj * x[j].y;
    }
    M = mc;
  }
  if (n == 1) return;  // uniform across the workgroup, before any barrier
  s_o[wave][lane] = make_float2(o0, o1);
  if (lane == 0) {
    s_max[wave] = M;
    s_tot[wave] = tot;
  }
  __syncthreads();
  if (wave == 0) {
    const float Mx = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    float T = 0.f, r0 = 0.f, r1 = 0.f;
    if (Mx != kNegInf) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = s_max[w] == kNegInf ? 0.f : fast_exp2((s_max[w] - Mx) * kLog2e);
        T += s_tot[w] * f;
        r0 += s_o[w][lane].x * f;
        r1 += s_o[w][lane].y * f;
      }
    }
    const float inv = T > 0.f ? 1.f / T : 0.f;
    reinterpret_cast<uint32_t*>(a.out)[(size_t)bh * (kD / 2) + lane] = pack_bf16x2(r0 * inv, r1 * inv);
    if (lane == 0) a.lse[bh] = T > 0.f ? Mx + __logf(T) : kNegInf;
  }
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
    hipLaunchKernelGGL((decode_split_kernel<G, true, kRingFp8>), dim3(a.grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<G, false, kRingBf16>), dim3(a.grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// One or two query heads per KV head make each page a matrix-vector product:
// the vector-ALU kernel here. Larger groups are small dense contractions and
// run on the matrix cores (decode_mfma.hip).
hipError_t launch_decode_split(const DecodeArgs& a, int group, int fp8, hipStream_t s) {
  switch (group) {
    case 1: return launch_split_g<1>(a, fp8, s);
    case 2: return launch_split_g<2>(a, fp8, s);
    case 4:
    case 8:
    case 16: return launch_decode_split_mfma(a, group, fp8, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_lse_merge(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(lse_merge_kernel, dim3(a.B * a.Hq), dim3(256), 0, s, a);
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
