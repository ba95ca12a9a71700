// bf16 exact-attention prefill on gfx950 matrix cores.
//
// Method ("FIA / FlashAttention" Q&A, section 1; "FasterTransformer vs
// FlashAttention", section 3): the Q block is loaded once, K/V blocks stream
// through on-chip memory, a running row max and normaliser (online softmax)
// keep the blocked result equal to the global softmax, and only the final
// output (plus its LogSumExp) is written to HBM. The N x N score matrix never
// leaves registers.
//
// gfx950 design.
//  * Workgroup = 4 wavefronts = 128 query rows (32 per wavefront); K/V tiles
//    of 64 keys are staged in LDS (K row-major, V transposed) and shared by
//    the 4 wavefronts.
//  * Both contractions use v_mfma_f32_32x32x16_bf16 (fp32 accumulate) in the
//    transposed form S^T = K Q^T and O^T = V^T P^T. In the 32x32 accumulator
//    layout a lane then owns one query column and 16 keys of it, so the row
//    max and row sum are in-lane plus one exchange with the partner lane
//    (lane ^ 32), and P^T leaves the first MFMA already in the B-operand
//    layout of the second (no LDS round trip). To make the 8 keys a lane owns
//    contiguous, the K rows are fed to the first MFMA in a fixed permuted
//    order (kperm below); the order of a contraction's k index is free as
//    long as both operands agree.
//  * Scores are scaled into log2 units once (scale*log2e folded into the exp
//    argument's FMA) and exponentiated with v_exp_f32. The running max is
//    lazy: it moves only when a tile's max exceeds it by more than kTau, so
//    the O^T rescale (64 multiplies per lane) happens only on the first tiles
//    of a row. Two normalisers are kept: the sum of the bf16-rounded P that
//    the second MFMA consumes (one v_dot2 with ones per pair) divides O, so
//    the normalisation matches the weights applied; the fp32 sum of P gives
//    the LSE.
//  * K/V for tile t+1 are fetched from HBM into registers while tile t is
//    computed; LDS writes of V go through a 16-byte XOR swizzle so the
//    transposing stores do not collide in the same banks.
//  * Grid: one workgroup per (query tile, batch, head). With causal masking
//    the heaviest query tiles (most keys) are issued first. Heads are ordered
//    so that workgroups with equal id mod 8 -- which the dispatcher places on
//    the same XCD -- share a KV head, keeping its K/V in that XCD's L2.
#include "fa_internal.h"
#include "hip_common.h"

namespace fa {

namespace {

constexpr int kD = 128;   // head dim
constexpr int kBr = 128;  // query rows per workgroup
constexpr int kBc = 64;   // keys per tile
constexpr int kKst = kD + 8;   // K row stride in LDS (bf16 elements) = 272 B
constexpr int kVst = kBc + 8;  // V^T row stride in LDS (bf16 elements) = 144 B
constexpr float kTau = 8.0f;   // lazy max threshold (log2 units)

// MFMA row r of the S^T tile reads key kperm(r): with it, accumulator
// register i of lane l holds key 16*(i/8) + 8*(l/32) + (i%8).
__device__ __forceinline__ int kperm(int r) {
  const int a = r >> 3, hh = (r >> 2) & 1, c = r & 3;
  return 16 * (a >> 1) + 8 * hh + 4 * (a & 1) + c;
}

// Byte offset of V^T element (d, key) inside the V^T LDS tile, with the
// 16-byte column unit XOR-swizzled by the row.
__device__ __forceinline__ int vt_off(int d, int key) {
  const int unit = (key >> 3) ^ ((d >> 4) & 7);
  return d * (kVst * 2) + unit * 16 + (key & 7) * 2;
}

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(256) void prefill_bf16_kernel(PrefillArgs a, int n_qtiles, int nbh) {
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kBc * kKst];
  __shared__ __attribute__((aligned(16))) char vt_lds[kD * kVst * 2];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int hi = lane >> 5;     // which half of the wavefront
  const int col = lane & 31;    // query column of this lane in the 32x32 tiles

  // ---- work unit
  const int L = blockIdx.x;
  const int qt = a.causal ? (n_qtiles - 1 - L / nbh) : (L / nbh);
  const int e = L % nbh;
  int b, h, g;
  if (a.has_map) {
    b = e / a.Hq;
    h = e % a.Hq;
    g = a.kv_map[h];
  } else {
    const int G = a.Hq / a.Hkv;
    const int bg = e % (a.B * a.Hkv);
    const int j = e / (a.B * a.Hkv);
    b = bg / a.Hkv;
    g = bg % a.Hkv;
    h = g * G + j;
  }
  const int q0 = qt * kBr;
  const int off = a.Sk - a.Sq;  // causal: key j visible to query i iff j <= i + off
  int kend = a.Sk;
  if (a.causal) kend = min(a.Sk, q0 + kBr + off);
  const int n_kt = kend > 0 ? (kend + kBc - 1) / kBc : 0;

  const uint16_t* Q = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)b * a.Hq + h) * (size_t)a.Sq * kD;
  const uint16_t* K = reinterpret_cast<const uint16_t*>(a.k) + ((size_t)b * a.Hkv + g) * (size_t)a.Sk * kD;
  const uint16_t* V = reinterpret_cast<const uint16_t*>(a.v) + ((size_t)b * a.Hkv + g) * (size_t)a.Sk * kD;

  // ---- Q^T as the B operand of S^T = K Q^T: lane holds query (q0+32w+col),
  // dims 16*kk + 8*hi + 0..7 for kk = 0..7.
  const int qrow = q0 + wave * 32 + col;
  bf16x8_t qf[8];
  {
    const bool live = qrow < a.Sq;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (live) v = *reinterpret_cast<const uint4*>(Q + (size_t)qrow * kD + 16 * kk + 8 * hi);
      qf[kk] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m = kNegInf;  // running max of this query row, log2 units (same in lane and lane^32)
  float lr = 0.f;     // this lane's share of sum(bf16(p)): normalises O (matches the MFMA weights)
  float le = 0.f;     // this lane's share of sum(p) in fp32: gives the LSE
  const float c = a.scale * kLog2e;

  // ---- global -> register staging of one K/V tile.
  // K: 4 rounds of 16-byte chunks, chunk (it*256 + tid) = key (chunk>>4), dims 8*(chunk&15).
  // V: thread owns keys 4*(tid>>4)+0..3, dims 8*(tid&15)+0..7.
  uint4 kreg[4], vreg[4];
  const int vkq = tid >> 4, vdc = tid & 15;
  auto fetch = [&](int k0) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int chunk = it * 256 + tid;
      const int key = k0 + (chunk >> 4);
      kreg[it] = key < a.Sk ? *reinterpret_cast<const uint4*>(K + (size_t)key * kD + 8 * (chunk & 15))
                            : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = k0 + 4 * vkq + j;
      vreg[j] = key < a.Sk ? *reinterpret_cast<const uint4*>(V + (size_t)key * kD + 8 * vdc)
                           : make_uint4(0, 0, 0, 0);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int chunk = it * 256 + tid;
      *reinterpret_cast<uint4*>(&k_lds[(chunk >> 4) * kKst + 8 * (chunk & 15)]) = kreg[it];
    }
    const uint32_t v0[4] = {vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w};
    const uint32_t v1[4] = {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w};
    const uint32_t v2[4] = {vreg[2].x, vreg[2].y, vreg[2].z, vreg[2].w};
    const uint32_t v3[4] = {vreg[3].x, vreg[3].y, vreg[3].z, vreg[3].w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int d0 = 8 * vdc + 2 * w;
      // keys 4*vkq .. +3 of dims d0 (low halves) and d0+1 (high halves)
      const uint2 lo = make_uint2(perm_b32(v1[w], v0[w], 0x05040100u), perm_b32(v3[w], v2[w], 0x05040100u));
      const uint2 hv = make_uint2(perm_b32(v1[w], v0[w], 0x07060302u), perm_b32(v3[w], v2[w], 0x07060302u));
      *reinterpret_cast<uint2*>(vt_lds + vt_off(d0, 4 * vkq)) = lo;
      *reinterpret_cast<uint2*>(vt_lds + vt_off(d0 + 1, 4 * vkq)) = hv;
    }
  };

  const int krow0 = kperm(col);  // K row this lane feeds for MFMA row `col`
  if (n_kt > 0) fetch(0);
  for (int t = 0; t < n_kt; ++t) {
    const int k0 = t * kBc;
    __syncthreads();  // previous tile's LDS reads are done
    stage();
    __syncthreads();
    if (t + 1 < n_kt) fetch(k0 + kBc);

    // Wavefront-uniform skip of tiles entirely above this wavefront's diagonal.
    const int wq0 = q0 + wave * 32;
    if (a.causal && k0 > wq0 + 31 + off) continue;

    // ---- S^T = K Q^T for the two 32-key halves of the tile.
    f32x16_t s0, s1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = 0.f;
      s1[i] = 0.f;
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(&k_lds[krow0 * kKst + 16 * kk + 8 * hi]);
      const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(&k_lds[(32 + krow0) * kKst + 16 * kk + 8 * hi]);
      s0 = mfma32(a0, qf[kk], s0);
      s1 = mfma32(a1, qf[kk], s1);
    }

    // ---- mask (ragged key tail, causal diagonal)
    const bool need_mask = (k0 + kBc > a.Sk) || (a.causal && k0 + kBc - 1 > wq0 + off);
    if (need_mask) {
      const int lim = a.causal ? min(a.Sk - 1, qrow + off) : a.Sk - 1;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 16 * (i >> 3) + 8 * hi + (i & 7);
        if (key > lim) s0[i] = kNegInf;
        if (key + 32 > lim) s1[i] = kNegInf;
      }
    }

    // ---- online softmax (lazy max)
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
    mx = fmaxf(mx, shfl_xor_f32(mx, 32));
    const float mxs = mx * c;
    const bool need = mxs > m + kTau;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float mn = need ? mxs : m;
      const float alpha = need ? fast_exp2(m - mn) : 1.f;
      lr *= alpha;
      le *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      m = mn;
    }
    const float mu = (m == kNegInf) ? 0.f : m;

    // P^T in bf16 as B operands of O^T = V^T P^T: pf[ks] covers keys 16ks..16ks+15.
    bf16x8_t pf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const f32x16_t& sv = (ks < 2) ? s0 : s1;
      const int base = 8 * (ks & 1);
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = fast_exp2(__builtin_fmaf(sv[base + 2 * j], c, -mu));
        const float p1 = fast_exp2(__builtin_fmaf(sv[base + 2 * j + 1], c, -mu));
        w[j] = pack_bf16x2(p0, p1);
        lr = dot2_bf16(w[j], 0x3f803f80u, lr);  // + bf16(p0) + bf16(p1)
        le += p0 + p1;
      }
      pf[ks] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8_t va = *reinterpret_cast<const bf16x8_t*>(vt_lds + vt_off(32 * db + col, 16 * ks + 8 * hi));
        o[db] = mfma32(va, pf[ks], o[db]);
      }
  }

  // ---- epilogue: O = O^T / sum(bf16 p), LSE = (m + log2 sum(p)) ln 2
  const float lrt = lr + shfl_xor_f32(lr, 32);
  const float let_ = le + shfl_xor_f32(le, 32);
  if (qrow >= a.Sq) return;
  const float inv = lrt > 0.f ? 1.f / lrt : 0.f;
  uint16_t* O = reinterpret_cast<uint16_t*>(a.out) + ((size_t)b * a.Hq + h) * (size_t)a.Sq * kD + (size_t)qrow * kD;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d = 32 * db + 8 * gq + 4 * hi;
      const uint2 w = make_uint2(pack_bf16x2(o[db][4 * gq] * inv, o[db][4 * gq + 1] * inv),
                                 pack_bf16x2(o[db][4 * gq + 2] * inv, o[db][4 * gq + 3] * inv));
      *reinterpret_cast<uint2*>(O + d) = w;
    }
  if (hi == 0)
    a.lse[((size_t)b * a.Hq + h) * a.Sq + qrow] = let_ > 0.f ? (m + __log2f(let_)) * kLn2 : kNegInf;
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
  const int n_qtiles = (a.Sq + kBr - 1) / kBr;
  const int nbh = a.B * a.Hq;
  const long long blocks = (long long)n_qtiles * nbh;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(prefill_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a, n_qtiles, nbh);
  return hipGetLastError();
}

}  // namespace fa
