// Paged Flash-Decoding split kernel on MFMA, for query-head groups of 4 to 16
// heads per KV head.
//
// Method ("Flash Attention & Paged Attention" blog, "FA and the decode
// phase"): the KV sequence of a request is split; each work item (request b,
// KV head g, a range of 64-token pages) produces a partial output and its
// LogSumExp, merged later by the LSE merge kernel. The cache is paged
// ("2. PagedAttention"; 64-token pages per the "FlashAttention breakthrough
// architecture" article).
//
// gfx950 design. With G query heads sharing a KV head, each page is a small
// dense contraction: S[64 tokens x G heads] = K Q^T, then O[G x 128] += P V.
// On the vector ALU every score would be reduced across the 16 lanes that
// share a token, and the softmax paid 16 times over; on the matrix cores the
// whole step costs 12 MFMAs per wavefront and page, and each score lives in
// one lane. The heads are padded to the 16 columns of the 16x16 MFMAs.
//  * Wavefront w takes tokens 16w..16w+15 of every page of the item.
//  * QK: v_mfma_f32_16x16x32_bf16, A = K (lane: token l%16, 8 dims), read
//    from HBM straight into registers (fp8 codes converted exactly to bf16);
//    B = Q^T, loaded once. The result gives lane l the scores of head l%16
//    for tokens 4(l/16)..+3.
//  * That is exactly the A-operand layout of v_mfma_f32_16x16x16_bf16, so P
//    feeds O = P V without any lane exchange. V must arrive transposed
//    (4 tokens of one dim per lane): it goes through a per-wavefront LDS ring
//    and gfx950's transposing read ds_read_b64_tr_b16. bf16 pages travel
//    HBM -> LDS with buffer_load ... lds; fp8 pages are converted in registers
//    and written to LDS as bf16. The ring is private to the wavefront, so no
//    barrier is needed until the epilogue.
//  * Each page's buffer resources end at the page's last valid token, so the
//    tail of a partial page reads as zeros (its NaN-or-anything contents never
//    reach an MFMA); tail scores are masked to -inf.
//  * Online softmax in log2 units with the lazy running max (it moves only
//    when a score exceeds it by more than kTau); the fp8 K scale is folded
//    into the score multiplier and the V scale into P.
//  * The four wavefronts' (m, l, O) are merged through LDS into the item's
//    normalised partial output and LSE.
#include "decode_common.h"
#include "fa_internal.h"
#include "hip_common.h"

namespace fa {

namespace {

constexpr int kD = 128;
constexpr float kTau = 8.0f;  // lazy max threshold, log2 units
constexpr int kNT = 2;        // cache policy: nontemporal (KV bytes are read once per step)

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_qk(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_pv(bf16x4_t a, bf16x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Transposing LDS read: within each group of 16 lanes, lane i receives
// element (i & 3) of the 8-byte chunks addressed by lanes 4j + (i >> 2).
__device__ __forceinline__ bf16x4_t lds_read_tr16(const char* p) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p));
  return __builtin_bit_cast(bf16x4_t, v);
}

// 16 fp8 (e4m3fn) codes -> two groups of 8 bf16 (exact).
__device__ __forceinline__ uint32_t fp8x2_lo(uint32_t x) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false));
}
__device__ __forceinline__ uint32_t fp8x2_hi(uint32_t x) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true));
}
__device__ __forceinline__ void fp8x16_to_bf16(uint4 w, bf16x8_t& lo, bf16x8_t& hi) {
  lo = __builtin_bit_cast(bf16x8_t, make_uint4(fp8x2_lo(w.x), fp8x2_hi(w.x), fp8x2_lo(w.y), fp8x2_hi(w.y)));
  hi = __builtin_bit_cast(bf16x8_t, make_uint4(fp8x2_lo(w.z), fp8x2_hi(w.z), fp8x2_lo(w.w), fp8x2_hi(w.w)));
}

// Wait until at most 8 * n vector-memory instructions are outstanding
// (n = 0..3): the bf16 direct-to-LDS V loads of a page are done once only
// the 8 instructions (4 K, 4 V) of each of the n pages issued after it may
// still be in flight. The compiler does not track these LDS writes.
__device__ __forceinline__ void wait_vmem_pages(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
  }
}

// HBM -> LDS without registers: lane l's 16 bytes at voffset land at
// dst + 16 l. (Kept out of the kernel template: called inside it directly,
// the host compilation pass drops the kernel's launch stub.)
__device__ __forceinline__ void load_to_lds16(__amdgpu_buffer_rsrc_t r, char* dst, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst), 16, voffset, 0, 0, kNT);
}

template <bool FP8>
struct MPage {
  uint4 k[FP8 ? 2 : 4];  // this lane's K fragments (16 B each)
  uint4 v[FP8 ? 2 : 1];  // fp8: this lane's V codes (bf16 V goes straight to LDS)
  int nvalid;            // tokens of the page that belong to the request
  float c, vsc;          // score multiplier (scale*log2e*k_scale), V scale
};

template <int G, bool FP8, int NB>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeArgs a) {
  static_assert(G >= 1 && G <= 16, "heads per KV head must fit the 16 MFMA columns");
  static_assert(NB >= 2 && NB <= 4, "ring depth");
  constexpr int kElem = FP8 ? 1 : 2;
  constexpr int kRowB = kD * kElem;    // bytes of one token row of a (page, KV head) block
  constexpr int kBlk = 64 * kRowB;     // bytes of a (page, KV head) block
  constexpr int kVq = 16 * kD * 2;     // LDS bytes of a wavefront's 16 V rows in bf16
  constexpr int kSlots = FP8 ? 1 : NB; // LDS V slots per wavefront
  constexpr int kRingB = 4 * kSlots * kVq;
  constexpr int kEpiB = (2 * 64 + 4 * G * kD) * 4;
  constexpr int kLdsB = kRingB > kEpiB ? kRingB : kEpiB;
  __shared__ __attribute__((aligned(16))) char lds[kLdsB];

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
    const int col = lane & 15, grp = lane >> 4;
    char* vring = lds + wave * kSlots * kVq;

    // ---- Q^T as the B operand of S = K Q^T: lane (col = head, grp), MFMA kk,
    // k-element e is dim dim_of(kk, grp, e); heads past G are zero columns.
    // The dim order of the contraction is free; it is chosen so that each K
    // fragment is one 16-byte load (fp8: one load feeds two MFMAs).
    auto dim0 = [&](int kk) { return FP8 ? 64 * (kk >> 1) + 16 * grp + 8 * (kk & 1) : 32 * kk + 8 * grp; };
    bf16x8_t qf[4];
    {
      const uint16_t* qh = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)b * a.Hq + g * G + (col < G ? col : 0)) * kD;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (col < G) v = *reinterpret_cast<const uint4*>(qh + dim0(kk));
        qf[kk] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
    const float c_base = a.scale * kLog2e;

    // ---- per-lane state: m, l of head `col` (log2 units; equal in the four
    // lanes of a head), O of heads 4*grp + e and dims 16*nb + col.
    float m = kNegInf, l = 0.f;
    f32x4_t acc[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const char* kpool = reinterpret_cast<const char*>(a.k_pages);
    const char* vpool = reinterpret_cast<const char*>(a.v_pages);
    const int32_t* table = a.page_table + (size_t)b * a.stride;

    // Byte offsets inside a (page, KV head) block.
    //   K fragment: token 16*wave + col, dims dim0(kk) .. +7 (fp8: +15).
    //   bf16 V direct load i: LDS row r = 4i + grp of the slot, 16-byte
    //     position col holds global unit col ^ 2*(r & 7) of token 16*wave + r
    //     (32-byte segments XOR-swizzled by row, for conflict-free
    //     transposing reads).
    //   fp8 V load m: token 16*wave + 8m + lane/8, 16 codes at 16*(lane & 7).
    int k_off[FP8 ? 2 : 4];
#pragma unroll
    for (int i = 0; i < (FP8 ? 2 : 4); ++i)
      k_off[i] = (16 * wave + col) * kRowB + (FP8 ? 64 * i + 16 * grp : (32 * i + 8 * grp) * 2);
    int v_off[FP8 ? 2 : 4];
#pragma unroll
    for (int i = 0; i < (FP8 ? 2 : 4); ++i) {
      if constexpr (FP8) {
        v_off[i] = (16 * wave + 8 * i + (lane >> 3)) * kRowB + 16 * (lane & 7);
      } else {
        const int r = 4 * i + grp;
        v_off[i] = (16 * wave + r) * kRowB + 16 * (col ^ (2 * (r & 7)));
      }
    }
    // Transposing read of dim block nb: lane (grp, col) addresses row
    // 4*grp + (col >> 2), dims 16*nb + 4*(col & 3) .. +3 (after the swizzle).
    const int tr_row = 4 * grp + (col >> 2);
    const int tr_base = tr_row * (kD * 2) + 8 * (col & 3);
    const int tr_swz = tr_row & 7;

    // ---- Page ids (and fp8 scales), 64 pages per window: lane i holds page
    // w0 + i, read with one vector load each.
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

    // ---- Ring of NB pages: page p lives in buf[(p - p0) % NB] (and, bf16, in
    // LDS slot (p - p0) % NB); its loads are issued NB-1 pages ahead of use.
    MPage<FP8> buf[NB];
    auto issue = [&](MPage<FP8>& d, int p, int slot) {
      if (p - w0 == 64) {
        w0 += 64;
        load_window();
      }
      const int pid = __builtin_amdgcn_readlane(tbl, p - w0);
      const bool ok = (unsigned)pid < (unsigned)a.num_pages;
      d.nvalid = ok ? min(64, L - p * 64) : 0;
      if constexpr (FP8) {
        d.c = c_base * __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, kscl), p - w0));
        d.vsc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, vscl), p - w0));
      } else {
        d.c = c_base;
        d.vsc = 1.f;
      }
      // The block offset is uniform; readfirstlane makes that visible to the
      // compiler (otherwise each buffer load gets a waterfall loop).
      const size_t off_v = ((size_t)(ok ? pid : 0) * a.Hkv + g) * kBlk;
      const size_t off = ((size_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(off_v >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)off_v);
      // Resources end at the last valid token: the tail reads as zeros.
      const int nbytes = __builtin_amdgcn_readfirstlane(d.nvalid * kRowB);
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kpool + off), (short)0, nbytes, 0x00020000);
      const __amdgpu_buffer_rsrc_t rv =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vpool + off), (short)0, nbytes, 0x00020000);
#pragma unroll
      for (int i = 0; i < (FP8 ? 2 : 4); ++i) {
        const u32x4_t t = __builtin_amdgcn_raw_buffer_load_b128(rk, k_off[i], 0, kNT);
        d.k[i] = make_uint4(t.x, t.y, t.z, t.w);
      }
      if constexpr (FP8) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const u32x4_t t = __builtin_amdgcn_raw_buffer_load_b128(rv, v_off[i], 0, kNT);
          d.v[i] = make_uint4(t.x, t.y, t.z, t.w);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          load_to_lds16(rv, vring + slot * kVq + i * 1024, v_off[i]);
      }
    };

    auto consume = [&](MPage<FP8>& cur, int p, int slot, int younger_pages) {
      // S = K Q^T for this wavefront's 16 tokens.
      bf16x8_t kf[4];
      if constexpr (FP8) {
        fp8x16_to_bf16(cur.k[0], kf[0], kf[1]);
        fp8x16_to_bf16(cur.k[1], kf[2], kf[3]);
      } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) kf[kk] = __builtin_bit_cast(bf16x8_t, cur.k[kk]);
      }
      f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) s = mfma_qk(kf[kk], qf[kk], s);

      // fp8: this page's V, converted to bf16, into the wavefront's LDS slot
      // (row t = 8i + lane/8, 32-byte segment lane & 7 stored at (lane & 7) ^ (t & 7)).
      if constexpr (FP8) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          bf16x8_t lo, hi;
          fp8x16_to_bf16(cur.v[i], lo, hi);
          const int t = 8 * i + (lane >> 3);
          char* dst = vring + t * (kD * 2) + 32 * ((lane & 7) ^ (t & 7));
          *reinterpret_cast<bf16x8_t*>(dst) = lo;
          *reinterpret_cast<bf16x8_t*>(dst + 16) = hi;
        }
      }

      // Tail tokens of a partial page: scores -inf, weights 0.
      const bool partial = cur.nvalid < 64;
      bool ok[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) ok[e] = 16 * wave + 4 * grp + e < cur.nvalid;
      if (partial) {
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] = ok[e] ? s[e] : kNegInf;
      }

      // Lazy running max of head `col`: c*s with c >= 0.
      const float c = cur.c;
      const float lmax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      if (__builtin_amdgcn_ballot_w64(lmax * c > m + kTau) != 0) {
        float x = fmaxf(lmax, shfl_xor_f32(lmax, 16));
        x = fmaxf(x, shfl_xor_f32(x, 32));
        const float mn = fmaxf(m, x * c);
        const float alpha = fast_exp2(m - mn);  // 0 while m is -inf
        l *= alpha;
        m = mn;
        // O rows are heads 4*grp + e: their factors come from lanes 4*grp + e.
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ae = __shfl(alpha, 4 * grp + e, 64);
#pragma unroll
          for (int nb = 0; nb < 8; ++nb) acc[nb][e] *= ae;
        }
      }

      // P = 2^(c*s - m) (fp8: times the V scale), already in A-operand layout.
      float pe[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pe[e] = fast_exp2(__builtin_fmaf(s[e], c, -m));
      if (partial) {
#pragma unroll
        for (int e = 0; e < 4; ++e) pe[e] = ok[e] ? pe[e] : 0.f;
      }
      l += (pe[0] + pe[1]) + (pe[2] + pe[3]);
      const float vsc = cur.vsc;
      const bf16x4_t pa = __builtin_bit_cast(
          bf16x4_t, make_uint2(pack_bf16x2(pe[0] * vsc, pe[1] * vsc), pack_bf16x2(pe[2] * vsc, pe[3] * vsc)));

      // O += P V, V^T blocks of 16 dims through the transposing read.
      if constexpr (!FP8) wait_vmem_pages(younger_pages);
      const char* vs = vring + slot * kVq + tr_base;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const bf16x4_t vb = lds_read_tr16(vs + 32 * (nb ^ tr_swz));
        acc[nb] = mfma_pv(pa, vb, acc[nb]);
      }
    };

#pragma unroll
    for (int j = 0; j < NB - 1; ++j)
      if (p0 + j < p1) issue(buf[j], p0 + j, j);
    // Unrolled by NB so that buffer and slot indices are compile-time constants.
    for (int p = p0; p < p1; p += NB) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if (p + j < p1) {
          const int nxt = p + j + NB - 1;
          if (nxt < p1) issue(buf[(j + NB - 1) % NB], nxt, FP8 ? 0 : (j + NB - 1) % NB);
          consume(buf[j], p + j, FP8 ? 0 : j, min(NB - 1, p1 - 1 - (p + j)));
        }
      }
    }

    // ---- Epilogue: l summed over the four lanes of each head, then the four
    // wavefronts' (m, l, O) merged through LDS into this split's normalised
    // partial output and LSE.
    l += shfl_xor_f32(l, 16);
    l += shfl_xor_f32(l, 32);
    __syncthreads();  // every wavefront is done with its ring
    float* s_m = reinterpret_cast<float*>(lds);  // [4][16]
    float* s_l = s_m + 64;                       // [4][16]
    float* s_o = s_l + 64;                       // [4][G][128]
    if (grp == 0) {
      s_m[wave * 16 + col] = m;
      s_l[wave * 16 + col] = l;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int h = 4 * grp + e;
      if (h < G) {
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) s_o[(wave * G + h) * kD + 16 * nb + col] = acc[nb][e];
      }
    }
    __syncthreads();
    finish_work_item<G>(a, b, g, split, s_m, s_l, s_o);
    if (__builtin_amdgcn_ballot_w64(bad_page != 0) != 0 && lane == 0) report_status(a.status, kStatusBadPage);
    __syncthreads();  // the next item reuses this workgroup's LDS
  }
}

template <int G>
hipError_t launch_g(const DecodeArgs& a, int fp8, hipStream_t s) {
  if (fp8)
    hipLaunchKernelGGL((decode_mfma_kernel<G, true, 4>), dim3(a.grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<G, false, 3>), dim3(a.grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_split_mfma(const DecodeArgs& a, int group, int fp8, hipStream_t s) {
  switch (group) {
    case 4: return launch_g<4>(a, fp8, s);
    case 8: return launch_g<8>(a, fp8, s);
    case 16: return launch_g<16>(a, fp8, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
