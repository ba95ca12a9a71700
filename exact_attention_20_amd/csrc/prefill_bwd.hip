// Backward of exact attention (bf16, D = 128) on gfx950 matrix cores.
//
// Recomputation ("Flash Attention & Paged Attention" blog, "1. FlashAttention";
// "FasterTransformer vs FlashAttention", section 3): the backward keeps no
// N x N matrix; from the forward's LSE it rebuilds P = exp(scale S - LSE)
// tile by tile, and with D_i = sum_d dO_id O_id (the row term of the softmax
// Jacobian) it forms dS = P * (dP - D) with dP = dO V^T, then
//   dQ = scale dS K,   dK = scale dS^T Q,   dV = P^T dO.
//
// Two kernels, no atomics:
//  * bwd_dq_kernel: shaped like the forward kernel. 8 wavefronts x 32 query
//    rows; it first forms D_i from the dO row it holds and the O row (and
//    writes it for the second kernel); 64-key tiles of K and V stream
//    through LDS. Per tile,
//    S^T = K Q^T and dP^T = V dO^T (K, V rows from LDS in the permuted row
//    order that makes each accumulator usable as a later operand; Q and dO in
//    registers), dS^T = P^T (dP^T - D) packed to bf16, and dQ^T += K^T dS^T
//    with K^T from gfx950's transposing LDS read (as V^T in the forward).
//  * bwd_dkdv_kernel: the transposed twin. 8 wavefronts x 32 keys, their K
//    rows in registers and the workgroup's V rows resident in LDS; 64-row
//    tiles of Q and dO (and their LSE, D)
//    stream through LDS for every query head that reads this KV head. Per
//    32-row half, S = Q K^T and dP = dO V^T (Q, dO rows in permuted order),
//    then dV^T += dO^T P and dK^T += Q^T dS with dO^T, Q^T from transposing
//    reads.
// S and dP are computed in both kernels (7 products instead of 5) in exchange
// for no atomic accumulation of dQ.
#include <mutex>
#include <type_traits>

#include "bf16_mfma.h"
#include "fa_internal.h"
#include "hip_common.h"

namespace fa {

namespace {

constexpr int kD = 128;
constexpr int kBc = 64;       // keys per tile (dQ kernel), query rows per tile (dK/dV kernel)
constexpr int kRow = kD * 2;  // 256 B per bf16 row; 16-byte units XOR-swizzled by swz(row)
constexpr int kTile = kBc * kRow;  // 16 KB
constexpr int NW = 8;

struct BwdArgs {
  const uint16_t* q;    // [B, Hq, Sq, D]
  const uint16_t* k;    // [B, Hkv, Sk, D]
  const uint16_t* v;
  const uint16_t* o;    // [B, Hq, Sq, D] forward output
  const uint16_t* dO;   // [B, Hq, Sq, D]
  const float* lse;     // [B, Hq, Sq] forward LSE (natural log)
  float* delta;         // [B, Hq, Sq] -D_i (written by the dQ kernel, read by dK/dV)
  float* lse2;          // [B, Hq, Sq] LSE * log2 e, +inf for a row without keys (likewise)
  uint16_t* dq;         // [B, Hq, Sq, D]
  uint16_t* dk;         // [B, Hkv, Sk, D]
  uint16_t* dv;
  int B, Hq, Hkv, Sq, Sk, causal;
  float scale;
};

// Unit c of row r sits at unit c ^ swz(r). The LDS serves 256 bytes (64
// banks) per clock. swz is a bijection on every 16 aligned rows, so the 16
// lanes of a row read (one unit of 16 different rows) hit 16 distinct
// 16-byte bank groups. Its top two bits are r & 3, so the four consecutive
// rows that a transposing read spans land in four distinct 64-byte blocks.
// (With r & 15 those four rows only permuted units inside one block: four
// lanes per bank.)
__device__ __forceinline__ int swz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

// Direct HBM -> LDS load of a 64-row tile: 16 blocks of 1 KB shared by the
// W wavefronts; lane l fills LDS unit (l & 15) of row 4j + (l >> 4) with the
// global unit that the row's swizzle stores there.
template <int W = NW>
__device__ __forceinline__ void load_rows(const __amdgpu_buffer_rsrc_t& rs, int r0, char* buf, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 16 / W; ++i) {
    const int j = wave * (16 / W) + i;
    const int r = 4 * j + (lane >> 4);
    const int unit = (lane & 15) ^ swz(r);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(buf + j * 1024), 16,
                                             (r0 + r) * kRow + unit * 16, 0, 0, 0);
  }
}

// This lane's index, formed where it is used. The asm is opaque, so the
// compiler neither hoists it nor keeps a copy live across a loop (where such
// a copy was spilled, and its reload waited for every load in flight).
__device__ __forceinline__ int lane_here() {
  int lo, id;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0" : "=v"(lo));
  asm volatile("v_mbcnt_hi_u32_b32 %0, -1, %1" : "=v"(id) : "v"(lo));
  return id;
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Row-operand offsets (A operand rows in kperm order, dims 16*kk + 8*hi).
__device__ __forceinline__ void row_offsets(int col, int hi, int (&off)[8]) {
  const int R = kperm(col);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) off[kk] = R * kRow + 16 * ((2 * kk + hi) ^ swz(R));
}
// Transposing-read offsets (A operand rows = dims 32*db + lane%32, k = rows
// 16*ks + 8*hi + e; add 16*ks rows): lane L of 16-lane group g addresses row
// 8*(g>>1) + 4*r + (L>>2), dims 32*db + 16*(g&1) + 4*(L&3). swz(r) depends
// on r & 15 only, so the offset does not depend on ks.
__device__ __forceinline__ void tr_offsets(int lane, int (&off)[4][2]) {
  const int g = lane >> 4, L = lane & 15;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int R = 8 * (g >> 1) + 4 * r + (L >> 2);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int u = 4 * db + 2 * (g & 1) + ((L & 3) >> 1);
      off[db][r] = R * kRow + 16 * (u ^ swz(R)) + 8 * (L & 1);
    }
  }
}
// The two reads (rows +0..3 and +4..7 of the 8-row group) have independent
// swizzles, hence two offsets; shifting both by 16 rows keeps them valid.
__device__ __forceinline__ bf16x8_t tr_operand(const char* base, int off0, int off1) {
  const uint2 v0 = lds_read_tr16(base + off0);
  const uint2 v1 = lds_read_tr16(base + off1);
  return __builtin_bit_cast(bf16x8_t, make_uint4(v0.x, v0.y, v1.x, v1.y));
}
// The same offsets in XOR form, one register each: with s = swz(row), unit
// (2*kk + hi) ^ s sits at byte 32*(kk ^ (s>>1)) + 16*(hi ^ (s&1)), so the
// kk-th row offset is X ^ (32*kk); the transposing offsets are Y_r ^ (64*db).
__device__ __forceinline__ int row_base(int R, int hi) {
  const int sw = swz(R);
  return R * kRow + 32 * (sw >> 1) + 16 * (hi ^ (sw & 1));
}
__device__ __forceinline__ void tr_bases(int lane, int (&y)[2]) {
  const int g = lane >> 4, L = lane & 15;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int R = 8 * (g >> 1) + 4 * r + (L >> 2);
    const int c0 = 32 * (g & 1) + 16 * ((L & 3) >> 1);
    y[r] = R * kRow + 8 * (L & 1) + (c0 ^ (16 * swz(R)));
  }
}

__device__ __forceinline__ bf16x8_t pack8(const f32x16_t& x, int base) {
  return __builtin_bit_cast(bf16x8_t, make_uint4(pack_bf16x2(x[base], x[base + 1]), pack_bf16x2(x[base + 2], x[base + 3]),
                                                 pack_bf16x2(x[base + 4], x[base + 5]), pack_bf16x2(x[base + 6], x[base + 7])));
}
// Store a 32 x 128 block held as C^T accumulators (lane: row `row`, dims
// 32*db + 8*gq + 4*hi .. +3) as bf16, multiplied by f.
__device__ __forceinline__ void store_rows(uint16_t* dst, const f32x16_t (&acc)[4], int hi, float f) {
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d = 32 * db + 8 * gq + 4 * hi;
      *reinterpret_cast<uint2*>(dst + d) = make_uint2(pack_bf16x2(acc[db][4 * gq] * f, acc[db][4 * gq + 1] * f),
                                                      pack_bf16x2(acc[db][4 * gq + 2] * f, acc[db][4 * gq + 3] * f));
    }
}

// ---------------------------------------------------------------- dQ
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdArgs a, int n_qtiles, int nbh) {
  // Two K and two V tile buffers, each its own LDS variable: the compiler can
  // then tell a tile's LDS reads from the loads filling the other pair and
  // does not make the reads wait for them.
  __shared__ __attribute__((aligned(16))) char k_lds0[kTile];
  __shared__ __attribute__((aligned(16))) char k_lds1[kTile];
  __shared__ __attribute__((aligned(16))) char v_lds0[kTile];
  __shared__ __attribute__((aligned(16))) char v_lds1[kTile];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hi = lane >> 5, col = lane & 31;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform copy
  constexpr int BR = 32 * NW;

  const int L = blockIdx.x;
  const int qt = a.causal ? (n_qtiles - 1 - L / nbh) : (L / nbh);
  const int e = L % nbh;
  const int G = a.Hq / a.Hkv;
  const int bg = e % (a.B * a.Hkv), j = e / (a.B * a.Hkv);
  const int b = bg / a.Hkv, g = bg % a.Hkv, h = g * G + j;
  const int Sq = a.Sq, Sk = a.Sk, off = Sk - Sq;
  const int q0 = qt * BR;
  int kend = Sk;
  if (a.causal) kend = min(Sk, q0 + BR + off);
  const int n_kt = kend > 0 ? (kend + kBc - 1) / kBc : 0;
  const size_t bh = (size_t)b * a.Hq + h, bgk = (size_t)b * a.Hkv + g;

  // Q and dO of this lane's row (B operands, dims 16*kk + 8*hi), its LSE in
  // log2 units (+inf for a row without keys, so that P = 0) and D.
  const int qrow = q0 + 32 * wave + col;
  bf16x8_t qreg[8], dreg[8];
  // D_i = sum_d dO_id O_id (fp32, bf16 pair products) from the dO row in
  // registers and the O row: half of the dims per half-wavefront, summed
  // across the halves; written for the dK/dV kernel.
  float lse2 = __builtin_inff(), dl = 0.f;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    uint4 x = make_uint4(0, 0, 0, 0), y = make_uint4(0, 0, 0, 0), z = make_uint4(0, 0, 0, 0);
    if (qrow < Sq) {
      x = *reinterpret_cast<const uint4*>(a.q + (bh * Sq + qrow) * kD + 16 * kk + 8 * hi);
      y = *reinterpret_cast<const uint4*>(a.dO + (bh * Sq + qrow) * kD + 16 * kk + 8 * hi);
      z = *reinterpret_cast<const uint4*>(a.o + (bh * Sq + qrow) * kD + 16 * kk + 8 * hi);
    }
    qreg[kk] = __builtin_bit_cast(bf16x8_t, x);
    dreg[kk] = __builtin_bit_cast(bf16x8_t, y);
    dl = dot2_bf16(y.x, z.x, dl);
    dl = dot2_bf16(y.y, z.y, dl);
    dl = dot2_bf16(y.z, z.z, dl);
    dl = dot2_bf16(y.w, z.w, dl);
  }
  dl = xor32_sum(dl);
  if (qrow < Sq) {
    const float l = a.lse[bh * Sq + qrow];
    lse2 = l == kNegInf ? __builtin_inff() : l * kLog2e;
    if (hi == 0) {
      a.delta[bh * Sq + qrow] = -dl;  // negated: the dK/dV kernel starts dP from it
      a.lse2[bh * Sq + qrow] = lse2;
    }
  }
  const float c = a.scale * kLog2e;

  f32x16_t acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  const __amdgpu_buffer_rsrc_t k_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.k + bgk * (size_t)Sk * kD), (short)0, Sk * kRow, 0x00020000);
  const __amdgpu_buffer_rsrc_t v_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.v + bgk * (size_t)Sk * kD), (short)0, Sk * kRow, 0x00020000);
  int r_off[8], t_off[4][2];
  row_offsets(col, hi, r_off);
  tr_offsets(lane, t_off);

  if (n_kt > 0) {
    load_rows(k_rs, 0, k_lds0, wave, lane);
    load_rows(v_rs, 0, v_lds0, wave, lane);
  }
  wait_vmem();
  __syncthreads();

  // Key tiles [0, n_full) are seen whole by every row of the workgroup (its
  // first row has the smallest key limit; rows past Sq have lse2 = +inf and
  // give 0 either way). They run a loop without the mask: vector-ALU work
  // does not overlap the matrix cores' on a SIMD, and the per-element key
  // index, compare and select were 40% of this loop's VALU work. The few
  // tiles at the diagonal or the Sk tail run the masked copy. Each tile ends
  // in one barrier, in either loop.
  const int lim_wg = a.causal ? min(Sk - 1, q0 + off) : Sk - 1;
  const int n_full = max(0, min(n_kt, (lim_wg + 1) / kBc));
  auto tile = [&](int t, auto masked, auto par) {
    constexpr int PAR = decltype(par)::value;  // t & 1
    // The lane offsets pass through here unchanged: otherwise the compiler
    // forms a copy of them per buffer outside the loop, which spills.
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) asm volatile("" : "+v"(r_off[kk]));
#pragma unroll
    for (int db = 0; db < 4; ++db) asm volatile("" : "+v"(t_off[db][0]), "+v"(t_off[db][1]));
    if (t + 1 < n_kt) {
      load_rows(k_rs, (t + 1) * kBc, PAR ? k_lds0 : k_lds1, wave, lane);
      load_rows(v_rs, (t + 1) * kBc, PAR ? v_lds0 : v_lds1, wave, lane);
    }
    const char* kl = PAR ? k_lds1 : k_lds0;
    const char* vl = PAR ? v_lds1 : v_lds0;
    // S^T = K Q^T and dP^T = V dO^T: register i of lane l, half h2, is key
    // 32*h2 + 16*(i/8) + 8*hi + (i%8) of the tile, query row `qrow`.
    f32x16_t s[2], dp[2];
    // dP^T starts from -D instead of zero: every accumulator register of this
    // lane belongs to query row `qrow`, so the products leave dP - D directly
    // (16 moves per tile in place of 32 subtractions). The splat is formed
    // here each tile: kept across the loop it would hold 16 more registers.
    float ndl1 = -dl;
    asm volatile("" : "+v"(ndl1));
    f32x16_t ndl;
#pragma unroll
    for (int i = 0; i < 16; ++i) ndl[i] = ndl1;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(kl + r_off[kk] + 32 * h2 * kRow);
        const bf16x8_t va = *reinterpret_cast<const bf16x8_t*>(vl + r_off[kk] + 32 * h2 * kRow);
        s[h2] = kk == 0 ? mfma32_first(ka, qreg[kk]) : mfma32(ka, qreg[kk], s[h2]);
        dp[h2] = mfma32(va, dreg[kk], kk == 0 ? ndl : dp[h2]);
      }
    }
    // P^T = exp2(S^T c - lse2) with the causal / ragged-tail mask (masked
    // tiles only), dS^T.
    bf16x8_t dsf[4];
    auto ds_tile = [&](auto masked) {
      // Key t*kBc + 8*hi + k is visible to this lane's row iff k <= rel, for
      // k = 32*h2 + 16*(i/8) + i%8 (a constant per element). rel is formed
      // here from the lane index, so nothing of it stays live across the
      // loop (a per-lane key limit kept there was spilled with an operand).
      int rel = 0;
      if constexpr (decltype(masked)::value) {
        const int lh = lane_here();
        const int row = q0 + 32 * wave_s + (lh & 31);
        const int lim = a.causal ? min(Sk - 1, row + off) : Sk - 1;
        rel = lim - t * kBc - 8 * (lh >> 5);
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float arg = __builtin_fmaf(s[h2][i], c, -lse2);
          if constexpr (decltype(masked)::value) {
            // Masked entries get a -inf argument (exp2 -> 0): a select, not a branch per element.
            arg = 32 * h2 + 16 * (i >> 3) + (i & 7) > rel ? kNegInf : arg;
          }
          s[h2][i] = fast_exp2(arg) * dp[h2][i];  // P (dP - D)
        }
        dsf[2 * h2] = pack8(s[h2], 0);
        dsf[2 * h2 + 1] = pack8(s[h2], 8);
      }
    };
    ds_tile(masked);
    // dQ^T += K^T dS^T (k = keys 16*ks + 8*hi + e).
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8_t kt = tr_operand(kl + 16 * ks * kRow, t_off[db][0], t_off[db][1]);
        acc[db] = mfma32(kt, dsf[ks], acc[db]);
      }
    wait_vmem();
    __syncthreads();
  };
  // Unrolled by two, so that every tile names its buffers at compile time.
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  int t = 0;
  for (; t + 1 < n_full; t += 2) {
    tile(t, std::false_type{}, P0{});
    tile(t + 1, std::false_type{}, P1{});
  }
  for (; t < n_kt; ++t) {
    if (t & 1)
      tile(t, std::bool_constant<true>{}, P1{});
    else if (t < n_full)
      tile(t, std::false_type{}, P0{});
    else
      tile(t, std::true_type{}, P0{});
  }
  if (qrow < Sq) store_rows(a.dq + (bh * Sq + qrow) * kD, acc, hi, a.scale);
}

// ---------------------------------------------------------------- dK, dV
// KW wavefronts of 32 keys each, two per SIMD. (Four wavefronts, one per
// SIMD with the full register file, avoid the few spills of this
// configuration but measured 16% slower overall.)
constexpr int KW = 8;
__global__ __launch_bounds__(64 * KW) __attribute__((amdgpu_waves_per_eu(KW / 4, KW / 4)))
void bwd_dkdv_kernel(BwdArgs a, int n_ktiles, int nbg) {
  // Double-buffered Q, dO, LSE and D tiles, each buffer its own LDS variable
  // (named at compile time by the step loops, unrolled by two), so that a
  // step's LDS reads do not wait for the loads filling the other buffers.
  // The Q/dO ring is read every step through row and transposing offsets.
  // Its wider alignment places it first, below 64 KB, where a DS
  // instruction's 16-bit offset holds each buffer's base; the resident V
  // block follows it. The other way round every ring read took an add.
  __shared__ __attribute__((aligned(1024))) char q_lds0[kTile];
  __shared__ __attribute__((aligned(1024))) char q_lds1[kTile];
  __shared__ __attribute__((aligned(1024))) char o_lds0[kTile];  // dO
  __shared__ __attribute__((aligned(1024))) char o_lds1[kTile];
  __shared__ __attribute__((aligned(16))) float st_lse0[kBc];
  __shared__ __attribute__((aligned(16))) float st_lse1[kBc];
  __shared__ __attribute__((aligned(16))) float st_d0[kBc];
  __shared__ __attribute__((aligned(16))) float st_d1[kBc];
  __shared__ __attribute__((aligned(16))) char v_res[32 * KW * kRow];  // this workgroup's V rows
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hi = lane >> 5, col = lane & 31;
  constexpr int BK = 32 * KW;  // keys per workgroup
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform copy (scalar branches)

  // Key tiles with the most query rows first (causal: the first ones).
  const int L = blockIdx.x;
  const int kt = a.causal ? L / nbg : (n_ktiles - 1 - L / nbg);
  const int e = L % nbg;
  const int b = e / a.Hkv, g = e % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int Sq = a.Sq, Sk = a.Sk, off = Sk - Sq;
  const int kw0 = kt * BK + 32 * wave;  // this wavefront's first key
  const int key = kw0 + col;           // this lane's key (column)
  const size_t bgk = (size_t)b * a.Hkv + g;

  // K of this lane's key in registers (B operand of S = Q K^T, dims
  // 16*kk + 8*hi); the workgroup's V rows resident in LDS (B operand of
  // dP = dO V^T, read per step), rows past Sk zero.
  bf16x8_t kreg[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    uint4 x = make_uint4(0, 0, 0, 0);
    if (key < Sk) x = *reinterpret_cast<const uint4*>(a.k + (bgk * Sk + key) * kD + 16 * kk + 8 * hi);
    kreg[kk] = __builtin_bit_cast(bf16x8_t, x);
  }
  {
    const __amdgpu_buffer_rsrc_t vs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.v + bgk * (size_t)Sk * kD), (short)0, Sk * kRow, 0x00020000);
#pragma unroll
    for (int c4 = 0; c4 < BK / 64; ++c4) load_rows<KW>(vs, kt * BK + 64 * c4, v_res + c4 * kTile, wave, lane);
  }
  f32x16_t dk[4], dv[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dk[db][i] = 0.f;
      dv[db][i] = 0.f;
    }
  const float c = a.scale * kLog2e;

  // Query tiles that can see any key of this workgroup: rows q with
  // q + off >= first key.
  const int n_qt = (Sq + kBc - 1) / kBc;
  const int qt0 = a.causal ? max(0, (kt * BK - off) / kBc) : 0;
  const int per_head = max(0, n_qt - qt0);
  const int n_steps = per_head * G;
  // Query tiles [q_lo, q_hi) are seen whole by every key of the workgroup
  // (no causal cut inside, no row past Sq, no key past Sk); their steps run a
  // loop without the mask, after the masked steps of the other tiles (the
  // diagonal band and the Sq tail). Step s < G*n_mask is masked tile
  // s % n_mask of query head s / n_mask; later steps take the whole tiles
  // head by head.
  const int klast = kt * BK + BK - 1;
  int q_lo = qt0, q_hi = qt0;
  if (klast < Sk) {
    const int need = klast - off;  // a whole tile starts at a row >= need
    const int qf = a.causal ? max(qt0, need <= 0 ? 0 : (need + kBc - 1) / kBc) : qt0;
    const int qe = Sq / kBc;  // tiles wholly below Sq
    if (qf < qe) {
      q_lo = qf;
      q_hi = qe;
    }
  }
  const int n_full = q_hi - q_lo, n_mask = per_head - n_full;
  const int n_mask_steps = G * n_mask;
  auto step_tile = [&](int step, int& jh, int& qt) {
    if (step < n_mask_steps) {
      jh = step / n_mask;
      const int i = step % n_mask;
      qt = i < q_lo - qt0 ? qt0 + i : q_hi + (i - (q_lo - qt0));
    } else {
      jh = (step - n_mask_steps) / n_full;
      qt = q_lo + (step - n_mask_steps) % n_full;
    }
  };

  int r_base = row_base(kperm(col), hi);
  int t_base[2];
  tr_bases(lane, t_base);

  auto issue = [&](int step, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    int jh, qt;
    step_tile(step, jh, qt);
    // The lane's load offsets are re-formed here on every call: hoisted out
    // of the step loops by the compiler, they were spilled and reloaded.
    const int ln = lane_here();
    const size_t bh = (size_t)b * a.Hq + g * G + jh;
    const __amdgpu_buffer_rsrc_t qs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.q + bh * (size_t)Sq * kD), (short)0, Sq * kRow, 0x00020000);
    const __amdgpu_buffer_rsrc_t ds = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.dO + bh * (size_t)Sq * kD), (short)0, Sq * kRow, 0x00020000);
    load_rows<KW>(qs, qt * kBc, buf ? q_lds1 : q_lds0, wave_u, ln);
    load_rows<KW>(ds, qt * kBc, buf ? o_lds1 : o_lds0, wave_u, ln);
    if (wave_u == 0) {
      const __amdgpu_buffer_rsrc_t ls = __builtin_amdgcn_make_buffer_rsrc(
          a.lse2 + bh * (size_t)Sq, (short)0, Sq * 4, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ls, (__attribute__((address_space(3))) void*)(buf ? st_lse1 : st_lse0), 4,
                                               (qt * kBc + ln) * 4, 0, 0, 0);
    } else if (wave_u == 1) {
      const __amdgpu_buffer_rsrc_t dsr = __builtin_amdgcn_make_buffer_rsrc(
          a.delta + bh * (size_t)Sq, (short)0, Sq * 4, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(dsr, (__attribute__((address_space(3))) void*)(buf ? st_d1 : st_d0), 4,
                                               (qt * kBc + ln) * 4, 0, 0, 0);
    }
  };

  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  if (n_steps > 0) issue(0, P0{});
  wait_vmem();
  __syncthreads();

  auto step = [&](int st, auto masked, auto par) {
    constexpr int buf = decltype(par)::value;  // st & 1
    // The per-step offsets base ^ const are cheap to form where they are
    // used; kept from outside the loop they would be spilled.
    asm volatile("" : "+v"(r_base), "+v"(t_base[0]), "+v"(t_base[1]));
    if (st + 1 < n_steps) issue(st + 1, std::integral_constant<int, buf ^ 1>{});
    int jh_unused, qt_cur;
    step_tile(st, jh_unused, qt_cur);
    const int q0 = qt_cur * kBc;
    const char* ql = buf ? q_lds1 : q_lds0;
    const char* ol = buf ? o_lds1 : o_lds0;
    const float* sl = buf ? st_lse1 : st_lse0;
    const float* sd = buf ? st_d1 : st_d0;
#pragma unroll
    for (int hq = 0; hq < 2; ++hq) {
      // S = Q K^T and dP = dO V^T for rows 32*hq .. +31 of the tile: register
      // i of lane l is row 32*hq + 16*(i/8) + 8*hi + (i%8), key `key`.
      // S first, then dP: only one product's operands are live at a time.
      f32x16_t s, dp;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int ro = (r_base ^ (32 * kk)) + 32 * hq * kRow;
        const bf16x8_t qa = *reinterpret_cast<const bf16x8_t*>(ql + ro);
        s = kk == 0 ? mfma32_first(qa, kreg[kk]) : mfma32(qa, kreg[kk], s);
      }
      // This lane's V row in v_res, formed here from the lane index: kept
      // across the loop, it was spilled, and its reload mid-step waited for
      // the prefetch loads.
      const int lh = lane_here();
      const int v_base = row_base(32 * wave_u + (lh & 31), lh >> 5);
      // dP starts from the staged -D of each register's row, so the products
      // leave dP - D directly (no subtraction per element).
      f32x16_t nd;
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        const int rb = 32 * hq + 16 * h8 + 8 * hi;
        const float4 d0 = *reinterpret_cast<const float4*>(sd + rb);
        const float4 d1 = *reinterpret_cast<const float4*>(sd + rb + 4);
        nd[8 * h8 + 0] = d0.x;
        nd[8 * h8 + 1] = d0.y;
        nd[8 * h8 + 2] = d0.z;
        nd[8 * h8 + 3] = d0.w;
        nd[8 * h8 + 4] = d1.x;
        nd[8 * h8 + 5] = d1.y;
        nd[8 * h8 + 6] = d1.z;
        nd[8 * h8 + 7] = d1.w;
      }
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int ro = (r_base ^ (32 * kk)) + 32 * hq * kRow;
        const bf16x8_t oa = *reinterpret_cast<const bf16x8_t*>(ol + ro);
        const bf16x8_t vb = *reinterpret_cast<const bf16x8_t*>(v_res + (v_base ^ (32 * kk)));
        dp = mfma32(oa, vb, kk == 0 ? nd : dp);
      }
      // P and dS; rows past Sq, masked keys and keys past Sk give 0.
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        const int rb = 32 * hq + 16 * h8 + 8 * hi;  // first row of these 8 registers
        const float4 l0 = *reinterpret_cast<const float4*>(sl + rb);
        const float4 l1 = *reinterpret_cast<const float4*>(sl + rb + 4);
        const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
        // Rows x of these 8 that this lane's key sees: x in [xlo, xhi) (row
        // below Sq, causal key <= row + off, key below Sk). Masked entries
        // get a -inf argument (exp2 -> 0), and a row without keys (LSE -inf)
        // a +inf one: selects, where the per-element conditional form
        // compiled to a divergent branch for every element.
        // The staged LSE is already in log2 units (+inf for a row without
        // keys), formed once per row by the dQ kernel.
        if constexpr (!decltype(masked)::value) {
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            const int i = 8 * h8 + x;
            const float p = fast_exp2(__builtin_fmaf(s[i], c, -lv[x]));
            s[i] = p;
            dp[i] = p * dp[i];  // P (dP - D)
          }
        } else {
          const int key_h = kt * BK + 32 * wave_u + (lane_here() & 31);
          const int xlo = a.causal ? key_h - off - (q0 + rb) : 0;
          const int xhi = key_h < Sk ? Sq - (q0 + rb) : 0;
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            const int i = 8 * h8 + x;
            const float p = fast_exp2(((x >= xlo) & (x < xhi)) ? __builtin_fmaf(s[i], c, -lv[x]) : kNegInf);
            s[i] = p;
            dp[i] = p * dp[i];  // P (dP - D)
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // dV^T += dO^T P and dK^T += Q^T dS (k = rows 16*ks + 8*hi + e of this half).
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8_t pf = pack8(s, 8 * ks);
        const bf16x8_t sf = pack8(dp, 8 * ks);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int ro = (32 * hq + 16 * ks) * kRow;
          const int o0 = t_base[0] ^ (64 * db), o1 = t_base[1] ^ (64 * db);
          dv[db] = mfma32(tr_operand(ol + ro, o0, o1), pf, dv[db]);
          dk[db] = mfma32(tr_operand(ql + ro, o0, o1), sf, dk[db]);
        }
      }
    }
    wait_vmem();
    __syncthreads();
  };
  // Both loops unrolled by two (buffer = step & 1 at compile time).
  int st = 0;
  for (; st + 1 < n_mask_steps; st += 2) {
    step(st, std::true_type{}, P0{});
    step(st + 1, std::true_type{}, P1{});
  }
  if (st < n_mask_steps) {
    step(st, std::true_type{}, P0{});
    ++st;
  }
  if (st & 1) {
    if (st < n_steps) step(st, std::false_type{}, P1{});
    ++st;
  }
  for (; st + 1 < n_steps; st += 2) {
    step(st, std::false_type{}, P0{});
    step(st + 1, std::false_type{}, P1{});
  }
  if (st < n_steps) step(st, std::false_type{}, P0{});
  if (key < Sk) {
    store_rows(a.dk + (bgk * Sk + key) * kD, dk, hi, a.scale);
    store_rows(a.dv + (bgk * Sk + key) * kD, dv, hi, 1.f);
  }
}

}  // namespace

// Per-row arrays of the backward (-D_i, then LSE_i in log2 units) for the entry
// point that allocates nothing. Each GPU the library runs on holds its own
// copy until the process ends; every call on that GPU shares it, so calls
// that overlap on one GPU race. The dQ kernel writes every row < Sq before
// the dK/dV kernel reads any, and reads past Sq return zeros through the
// buffer bounds, so nothing in it needs clearing between calls.
static __device__ __align__(256) char scratch[kBwdScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxScratchDevices] = {};
}  // namespace

// Device address of `scratch` on the current device. In host code the array's
// name is only a host-side handle, so the address is asked of the runtime once
// per device, with that device current, and kept.
hipError_t bwd_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255) != 0) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *ptr = g_scratch_addr[dev];
  return hipSuccess;
}

hipError_t launch_attention_bwd(const BwdLaunch& l, hipStream_t s) {
  BwdArgs a;
  a.q = reinterpret_cast<const uint16_t*>(l.q);
  a.k = reinterpret_cast<const uint16_t*>(l.k);
  a.v = reinterpret_cast<const uint16_t*>(l.v);
  a.o = reinterpret_cast<const uint16_t*>(l.o);
  a.dO = reinterpret_cast<const uint16_t*>(l.dO);
  a.lse = l.lse;
  a.delta = l.delta;
  a.lse2 = l.lse2;
  a.dq = reinterpret_cast<uint16_t*>(l.dq);
  a.dk = reinterpret_cast<uint16_t*>(l.dk);
  a.dv = reinterpret_cast<uint16_t*>(l.dv);
  a.B = l.B; a.Hq = l.Hq; a.Hkv = l.Hkv; a.Sq = l.Sq; a.Sk = l.Sk; a.causal = l.causal;
  a.scale = l.scale;
  const int64_t rows = (int64_t)l.B * l.Hq * l.Sq;
  if (rows > 0) {
    const int n_qtiles = (l.Sq + 32 * NW - 1) / (32 * NW);
    const int nbh = l.B * l.Hq;
    hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)((int64_t)n_qtiles * nbh)), dim3(64 * NW), 0, s, a, n_qtiles, nbh);
  }
  if (l.Sk > 0) {
    const int n_ktiles = (l.Sk + 32 * KW - 1) / (32 * KW);
    const int nbg = l.B * l.Hkv;
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)((int64_t)n_ktiles * nbg)), dim3(64 * KW), 0, s, a, n_ktiles, nbg);
  }
  return hipGetLastError();
}

}  // namespace fa
