// fp8 exact-attention prefill on gfx950 matrix cores (e4m3 inputs, fp32 accumulation).
//
// Same method as the bf16 kernel ("FIA / FlashAttention" Q&A, section 1;
// "FasterTransformer vs FlashAttention", section 3: Q block outer, K/V
// blocks streamed through on-chip memory, running max and normaliser), with
// Q, K and V stored as OCP e4m3fn codes and a fp32 dequantisation scale per
// (batch, head) ("FIA / FlashAttention" Q&A, section 3: FP8 inference
// kernels). Both contractions run on v_mfma_f32_32x32x64_f8f6f4: S^T = K Q^T
// on the fp8 inputs, and O^T = V^T P^T with the probabilities P rounded to
// e4m3 (nearest even) for the second product. The score multiplier absorbs
// q_scale * k_scale, the final division absorbs v_scale.
//
// gfx950 design.
//  * Workgroup = 8 wavefronts x 32 query rows; K/V tiles of 64 keys (8 KB
//    each in fp8) go HBM -> LDS with buffer_load ... lds, two buffers each.
//  * One 32x32x64 MFMA covers 64 of the contraction; A and B lanes pair up
//    by (lane / 32, byte), whatever the hardware's internal k order, so:
//    - S^T: lane (row = key, h = lane / 32) of K holds dims 64*kk + 32*h ..
//      +31 (32 contiguous bytes, two 16-byte LDS reads); Q^T lanes hold the
//      same dims of their query row, in registers for the whole row block.
//    - O^T: the 32 scores a lane owns after the first product (query column
//      lane % 32, keys 32*h2 + 8*(i/4) + 4*(lane/32) + i%4 for register i of
//      half h2) become its 32 P bytes, byte e = 16*h2 + i; the V^T lanes with
//      the same lane / 32 must hold V of exactly those keys in the same byte
//      order, which gfx950's transposing byte read (ds_read_b64_tr_b8)
//      delivers: within 16 lanes, lane i receives byte i % 8 of the 8-byte
//      chunks addressed by lanes 2j + i / 8, j = 0..7. Source lanes 2j and
//      2j + 1 address the same key at adjacent 8-dim blocks, so lane i gets
//      8 keys of dim d0 + i.
//  * The normaliser is the fp32 sum of the unrounded P (no fp8 dot product
//    on this chip); the LSE uses the same sum.
//  * LDS rows are 128 bytes with their 16-byte units XOR-swizzled per row
//    (different functions for K and V, matched to their read patterns) so the
//    lanes of one read pass use distinct banks.
#include <type_traits>

#include "fa_internal.h"
#include "hip_common.h"

namespace fa {

namespace {

constexpr int kD = 128;
constexpr int kBc = 64;         // keys per tile
constexpr int kRow = kD;        // bytes per fp8 row
constexpr int kTile = kBc * kRow;  // 8 KB
constexpr float kTau = 8.0f;    // lazy max threshold (log2 units): P <= 2^8 < 448
constexpr float kSumBound = 256.0f;  // 2^kTau: a sum of weights at or below it bounds each of them

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16_t mfma8(i32x8_t a, i32x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma8_first(i32x8_t a, i32x8_t b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, f32x16_t{}, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ i32x2_t lds_read_tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2_t*)(p));
}

// 16-byte unit swizzles (unit u of row r is stored at unit u ^ f(r)).
__device__ __forceinline__ int swz_k(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz_v(int r) { return (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2) | ((r >> 2) & 1); }

// Key of P byte e for lanes with lane / 32 == h (see the header).
__device__ __forceinline__ int key_of_byte(int h, int e) {
  return 32 * (e >> 4) + 8 * ((e & 15) >> 2) + 4 * h + (e & 3);
}

struct Fp8Args {
  const uint8_t* q;        // [B, Hq, Sq, D] e4m3fn
  const uint8_t* k;        // [B, Hkv, Sk, D]
  const uint8_t* v;
  const float* q_scale;    // [B, Hq]
  const float* k_scale;    // [B, Hkv]
  const float* v_scale;    // [B, Hkv]
  uint16_t* out;           // [B, Hq, Sq, D] bf16
  float* lse;              // [B, Hq, Sq]
  int B, Hq, Hkv, Sq, Sk, causal;
  float scale;
};

constexpr int NW = 8;
constexpr int BR = 32 * NW;

__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_fp8_kernel(Fp8Args a, int n_qtiles, int nbh) {
  __shared__ __attribute__((aligned(16))) char k_lds[2 * kTile];
  __shared__ __attribute__((aligned(16))) char v_lds[2 * kTile];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int hi = lane >> 5, col = lane & 31;

  // ---- work unit: heaviest causal tiles first; equal ids mod 8 share a KV head
  const int L = blockIdx.x;
  const int qt = a.causal ? (n_qtiles - 1 - L / nbh) : (L / nbh);
  const int e_ = L % nbh;
  const int G = a.Hq / a.Hkv;
  const int bg = e_ % (a.B * a.Hkv), j_ = e_ / (a.B * a.Hkv);
  const int b = bg / a.Hkv, g = bg % a.Hkv, h = g * G + j_;
  const int Sq = a.Sq, Sk = a.Sk;
  const int q0 = qt * BR;
  const int off = Sk - Sq;
  int kend = Sk;
  if (a.causal) kend = min(Sk, q0 + BR + off);
  const int n_kt = kend > 0 ? (kend + kBc - 1) / kBc : 0;

  const size_t bh = (size_t)b * a.Hq + h;
  const uint8_t* Q = a.q + bh * (size_t)Sq * kD;
  const uint8_t* K = a.k + ((size_t)b * a.Hkv + g) * (size_t)Sk * kD;
  const uint8_t* V = a.v + ((size_t)b * a.Hkv + g) * (size_t)Sk * kD;
  const float qs = a.q_scale[bh], ks = a.k_scale[(size_t)b * a.Hkv + g], vs = a.v_scale[(size_t)b * a.Hkv + g];
  const float c = a.scale * qs * ks * kLog2e;

  // ---- Q^T (B operand): query row q0 + 32*wave + col, dims 64*kk + 32*hi .. +31
  const int qrow = q0 + 32 * wave + col;
  i32x8_t qreg[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    uint4 lo = make_uint4(0, 0, 0, 0), up = make_uint4(0, 0, 0, 0);
    if (qrow < Sq) {
      const uint4* p = reinterpret_cast<const uint4*>(Q + (size_t)qrow * kD + 64 * kk + 32 * hi);
      lo = p[0];
      up = p[1];
    }
    qreg[kk] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)up.x, (int)up.y, (int)up.z, (int)up.w};
  }

  float m = kNegInf, le[4] = {0.f, 0.f, 0.f, 0.f};
  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;

  // ---- direct HBM -> LDS loads: one 1 KB block (8 rows) per wavefront and
  // tile; lane l fills LDS unit (l & 7) of row 8*wave + (l >> 3), fetching the
  // global unit that the row's swizzle stores there.
  const __amdgpu_buffer_rsrc_t k_rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(K), (short)0, Sk * kRow, 0x00020000);
  const __amdgpu_buffer_rsrc_t v_rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(V), (short)0, Sk * kRow, 0x00020000);
  const int dl_row = 8 * wave + (lane >> 3), dl_pos = lane & 7;
  auto load_tile = [&](const __amdgpu_buffer_rsrc_t& rs, int k0, char* buf, bool is_v) {
    const int unit = dl_pos ^ (is_v ? swz_v(dl_row) : swz_k(dl_row));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(buf + wave * 1024), 16,
                                             (k0 + dl_row) * kRow + unit * 16, 0, 0, 0);
  };
  auto load_k = [&](int t) { load_tile(k_rs, t * kBc, k_lds + (t & 1) * kTile, false); };
  auto load_v = [&](int t) { load_tile(v_rs, t * kBc, v_lds + (t & 1) * kTile, true); };
  auto wait_loads = [] { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // K read offsets: row 32*h2 + col, units 4*kk + 2*hi and +1.
  int k_off[2][2][2];  // [h2][kk][unit]
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int r = 32 * h2 + col;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int x = 0; x < 2; ++x) k_off[h2][kk][x] = r * kRow + 16 * ((4 * kk + 2 * hi + x) ^ swz_k(r));
  }
  // V transposing-read offsets: group gq = lane >> 4, index i = lane & 15 as
  // source lane 2j + s: key key_of_byte(gq >> 1, 8*rr + j), unit 2*db + (gq & 1), half s.
  int v_off[4][4];  // [db][rr]
  {
    const int gq = lane >> 4, i = lane & 15, jj = i >> 1, s = i & 1;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int key = key_of_byte(gq >> 1, 8 * rr + jj);
#pragma unroll
      for (int db = 0; db < 4; ++db) v_off[db][rr] = key * kRow + 16 * ((2 * db + (gq & 1)) ^ swz_v(key)) + 8 * s;
    }
  }

  auto qk = [&](int kbuf, f32x16_t (&s)[2]) {
    const char* kl = k_lds + kbuf * kTile;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint4 x0 = *reinterpret_cast<const uint4*>(kl + k_off[h2][kk][0]);
        const uint4 x1 = *reinterpret_cast<const uint4*>(kl + k_off[h2][kk][1]);
        const i32x8_t av = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        s[h2] = kk == 0 ? mfma8_first(av, qreg[kk]) : mfma8(av, qreg[kk], s[h2]);
      }
  };

  const int wq0 = q0 + 32 * wave;
  auto active = [&](int t) { return !(a.causal && t * kBc > wq0 + 31 + off); };
  auto mask = [&](int t, f32x16_t (&s)[2]) {
    const int lim = a.causal ? min(Sk - 1, qrow + off) : Sk - 1;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (t * kBc + 32 * h2 + 8 * (i >> 2) + 4 * hi + (i & 3) > lim) s[h2][i] = kNegInf;
  };
  auto update_max = [&](const f32x16_t (&s)[2]) {
    // Max over the lane's 32 scores as a tree of 3-input maxes (v_max3_f32).
    auto max3 = [](float x, float y, float z) { return fmaxf(fmaxf(x, y), z); };
    auto sv = [&](int i) { return s[i >> 4][i & 15]; };
    float t[11];
#pragma unroll
    for (int i = 0; i < 10; ++i) t[i] = max3(sv(3 * i), sv(3 * i + 1), sv(3 * i + 2));
    t[10] = fmaxf(sv(30), sv(31));
    float mx = fmaxf(max3(max3(t[0], t[1], t[2]), max3(t[3], t[4], t[5]), max3(t[6], t[7], t[8])), fmaxf(t[9], t[10]));
    mx = xor32_max(mx) * c;
    const bool need = mx > m + kTau;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(need) != 0, 0)) {
      asm volatile("");
      const float mn = need ? mx : m;
      const float alpha = need ? fast_exp2(m - mn) : 1.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) le[j] *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      m = mn;
    }
  };
  // P = exp2(s*c - m) -> e4m3 bytes (byte 16*h2 + i) with the running max as
  // it stands, and the tile's fp32 sums te[w] (each over 8 of the lane's
  // scores).
  // P bytes of the current tile, kept in one place across tiles: each
  // conversion below keeps the other half of its register, so giving it the
  // previous tile's word (overwritten in full by the pair of conversions)
  // saves a register clear or copy per word.
  int pw[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  auto exps = [&](const f32x16_t (&s)[2], float (&te)[4]) {
    const float mu = m == kNegInf ? 0.f : m;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float p[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) p[x] = fast_exp2(__builtin_fmaf(s[h2][4 * w + x], c, -mu));
        int& word = pw[4 * h2 + w];
        word = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], word, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], word, true);
        const float g = (p[0] + p[1]) + (p[2] + p[3]);
        te[w] = h2 == 0 ? g : te[w] + g;
      }
  };
  // O^T += V^T P^T; with kb >= 0 the next tile's S^T from K buffer kb is
  // computed in the same straight-line block, one QK product after each PV
  // product.
  auto pv_qk = [&](int vbuf, int kb, f32x16_t (&n)[2]) {
    const i32x8_t pf = {pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};
    const char* vl = v_lds + vbuf * kTile;
    const char* kl = k_lds + (kb < 0 ? 0 : kb) * kTile;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const i32x2_t r0 = lds_read_tr8(vl + v_off[db][0]);
      const i32x2_t r1 = lds_read_tr8(vl + v_off[db][1]);
      const i32x2_t r2 = lds_read_tr8(vl + v_off[db][2]);
      const i32x2_t r3 = lds_read_tr8(vl + v_off[db][3]);
      const i32x8_t va = {r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y};
      o[db] = mfma8(va, pf, o[db]);
      if (kb >= 0) {
        const int h2 = db >> 1, kk = db & 1;
        const uint4 x0 = *reinterpret_cast<const uint4*>(kl + k_off[h2][kk][0]);
        const uint4 x1 = *reinterpret_cast<const uint4*>(kl + k_off[h2][kk][1]);
        const i32x8_t av = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        n[h2] = kk == 0 ? mfma8_first(av, qreg[kk]) : mfma8(av, qreg[kk], n[h2]);
      }
    }
  };
  auto add_sums = [&](const float (&te)[4]) {
#pragma unroll
    for (int w = 0; w < 4; ++w) le[w] += te[w];
  };

  auto prefetch = [&](int t) {
    if (t + 2 < n_kt) load_k(t + 2);
    if (t + 1 < n_kt) load_v(t + 1);
  };

  // ---- prologue
  f32x16_t sc[2];
  if (n_kt > 0) {
    load_k(0);
    load_v(0);
    if (n_kt > 1) load_k(1);
  }
  wait_loads();
  __syncthreads();
  if (n_kt > 0 && active(0)) qk(0, sc);
  __syncthreads();

  // Tiles below the whole workgroup's diagonal and inside Sk need no mask:
  // a branch-free main loop, unrolled by two so the two score arrays swap
  // roles (no copies) and the buffer parity is a compile-time constant. The
  // next tile's scores are computed even past the last tile (from a stale
  // buffer, then discarded).
  int n_main = Sk / kBc;
  if (a.causal) n_main = min(n_main, max(0, (q0 + off + 1) / kBc));
  n_main = min(n_main, n_kt);
  auto main_step = [&](auto par, int t, f32x16_t (&cur)[2], f32x16_t (&nxt)[2]) {
    constexpr int PAR = decltype(par)::value;
    prefetch(t);
    // The lazy max only has to keep every weight at or below 2^kTau, and a
    // lane's sum of 8 weights bounds each of them: the tile's weights are
    // first formed with the max as it stands, and only if some sum exceeds
    // 2^kTau (the first tile of a row, or scores that rose by about kTau) is
    // the tile redone with the row max and the lazy move of the max. That
    // takes the max tree and its cross-lane exchange and vote off the common
    // path, where they stood between the scores and the first exponential.
    float te[4];
    bool redo = true;
    if (__builtin_amdgcn_ballot_w64(m == kNegInf) == 0) {
      exps(cur, te);
      const float big = fmaxf(fmaxf(te[0], te[1]), fmaxf(te[2], te[3]));
      redo = __builtin_amdgcn_ballot_w64(!(big <= kSumBound)) != 0;
    }
    if (__builtin_expect(redo, 0)) {
      update_max(cur);
      exps(cur, te);
    }
    add_sums(te);
    pv_qk(PAR, 1 - PAR, nxt);
    wait_loads();
    __syncthreads();
  };
  int t = 0;
  {
    f32x16_t sn[2];
    for (; t + 1 < n_main; t += 2) {
      main_step(std::integral_constant<int, 0>{}, t, sc, sn);
      main_step(std::integral_constant<int, 1>{}, t + 1, sn, sc);
    }
    if (t < n_main) {
      main_step(std::integral_constant<int, 0>{}, t, sc, sn);
      sc[0] = sn[0];
      sc[1] = sn[1];
      ++t;
    }
  }
  // Diagonal and ragged-tail tiles: masked, per-wavefront skipping.
  for (; t < n_kt; ++t) {
    f32x16_t sn[2];
    prefetch(t);
    const bool use = active(t);
    const bool next = t + 1 < n_kt && active(t + 1);
    if (use) {
      mask(t, sc);
      update_max(sc);
      float te[4];
      exps(sc, te);
      add_sums(te);
      pv_qk(t & 1, next ? (t + 1) & 1 : -1, sn);
    } else if (next) {
      qk((t + 1) & 1, sn);
    }
    if (next) {
      sc[0] = sn[0];
      sc[1] = sn[1];
    }
    wait_loads();
    __syncthreads();
  }

  // ---- epilogue: O = v_scale * O^T / sum(p), LSE = (m + log2 sum(p)) ln 2
  const float lt = xor32_sum((le[0] + le[1]) + (le[2] + le[3]));
  if (qrow < Sq) {
    const float inv = lt > 0.f ? vs / lt : 0.f;
    uint16_t* O = a.out + (bh * (size_t)Sq + qrow) * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = 32 * db + 8 * gq + 4 * hi;
        *reinterpret_cast<uint2*>(O + d) = make_uint2(pack_bf16x2(o[db][4 * gq] * inv, o[db][4 * gq + 1] * inv),
                                                      pack_bf16x2(o[db][4 * gq + 2] * inv, o[db][4 * gq + 3] * inv));
      }
    if (hi == 0) a.lse[bh * Sq + qrow] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : kNegInf;
  }
}

}  // namespace

hipError_t launch_prefill_fp8(const void* q, const void* k, const void* v, const float* q_scale,
                              const float* k_scale, const float* v_scale, void* out, float* lse, int B,
                              int Hq, int Hkv, int Sq, int Sk, int causal, float scale, hipStream_t s) {
  Fp8Args a;
  a.q = reinterpret_cast<const uint8_t*>(q);
  a.k = reinterpret_cast<const uint8_t*>(k);
  a.v = reinterpret_cast<const uint8_t*>(v);
  a.q_scale = q_scale; a.k_scale = k_scale; a.v_scale = v_scale;
  a.out = reinterpret_cast<uint16_t*>(out);
  a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Sq = Sq; a.Sk = Sk; a.causal = causal;
  a.scale = scale;
  const int n_qtiles = (Sq + BR - 1) / BR;
  const int nbh = B * Hq;
  const long long blocks = (long long)n_qtiles * nbh;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(prefill_fp8_kernel, dim3((unsigned)blocks), dim3(64 * NW), 0, s, a, n_qtiles, nbh);
  return hipGetLastError();
}

}  // namespace fa
