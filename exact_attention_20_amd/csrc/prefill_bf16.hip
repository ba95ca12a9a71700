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
//  * Workgroup = NW wavefronts, each owning QB blocks of 32 query rows, so
//    BR = 32*NW*QB rows per workgroup. Each wavefront keeps its Q rows in
//    registers for the whole row block; K/V tiles of 64 keys are shared by
//    all wavefronts through LDS (64 KB: two K and two V buffers); every K or
//    V fragment a wavefront reads from LDS feeds QB matrix instructions.
//  * Both contractions use v_mfma_f32_32x32x16_bf16 (fp32 accumulate) in the
//    transposed form S^T = K Q^T and O^T = V^T P^T. In the 32x32 accumulator
//    layout a lane then owns one query column and 16 keys of it, so the row
//    max and row sums are in-lane plus one v_permlane32_swap with the partner
//    lane (lane ^ 32), and P^T leaves the first MFMA already in the B-operand
//    layout of the second (no LDS round trip). To make the 8 keys a lane owns
//    contiguous, the K rows are fed to the first MFMA in a fixed permuted
//    order (kperm below); the order of a contraction's k index is free as
//    long as both operands agree.
//  * K/V tiles travel HBM -> LDS with buffer_load ... lds (no registers, no
//    LDS store instructions); a buffer resource bounded by Sk rows returns
//    zeros past the last key. V reaches the second MFMA through gfx950's
//    transposing LDS read (ds_read_b64_tr_b16), so nothing is transposed in
//    registers. Rows are stored unpadded with their 16-byte units
//    XOR-swizzled so that the operand reads are free of bank conflicts.
//  * Software pipeline inside each wavefront: the scores of tile t+1 are
//    computed (MFMA) while the softmax of tile t runs on the VALU and its P*V
//    product is issued. K runs one tile ahead of V through two pairs of LDS
//    buffers whose next contents are in flight from HBM meanwhile; one
//    barrier per tile.
//  * Scores are scaled into log2 units once (scale*log2e folded into the exp
//    argument's FMA) and exponentiated with v_exp_f32. The running max is
//    lazy: it moves only when a tile's max exceeds it by more than kTau, so
//    the O^T rescale happens only on the first tiles of a row. Two normalisers
//    are kept: the sum of the bf16-rounded P that the second MFMA consumes
//    (one v_dot2 with ones per pair) divides O, so the normalisation matches
//    the weights applied; the fp32 sum of P gives the LSE. Dividing by the
//    fp32 sum alone would save the v_dot2s but leave a row dominated by one
//    key (whose weight, relative to the lazy max, is rarely a bf16 value)
//    with an error of up to 2^-9 |v| instead of 2^-9 |v - O|.
//  * Grid: one workgroup per (query tile, batch, head). With causal masking
//    the heaviest query tiles (most keys) are issued first. Heads are ordered
//    so that workgroups with equal id mod 8 -- which the dispatcher places on
//    the same XCD -- share a KV head, keeping its K/V in that XCD's L2.
#include <type_traits>

#include "bf16_mfma.h"
#include "fa_internal.h"
#include "hip_common.h"

namespace fa {

namespace {

constexpr int kD = 128;        // head dim
constexpr int kBc = 64;        // keys per tile
constexpr int kRow = kD * 2;   // K/V row in LDS: 256 B, unpadded, 16-byte units XOR-swizzled
constexpr float kTau = 8.0f;   // lazy max threshold (log2 units)
constexpr float kSumBound = 256.0f;  // 2^kTau: a tile sum at or below it bounds every weight

// Modes of the kernel:
//  kContig  contiguous [B, H, S, D] tensors, one work unit per (query tile, b, h);
//  kRagged  ragged paged prefill: work unit (request, query tile) from the
//           plan's list, the request's new tokens are packed rows [T, Hq, D]
//           of q and out, key tile t is page t of the request's table row;
//  kPrefix  shared-prefix pass of a cascade decode: one work unit per
//           PrefixItem; its query rows are the decode queries of a group's
//           requests, G query heads of each folded into rows (one dense tile
//           per KV head: "head-query fusion"), its keys a chunk of the
//           group's prefix pages, no mask; results go to partial slots.
constexpr int kContig = 0, kRagged = 1, kPrefix = 2;

#ifndef FA_PREFILL_PINGPONG
#define FA_PREFILL_PINGPONG 1
#endif
constexpr bool kPingPong = FA_PREFILL_PINGPONG != 0;
#ifndef FA_PREFILL_KV_DEPTH
#define FA_PREFILL_KV_DEPTH 3
#endif
constexpr int kKvDepth = FA_PREFILL_KV_DEPTH;  // K and V tile buffers each (ping-pong schedule)

template <int NW, int QB, int MODE, bool PP>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void prefill_bf16_kernel(PrefillArgs a, int n_qtiles, int nbh) {
  constexpr int NT = 64 * NW;                 // threads
  constexpr int BR = 32 * NW * QB;            // query rows per workgroup
  constexpr int KBUF = kBc * kRow;            // bytes per K buffer
  constexpr int VBUF = kBc * kRow;            // bytes per V buffer
  constexpr int BLK = (kBc * kRow / 1024) / NW;  // 1 KB direct-load blocks per wave per tile
  // Two K and two V tile buffers, each its own LDS variable: the compiler
  // then tags every access with the variable it touches, and a tile's reads
  // of one buffer need not wait for the loads still filling another (see
  // lds_step).
  __shared__ __attribute__((aligned(16))) char k_lds0[KBUF];
  __shared__ __attribute__((aligned(16))) char k_lds1[KBUF];
  __shared__ __attribute__((aligned(16))) char v_lds0[VBUF];
  __shared__ __attribute__((aligned(16))) char v_lds1[VBUF];
  // Two more of each for the ping-pong schedule's deeper prefetch (unused,
  // and so not allocated, by the other schedule).
  __shared__ __attribute__((aligned(16))) char k_lds2[KBUF];
  __shared__ __attribute__((aligned(16))) char k_lds3[KBUF];
  __shared__ __attribute__((aligned(16))) char v_lds2[VBUF];
  __shared__ __attribute__((aligned(16))) char v_lds3[VBUF];

  constexpr bool PAGED = MODE != kContig;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int hi = lane >> 5;     // which half of the wavefront
  const int col = lane & 31;    // query column of this lane in the 32x32 tiles

  // ---- work unit
  const int L = blockIdx.x;
  int b, h, g, qt, Sq, Sk, causal;
  size_t tok0 = 0;  // ragged: packed row of the request's first new token
  int p_first = 0;  // paged: table entry of key tile 0
  int slot = 0, req_off = 0, row0 = 0;  // prefix pass
  if constexpr (MODE == kPrefix) {
    const PrefixItem it = reinterpret_cast<const PrefixItem*>(a.items)[L];
    b = it.first_req;  // its page-table row holds the group's prefix pages
    g = it.g;
    h = 0;
    qt = 0;
    Sq = it.nrows;
    Sk = (it.page_end - it.page_begin) * kBc;
    causal = 0;
    p_first = it.page_begin;
    slot = it.slot;
    req_off = it.req_off;
    row0 = it.row0;
  } else if constexpr (MODE == kRagged) {
    // Items are ordered heaviest first; within one, e enumerates query head
    // h = g*G + e/Hkv with g = e % Hkv, so workgroups with equal id mod 8
    // (one XCD) share a KV head when Hq is a multiple of 8.
    const int item = L / a.Hq, e = L % a.Hq;
    b = a.items[2 * item];
    qt = a.items[2 * item + 1];
    g = e % a.Hkv;
    h = g * (a.Hq / a.Hkv) + e / a.Hkv;
    const int c0 = a.cu_q[b];
    tok0 = (size_t)c0;
    Sq = a.cu_q[b + 1] - c0;
    Sk = a.seqlens[b];
    causal = 1;
  } else {
    qt = a.causal ? (n_qtiles - 1 - L / nbh) : (L / nbh);
    const int e = L % nbh;
    if (a.has_map) {
      b = e / a.Hq;
      h = e % a.Hq;
      g = a.kv_map[h];
    } else {
      // e = (b*Hkv + g) + B*Hkv*j enumerates query head h = g*G + j, so heads
      // with equal e % 8 share KV heads when B*Hkv is a multiple of 8.
      const int G = a.Hq / a.Hkv;
      const int bg = e % (a.B * a.Hkv);
      const int j = e / (a.B * a.Hkv);
      b = bg / a.Hkv;
      g = bg % a.Hkv;
      h = g * G + j;
    }
    Sq = a.Sq;
    Sk = a.Sk;
    causal = a.causal;
  }
  const int q0 = qt * BR;
  const int off = Sk - Sq;  // causal: key j visible to query i iff j <= i + off
  int kend = Sk;
  if (causal) kend = min(Sk, q0 + BR + off);
  const int n_kt = kend > 0 ? (kend + kBc - 1) / kBc : 0;

  // Query/output rows: contiguous [Sq, D] per head, packed [T, Hq, D], or
  // (prefix pass) row r = decode query (request, head) of the group, found
  // through the group's member list, as a row of q [B * Hq, D].
  const size_t row_stride = MODE == kRagged ? (size_t)a.Hq * kD : (size_t)kD;
  const size_t qo_base = MODE == kPrefix   ? 0
                         : MODE == kRagged ? (tok0 * a.Hq + h) * kD
                                           : ((size_t)b * a.Hq + h) * (size_t)Sq * kD;
  const uint16_t* Q = reinterpret_cast<const uint16_t*>(a.q) + qo_base;
  auto prefix_row = [&](int r) -> size_t {
    const int G = a.Hq / a.Hkv;
    const int f = row0 + r;
    const int req = a.group_reqs[req_off + f / G];
    return (size_t)req * a.Hq + g * G + f % G;
  };
  auto q_row_ptr = [&](int r) {
    return MODE == kPrefix ? reinterpret_cast<const uint16_t*>(a.q) + prefix_row(r) * kD : Q + (size_t)r * row_stride;
  };

  // ---- Q: the B operand of S^T = K Q^T for lane (col, hi) in query block
  // qb is row 32*(QB*wave + qb) + col of the tile, dims 16*kk + 8*hi + 0..7.
  // It is the same for every key tile, so it is read once from HBM straight
  // into registers (no LDS space, no LDS reads in the loop).
  bf16x8_t qreg[QB][8];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = q0 + 32 * (QB * wave + qb) + col;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r < Sq) v = *reinterpret_cast<const uint4*>(q_row_ptr(r) + 16 * kk + 8 * hi);
      qreg[qb][kk] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // Per query block: first row, this lane's row, running max (log2 units,
  // same in lane and lane^32), shares of the two normalisers, O^T.
  int wq0[QB], qrow[QB];
  // The normalisers are kept as 4 partial sums each, so that their updates
  // form 4 short dependency chains instead of one long one.
  float m[QB], lr[QB][4], le[QB][4];
  f32x16_t o[QB][4];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    wq0[qb] = q0 + (QB * wave + qb) * 32;
    qrow[qb] = wq0[qb] + col;
    m[qb] = kNegInf;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lr[qb][j] = 0.f;  // sum(bf16(p)): normalises O (matches the MFMA weights)
      le[qb][j] = 0.f;  // sum(p) in fp32: gives the LSE
    }
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[qb][db][i] = 0.f;
  }
  const float c = a.scale * kLog2e;

  // ---- K/V tiles: one direct load moves 1 KB, lane l filling LDS unit
  // (l & 15) of row 4j + (l >> 4). K: unit c of row r sits at c ^ (r & 15);
  // V: at c ^ 4*(r & 3); each lane fetches the global unit that belongs in the
  // LDS slot it fills.
  //
  // Contiguous K/V: one buffer resource over the head's Sk rows; loads past
  // the last key return zeros. Paged: one resource per tile over its page,
  // bounded by the page's valid rows (zeros past the request's last key, so
  // stale or NaN tail slots are never read); a page id outside the pool
  // gives an empty resource (all zeros) instead of a stray access.
  const size_t kv_base = ((size_t)b * a.Hkv + g) * (size_t)Sk * kD;
  const __amdgpu_buffer_rsrc_t k_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(a.k) + (PAGED ? 0 : kv_base)), (short)0,
      PAGED ? 0 : Sk * kRow, 0x00020000);
  const __amdgpu_buffer_rsrc_t v_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(a.v) + (PAGED ? 0 : kv_base)), (short)0,
      PAGED ? 0 : Sk * kRow, 0x00020000);
  // The page table is read-only for the whole kernel, so it is read through
  // the constant address space: uniform indices then give scalar loads,
  // which do not wait behind the tile loads in flight.
  const_i32* ptab = (const_i32*)(a.page_table) + (size_t)b * a.stride;
  // A page id outside the pool reads as zeros; that it happened is noted here
  // (a scalar OR) and reported once after the loop: a memory atomic inside
  // the loop, even never taken, made the compiler's waits for the tile loads
  // conservative (the paged prefill ran 11% slower).
  bool bad_page = false;
  auto page_rsrc = [&](const void* pool, int t) {
    const int pt = p_first + t;
    const int pid = pt < a.stride ? ptab[pt] : -1;
    const bool valid = (unsigned)pid < (unsigned)a.num_pages;
    bad_page |= !valid;
    const char* base = reinterpret_cast<const char*>(pool) +
                       ((size_t)(valid ? pid : 0) * a.Hkv + g) * (size_t)(kBc * kRow);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0,
                                             valid ? min(kBc, Sk - t * kBc) * kRow : 0, 0x00020000);
  };
  const int dl_row = lane >> 4, dl_pos = lane & 15;
  auto load_tile = [&](const __amdgpu_buffer_rsrc_t& rs, int k0, char* buf, bool is_v) {
#pragma unroll
    for (int i = 0; i < BLK; ++i) {
      const int j = wave * BLK + i;
      const int r = 4 * j + dl_row;
      const int unit = is_v ? (dl_pos ^ (4 * (r & 3))) : (dl_pos ^ (r & 15));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(buf + j * 1024), 16, (k0 + r) * kRow + unit * 16, 0, 0, 0);
    }
  };
  // Key tile t lives in K buffer t & 1, value tile t in V buffer t & 1.
  auto kbuf = [&](int t) { return (t & 1) ? k_lds1 : k_lds0; };
  auto vbuf = [&](int t) { return (t & 1) ? v_lds1 : v_lds0; };
  auto load_k = [&](int t, char* dst) {
    if constexpr (PAGED)
      load_tile(page_rsrc(a.k, t), 0, dst, false);
    else
      load_tile(k_rs, t * kBc, dst, false);
  };
  auto load_v = [&](int t, char* dst) {
    if constexpr (PAGED)
      load_tile(page_rsrc(a.v, t), 0, dst, true);
    else
      load_tile(v_rs, t * kBc, dst, true);
  };
  // This wavefront's direct loads have landed in LDS (waited for explicitly
  // before the barrier that publishes them).
  auto wait_loads = [] { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // Per-lane LDS read addresses.
  // K (A operand of S^T = K Q^T): MFMA row `col` feeds key R = kperm(col),
  //   global unit 2*kk + hi of that row, stored at unit (2*kk + hi) ^ (R & 15);
  //   the second 32-key half is 32 rows further.
  int k_off[8];
  {
    const int R = kperm(col);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) k_off[kk] = R * kRow + 16 * ((2 * kk + hi) ^ (R & 15));
  }
  // V (A operand of O^T = V^T P^T, rows d = 32*db + col, k-slots = keys
  // 16*ks + 8*hi + 0..7): two transposing reads per operand; lane L of each
  // 16-lane group g addresses key 16*ks + 8*(g>>1) + 4*r + (L>>2) and dims
  // 32*db + 16*(g&1) + 4*(L&3) .. +3, so lane i of the group receives keys
  // +4r .. +4r+3 of dim 32*db + 16*(g&1) + i. With (L>>2) = key & 3 the
  // swizzle moves the 64-byte block db to db ^ (L>>2).
  int v_off[4];
  {
    const int vg = lane >> 4, vL = lane & 15, q4 = vL >> 2;
    const int v_lane = (8 * (vg >> 1) + q4) * kRow + 16 * (2 * (vg & 1) + ((vL & 3) >> 1)) + 8 * (vL & 1);
#pragma unroll
    for (int db = 0; db < 4; ++db) v_off[db] = v_lane + 64 * (db ^ q4);
  }

  // Tile t holds work for query block qb unless it lies wholly above its diagonal.
  // A wavefront's query block takes part in tile t unless all its rows lie
  // past Sq (the padding of a unit's last row tile) or, causal, before the
  // tile's first key.
  auto blk_active = [&](int t, int qb) { return wq0[qb] < Sq && !(causal && t * kBc > wq0[qb] + 31 + off); };
  auto any_active = [&](int t) { return blk_active(t, QB - 1); };

  // S^T for every query block from K buffer kbuf.
  auto qk = [&](const char* kl, f32x16_t (&s)[QB][2]) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(kl + k_off[kk]);
      const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(kl + k_off[kk] + 32 * kRow);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const bf16x8_t qf = qreg[qb][kk];
        s[qb][0] = kk == 0 ? mfma32_first(a0, qf) : mfma32(a0, qf, s[qb][0]);
        s[qb][1] = kk == 0 ? mfma32_first(a1, qf) : mfma32(a1, qf, s[qb][1]);
      }
    }
  };

  // Causal / ragged-tail mask of tile t's scores for query block qb.
  auto mask = [&](int t, int qb, f32x16_t& s0, f32x16_t& s1) {
    const int k0 = t * kBc;
    const int lim = causal ? min(Sk - 1, qrow[qb] + off) : Sk - 1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = k0 + 16 * (i >> 3) + 8 * hi + (i & 7);
      if (key > lim) s0[i] = kNegInf;
      if (key + 32 > lim) s1[i] = kNegInf;
    }
  };

  // Row max of the tile and the lazy move of block qb's running max.
  auto update_max = [&](int qb, const f32x16_t& s0, const f32x16_t& s1) {
    // balanced max tree over the 32 scores of this lane
    float t8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t8[i] = fmaxf(fmaxf(s0[2 * i], s0[2 * i + 1]), fmaxf(s1[2 * i], s1[2 * i + 1]));
    float mx = fmaxf(fmaxf(fmaxf(t8[0], t8[1]), fmaxf(t8[2], t8[3])), fmaxf(fmaxf(t8[4], t8[5]), fmaxf(t8[6], t8[7])));
    mx = xor32_max(mx);
    const float mxs = mx * c;
    const bool need = mxs > m[qb] + kTau;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(need) != 0, 0)) {
      // Rarely taken once the max has settled: kept as a branch (the empty
      // volatile asm stops the compiler from turning it into unconditional
      // multiplies by alpha = 1).
      asm volatile("");
      const float mn = need ? mxs : m[qb];
      const float alpha = need ? fast_exp2(m[qb] - mn) : 1.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lr[qb][j] *= alpha;
        le[qb][j] *= alpha;
      }
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[qb][db][i] *= alpha;
      m[qb] = mn;
    }
  };

  // P = exp2(s*c - m) in bf16 for the query blocks selected by `use`, both
  // normalisers, and O^T += V^T P^T from V buffer vbuf. With kb >= 0 the
  // scores of the next tile are computed from K buffer kb in the same
  // straight-line block, so the scheduler can interleave those MFMAs with
  // this tile's exponentials.
  auto exp_pv_qk = [&](const char* vl, const f32x16_t (&s)[QB][2], const bool (&use)[QB], const char* kl,
                       bool next_qk, f32x16_t (&n)[QB][2]) {
    float mu[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mu[qb] = (m[qb] == kNegInf) ? 0.f : m[qb];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8_t pf[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (!use[qb]) continue;
        const f32x16_t& sv = s[qb][ks >> 1];
        const int base = 8 * (ks & 1);
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = fast_exp2(__builtin_fmaf(sv[base + 2 * j], c, -mu[qb]));
          const float p1 = fast_exp2(__builtin_fmaf(sv[base + 2 * j + 1], c, -mu[qb]));
          w[j] = pack_bf16x2(p0, p1);
          lr[qb][j] = dot2_bf16(w[j], 0x3f803f80u, lr[qb][j]);  // + bf16(p0) + bf16(p1)
          le[qb][j] += p0 + p1;
        }
        pf[qb] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const char* vp = vl + v_off[db] + 16 * ks * kRow;
        const uint2 v0 = lds_read_tr16(vp);
        const uint2 v1 = lds_read_tr16(vp + 4 * kRow);
        const bf16x8_t va = __builtin_bit_cast(bf16x8_t, make_uint4(v0.x, v0.y, v1.x, v1.y));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          if (use[qb]) o[qb][db] = mfma32(va, pf[qb], o[qb][db]);
      }
      if (next_qk) {
#pragma unroll
        for (int kk = 2 * ks; kk < 2 * ks + 2; ++kk) {
          const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(kl + k_off[kk]);
          const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(kl + k_off[kk] + 32 * kRow);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const bf16x8_t qf = qreg[qb][kk];
            n[qb][0] = kk == 0 ? mfma32_first(a0, qf) : mfma32(a0, qf, n[qb][0]);
            n[qb][1] = kk == 0 ? mfma32_first(a1, qf) : mfma32(a1, qf, n[qb][1]);
          }
        }
      }
    }
  };

  // One tile's LDS traffic: start the loads of K(t+2) over K(t) and of
  // V(t+1) over V(t-1) (both buffers were last read in iteration t-1, before
  // its closing barrier), then run `body` on the buffers this tile reads,
  // V(t) and K(t+1). The four buffers are distinct (separate LDS variables,
  // and restrict here): when the compiler cannot tell that the loads just
  // started write other addresses than a read, it makes the tile's first
  // transposing LDS read wait for them, which exposes their whole latency.
  auto lds_step = [&](int t, const char* __restrict__ vl, const char* __restrict__ kl, char* __restrict__ kw,
                      char* __restrict__ vw, auto&& body) {
    if (t + 2 < n_kt) load_k(t + 2, kw);
    if (t + 1 < n_kt) load_v(t + 1, vw);
    body(vl, kl);
  };

  // Tiles below the whole workgroup's diagonal and inside Sk need no mask
  // and have work for every query block: they run the branch-free main loop.
  int n_main = Sk / kBc;
  if (causal) n_main = min(n_main, max(0, (q0 + off + 1) / kBc));
  n_main = min(n_main, n_kt);

  if constexpr (PP) {
    static_assert(QB == 1 && NW == 8, "the ping-pong schedule pairs two 32-row wavefronts per SIMD");
    // ---- Ping-pong schedule. Waves 0-3 (group A) and 4-7 (group B) put one
    // wavefront of each group on every SIMD. A wavefront alternates a matrix
    // phase M(j) -- O^T += V^T P^T of tile j-1, then S^T = K Q^T of tile j --
    // with a vector phase V(j): mask, running max and P = exp2(S c - m) of
    // tile j in bf16 with both normalisers. The two groups run one phase
    // apart with a barrier between phases: in slot 2j group A runs M(j) while
    // B runs V(j-1), in slot 2j+1 A runs V(j) while B runs M(j). So on every
    // SIMD one wavefront issues matrix instructions while the other runs the
    // softmax; the matrix core then executes one wavefront's MFMAs while the
    // other's vector instructions issue, which one wavefront's dependent
    // chain (scores -> max -> exponentials -> P V) cannot do on its own.
    // Loads of K(j+1) and V(j) start in slot 2j (their buffers were last
    // read in slots 2j-2 and 2j-1) and are waited for at the end of slot
    // 2j+1, one slot before their first reader.
    const bool grp_a = __builtin_amdgcn_readfirstlane(wave) < 4;
    f32x16_t s0, s1;    // S^T of a tile between its M and V phases (keys 0-31, 32-63)
    uint32_t pw[4][4];  // P^T of a tile between its V phase and the next M phase: [k step][pair]

    auto m_phase = [&](int j, const char* vl, const char* kl) __attribute__((always_inline)) {
      const bool pv = j >= 1 && blk_active(j - 1, 0);
      const bool sq = j < n_kt && blk_active(j, 0);
      auto pv_step = [&](int ks) __attribute__((always_inline)) {
        const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, make_uint4(pw[ks][0], pw[ks][1], pw[ks][2], pw[ks][3]));
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const char* vp = vl + v_off[db] + 16 * ks * kRow;
          const uint2 v0 = lds_read_tr16(vp);
          const uint2 v1 = lds_read_tr16(vp + 4 * kRow);
          const bf16x8_t va = __builtin_bit_cast(bf16x8_t, make_uint4(v0.x, v0.y, v1.x, v1.y));
          o[0][db] = mfma32(va, pf, o[0][db]);
        }
      };
      auto qk_step = [&](int kk) __attribute__((always_inline)) {
        const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(kl + k_off[kk]);
        const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(kl + k_off[kk] + 32 * kRow);
        const bf16x8_t qf = qreg[0][kk];
        s0 = kk == 0 ? mfma32_first(a0, qf) : mfma32(a0, qf, s0);
        s1 = kk == 0 ? mfma32_first(a1, qf) : mfma32(a1, qf, s1);
      };
      if (pv && sq) {
        // Eight blocks of four MFMAs: block b is k step b of S^T (two
        // 32-key halves) and two of the four 32-dim blocks of O^T for k step
        // b/2 of P V. Each block's LDS operands are read one block ahead
        // (their latency hides behind the previous block's MFMAs), and the
        // scheduling barriers keep that order, so that no more than two
        // blocks' operands are live at once.
        struct Ops {
          bf16x8_t k0, k1, v0, v1;
        };
        auto read_ops = [&](int b) __attribute__((always_inline)) {
          Ops r;
          r.k0 = *reinterpret_cast<const bf16x8_t*>(kl + k_off[b]);
          r.k1 = *reinterpret_cast<const bf16x8_t*>(kl + k_off[b] + 32 * kRow);
          const int ks = b >> 1, db = 2 * (b & 1);
          const char* vp0 = vl + v_off[db] + 16 * ks * kRow;
          const char* vp1 = vl + v_off[db + 1] + 16 * ks * kRow;
          const uint2 a0 = lds_read_tr16(vp0), a1 = lds_read_tr16(vp0 + 4 * kRow);
          const uint2 b0 = lds_read_tr16(vp1), b1 = lds_read_tr16(vp1 + 4 * kRow);
          r.v0 = __builtin_bit_cast(bf16x8_t, make_uint4(a0.x, a0.y, a1.x, a1.y));
          r.v1 = __builtin_bit_cast(bf16x8_t, make_uint4(b0.x, b0.y, b1.x, b1.y));
          return r;
        };
        Ops cur = read_ops(0);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          Ops nxt;
          if (b < 7) nxt = read_ops(b + 1);
          __builtin_amdgcn_sched_barrier(0);
          const bf16x8_t qf = qreg[0][b];
          s0 = b == 0 ? mfma32_first(cur.k0, qf) : mfma32(cur.k0, qf, s0);
          s1 = b == 0 ? mfma32_first(cur.k1, qf) : mfma32(cur.k1, qf, s1);
          const int ks = b >> 1, db = 2 * (b & 1);
          const bf16x8_t pf =
              __builtin_bit_cast(bf16x8_t, make_uint4(pw[ks][0], pw[ks][1], pw[ks][2], pw[ks][3]));
          o[0][db] = mfma32(cur.v0, pf, o[0][db]);
          o[0][db + 1] = mfma32(cur.v1, pf, o[0][db + 1]);
          __builtin_amdgcn_sched_barrier(0);
          if (b < 7) cur = nxt;
        }
      } else if (pv) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) pv_step(ks);
      } else if (sq) {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) qk_step(kk);
      }
    };

    // P of the tile with the running max as it stands, and the tile's shares
    // of both normalisers (tr: sum of bf16(p), te: fp32 sum of p).
    auto exps = [&](float (&tr)[4], float (&te)[4]) __attribute__((always_inline)) {
      const float mu = m[0] == kNegInf ? 0.f : m[0];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const f32x16_t& sv = (ks >> 1) ? s1 : s0;
        const int base = 8 * (ks & 1);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float p0 = fast_exp2(__builtin_fmaf(sv[base + 2 * jj], c, -mu));
          const float p1 = fast_exp2(__builtin_fmaf(sv[base + 2 * jj + 1], c, -mu));
          pw[ks][jj] = pack_bf16x2(p0, p1);
          // + bf16(p0) + bf16(p1); the first step starts both sums (no add of zero)
          tr[jj] = dot2_bf16(pw[ks][jj], 0x3f803f80u, ks == 0 ? 0.f : tr[jj]);
          te[jj] = ks == 0 ? p0 + p1 : te[jj] + (p0 + p1);
        }
      }
    };
    // The running max is lazy: it only has to keep every weight p = exp2(s c - m)
    // at or below 2^kTau. The tile's weights are first formed with the max as it
    // stands; a lane's fp32 tile sum bounds each of its weights, so if no lane's
    // sum exceeds 2^kTau the tile is kept without ever forming its row max. Else
    // (the first tile of a row, or scores that rose past the max by about kTau)
    // the tile is redone the long way: row max, lazy move of the max with the
    // rescale of O and the normalisers, weights again. This takes the max tree,
    // its cross-lane exchange and the wave-wide vote off the common path, where
    // they stood between the scores and the first exponential.
    auto v_phase = [&](int j) __attribute__((always_inline)) {
      if (j < 0 || j >= n_kt || !blk_active(j, 0)) return;
      if (j >= n_main) mask(j, 0, s0, s1);
      float tr[4], te[4];
      bool redo = true;
      if (__builtin_amdgcn_ballot_w64(m[0] == kNegInf) == 0) {
        exps(tr, te);
        const float big = fmaxf(fmaxf(te[0], te[1]), fmaxf(te[2], te[3]));
        redo = __builtin_amdgcn_ballot_w64(!(big <= kSumBound)) != 0;
      }
      if (__builtin_expect(redo, 0)) {
        update_max(0, s0, s1);
        exps(tr, te);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        lr[0][jj] += tr[jj];
        le[0][jj] += te[jj];
      }
    };

    // Barrier between the two slots of an iteration: it only keeps the
    // groups in step (nothing in LDS changes hands there), so no memory
    // fence, and the scheduler moves no work across it.
    auto phase_barrier = [] __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    // K and V each have NB buffers; tile t lives in buffer t % NB. Iteration j
    // reads K(j) and V(j-1) and starts the loads of K(j+NB-1) and V(j+NB-2),
    // whose buffers held K(j-1) and V(j-2), last read in iteration j-1. So a
    // tile's loads have NB-1 iterations to land. Every iteration starts the
    // same number of loads (tiles past the last one read through an empty
    // buffer resource: no memory access, zeros), so the wait at its end is
    // one count: the loads of the last NB-2 iterations may still be in flight.
    constexpr int NB = kKvDepth;
    static_assert(NB >= 2 && NB <= 4, "two to four K and V buffers");
    static_assert(BLK == 2, "the vmcnt arithmetic below counts 2 + 2 loads per iteration");
    const __amdgpu_buffer_rsrc_t none_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(a.k)), (short)0, 0, 0x00020000);
    auto kb = [&](auto i) __attribute__((always_inline)) -> char* {
      constexpr int I = ((decltype(i)::value % NB) + NB) % NB;
      if constexpr (I == 0) return k_lds0;
      else if constexpr (I == 1) return k_lds1;
      else if constexpr (I == 2) return k_lds2;
      else return k_lds3;
    };
    auto vb = [&](auto i) __attribute__((always_inline)) -> char* {
      constexpr int I = ((decltype(i)::value % NB) + NB) % NB;
      if constexpr (I == 0) return v_lds0;
      else if constexpr (I == 1) return v_lds1;
      else if constexpr (I == 2) return v_lds2;
      else return v_lds3;
    };
    auto load_kt = [&](int t, char* dst) __attribute__((always_inline)) {
      if (t >= 0 && t < n_kt) load_k(t, dst);
      else load_tile(none_rs, 0, dst, false);
    };
    auto load_vt = [&](int t, char* dst) __attribute__((always_inline)) {
      if (t >= 0 && t < n_kt) load_v(t, dst);
      else load_tile(none_rs, 0, dst, true);
    };
    // End of an iteration: this wavefront's loads for the next iteration have
    // landed (the 4 loads of each of the NB-2 later iterations may still be
    // in flight) and its LDS reads are done; the barrier publishes both. No
    // memory fence: a workgroup fence would also wait for those later loads.
    auto iter_barrier = [] __attribute__((always_inline)) {
      if constexpr (NB == 2)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      else if constexpr (NB == 3)
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
    };
    // Iteration j: slot 2j then slot 2j+1. Each group has a loop of its own
    // (the branch is outside the loop), so that the registers of each are
    // allocated for its own order of phases.
    auto slots = [&](auto grp, int j, const char* __restrict__ vl, const char* __restrict__ kl,
                     char* __restrict__ kw, char* __restrict__ vw) __attribute__((always_inline)) {
      constexpr bool A = decltype(grp)::value;
      load_kt(j + NB - 1, kw);
      load_vt(j + NB - 2, vw);
      if constexpr (A)
        m_phase(j, vl, kl);
      else
        v_phase(j - 1);
      phase_barrier();
      if constexpr (A)
        v_phase(j);
      else
        m_phase(j, vl, kl);
      iter_barrier();
    };
    // Unrolled by NB so that every buffer is a fixed LDS variable; the
    // iterations past n_kt do nothing but keep the barriers in step.
    auto iter = [&](auto grp, auto r, int j) __attribute__((always_inline)) {
      constexpr int R = decltype(r)::value;  // j % NB
      slots(grp, j, vb(std::integral_constant<int, R - 1>{}), kb(std::integral_constant<int, R>{}),
            kb(std::integral_constant<int, R - 1>{}), vb(std::integral_constant<int, R - 2>{}));
    };
    auto run = [&](auto grp) __attribute__((always_inline)) {
      for (int j = 0; j <= n_kt; j += NB) {
        iter(grp, std::integral_constant<int, 0>{}, j);
        iter(grp, std::integral_constant<int, 1>{}, j + 1);
        if constexpr (NB > 2) iter(grp, std::integral_constant<int, 2>{}, j + 2);
        if constexpr (NB > 3) iter(grp, std::integral_constant<int, 3>{}, j + 3);
      }
    };
    // Prologue: the loads that iterations 1-NB .. -1 would have started,
    // K(0) .. K(NB-2) and V(-1) .. V(NB-3) (V(-1) empty), then K(0) is waited for.
    load_kt(0, kb(std::integral_constant<int, 0>{}));
    load_vt(-1, vb(std::integral_constant<int, -1>{}));
    if constexpr (NB > 2) {
      load_kt(1, kb(std::integral_constant<int, 1>{}));
      load_vt(0, vb(std::integral_constant<int, 0>{}));
    }
    if constexpr (NB > 3) {
      load_kt(2, kb(std::integral_constant<int, 2>{}));
      load_vt(1, vb(std::integral_constant<int, 1>{}));
    }
    iter_barrier();
    if (grp_a)
      run(std::true_type{});
    else
      run(std::false_type{});
    // Every load has landed (the last ones were of empty tiles, writing zeros)
    // before the epilogue reuses the buffers.
    wait_loads();
    __syncthreads();
  } else {
    // ---- prologue: K(0), K(1), V(0) in LDS, then S(0).
    f32x16_t sc[QB][2];
    if (n_kt > 0) {
      load_k(0, kbuf(0));
      load_v(0, vbuf(0));
      if (n_kt > 1) load_k(1, kbuf(1));
    }
    wait_loads();
    __syncthreads();  // K(0), K(1), V(0) visible to every wavefront
    if (n_kt > 0 && any_active(0)) qk(kbuf(0), sc);
    __syncthreads();  // every wavefront has read K(0) before K(2) replaces it

    bool all[QB];
  #pragma unroll
    for (int qb = 0; qb < QB; ++qb) all[qb] = true;
    // One tile of the main loop with buffer parity PAR known at compile time
    // (LDS offsets become immediates); the scores of tile t arrive in `cur`
    // and those of tile t+1 leave in `nxt`. The next tile's scores are
    // computed even past the last tile (from a stale buffer, then discarded)
    // to keep this block free of branches.
    auto main_step = [&](auto par, int t, f32x16_t (&cur)[QB][2], f32x16_t (&nxt)[QB][2]) {
      constexpr int PAR = decltype(par)::value;
      lds_step(t, PAR ? v_lds1 : v_lds0, PAR ? k_lds0 : k_lds1, PAR ? k_lds1 : k_lds0, PAR ? v_lds0 : v_lds1,
               [&](const char* vl, const char* kl) {
  #pragma unroll
                 for (int qb = 0; qb < QB; ++qb) update_max(qb, cur[qb][0], cur[qb][1]);
                 exp_pv_qk(vl, cur, all, kl, true, nxt);
               });
      wait_loads();
      __syncthreads();
    };
    // Unrolled by two so the two score arrays swap roles instead of being
    // copied, and t starts at 0, so tile t uses buffer t & 1 = its position.
    int t = 0;
    {
      f32x16_t sn[QB][2];
      for (; t + 1 < n_main; t += 2) {
        main_step(std::integral_constant<int, 0>{}, t, sc, sn);
        main_step(std::integral_constant<int, 1>{}, t + 1, sn, sc);
      }
      if (t < n_main) {
        main_step(std::integral_constant<int, 0>{}, t, sc, sn);
  #pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          sc[qb][0] = sn[qb][0];
          sc[qb][1] = sn[qb][1];
        }
        ++t;
      }
    }
    for (; t < n_kt; ++t) {
      f32x16_t sn[QB][2];
      const bool next = t + 1 < n_kt && any_active(t + 1);
      lds_step(t, vbuf(t), kbuf(t + 1), kbuf(t), vbuf(t + 1), [&](const char* vl, const char* kl) {
        bool use[QB];
        bool any = false;
  #pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          use[qb] = blk_active(t, qb);
          any |= use[qb];
          if (use[qb]) {
            mask(t, qb, sc[qb][0], sc[qb][1]);
            update_max(qb, sc[qb][0], sc[qb][1]);
          }
        }
        if (any)
          exp_pv_qk(vl, sc, use, kl, next, sn);
        else if (next)
          qk(kl, sn);
      });
      if (next) {
  #pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          sc[qb][0] = sn[qb][0];
          sc[qb][1] = sn[qb][1];
        }
      }
      wait_loads();
      __syncthreads();
    }

  }

  if constexpr (PAGED) {
    if (bad_page && lane == 0) report_status(a.status, kStatusBadPage);
  }

  // ---- epilogue: O = O^T / sum(bf16 p), LSE = (m + log2 sum(p)) ln 2
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lrt = xor32_sum((lr[qb][0] + lr[qb][1]) + (lr[qb][2] + lr[qb][3]));
    const float let_ = xor32_sum((le[qb][0] + le[qb][1]) + (le[qb][2] + le[qb][3]));
    const float inv = lrt > 0.f ? 1.f / lrt : 0.f;
    const float lse_val = let_ > 0.f ? (m[qb] + __log2f(let_)) * kLn2 : kNegInf;
    if constexpr (MODE == kPrefix) {
      if (qrow[qb] >= Sq) continue;
      // The request's only slot: final bf16 output; else this chunk's
      // normalised partial output and LSE for the merge.
      const size_t pr = prefix_row(qrow[qb]);
      const int req = (int)(pr / a.Hq);
      if (a.splits[req] == 1) {
        uint16_t* O = reinterpret_cast<uint16_t*>(a.out) + pr * kD;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int d = 32 * db + 8 * gq + 4 * hi;
            *reinterpret_cast<uint2*>(O + d) =
                make_uint2(pack_bf16x2(o[qb][db][4 * gq] * inv, o[qb][db][4 * gq + 1] * inv),
                           pack_bf16x2(o[qb][db][4 * gq + 2] * inv, o[qb][db][4 * gq + 3] * inv));
          }
        if (hi == 0) a.lse[pr] = lse_val;
      } else {
        float* P = a.part_o + (pr * a.num_splits + slot) * kD;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int d = 32 * db + 8 * gq + 4 * hi;
            *reinterpret_cast<float4*>(P + d) = make_float4(o[qb][db][4 * gq] * inv, o[qb][db][4 * gq + 1] * inv,
                                                            o[qb][db][4 * gq + 2] * inv, o[qb][db][4 * gq + 3] * inv);
          }
        if (hi == 0) a.part_lse[pr * a.num_splits + slot] = lse_val;
      }
      continue;
    }
    // The block's 32 bf16 output rows go through this wavefront's 8 KB of
    // the (now idle) K/V buffers, so that each store writes whole 256-byte
    // rows: lane (col, hi) holds dims 32*db + 8*gq + 4*hi .. +3 of row col,
    // stored in 16-byte unit 4*db + gq (XOR-swizzled by row & 15, which
    // keeps both the writes and the row reads free of bank conflicts). A
    // wavefront's LDS operations complete in order, so no barrier is needed.
    char* st = (wave < 2 ? k_lds0 : wave < 4 ? k_lds1 : wave < 6 ? v_lds0 : v_lds1) + (wave & 1) * (32 * kRow);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const uint2 w = make_uint2(pack_bf16x2(o[qb][db][4 * gq] * inv, o[qb][db][4 * gq + 1] * inv),
                                   pack_bf16x2(o[qb][db][4 * gq + 2] * inv, o[qb][db][4 * gq + 3] * inv));
        *reinterpret_cast<uint2*>(st + col * kRow + 16 * ((4 * db + gq) ^ (col & 15)) + 8 * hi) = w;
      }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rr = 4 * i + (lane >> 4), u = lane & 15;
      const uint4 v = *reinterpret_cast<const uint4*>(st + rr * kRow + 16 * (u ^ (rr & 15)));
      if (wq0[qb] + rr < Sq)
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.out) + qo_base + (size_t)(wq0[qb] + rr) * row_stride +
                                  8 * u) = v;
    }
    const size_t lse_idx = PAGED ? (tok0 + qrow[qb]) * a.Hq + h : ((size_t)b * a.Hq + h) * Sq + qrow[qb];
    if (hi == 0 && qrow[qb] < Sq) a.lse[lse_idx] = lse_val;
  }
}

template <int NW, int QB>
hipError_t launch_cfg(const PrefillArgs& a, hipStream_t s) {
  constexpr int BR = 32 * NW * QB;
  const int n_qtiles = (a.Sq + BR - 1) / BR;
  const int nbh = a.B * a.Hq;
  const long long blocks = (long long)n_qtiles * nbh;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((prefill_bf16_kernel<NW, QB, kContig, kPingPong>), dim3((unsigned)blocks), dim3(64 * NW), 0, s, a,
                     n_qtiles, nbh);
  return hipGetLastError();
}

template <int NW, int QB>
hipError_t launch_paged_cfg(const PrefillArgs& a, int n_items, hipStream_t s) {
  static_assert(32 * NW * QB == kPrefillRows, "the plan's tile height must match the kernel's");
  const long long blocks = (long long)n_items * a.Hq;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((prefill_bf16_kernel<NW, QB, kRagged, kPingPong>), dim3((unsigned)blocks), dim3(64 * NW), 0, s, a,
                     0, 0);
  return hipGetLastError();
}

template <int NW, int QB>
hipError_t launch_prefix_cfg(const PrefillArgs& a, int n_items, hipStream_t s) {
  static_assert(32 * NW * QB == kPrefillRows, "the plan's tile height must match the kernel's");
  if (n_items == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_bf16_kernel<NW, QB, kPrefix, false>), dim3((unsigned)n_items), dim3(64 * NW), 0, s, a, 0, 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
  return launch_cfg<8, 1>(a, s);
}

hipError_t launch_prefill_paged_bf16(const PrefillArgs& a, int n_items, hipStream_t s) {
  return launch_paged_cfg<8, 1>(a, n_items, s);
}

hipError_t launch_prefix_bf16(const PrefillArgs& a, int n_items, hipStream_t s) {
  return launch_prefix_cfg<8, 1>(a, n_items, s);
}

}  // namespace fa
