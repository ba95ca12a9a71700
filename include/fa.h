/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library (libfa.so).
 *
 * Exact attention O = softmax(Q K^T / sqrt(d)) V, forward only, in three forms:
 *   - prefill: every query row of a [B, Hq, Sq, D] block against its KV head,
 *     optionally causal, tiled so the score matrix never reaches HBM;
 *   - ragged paged prefill: the new tokens of a batch of requests against
 *     their paged KV caches (after appending their own K/V to the pages);
 *   - paged Flash-Decoding: one query token per request against a KV cache
 *     held in 64-token pages behind a page table, split along the sequence,
 *     partial results merged by their LogSumExp.
 *
 * Sources (titles of the pages this follows):
 *   "FIA / FlashAttention" help-centre Q&A: section 1 (the attention formula,
 *     exactness, IO-aware tiling with online softmax), section 2 (FIA: a plan
 *     step that preprocesses ragged lengths and balances load, then a run
 *     step), section 3 (GQA, FP8 inference kernels), section 4 (the causal
 *     packed-QKV call and the plan/run decode calls).
 *   "Flash Attention & Paged Attention" blog: "FA and the decode phase"
 *     (Flash-Decoding) and "2. PagedAttention" (pages + logical page table).
 *   "FasterTransformer vs FlashAttention" article, section 3 (the blocked
 *     loop: Q block outer, K/V blocks inner, running max and normaliser).
 *   "FlashAttention breakthrough architecture" article: 64-token pages,
 *     num_splits as the split-KV parallelism knob, cache_seqlens.
 *
 * Conventions for every call:
 *   - Tensor arguments are raw DEVICE pointers unless marked "host". The
 *     caller owns all device memory (inputs, outputs and the decode
 *     workspace); the library allocates only the small host-side plan object.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default
 *     stream. All device work is enqueued asynchronously on it; faults in
 *     device code surface at the caller's next synchronisation.
 *   - Return value: FA_OK or an fa_status error code. Every argument check
 *     happens before any device work is enqueued, so an error return means
 *     nothing was launched. fa_last_error() gives a message (thread-local).
 *   - No call throws across the ABI. Calls are re-entrant; concurrent decode
 *     runs need distinct workspaces.
 *   - LSE outputs are natural-log LogSumExp of the scaled, unmasked scores of
 *     a query row: LSE_i = ln sum_j exp(scale * q_i . k_j).
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, inconsistent shapes */
  FA_ERR_UNSUPPORTED = 2,      /* valid request outside what the kernels cover */
  FA_ERR_WORKSPACE = 3,        /* decode workspace too small */
  FA_ERR_HIP = 4               /* a HIP runtime call failed (message has the HIP error) */
} fa_status;

typedef enum {
  FA_DTYPE_F32 = 0,
  FA_DTYPE_BF16 = 1,
  FA_DTYPE_FP8_E4M3FN = 2 /* OCP e4m3fn codes (uint8), KV cache only */
} fa_dtype;

/* Message for the last error on the calling thread ("" after success). */
const char* fa_last_error(void);

/* Bits of the device status word (fa_device_status). */
enum {
  FA_STATUS_BAD_PAGE = 1,     /* a page-table entry outside [0, num_pages) was met */
  FA_STATUS_BAD_POSITION = 2  /* an appended token's position was negative or past its table row */
};

/*
 * fa_device_status -- the bits the kernels OR-ed into the current device's
 * status word, since it was last cleared, when they met bad DEVICE metadata
 * in the logical-to-physical page table ("Flash Attention & Paged Attention"
 * blog, "2. PagedAttention"). Host checks only see the host copies a plan is
 * built from; the kernels read such a page as zeros (attention) or do not
 * write it (KV append), and set a bit here.
 *   flags_out  host; receives the word
 *   clear      nonzero: reset the word to 0 after reading it
 * Synchronizes the current device first, so every call enqueued before it
 * has finished. One word per device, shared by every call on that device.
 */
int fa_device_status(unsigned int* flags_out, int clear);

/* Library ABI version (bumped on any signature change). */
int fa_abi_version(void);

/*
 * fa_prefill_fwd -- exact attention forward over contiguous BHSD tensors.
 * (FIA / FlashAttention Q&A, sections 1 and 4; FasterTransformer vs
 * FlashAttention, section 3: the Q-block-outer, KV-block-inner loop.)
 *
 *   q    [B, Hq,  Sq, D]  dtype, contiguous
 *   k, v [B, Hkv, Sk, D]  dtype, contiguous
 *   out  [B, Hq,  Sq, D]  dtype (bf16 rounded to nearest even), written
 *   lse  [B, Hq,  Sq]     fp32 natural-log LSE per query row, written
 *   dtype        FA_DTYPE_F32 (D = 64 or 128) or FA_DTYPE_BF16 (D = 128);
 *                accumulation is fp32 in both.
 *   causal       0/1. Causal masking is aligned bottom-right: key j is
 *                visible to query i iff j <= i + (Sk - Sq). A query row that
 *                sees no key gets out = 0 and lse = -inf.
 *   scale        score multiplier; <= 0 selects 1/sqrt(D).
 *   kv_head_map  host int32[Hq]: KV head read by each query head (GQA), or
 *                NULL for contiguous groups h / (Hq / Hkv) (then Hq % Hkv
 *                must be 0). Entries must lie in [0, Hkv).
 * Limits: B, Hq, Hkv >= 1; Hq, Hkv <= 256; Sq, Sk >= 0 (0 is a no-op for
 * Sq = 0; Sk = 0 gives out = 0, lse = -inf); B*Hq*Sq*D and B*Hkv*Sk*D must fit in
 * int64 and Sq, Sk < 2^31; bf16 also needs Sk < 2^23 (FA_ERR_UNSUPPORTED).
 */
int fa_prefill_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                   int B, int Hq, int Hkv, int Sq, int Sk, int D, int dtype, int causal,
                   float scale, const int32_t* kv_head_map, void* stream);

/*
 * fa_prefill_fp8_fwd -- exact attention forward with fp8 (OCP e4m3fn) inputs
 * on the fp8 matrix cores. ("FIA / FlashAttention" Q&A, section 3: FP8
 * inference kernels; section 1 for the method.)
 *
 *   q    [B, Hq,  Sq, 128]  uint8 e4m3fn codes; value = code * q_scale[b, h]
 *   k, v [B, Hkv, Sk, 128]  uint8 e4m3fn codes; value = code * k_scale / v_scale[b, g]
 *   q_scale [B, Hq], k_scale / v_scale [B, Hkv]  fp32 device arrays, finite and > 0
 *   out  [B, Hq, Sq, 128] bf16 (nearest even), lse [B, Hq, Sq] fp32 natural log
 *   causal, scale as for fa_prefill_fwd (bottom-right mask; <= 0 selects 1/sqrt(128));
 *   query head h reads KV head h / (Hq / Hkv).
 * Both products run on the fp8 matrix cores with fp32 accumulation. The
 * matrix core sums each block of 64 products exactly when they are of
 * similar size, but drops the low bits of products far below the largest of
 * their block (measured on gfx950: error up to about 2^-12.4 of that largest
 * product). So a score, and the LSE with it, carries an absolute error of up
 * to about 2^-12 * scale * sum over its two blocks of max_d |q_d k_d|: below
 * 1e-4 for inputs without outlier dims, but not small when one dim carries a
 * large score. The softmax weights P are rounded to e4m3 (nearest even) for
 * the P V product, and O is divided by the fp32 sum of the unrounded
 * weights. Each weight carries a relative error of at most 2^-4 before
 * normalisation, so |O - O_exact| <= 2^-4 * sum_j w_j |v_j| (plus bf16
 * rounding and the score error above) per element, with w the exact weights.
 * Limits: D = 128; Sk * 128 < 2^31.
 */
int fa_prefill_fp8_fwd(const void* q, const void* k, const void* v, const float* q_scale,
                       const float* k_scale, const float* v_scale, void* out, float* lse, int B,
                       int Hq, int Hkv, int Sq, int Sk, int D, int causal, float scale,
                       void* stream);

/*
 * fa_prefill_bwd -- gradients of the bf16 prefill: dQ, dK, dV from dO.
 * ("Flash Attention & Paged Attention" blog, "1. FlashAttention" and
 * "FasterTransformer vs FlashAttention", section 3: recomputation -- the
 * backward rebuilds the attention weights from the LSE the forward saved
 * instead of storing the N x N matrix; "FIA / FlashAttention" Q&A, section
 * 3: FlashAttention's backward is what training needs.)
 *
 *   q, k, v   as given to fa_prefill_fwd (bf16, D = 128, contiguous BHSD)
 *   o, lse    fa_prefill_fwd's outputs for them (same causal flag and scale)
 *   dout      [B, Hq, Sq, 128] bf16 upstream gradient dO
 *   dq        [B, Hq, Sq, 128] bf16, written
 *   dk, dv    [B, Hkv, Sk, 128] bf16, written; a KV head's gradient sums the
 *             query heads h with h / (Hq / Hkv) equal to it
 *   workspace device buffer of >= fa_prefill_bwd_workspace_size(B, Hq, Sq)
 *             bytes (holds -D_i, D_i = sum_d dO_id O_id, and LSE_i in log2 units,
 *             written by the first kernel for the second)
 * dS = P * (dP - D) with P = exp(scale S - LSE), dP = dO V^T; dQ = scale dS K,
 * dK = scale dS^T Q, dV = P^T dO; fp32 accumulation, bf16 products (P and dS
 * are rounded to bf16 for the matrix cores). Two kernels on `stream`, no
 * atomics. Limits: D = 128, Hq % Hkv == 0, Sq and Sk below 2^23.
 */
size_t fa_prefill_bwd_workspace_size(int B, int Hq, int Sq);

int fa_prefill_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq,
                   int Sk, int D, int causal, float scale, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * fa_prefill_bwd_noalloc -- fa_prefill_bwd without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving or training loops, harnesses that forbid hipMalloc). The two
 * per-row arrays the workspace would hold live in a static device array of
 * 32 MiB (one per GPU, held until the process ends), so
 * fa_prefill_bwd_workspace_size(B, Hq, Sq) must not exceed 32 MiB:
 * B * Hq * Sq up to about 4.19M rows. Larger calls return FA_ERR_WORKSPACE
 * and launch nothing. Arguments, results and errors are otherwise those of
 * fa_prefill_bwd, and the same kernels run. This call allocates nothing: no
 * hipMalloc, no hipFree, no library allocation. Every call on a GPU shares
 * that GPU's array; calls that overlap on one GPU (two streams, two threads)
 * race and must be serialised by the caller. The array's address is looked
 * up on the first call on each device (FA_ERR_HIP if that fails).
 */
int fa_prefill_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                           int Hq, int Hkv, int Sq, int Sk, int D, int causal, float scale,
                           void* stream);

/*
 * Paged Flash-Decoding: plan once per batch composition, then run.
 * ("FIA / FlashAttention" Q&A, section 2: plan preprocesses ragged lengths
 * and balances load, run executes the batch; "Flash Attention & Paged
 * Attention", Flash-Decoding and PagedAttention sections.)
 *
 * KV cache layout: k_pages / v_pages are pools [P, Hkv, 64, D] (one 64-token
 * page of one KV head is a contiguous [64, D] block); page_table is int32
 * [B, max_pages_per_req], logical page j of request b at physical page
 * page_table[b * max_pages_per_req + j]; only entries j < ceil(L_b / 64) are
 * read. Tokens past L_b on the last page are never read into the result
 * (their contents may be anything, NaN included).
 */
typedef struct fa_decode_plan_s fa_decode_plan_t;

/*
 * Bytes of device workspace a plan for this batch shape needs; pass the same
 * arguments later to fa_decode_plan. Returns 0 on invalid arguments.
 * num_splits_request as in fa_decode_plan; num_cus = 0 means "the current
 * device's CU count" (a HIP query), else the value given.
 */
size_t fa_decode_workspace_size(const int32_t* seqlens_host, int B, int Hq, int Hkv, int D,
                                int num_splits_request, int num_cus);

/*
 * fa_decode_plan -- split every request's pages into chunks and balance them.
 *   seqlens_host       host int32[B], context length L_b >= 0 of each request
 *   page_table_host    host int32[B * max_pages_per_req] or NULL. When given,
 *                      every entry the run will read is checked to lie in
 *                      [0, num_pages); violations return
 *                      FA_ERR_INVALID_ARGUMENT (the device kernel also skips
 *                      out-of-range ids, so a bad table cannot fault).
 *   max_pages_per_req  row stride of the page table; ceil(L_b/64) must fit.
 *   num_pages          P, pages in each pool.
 *   Hq, Hkv, D         heads and head size; Hq % Hkv == 0, Hq/Hkv in
 *                      {1, 2, 4, 8, 16}, D = 128.
 *   kv_dtype           FA_DTYPE_BF16 or FA_DTYPE_FP8_E4M3FN.
 *   num_splits_request 0 = let the plan choose the chunk size for the
 *                      device's CUs; k > 0 = split every request into
 *                      min(k, pages_b) near-equal page ranges.
 *   num_cus            0 = query the current device, else use this count.
 *   workspace          16-byte aligned device buffer of >=
 *                      fa_decode_workspace_size bytes; the plan uploads its
 *                      work list there with one hipMemcpyAsync on `stream`.
 *   plan_out           receives a host plan object (free with
 *                      fa_decode_plan_destroy, after the runs that use it).
 *   num_splits_out     receives the largest split count of any request: the
 *                      stride of the partial-result buffers, to be passed to
 *                      fa_decode_run.
 */
int fa_decode_plan(const int32_t* seqlens_host, const int32_t* page_table_host, int B,
                   int max_pages_per_req, int num_pages, int Hq, int Hkv, int D, int kv_dtype,
                   int num_splits_request, int num_cus, void* workspace,
                   size_t workspace_bytes, void* stream, fa_decode_plan_t** plan_out,
                   int* num_splits_out);

void fa_decode_plan_destroy(fa_decode_plan_t* plan);

/*
 * Host view of a plan, for inspection and tests. Copies up to `capacity`
 * work items into items_out as int32 quadruples
 * (request b, kv head g | split << 8, first page, end page (exclusive)) and
 * each request's split count into splits_out[B] (either pointer may be NULL).
 * Items with b = -1 are padding (see fa_decode_plan_host).
 * Returns the number of work items, or -1 on a NULL plan.
 */
int fa_decode_plan_items(const fa_decode_plan_t* plan, int32_t* items_out, int capacity,
                         int32_t* splits_out, int* chunk_pages_out);

/*
 * Pure host planning (no device, no HIP call): the same work list
 * fa_decode_plan computes, for a given CU count. Writes up to `capacity`
 * quadruples as in fa_decode_plan_items and each request's split count into
 * splits_out[B]. Returns the number of work items, or a negative fa_status
 * on invalid arguments.
 *   grid_out  receives the number of split-kernel workgroups; workgroup w
 *             runs items w, w + grid, w + 2 grid, ... In the usual plan grid
 *             equals the item count (one item each, longest first). When
 *             every item fits one round of the resident workgroups, the
 *             auto plan may instead cut each KV head's pages, concatenated
 *             over the requests, into windows of equal estimated cost (pages
 *             plus a fixed cost per item), one per workgroup; a window that
 *             crosses a request boundary is two items in successive rounds,
 *             and rounds are padded with b = -1 items. chunk_pages_out then
 *             receives that cost bound.
 */
int fa_decode_plan_host(const int32_t* seqlens_host, int B, int max_pages_per_req, int Hq,
                        int Hkv, int num_splits_request, int num_cus, int32_t* items_out,
                        int capacity, int32_t* splits_out, int* num_splits_out,
                        int* chunk_pages_out, int* grid_out);

/*
 * fa_decode_run -- split-KV decode plus LSE merge; two kernels on `stream`,
 * no host synchronisation, no allocation (so it can be captured in a graph).
 *   q          [B, Hq, D] bf16, one query token per request
 *   k_pages    [P, Hkv, 64, D] bf16, or uint8 e4m3fn codes (per plan dtype)
 *   v_pages    same as k_pages
 *   k_scale    fp32 [P, Hkv] dequantisation scale per page and KV head
 *              (value = code * scale); required for fp8, ignored for bf16.
 *              Scales must be finite and >= 0 (a quantiser's max|x|/448 is);
 *              negative scales give undefined results.
 *   v_scale    same for V
 *   page_table int32 [B, max_pages_per_req] (device copy of the plan's table)
 *   seqlens    int32 [B] device copy of the lengths given to the plan (the
 *              kernel masks tokens >= seqlens[b]; they must match the plan)
 *   num_splits must equal the plan's *num_splits_out
 *   scale      score multiplier; <= 0 selects 1/sqrt(D)
 *   out        [B, Hq, D] bf16, written; lse [B, Hq] fp32, written. A request
 *              with L_b = 0 gets out = 0 and lse = -inf.
 *   workspace  the buffer given to the plan (it holds the work list and the
 *              per-split partial results); any other pointer is rejected
 *              with FA_ERR_INVALID_ARGUMENT
 */
int fa_decode_run(const fa_decode_plan_t* plan, const void* q, const void* k_pages,
                  const void* v_pages, const float* k_scale, const float* v_scale,
                  const int32_t* page_table, const int32_t* seqlens, int num_splits, float scale,
                  void* out, float* lse, void* workspace, void* stream);

/*
 * Ragged prefill over a paged KV cache: append, plan, run.
 * ("Flash Attention & Paged Attention" blog, "FA and the prefill phase":
 * prefill attends over the whole prompt and leaves the computed K and V in
 * device memory as the KV cache that decode reuses; "2. PagedAttention":
 * that cache lives in fixed-size pages behind a page table; "FIA /
 * FlashAttention" Q&A, section 2: variable-length batches, a plan step that
 * preprocesses the lengths and balances the work, then a run step.)
 *
 * A batch holds B requests. Request b brings n_b new tokens (n_b >= 0) and
 * ends up with L_b >= n_b tokens in its cache; the new tokens are the last
 * n_b of those, at positions L_b - n_b .. L_b - 1, after a cached prefix of
 * L_b - n_b tokens. The new tokens of all requests are packed along one axis
 * of T = sum n_b rows in request order:
 *   cu_seqlens_q  int32 [B + 1], cu[0] = 0, cu[b+1] = cu[b] + n_b
 *   seqlens       int32 [B], L_b (prefix plus new tokens)
 * KV pools and page table are laid out as for decode above (pools
 * [P, Hkv, 64, D] bf16, page_table int32 [B, max_pages_per_req]); entry j of
 * row b is read for j < ceil(L_b / 64). D = 128 and Hq % Hkv == 0; query
 * head h reads KV head h / (Hq / Hkv).
 */

/*
 * fa_kv_append -- write the new tokens' K and V into their pages.
 *   k_new, v_new  [T, Hkv, D] bf16, packed as cu_seqlens_q says
 *   k_pages, v_pages  pools, updated in place: new token i of request b goes
 *                 to slot t % 64 of page page_table[b][t / 64], t = L_b - n_b + i.
 *   page_table, seqlens, cu_seqlens_q  DEVICE int32 arrays as above
 *   B, total_q    requests and T (= cu_seqlens_q[B])
 * A bit-exact copy; nothing else in the pools changes. Tokens whose page id
 * lies outside [0, num_pages), whose position is negative (n_b > L_b) or
 * whose page index reaches max_pages_per_req are skipped, so bad device
 * metadata cannot make the kernel write outside the pools. One kernel on
 * `stream`; total_q = 0 is a no-op. Pages shared by several requests'
 * positions must not be written by two of them in one call.
 */
int fa_kv_append(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                 const int32_t* page_table, const int32_t* seqlens, const int32_t* cu_seqlens_q,
                 int B, int total_q, int max_pages_per_req, int num_pages, int Hkv, int D,
                 void* stream);

typedef struct fa_prefill_plan_s fa_prefill_plan_t;

/*
 * Pure host planning for the ragged prefill (no device, no HIP call).
 * The work is cut into items (request b, query tile qt) of 256 new tokens
 * each (the last tile of a request may be shorter; a request with n_b = 0
 * has none), ordered by decreasing key count so that the longest items
 * start first. Writes up to `capacity` pairs (b, qt) into items_out (may be
 * NULL) and returns the number of items, or a negative fa_status when the
 * lengths are inconsistent (cu not starting at 0 or decreasing, n_b > L_b,
 * a negative length).
 */
int fa_prefill_paged_plan_host(const int32_t* seqlens_host, const int32_t* cu_seqlens_q_host,
                               int B, int32_t* items_out, int capacity);

/* Bytes of device workspace fa_prefill_paged_plan needs (0 on invalid arguments). */
size_t fa_prefill_paged_workspace_size(const int32_t* seqlens_host,
                                       const int32_t* cu_seqlens_q_host, int B);

/*
 * fa_prefill_paged_plan -- build and upload the work list of a ragged batch.
 *   seqlens_host, cu_seqlens_q_host  host copies of the batch's lengths
 *   page_table_host  host int32 [B, max_pages_per_req] or NULL; when given,
 *                    every entry the run reads is checked to lie in
 *                    [0, num_pages) (FA_ERR_INVALID_ARGUMENT otherwise).
 *   Hq, Hkv, D       heads and head size (D = 128, Hq % Hkv == 0, <= 256)
 *   workspace        16-byte aligned device buffer of >=
 *                    fa_prefill_paged_workspace_size bytes; the work list is
 *                    uploaded there with one hipMemcpyAsync on `stream`
 *                    followed by a wait on it. fa_prefill_paged_run must be
 *                    given this same buffer (FA_ERR_INVALID_ARGUMENT otherwise).
 *   plan_out         receives a host plan object (fa_prefill_paged_plan_destroy).
 */
int fa_prefill_paged_plan(const int32_t* seqlens_host, const int32_t* cu_seqlens_q_host,
                          const int32_t* page_table_host, int B, int max_pages_per_req,
                          int num_pages, int Hq, int Hkv, int D, void* workspace,
                          size_t workspace_bytes, void* stream, fa_prefill_plan_t** plan_out);

void fa_prefill_paged_plan_destroy(fa_prefill_plan_t* plan);

/*
 * fa_prefill_paged_run -- causal attention of every new token over its
 * request's whole cache (prefix and new tokens), one kernel on `stream`, no
 * allocation and no host synchronisation.
 *   q            [T, Hq, D] bf16, packed new tokens
 *   k_pages, v_pages  pools already holding all L_b tokens of every request
 *                (call fa_kv_append first for the new ones)
 *   page_table, seqlens, cu_seqlens_q  device copies of what the plan saw
 *   scale        score multiplier; <= 0 selects 1/sqrt(D)
 *   out          [T, Hq, D] bf16, written (rounded to nearest even)
 *   lse          [T, Hq] fp32 natural-log LSE, written
 * New token i of request b sees keys 0 .. L_b - n_b + i: the causal mask
 * aligned bottom-right, as in fa_prefill_fwd with Sq = n_b, Sk = L_b.
 * Page ids outside [0, num_pages) read as zeros (never out of bounds).
 */
int fa_prefill_paged_run(const fa_prefill_plan_t* plan, const void* q, const void* k_pages,
                         const void* v_pages, const int32_t* page_table, const int32_t* seqlens,
                         const int32_t* cu_seqlens_q, float scale, void* out, float* lse,
                         void* workspace, void* stream);

/*
 * Shared-prefix (cascade) decode: requests that share a prompt prefix.
 * ("FIA / FlashAttention" Q&A, section 3's comparison table: prefix sharing
 * and head-query fusion as inference optimisations; "Flash Attention & Paged
 * Attention", Flash-Decoding: partial results over parts of the KV sequence
 * are combined exactly by their LogSumExp.)
 *
 * The batch is a paged decode batch as above. Requests are put in groups;
 * every request of group j starts its page-table row with the same
 * prefix_pages[j] physical pages (a prefix of 64 * prefix_pages[j] tokens,
 * whole pages only, held once in the pool). The result is exactly decode
 * attention over each request's whole cache, as fa_decode_run computes it;
 * only the work is organised differently: a group's prefix is attended once
 * for all its decode queries (the G query heads of every member folded into
 * the rows of one dense matrix-core tile per KV head), each request's suffix
 * goes through the split-KV kernel, and the LSE merge combines prefix and
 * suffix partials. bf16 KV only; Hq, Hkv, D as for fa_decode_plan.
 *
 *   prefix_group_host  host int32[B]: group of each request, or -1 (no prefix)
 *   prefix_pages_host  host int32[n_groups]: prefix length of each group in
 *                      pages (0 allowed); every member needs L_b >= 64 * that.
 *   n_groups           number of groups (0: an ordinary decode plan)
 * The plan checks, on the host page table, that every member shares its
 * group's prefix pages (FA_ERR_INVALID_ARGUMENT otherwise). The plan object
 * is used with fa_decode_run and freed with fa_decode_plan_destroy like any
 * decode plan (the workspace rules of fa_decode_plan apply); fa_decode_run
 * then launches three kernels (prefix pass, split-KV kernel, merge).
 */
size_t fa_decode_cascade_workspace_size(const int32_t* seqlens_host, int B, int max_pages_per_req,
                                        int Hq, int Hkv, int D, const int32_t* prefix_group_host,
                                        const int32_t* prefix_pages_host, int n_groups,
                                        int num_cus);

int fa_decode_plan_cascade(const int32_t* seqlens_host, const int32_t* page_table_host, int B,
                           int max_pages_per_req, int num_pages, int Hq, int Hkv, int D,
                           const int32_t* prefix_group_host, const int32_t* prefix_pages_host,
                           int n_groups, int num_cus, void* workspace, size_t workspace_bytes,
                           void* stream, fa_decode_plan_t** plan_out, int* num_splits_out);

/*
 * Pure host cascade planning (no device, no HIP call), for inspection and
 * tests. Writes up to `capacity` suffix work items as in
 * fa_decode_plan_items, up to `prefix_capacity` prefix items as int32
 * octets (member-list offset, KV head, first folded row, rows, first page,
 * end page, partial slot, a member request), each request's slot count
 * into splits_out[B], the prefix item count and the largest slot count.
 * Returns the number of suffix items or a negative fa_status.
 */
int fa_decode_plan_cascade_host(const int32_t* seqlens_host, int B, int max_pages_per_req, int Hq,
                                int Hkv, const int32_t* prefix_group_host,
                                const int32_t* prefix_pages_host, int n_groups, int num_cus,
                                int32_t* items_out, int capacity, int32_t* prefix_items_out,
                                int prefix_capacity, int32_t* splits_out,
                                int* n_prefix_items_out, int* num_splits_out);

/*
 * fa_debug_gather_kv -- copy the L_b logical tokens of one request and KV
 * head out of a paged pool into dst [L_b, D] (same element type as the
 * pool): logical token t is slot t mod 64 of physical page
 * page_table[b][t / 64] ("Flash Attention & Paged Attention" blog,
 * "2. PagedAttention": a logical-to-physical table over fixed-size pages;
 * "FlashAttention breakthrough architecture", paged storage: 64-token
 * blocks). A small kernel of its own, for the bit-exact test of the page
 * layout; the attention kernels do their own lookups. max_pages_per_req and
 * num_pages as for the plan; ids outside [0, num_pages) leave their tokens'
 * dst rows untouched.
 */
int fa_debug_gather_kv(const void* pages, int kv_dtype, const int32_t* page_table,
                       int max_pages_per_req, int num_pages, int Hkv, int D, int b, int L_b,
                       int kv_head, void* dst, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
