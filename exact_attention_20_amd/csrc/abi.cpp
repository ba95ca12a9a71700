// C ABI of libfa.so: argument validation, plan objects and kernel dispatch.
// The public contract (argument meaning, layouts, ownership, errors) is in
// include/fa.h; this file implements it. No device work is enqueued until
// every check has passed.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "fa.h"
#include "fa_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return FA_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(FA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Plan workspaces hold 16-byte work items and float4 partial results.
bool misaligned(const void* p) { return ((uintptr_t)p & 15) != 0; }

int device_cus(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  e = hipDeviceGetAttribute(out, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(CU count)");
  return FA_OK;
}

}  // namespace

struct fa_decode_plan_s {
  int B, stride, num_pages, Hq, Hkv, D, kv_dtype, num_splits, chunk_pages;
  int grid;  // split-kernel workgroups (each runs items w, w + grid, ...)
  std::vector<fa::WorkItem> items;
  std::vector<int32_t> splits;
  std::vector<fa::PrefixItem> prefix_items;  // cascade plans only
  std::vector<int32_t> group_reqs;
  fa::WorkspaceLayout layout;
  const void* workspace;  // the buffer holding this plan's work list
};

struct fa_prefill_plan_s {
  int B, stride, num_pages, Hq, Hkv, D, n_items;
  size_t bytes;           // workspace bytes the work list occupies
  const void* workspace;  // the buffer holding the work list
};

extern "C" {

const char* fa_last_error(void) { return g_err.c_str(); }

int fa_device_status(unsigned int* flags_out, int clear) {
  if (!flags_out) return fail(FA_ERR_INVALID_ARGUMENT, "fa_device_status: flags_out is null");
  unsigned* p = nullptr;
  hipError_t e = fa::device_status_ptr(&p);
  if (e != hipSuccess) return hip_fail(e, "fa_device_status: device status word");
  e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "fa_device_status: synchronize");
  unsigned v = 0;
  e = hipMemcpy(&v, p, sizeof v, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "fa_device_status: read");
  if (clear && v != 0) {
    const unsigned zero = 0;
    e = hipMemcpy(p, &zero, sizeof zero, hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "fa_device_status: clear");
  }
  *flags_out = v;
  return ok();
}

int fa_abi_version(void) { return 2; }

int fa_prefill_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                   int Hq, int Hkv, int Sq, int Sk, int D, int dtype, int causal, float scale,
                   const int32_t* kv_head_map, void* stream) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 0 || Sk < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_fwd: need B,Hq,Hkv >= 1 and Sq,Sk >= 0 (got B=%d Hq=%d Hkv=%d Sq=%d Sk=%d)", B, Hq, Hkv, Sq, Sk);
  if (Hq > fa::kMaxHeads || Hkv > fa::kMaxHeads)
    return fail(FA_ERR_UNSUPPORTED, "fa_prefill_fwd: Hq and Hkv must be <= %d", fa::kMaxHeads);
  if (causal != 0 && causal != 1)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_fwd: causal must be 0 or 1");
  if (!(std::isfinite(scale)))
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_fwd: scale is not finite");
  if (dtype == FA_DTYPE_F32) {
    if (D != 64 && D != 128)
      return fail(FA_ERR_UNSUPPORTED, "fa_prefill_fwd: fp32 supports D in {64,128} (got %d)", D);
  } else if (dtype == FA_DTYPE_BF16) {
    if (D != 128) return fail(FA_ERR_UNSUPPORTED, "fa_prefill_fwd: bf16 supports D=128 (got %d)", D);
    // K/V tiles are read through a buffer resource of Sk * 256 bytes per head.
    if ((long long)Sk * 256 > 0x7fffffffLL)
      return fail(FA_ERR_UNSUPPORTED, "fa_prefill_fwd: bf16 needs Sk below 2^23 (got %d)", Sk);
  } else {
    return fail(FA_ERR_UNSUPPORTED, "fa_prefill_fwd: dtype %d not supported (F32 or BF16)", dtype);
  }
  fa::PrefillArgs a;
  std::memset(&a, 0, sizeof a);
  if (kv_head_map) {
    for (int h = 0; h < Hq; ++h) {
      if (kv_head_map[h] < 0 || kv_head_map[h] >= Hkv)
        return fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_fwd: kv_head_map[%d]=%d outside [0,%d)", h, kv_head_map[h], Hkv);
      a.kv_map[h] = (uint8_t)kv_head_map[h];
    }
    a.has_map = 1;
  } else if (Hq % Hkv != 0) {
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_fwd: Hq %% Hkv != 0 (%d, %d) and no kv_head_map", Hq, Hkv);
  }
  if (Sq == 0) return ok();
  if (!q || !out || !lse || (Sk > 0 && (!k || !v)))
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_fwd: null tensor pointer");
  a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Sq = Sq; a.Sk = Sk; a.D = D;
  a.causal = causal;
  a.scale = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)D));
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = dtype == FA_DTYPE_F32 ? fa::launch_prefill_f32(a, s) : fa::launch_prefill_bf16(a, s);
  if (e != hipSuccess) return hip_fail(e, "fa_prefill_fwd launch");
  return ok();
}

int fa_prefill_fp8_fwd(const void* q, const void* k, const void* v, const float* q_scale,
                       const float* k_scale, const float* v_scale, void* out, float* lse, int B, int Hq,
                       int Hkv, int Sq, int Sk, int D, int causal, float scale, void* stream) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 0 || Sk < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_fp8_fwd: need B,Hq,Hkv >= 1 and Sq,Sk >= 0");
  if (Hq > fa::kMaxHeads || Hkv > fa::kMaxHeads)
    return fail(FA_ERR_UNSUPPORTED, "fa_prefill_fp8_fwd: Hq and Hkv must be <= %d", fa::kMaxHeads);
  if (Hq % Hkv != 0) return fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_fp8_fwd: Hq %% Hkv != 0 (%d, %d)", Hq, Hkv);
  if (D != 128) return fail(FA_ERR_UNSUPPORTED, "fa_prefill_fp8_fwd: D=%d not supported (128)", D);
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_fp8_fwd: causal must be 0 or 1");
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_fp8_fwd: scale is not finite");
  if (Sq == 0) return ok();
  if (!q || !out || !lse || !q_scale || (Sk > 0 && (!k || !v || !k_scale || !v_scale)))
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_fp8_fwd: null pointer");
  if ((long long)Sk * 128 > 0x7fffffffLL)
    return fail(FA_ERR_UNSUPPORTED, "fa_prefill_fp8_fwd: Sk * 128 must fit in 31 bits");
  const float sc = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)D));
  hipError_t e = fa::launch_prefill_fp8(q, k, v, q_scale, k_scale, v_scale, out, lse, B, Hq, Hkv, Sq, Sk, causal,
                                        sc, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fa_prefill_fp8_fwd launch");
  return ok();
}

size_t fa_prefill_bwd_workspace_size(int B, int Hq, int Sq) {
  if (B < 1 || Hq < 1 || Sq < 0) return 0;
  // -D_i, then LSE_i in log2 units, one fp32 array each.
  return 2 * (((size_t)B * Hq * (size_t)Sq * sizeof(float) + 255) / 256 * 256) + 256;
}

// Argument checks shared by the two backward entry points; FA_OK when a launch is needed.
static int check_bwd(const char* who, const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv,
                     int Sq, int Sk, int D, int causal, float scale) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 0 || Sk < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: need B,Hq,Hkv >= 1 and Sq,Sk >= 0", who);
  if (Hq > fa::kMaxHeads || Hkv > fa::kMaxHeads)
    return fail(FA_ERR_UNSUPPORTED, "%s: Hq and Hkv must be <= %d", who, fa::kMaxHeads);
  if (Hq % Hkv != 0) return fail(FA_ERR_INVALID_ARGUMENT, "%s: Hq %% Hkv != 0 (%d, %d)", who, Hq, Hkv);
  if (D != 128) return fail(FA_ERR_UNSUPPORTED, "%s: D=%d not supported (128)", who, D);
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARGUMENT, "%s: causal must be 0 or 1", who);
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARGUMENT, "%s: scale is not finite", who);
  if ((long long)std::max(Sq, Sk) * 256 > 0x7fffffffLL)
    return fail(FA_ERR_UNSUPPORTED, "%s: Sq and Sk must be below 2^23", who);
  if ((Sq > 0 && (!q || !o || !lse || !dout || !dq)) || (Sk > 0 && (!k || !v || !dk || !dv)))
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: null tensor pointer", who);
  return FA_OK;
}

static int launch_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Sk,
                      int D, int causal, float scale, void* workspace, const char* who, void* stream) {
  fa::BwdLaunch l;
  l.q = q; l.k = k; l.v = v; l.o = o; l.dO = dout; l.lse = lse;
  l.delta = (float*)workspace;
  l.lse2 = (float*)((char*)workspace + ((size_t)B * Hq * (size_t)Sq * sizeof(float) + 255) / 256 * 256);
  l.dq = dq; l.dk = dk; l.dv = dv;
  l.B = B; l.Hq = Hq; l.Hkv = Hkv; l.Sq = Sq; l.Sk = Sk; l.causal = causal;
  l.scale = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)D));
  hipError_t e = fa::launch_attention_bwd(l, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, who);
  return ok();
}

int fa_prefill_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Sk,
                   int D, int causal, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_bwd("fa_prefill_bwd", q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Sq, Sk, D, causal, scale);
  if (st != FA_OK) return st;
  if (Sq == 0 && Sk == 0) return ok();
  const size_t need = fa_prefill_bwd_workspace_size(B, Hq, Sq);
  if (!workspace || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "fa_prefill_bwd: workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  return launch_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Sq, Sk, D, causal, scale, workspace,
                    "fa_prefill_bwd launch", stream);
}

int fa_prefill_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq,
                           int Sk, int D, int causal, float scale, void* stream) {
  int st = check_bwd("fa_prefill_bwd_noalloc", q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Sq, Sk, D, causal,
                     scale);
  if (st != FA_OK) return st;
  if (Sq == 0 && Sk == 0) return ok();
  const size_t need = fa_prefill_bwd_workspace_size(B, Hq, Sq);
  if (need > fa::kBwdScratchBytes)
    return fail(FA_ERR_WORKSPACE,
                "fa_prefill_bwd_noalloc: needs %zu bytes of scratch, more than the static %zu "
                "(B*Hq*Sq <= %zu rows); use fa_prefill_bwd with a workspace",
                need, fa::kBwdScratchBytes, (fa::kBwdScratchBytes - 768) / 8);
  void* ws = nullptr;
  hipError_t e = fa::bwd_scratch(&ws);
  if (e != hipSuccess) return hip_fail(e, "fa_prefill_bwd_noalloc: scratch address");
  return launch_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Sq, Sk, D, causal, scale, ws,
                    "fa_prefill_bwd_noalloc launch", stream);
}

static int check_decode_shape(int B, int Hq, int Hkv, int D) {
  if (B < 1 || Hq < 1 || Hkv < 1)
    return fail(FA_ERR_INVALID_ARGUMENT, "decode: need B, Hq, Hkv >= 1");
  if (Hq > fa::kMaxHeads || Hkv > fa::kMaxHeads)
    return fail(FA_ERR_UNSUPPORTED, "decode: Hq and Hkv must be <= %d", fa::kMaxHeads);
  if (Hq % Hkv != 0) return fail(FA_ERR_INVALID_ARGUMENT, "decode: Hq %% Hkv != 0 (%d, %d)", Hq, Hkv);
  int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
    return fail(FA_ERR_UNSUPPORTED, "decode: group size Hq/Hkv=%d not in {1,2,4,8,16}", G);
  if (D != 128) return fail(FA_ERR_UNSUPPORTED, "decode: D=%d not supported (128)", D);
  return FA_OK;
}

size_t fa_decode_workspace_size(const int32_t* seqlens_host, int B, int Hq, int Hkv, int D,
                                int num_splits_request, int num_cus) {
  if (!seqlens_host || check_decode_shape(B, Hq, Hkv, D) != FA_OK || num_splits_request < 0) return 0;
  if (num_cus == 0 && device_cus(&num_cus) != FA_OK) return 0;
  int stride = 1;
  for (int b = 0; b < B; ++b) {
    if (seqlens_host[b] < 0) return 0;
    stride = std::max(stride, (int)(((int64_t)seqlens_host[b] + fa::kPage - 1) / fa::kPage));
  }
  fa::PlanResult r;
  if (fa::plan_decode_host(seqlens_host, B, stride, Hkv, num_splits_request, num_cus, nullptr, 0,
                           nullptr, &r) != 0)
    return 0;
  return fa::workspace_layout(r.n_items, B, Hq, D, r.num_splits).total;
}

int fa_decode_plan_host(const int32_t* seqlens_host, int B, int max_pages_per_req, int Hq, int Hkv,
                        int num_splits_request, int num_cus, int32_t* items_out, int capacity,
                        int32_t* splits_out, int* num_splits_out, int* chunk_pages_out, int* grid_out) {
  if (!seqlens_host || B < 1 || Hkv < 1 || Hq < 1 || max_pages_per_req < 1 || num_cus < 1 ||
      capacity < 0 || num_splits_request < 0) {
    fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_plan_host: invalid argument");
    return -FA_ERR_INVALID_ARGUMENT;
  }
  fa::PlanResult r;
  std::vector<fa::WorkItem> tmp;
  if (items_out && capacity > 0) tmp.resize(capacity);
  if (fa::plan_decode_host(seqlens_host, B, max_pages_per_req, Hkv, num_splits_request, num_cus,
                           tmp.empty() ? nullptr : tmp.data(), capacity, splits_out, &r) != 0) {
    fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_plan_host: bad lengths or page-table stride");
    return -FA_ERR_INVALID_ARGUMENT;
  }
  if (items_out) {
    int n = std::min(capacity, r.n_items);
    for (int i = 0; i < n; ++i) {
      items_out[4 * i + 0] = tmp[i].b;
      items_out[4 * i + 1] = tmp[i].g_split;
      items_out[4 * i + 2] = tmp[i].page_begin;
      items_out[4 * i + 3] = tmp[i].page_end;
    }
  }
  if (num_splits_out) *num_splits_out = r.num_splits;
  if (chunk_pages_out) *chunk_pages_out = r.chunk_pages;
  if (grid_out) *grid_out = r.grid;
  ok();
  return r.n_items;
}

int fa_decode_plan(const int32_t* seqlens_host, const int32_t* page_table_host, int B,
                   int max_pages_per_req, int num_pages, int Hq, int Hkv, int D, int kv_dtype,
                   int num_splits_request, int num_cus, void* workspace, size_t workspace_bytes,
                   void* stream, fa_decode_plan_t** plan_out, int* num_splits_out) {
  if (!plan_out || !num_splits_out)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_plan: plan_out and num_splits_out must be non-null");
  *plan_out = nullptr;
  int st = check_decode_shape(B, Hq, Hkv, D);
  if (st != FA_OK) return st;
  if (!seqlens_host) return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_plan: seqlens_host is null");
  if (max_pages_per_req < 1 || num_pages < 1)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_plan: need max_pages_per_req >= 1 and num_pages >= 1");
  if (kv_dtype != FA_DTYPE_BF16 && kv_dtype != FA_DTYPE_FP8_E4M3FN)
    return fail(FA_ERR_UNSUPPORTED, "fa_decode_plan: kv_dtype %d not supported (BF16 or FP8_E4M3FN)", kv_dtype);
  if (num_splits_request < 0) return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_plan: num_splits_request < 0");
  if (num_cus < 0) return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_plan: num_cus < 0");
  for (int b = 0; b < B; ++b) {
    if (seqlens_host[b] < 0) return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_plan: seqlens[%d] < 0", b);
    int64_t n = ((int64_t)seqlens_host[b] + fa::kPage - 1) / fa::kPage;
    if (n > max_pages_per_req)
      return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_plan: request %d needs %lld pages > max_pages_per_req %d", b, (long long)n, max_pages_per_req);
    if (page_table_host) {
      for (int64_t j = 0; j < n; ++j) {
        int32_t id = page_table_host[(int64_t)b * max_pages_per_req + j];
        if (id < 0 || id >= num_pages)
          return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_plan: page_table[%d][%lld]=%d outside [0,%d)", b, (long long)j, id, num_pages);
      }
    }
  }
  if (num_cus == 0) {
    st = device_cus(&num_cus);
    if (st != FA_OK) return st;
  }
  fa::PlanResult r;
  if (fa::plan_decode_host(seqlens_host, B, max_pages_per_req, Hkv, num_splits_request, num_cus,
                           nullptr, 0, nullptr, &r) != 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_plan: planning failed");
  fa_decode_plan_t* p = new (std::nothrow) fa_decode_plan_t;
  if (!p) return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_plan: out of host memory");
  p->items.resize(std::max(r.n_items, 1));
  p->splits.resize(B);
  fa::plan_decode_host(seqlens_host, B, max_pages_per_req, Hkv, num_splits_request, num_cus,
                       p->items.data(), r.n_items, p->splits.data(), &r);
  p->B = B; p->stride = max_pages_per_req; p->num_pages = num_pages;
  p->Hq = Hq; p->Hkv = Hkv; p->D = D; p->kv_dtype = kv_dtype;
  p->num_splits = r.num_splits; p->chunk_pages = r.chunk_pages;
  p->grid = r.grid;
  p->items.resize(r.n_items);
  p->layout = fa::workspace_layout(r.n_items, B, Hq, D, r.num_splits);
  if (!workspace || workspace_bytes < p->layout.total) {
    size_t need = p->layout.total;
    delete p;
    return fail(FA_ERR_WORKSPACE, "fa_decode_plan: workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  }
  if (misaligned(workspace)) {
    delete p;
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_plan: workspace must be 16-byte aligned");
  }
  p->workspace = workspace;
  // Work list and split counts into one host staging block, one upload.
  std::vector<char> stage(p->layout.part_o_off, 0);
  if (r.n_items) std::memcpy(stage.data() + p->layout.items_off, p->items.data(), sizeof(fa::WorkItem) * r.n_items);
  std::memcpy(stage.data() + p->layout.splits_off, p->splits.data(), sizeof(int32_t) * B);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(workspace, stage.data(), stage.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);  // staging block is freed on return
  if (e != hipSuccess) {
    delete p;
    return hip_fail(e, "fa_decode_plan upload");
  }
  *plan_out = p;
  *num_splits_out = r.num_splits;
  return ok();
}

void fa_decode_plan_destroy(fa_decode_plan_t* plan) { delete plan; }

int fa_decode_plan_items(const fa_decode_plan_t* plan, int32_t* items_out, int capacity,
                         int32_t* splits_out, int* chunk_pages_out) {
  if (!plan) return -1;
  int n = std::min<int>(capacity, (int)plan->items.size());
  for (int i = 0; items_out && i < n; ++i) {
    items_out[4 * i + 0] = plan->items[i].b;
    items_out[4 * i + 1] = plan->items[i].g_split;
    items_out[4 * i + 2] = plan->items[i].page_begin;
    items_out[4 * i + 3] = plan->items[i].page_end;
  }
  if (splits_out) std::memcpy(splits_out, plan->splits.data(), sizeof(int32_t) * plan->B);
  if (chunk_pages_out) *chunk_pages_out = plan->chunk_pages;
  return (int)plan->items.size();
}

int fa_decode_run(const fa_decode_plan_t* plan, const void* q, const void* k_pages,
                  const void* v_pages, const float* k_scale, const float* v_scale,
                  const int32_t* page_table, const int32_t* seqlens, int num_splits, float scale,
                  void* out, float* lse, void* workspace, void* stream) {
  if (!plan) return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_run: plan is null");
  if (num_splits != plan->num_splits)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_run: num_splits %d != plan's %d", num_splits, plan->num_splits);
  if (!q || !out || !lse || !workspace || !seqlens)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_run: null pointer (q/out/lse/workspace/seqlens)");
  if (workspace != plan->workspace)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_run: workspace is not the buffer the plan was built in");
  if ((!plan->items.empty() || !plan->prefix_items.empty()) && (!k_pages || !v_pages || !page_table))
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_run: null KV pool or page table");
  bool fp8 = plan->kv_dtype == FA_DTYPE_FP8_E4M3FN;
  if (fp8 && !plan->items.empty() && (!k_scale || !v_scale))
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_run: fp8 KV needs k_scale and v_scale");
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_run: scale is not finite");
  char* ws = (char*)workspace;
  fa::DecodeArgs a;
  a.items = (const fa::WorkItem*)(ws + plan->layout.items_off);
  a.n_items = (int)plan->items.size();
  a.grid = plan->grid;
  a.splits_per_req = (const int32_t*)(ws + plan->layout.splits_off);
  a.q = q; a.k_pages = k_pages; a.v_pages = v_pages; a.k_scale = k_scale; a.v_scale = v_scale;
  a.page_table = page_table; a.seqlens = seqlens;
  a.stride = plan->stride; a.num_pages = plan->num_pages;
  a.B = plan->B; a.Hq = plan->Hq; a.Hkv = plan->Hkv; a.D = plan->D;
  a.num_splits = plan->num_splits;
  a.scale = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)plan->D));
  a.part_o = (float*)(ws + plan->layout.part_o_off);
  a.part_lse = (float*)(ws + plan->layout.part_lse_off);
  a.out = out; a.lse = lse;
  hipError_t e = fa::device_status_ptr(&a.status);
  if (e != hipSuccess) return hip_fail(e, "fa_decode_run: device status word");
  hipStream_t s = (hipStream_t)stream;
  if (!plan->prefix_items.empty()) {
    // Cascade plan: the shared prefixes first, into their partial slots.
    fa::PrefillArgs pa;
    std::memset(&pa, 0, sizeof pa);
    pa.q = q; pa.k = k_pages; pa.v = v_pages; pa.out = out; pa.lse = lse;
    pa.B = plan->B; pa.Hq = plan->Hq; pa.Hkv = plan->Hkv; pa.D = plan->D;
    pa.scale = a.scale;
    pa.items = (const int32_t*)(ws + plan->layout.prefix_items_off);
    pa.page_table = page_table; pa.seqlens = seqlens;
    pa.stride = plan->stride; pa.num_pages = plan->num_pages;
    pa.group_reqs = (const int32_t*)(ws + plan->layout.group_reqs_off);
    pa.splits = a.splits_per_req;
    pa.part_o = a.part_o; pa.part_lse = a.part_lse; pa.num_splits = plan->num_splits;
    pa.status = a.status;
    e = fa::launch_prefix_bf16(pa, (int)plan->prefix_items.size(), s);
    if (e != hipSuccess) return hip_fail(e, "fa_decode_run prefix launch");
  }
  if (a.n_items > 0) e = fa::launch_decode_split(a, plan->Hq / plan->Hkv, fp8 ? 1 : 0, s);
  if (e != hipSuccess) return hip_fail(e, "fa_decode_run split launch");
  e = fa::launch_lse_merge(a, s);
  if (e != hipSuccess) return hip_fail(e, "fa_decode_run merge launch");
  return ok();
}

static int cascade_check(const char* who, const int32_t* seqlens_host, int B, int max_pages_per_req,
                         int Hq, int Hkv, int D, const int32_t* prefix_group_host,
                         const int32_t* prefix_pages_host, int n_groups, int num_cus) {
  int st = check_decode_shape(B, Hq, Hkv, D);
  if (st != FA_OK) return st;
  if (!seqlens_host || !prefix_group_host || (n_groups > 0 && !prefix_pages_host))
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: seqlens, prefix_group (and prefix_pages when n_groups > 0) are required", who);
  if (n_groups < 0 || max_pages_per_req < 1 || num_cus < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: need n_groups >= 0, max_pages_per_req >= 1, num_cus >= 0", who);
  for (int j = 0; j < n_groups; ++j)
    if (prefix_pages_host[j] < 0 || prefix_pages_host[j] > max_pages_per_req)
      return fail(FA_ERR_INVALID_ARGUMENT, "%s: prefix_pages[%d]=%d outside [0, %d]", who, j, prefix_pages_host[j], max_pages_per_req);
  for (int b = 0; b < B; ++b) {
    const int j = prefix_group_host[b];
    if (j < -1 || j >= n_groups)
      return fail(FA_ERR_INVALID_ARGUMENT, "%s: prefix_group[%d]=%d outside [-1, %d)", who, b, j, n_groups);
    if (seqlens_host[b] < 0) return fail(FA_ERR_INVALID_ARGUMENT, "%s: seqlens[%d] < 0", who, b);
    if (j >= 0 && seqlens_host[b] < (int64_t)fa::kPage * prefix_pages_host[j])
      return fail(FA_ERR_INVALID_ARGUMENT, "%s: request %d is shorter (%d) than its group's prefix (%d pages)", who, b, seqlens_host[b], prefix_pages_host[j]);
    if (((int64_t)seqlens_host[b] + fa::kPage - 1) / fa::kPage > max_pages_per_req)
      return fail(FA_ERR_INVALID_ARGUMENT, "%s: request %d needs more than max_pages_per_req pages", who, b);
  }
  return FA_OK;
}

size_t fa_decode_cascade_workspace_size(const int32_t* seqlens_host, int B, int max_pages_per_req, int Hq,
                                        int Hkv, int D, const int32_t* prefix_group_host,
                                        const int32_t* prefix_pages_host, int n_groups, int num_cus) {
  if (cascade_check("fa_decode_cascade_workspace_size", seqlens_host, B, max_pages_per_req, Hq, Hkv, D,
                    prefix_group_host, prefix_pages_host, n_groups, num_cus) != FA_OK)
    return 0;
  if (num_cus == 0 && device_cus(&num_cus) != FA_OK) return 0;
  fa::CascadePlan cp;
  if (fa::plan_cascade_host(seqlens_host, B, max_pages_per_req, Hq, Hkv, prefix_group_host, prefix_pages_host,
                            n_groups, num_cus, &cp) != 0)
    return 0;
  return fa::workspace_layout((int)cp.items.size(), B, Hq, D, cp.num_splits, (int)cp.prefix_items.size(),
                              (int)cp.group_reqs.size()).total;
}

int fa_decode_plan_cascade_host(const int32_t* seqlens_host, int B, int max_pages_per_req, int Hq, int Hkv,
                                const int32_t* prefix_group_host, const int32_t* prefix_pages_host,
                                int n_groups, int num_cus, int32_t* items_out, int capacity,
                                int32_t* prefix_items_out, int prefix_capacity, int32_t* splits_out,
                                int* n_prefix_items_out, int* num_splits_out) {
  if (num_cus < 1 || capacity < 0 || prefix_capacity < 0) {
    fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_plan_cascade_host: need num_cus >= 1 and capacities >= 0");
    return -FA_ERR_INVALID_ARGUMENT;
  }
  int st = cascade_check("fa_decode_plan_cascade_host", seqlens_host, B, max_pages_per_req, Hq, Hkv, 128,
                         prefix_group_host, prefix_pages_host, n_groups, num_cus);
  if (st != FA_OK) return -st;
  fa::CascadePlan cp;
  if (fa::plan_cascade_host(seqlens_host, B, max_pages_per_req, Hq, Hkv, prefix_group_host, prefix_pages_host,
                            n_groups, num_cus, &cp) != 0) {
    fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_plan_cascade_host: planning failed");
    return -FA_ERR_INVALID_ARGUMENT;
  }
  for (int i = 0; items_out && i < std::min<int>(capacity, (int)cp.items.size()); ++i) {
    items_out[4 * i + 0] = cp.items[i].b;
    items_out[4 * i + 1] = cp.items[i].g_split;
    items_out[4 * i + 2] = cp.items[i].page_begin;
    items_out[4 * i + 3] = cp.items[i].page_end;
  }
  for (int i = 0; prefix_items_out && i < std::min<int>(prefix_capacity, (int)cp.prefix_items.size()); ++i)
    std::memcpy(prefix_items_out + 8 * i, &cp.prefix_items[i], sizeof(fa::PrefixItem));
  if (splits_out) std::memcpy(splits_out, cp.splits.data(), sizeof(int32_t) * B);
  if (n_prefix_items_out) *n_prefix_items_out = (int)cp.prefix_items.size();
  if (num_splits_out) *num_splits_out = cp.num_splits;
  ok();
  return (int)cp.items.size();
}

int fa_decode_plan_cascade(const int32_t* seqlens_host, const int32_t* page_table_host, int B,
                           int max_pages_per_req, int num_pages, int Hq, int Hkv, int D,
                           const int32_t* prefix_group_host, const int32_t* prefix_pages_host,
                           int n_groups, int num_cus, void* workspace, size_t workspace_bytes,
                           void* stream, fa_decode_plan_t** plan_out, int* num_splits_out) {
  if (!plan_out || !num_splits_out)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_plan_cascade: plan_out and num_splits_out must be non-null");
  *plan_out = nullptr;
  int st = cascade_check("fa_decode_plan_cascade", seqlens_host, B, max_pages_per_req, Hq, Hkv, D,
                         prefix_group_host, prefix_pages_host, n_groups, num_cus);
  if (st != FA_OK) return st;
  if (!page_table_host || num_pages < 1)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_plan_cascade: the host page table and num_pages >= 1 are required");
  std::vector<int32_t> first(std::max(n_groups, 1), -1);
  for (int b = 0; b < B; ++b) {
    const int64_t n = ((int64_t)seqlens_host[b] + fa::kPage - 1) / fa::kPage;
    const int32_t* row = page_table_host + (int64_t)b * max_pages_per_req;
    for (int64_t j = 0; j < n; ++j)
      if (row[j] < 0 || row[j] >= num_pages)
        return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_plan_cascade: page_table[%d][%lld]=%d outside [0,%d)", b, (long long)j, row[j], num_pages);
    const int g = prefix_group_host[b];
    if (g < 0) continue;
    if (first[g] < 0) {
      first[g] = b;
      continue;
    }
    const int32_t* ref = page_table_host + (int64_t)first[g] * max_pages_per_req;
    for (int j = 0; j < prefix_pages_host[g]; ++j)
      if (row[j] != ref[j])
        return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_plan_cascade: request %d does not share page %d of group %d's prefix", b, j, g);
  }
  if (num_cus == 0) {
    st = device_cus(&num_cus);
    if (st != FA_OK) return st;
  }
  fa_decode_plan_t* p = new (std::nothrow) fa_decode_plan_t;
  if (!p) return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_plan_cascade: out of host memory");
  fa::CascadePlan cp;
  if (fa::plan_cascade_host(seqlens_host, B, max_pages_per_req, Hq, Hkv, prefix_group_host, prefix_pages_host,
                            n_groups, num_cus, &cp) != 0) {
    delete p;
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_plan_cascade: planning failed");
  }
  p->B = B; p->stride = max_pages_per_req; p->num_pages = num_pages;
  p->Hq = Hq; p->Hkv = Hkv; p->D = D; p->kv_dtype = FA_DTYPE_BF16;
  p->num_splits = cp.num_splits; p->chunk_pages = cp.prefix_chunk_pages;
  p->grid = (int)cp.items.size();
  p->items = std::move(cp.items);
  p->splits = std::move(cp.splits);
  p->prefix_items = std::move(cp.prefix_items);
  p->group_reqs = std::move(cp.group_reqs);
  p->layout = fa::workspace_layout((int)p->items.size(), B, Hq, D, p->num_splits, (int)p->prefix_items.size(),
                                   (int)p->group_reqs.size());
  if (!workspace || workspace_bytes < p->layout.total) {
    size_t need = p->layout.total;
    delete p;
    return fail(FA_ERR_WORKSPACE, "fa_decode_plan_cascade: workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  }
  if (misaligned(workspace)) {
    delete p;
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_plan_cascade: workspace must be 16-byte aligned");
  }
  p->workspace = workspace;
  // The metadata before and after the partial-result area, staged and
  // uploaded in two copies (the partials themselves need no initial value).
  const fa::WorkspaceLayout& w = p->layout;
  std::vector<char> head(w.part_o_off, 0), tail(w.total - w.prefix_items_off, 0);
  if (!p->items.empty()) std::memcpy(head.data() + w.items_off, p->items.data(), sizeof(fa::WorkItem) * p->items.size());
  std::memcpy(head.data() + w.splits_off, p->splits.data(), sizeof(int32_t) * B);
  if (!p->prefix_items.empty())
    std::memcpy(tail.data(), p->prefix_items.data(), sizeof(fa::PrefixItem) * p->prefix_items.size());
  if (!p->group_reqs.empty())
    std::memcpy(tail.data() + (w.group_reqs_off - w.prefix_items_off), p->group_reqs.data(),
                sizeof(int32_t) * p->group_reqs.size());
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(workspace, head.data(), head.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess && !tail.empty())
    e = hipMemcpyAsync((char*)workspace + w.prefix_items_off, tail.data(), tail.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);  // the staging block is freed on return
  if (e != hipSuccess) {
    delete p;
    return hip_fail(e, "fa_decode_plan_cascade upload");
  }
  *plan_out = p;
  *num_splits_out = p->num_splits;
  return ok();
}

static int check_ragged_shape(const char* who, int B, int Hq, int Hkv, int D) {
  if (B < 1 || Hq < 1 || Hkv < 1)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: need B, Hq, Hkv >= 1", who);
  if (Hq > fa::kMaxHeads || Hkv > fa::kMaxHeads)
    return fail(FA_ERR_UNSUPPORTED, "%s: Hq and Hkv must be <= %d", who, fa::kMaxHeads);
  if (Hq % Hkv != 0) return fail(FA_ERR_INVALID_ARGUMENT, "%s: Hq %% Hkv != 0 (%d, %d)", who, Hq, Hkv);
  if (D != 128) return fail(FA_ERR_UNSUPPORTED, "%s: D=%d not supported (128)", who, D);
  return FA_OK;
}

int fa_kv_append(const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                 const int32_t* page_table, const int32_t* seqlens, const int32_t* cu_seqlens_q,
                 int B, int total_q, int max_pages_per_req, int num_pages, int Hkv, int D,
                 void* stream) {
  if (B < 1 || Hkv < 1 || total_q < 0 || max_pages_per_req < 1 || num_pages < 1)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_kv_append: need B, Hkv, max_pages_per_req, num_pages >= 1 and total_q >= 0");
  if (D != 128) return fail(FA_ERR_UNSUPPORTED, "fa_kv_append: D=%d not supported (128)", D);
  if (total_q == 0) return ok();
  if (!k_new || !v_new || !k_pages || !v_pages || !page_table || !seqlens || !cu_seqlens_q)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_kv_append: null pointer");
  fa::AppendArgs a;
  a.k_new = k_new; a.v_new = v_new; a.k_pages = k_pages; a.v_pages = v_pages;
  a.page_table = page_table; a.seqlens = seqlens; a.cu_q = cu_seqlens_q;
  a.B = B; a.T = total_q; a.stride = max_pages_per_req; a.num_pages = num_pages; a.Hkv = Hkv; a.D = D;
  hipError_t e = fa::device_status_ptr(&a.status);
  if (e != hipSuccess) return hip_fail(e, "fa_kv_append: device status word");
  e = fa::launch_kv_append(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fa_kv_append launch");
  return ok();
}

int fa_prefill_paged_plan_host(const int32_t* seqlens_host, const int32_t* cu_seqlens_q_host,
                               int B, int32_t* items_out, int capacity) {
  if (!seqlens_host || !cu_seqlens_q_host || B < 1 || capacity < 0) {
    fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_paged_plan_host: invalid argument");
    return -FA_ERR_INVALID_ARGUMENT;
  }
  int n = fa::plan_prefill_host(seqlens_host, cu_seqlens_q_host, B, items_out, capacity);
  if (n < 0) {
    fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_paged_plan_host: inconsistent lengths (cu[0] != 0, n_b < 0 or n_b > L_b)");
    return -FA_ERR_INVALID_ARGUMENT;
  }
  ok();
  return n;
}

size_t fa_prefill_paged_workspace_size(const int32_t* seqlens_host,
                                       const int32_t* cu_seqlens_q_host, int B) {
  if (!seqlens_host || !cu_seqlens_q_host || B < 1) return 0;
  int n = fa::plan_prefill_host(seqlens_host, cu_seqlens_q_host, B, nullptr, 0);
  if (n < 0) return 0;
  return ((size_t)std::max(n, 1) * 2 * sizeof(int32_t) + 255) / 256 * 256;
}

int fa_prefill_paged_plan(const int32_t* seqlens_host, const int32_t* cu_seqlens_q_host,
                          const int32_t* page_table_host, int B, int max_pages_per_req,
                          int num_pages, int Hq, int Hkv, int D, void* workspace,
                          size_t workspace_bytes, void* stream, fa_prefill_plan_t** plan_out) {
  if (!plan_out) return fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_paged_plan: plan_out is null");
  *plan_out = nullptr;
  int st = check_ragged_shape("fa_prefill_paged_plan", B, Hq, Hkv, D);
  if (st != FA_OK) return st;
  if (!seqlens_host || !cu_seqlens_q_host)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_paged_plan: seqlens_host and cu_seqlens_q_host are required");
  if (max_pages_per_req < 1 || num_pages < 1)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_paged_plan: need max_pages_per_req >= 1 and num_pages >= 1");
  std::vector<int32_t> items;
  int n = fa::plan_prefill_host(seqlens_host, cu_seqlens_q_host, B, nullptr, 0);
  if (n < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_paged_plan: inconsistent lengths (cu[0] != 0, n_b < 0 or n_b > L_b)");
  for (int b = 0; b < B; ++b) {
    int64_t np = ((int64_t)seqlens_host[b] + fa::kPage - 1) / fa::kPage;
    if (np > max_pages_per_req)
      return fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_paged_plan: request %d needs %lld pages > max_pages_per_req %d", b, (long long)np, max_pages_per_req);
    if (page_table_host) {
      for (int64_t j = 0; j < np; ++j) {
        int32_t id = page_table_host[(int64_t)b * max_pages_per_req + j];
        if (id < 0 || id >= num_pages)
          return fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_paged_plan: page_table[%d][%lld]=%d outside [0,%d)", b, (long long)j, id, num_pages);
      }
    }
  }
  const size_t need = fa_prefill_paged_workspace_size(seqlens_host, cu_seqlens_q_host, B);
  if (!workspace || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "fa_prefill_paged_plan: workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  if (misaligned(workspace))
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_paged_plan: workspace must be 16-byte aligned");
  items.resize(2 * (size_t)std::max(n, 1), 0);
  fa::plan_prefill_host(seqlens_host, cu_seqlens_q_host, B, items.data(), n);
  fa_prefill_plan_t* p = new (std::nothrow) fa_prefill_plan_t;
  if (!p) return fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_paged_plan: out of host memory");
  p->B = B; p->stride = max_pages_per_req; p->num_pages = num_pages;
  p->Hq = Hq; p->Hkv = Hkv; p->D = D; p->n_items = n; p->bytes = need;
  p->workspace = workspace;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(workspace, items.data(), items.size() * sizeof(int32_t), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);  // the host list is freed on return
  if (e != hipSuccess) {
    delete p;
    return hip_fail(e, "fa_prefill_paged_plan upload");
  }
  *plan_out = p;
  return ok();
}

void fa_prefill_paged_plan_destroy(fa_prefill_plan_t* plan) { delete plan; }

int fa_prefill_paged_run(const fa_prefill_plan_t* plan, const void* q, const void* k_pages,
                         const void* v_pages, const int32_t* page_table, const int32_t* seqlens,
                         const int32_t* cu_seqlens_q, float scale, void* out, float* lse,
                         void* workspace, void* stream) {
  if (!plan) return fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_paged_run: plan is null");
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_paged_run: scale is not finite");
  if (workspace != plan->workspace)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_paged_run: workspace is not the buffer the plan was built in");
  if (plan->n_items == 0) return ok();
  if (!q || !k_pages || !v_pages || !page_table || !seqlens || !cu_seqlens_q || !out || !lse || !workspace)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_prefill_paged_run: null pointer");
  fa::PrefillArgs a;
  std::memset(&a, 0, sizeof a);
  a.q = q; a.k = k_pages; a.v = v_pages; a.out = out; a.lse = lse;
  a.B = plan->B; a.Hq = plan->Hq; a.Hkv = plan->Hkv; a.D = plan->D;
  a.causal = 1;
  a.scale = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)plan->D));
  a.items = (const int32_t*)workspace;
  a.page_table = page_table; a.seqlens = seqlens; a.cu_q = cu_seqlens_q;
  a.stride = plan->stride; a.num_pages = plan->num_pages;
  hipError_t e = fa::device_status_ptr(&a.status);
  if (e != hipSuccess) return hip_fail(e, "fa_prefill_paged_run: device status word");
  e = fa::launch_prefill_paged_bf16(a, plan->n_items, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fa_prefill_paged_run launch");
  return ok();
}

int fa_debug_gather_kv(const void* pages, int kv_dtype, const int32_t* page_table,
                       int max_pages_per_req, int num_pages, int Hkv, int D, int b, int L_b,
                       int kv_head, void* dst, void* stream) {
  if (kv_dtype != FA_DTYPE_BF16 && kv_dtype != FA_DTYPE_FP8_E4M3FN)
    return fail(FA_ERR_UNSUPPORTED, "fa_debug_gather_kv: kv_dtype %d not supported", kv_dtype);
  if (D != 128 || Hkv < 1 || b < 0 || L_b < 0 || kv_head < 0 || kv_head >= Hkv ||
      max_pages_per_req < 1 || num_pages < 1 ||
      ((int64_t)L_b + fa::kPage - 1) / fa::kPage > max_pages_per_req)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_debug_gather_kv: invalid shape arguments");
  if (L_b == 0) return ok();
  if (!pages || !page_table || !dst) return fail(FA_ERR_INVALID_ARGUMENT, "fa_debug_gather_kv: null pointer");
  hipError_t e = fa::launch_gather_kv(pages, kv_dtype == FA_DTYPE_BF16 ? 2 : 1, page_table,
                                      max_pages_per_req, num_pages, Hkv, D, b, L_b, kv_head, dst,
                                      (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fa_debug_gather_kv launch");
  return ok();
}

}  // extern "C"
