"""Thin Python binding over libfa.so, the gfx950 exact-attention library.

Argument marshalling only: torch tensors become device pointers, the current
torch stream becomes the hipStream_t, and status codes become exceptions.
Every step of the computation runs in the library's HIP kernels; there is no
fallback. If ``libfa.so`` is missing the import of this module still works
(so CPU-only tools can load it), but every call raises ``FAError`` -- build
it with ``python -m exact_attention_20_amd.build``.

Names mirror the C ABI in ``include/fa.h`` (``fa_prefill_fwd``,
``fa_decode_plan``, ``fa_decode_run``, ``fa_kv_append``,
``fa_prefill_paged_plan``, ``fa_prefill_paged_run``, ...) plus convenience
wrappers ``prefill``, ``decode`` and ``prefill_paged`` that allocate the
outputs.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

__all__ = [
    "FAError", "lib_path", "load", "F32", "BF16", "FP8_E4M3FN",
    "fa_prefill_fwd", "prefill", "DecodePlan", "fa_decode_plan", "fa_decode_run", "decode",
    "fa_decode_plan_host", "fa_decode_workspace_size", "fa_debug_gather_kv",
    "fa_kv_append", "PrefillPlan", "fa_prefill_paged_plan", "fa_prefill_paged_run",
    "fa_prefill_paged_plan_host", "fa_prefill_paged_workspace_size", "prefill_paged",
    "fa_decode_plan_cascade", "fa_decode_plan_cascade_host", "fa_decode_cascade_workspace_size",
    "fa_prefill_fp8_fwd", "prefill_fp8", "fa_prefill_bwd", "fa_prefill_bwd_workspace_size", "prefill_bwd",
    "fa_prefill_bwd_noalloc",
]

F32, BF16, FP8_E4M3FN = 0, 1, 2
_STATUS = {0: "FA_OK", 1: "FA_ERR_INVALID_ARGUMENT", 2: "FA_ERR_UNSUPPORTED",
           3: "FA_ERR_WORKSPACE", 4: "FA_ERR_HIP"}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class FAError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


def lib_path() -> str:
    """The in-tree libfa.so; FA_LIBRARY names another build of the same ABI
    (the CPU tests use it for a sanitizer build of the host code)."""
    return os.environ.get("FA_LIBRARY") or os.path.join(_HERE, "libfa.so")


def load():
    """Load libfa.so once and declare the C signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise FAError(-1, f"{path} is not built (python -m exact_attention_20_amd.build)")
    lib = C.CDLL(path)
    vp, i32p, f32p = C.c_void_p, C.POINTER(C.c_int32), C.POINTER(C.c_float)
    ci, cf, csz = C.c_int, C.c_float, C.c_size_t
    lib.fa_last_error.restype = C.c_char_p
    lib.fa_abi_version.restype = ci
    lib.fa_prefill_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, ci, cf, i32p, vp]
    lib.fa_prefill_fwd.restype = ci
    lib.fa_decode_workspace_size.argtypes = [i32p, ci, ci, ci, ci, ci, ci]
    lib.fa_decode_workspace_size.restype = csz
    lib.fa_decode_plan.argtypes = [i32p, i32p, ci, ci, ci, ci, ci, ci, ci, ci, ci, vp, csz, vp,
                                   C.POINTER(vp), C.POINTER(ci)]
    lib.fa_decode_plan.restype = ci
    lib.fa_decode_plan_destroy.argtypes = [vp]
    lib.fa_decode_plan_destroy.restype = None
    lib.fa_decode_plan_items.argtypes = [vp, i32p, ci, i32p, C.POINTER(ci)]
    lib.fa_decode_plan_items.restype = ci
    lib.fa_decode_plan_host.argtypes = [i32p, ci, ci, ci, ci, ci, ci, i32p, ci, i32p,
                                        C.POINTER(ci), C.POINTER(ci), C.POINTER(ci)]
    lib.fa_decode_plan_host.restype = ci
    lib.fa_decode_run.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ci, cf, vp, vp, vp, vp]
    lib.fa_decode_run.restype = ci
    lib.fa_debug_gather_kv.argtypes = [vp, ci, vp, ci, ci, ci, ci, ci, ci, ci, vp, vp]
    lib.fa_debug_gather_kv.restype = ci
    lib.fa_kv_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, vp]
    lib.fa_kv_append.restype = ci
    lib.fa_prefill_paged_plan_host.argtypes = [i32p, i32p, ci, i32p, ci]
    lib.fa_prefill_paged_plan_host.restype = ci
    lib.fa_prefill_paged_workspace_size.argtypes = [i32p, i32p, ci]
    lib.fa_prefill_paged_workspace_size.restype = csz
    lib.fa_prefill_paged_plan.argtypes = [i32p, i32p, i32p, ci, ci, ci, ci, ci, ci, vp, csz, vp,
                                          C.POINTER(vp)]
    lib.fa_prefill_paged_plan.restype = ci
    lib.fa_prefill_paged_plan_destroy.argtypes = [vp]
    lib.fa_prefill_paged_plan_destroy.restype = None
    lib.fa_prefill_paged_run.argtypes = [vp, vp, vp, vp, vp, vp, vp, cf, vp, vp, vp, vp]
    lib.fa_prefill_paged_run.restype = ci
    lib.fa_prefill_bwd_workspace_size.argtypes = [ci, ci, ci]
    lib.fa_prefill_bwd_workspace_size.restype = csz
    lib.fa_prefill_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, cf, vp, csz, vp]
    lib.fa_prefill_bwd.restype = ci
    lib.fa_prefill_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, cf, vp]
    lib.fa_prefill_bwd_noalloc.restype = ci
    lib.fa_prefill_fp8_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, cf, vp]
    lib.fa_prefill_fp8_fwd.restype = ci
    lib.fa_decode_cascade_workspace_size.argtypes = [i32p, ci, ci, ci, ci, ci, i32p, i32p, ci, ci]
    lib.fa_decode_cascade_workspace_size.restype = csz
    lib.fa_decode_plan_cascade.argtypes = [i32p, i32p, ci, ci, ci, ci, ci, ci, i32p, i32p, ci, ci, vp, csz,
                                           vp, C.POINTER(vp), C.POINTER(ci)]
    lib.fa_decode_plan_cascade.restype = ci
    lib.fa_decode_plan_cascade_host.argtypes = [i32p, ci, ci, ci, ci, i32p, i32p, ci, ci, i32p, ci, i32p, ci,
                                                i32p, C.POINTER(ci), C.POINTER(ci)]
    lib.fa_decode_plan_cascade_host.restype = ci
    lib.fa_device_status.argtypes = [C.POINTER(C.c_uint), ci]
    lib.fa_device_status.restype = ci
    _LIB = lib
    return lib


# Bits of the device status word (fa.h: FA_STATUS_*).
STATUS_BAD_PAGE = 1
STATUS_BAD_POSITION = 2


def device_status(clear=True):
    """The current device's status word: FA_STATUS_* bits the kernels set
    when they met bad device page-table metadata (read as zeros or skipped).
    Synchronizes the device; clears the word unless clear=False."""
    v = C.c_uint(0)
    _check(load().fa_device_status(C.byref(v), 1 if clear else 0))
    return v.value


def _check(status):
    if status != 0:
        raise FAError(status, load().fa_last_error().decode())


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _i32_host(x):
    a = torch.as_tensor(x, dtype=torch.int32, device="cpu").contiguous()
    return a, a.data_ptr()


def _need(t, name, dtype=None, device=True):
    if not isinstance(t, torch.Tensor):
        raise FAError(1, f"{name} must be a torch.Tensor")
    if not t.is_contiguous():
        raise FAError(1, f"{name} must be contiguous")
    if device and not t.is_cuda:
        raise FAError(1, f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise FAError(1, f"{name} must be {dtype} (got {t.dtype})")


_DT = {torch.float32: F32, torch.bfloat16: BF16}


# ------------------------------------------------------------------ prefill

def fa_prefill_fwd(q, k, v, out, lse, causal=True, scale=0.0, kv_head_map=None, stream=None):
    """Exact attention forward into caller-owned ``out`` [B,Hq,Sq,D] and ``lse`` [B,Hq,Sq]."""
    lib = load()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, n, q.dtype)
    _need(lse, "lse", torch.float32)
    if q.dtype not in _DT:
        raise FAError(2, f"dtype {q.dtype} not supported")
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    if k.shape != (B, Hkv, Sk, D) or v.shape != k.shape or out.shape != q.shape or lse.shape != (B, Hq, Sq):
        raise FAError(1, "inconsistent shapes")
    mp = None
    if kv_head_map is not None:
        hm, _ = _i32_host(kv_head_map)
        if hm.numel() != Hq:
            raise FAError(1, "kv_head_map needs Hq entries")
        mp = C.cast(hm.data_ptr(), C.POINTER(C.c_int32))
    _check(lib.fa_prefill_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Sq, Sk, D,
                              _DT[q.dtype], int(bool(causal)), float(scale or 0.0), mp, _stream(stream)))
    return out, lse


def prefill(q, k, v, causal=True, scale=None, kv_head_map=None, stream=None):
    """(out, lse) = exact attention of contiguous BHSD q, k, v (bf16 or fp32)."""
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    return fa_prefill_fwd(q, k, v, out, lse, causal, scale or 0.0, kv_head_map, stream)


# ------------------------------------------------------------------ decode

def fa_decode_workspace_size(seqlens, Hq, Hkv, D=128, num_splits=0, num_cus=0):
    sl, p = _i32_host(seqlens)
    n = load().fa_decode_workspace_size(C.cast(p, C.POINTER(C.c_int32)), sl.numel(), Hq, Hkv, D,
                                        num_splits, num_cus)
    if n == 0:
        raise FAError(1, "invalid arguments for the decode workspace")
    return n


def fa_decode_plan_host(seqlens, max_pages, Hq, Hkv, num_splits=0, num_cus=256):
    """Pure host planning: (items [n,4] int32 tensor, splits [B], num_splits, chunk_pages, grid).

    ``grid`` is the number of split-kernel workgroups; workgroup w runs items
    w, w + grid, ... (items with b = -1 are padding)."""
    lib = load()
    sl, p = _i32_host(seqlens)
    B = sl.numel()
    ns, ch, gr = C.c_int(0), C.c_int(0), C.c_int(0)
    i32 = C.POINTER(C.c_int32)
    n = lib.fa_decode_plan_host(C.cast(p, i32), B, max_pages, Hq, Hkv, num_splits, num_cus, None, 0,
                                None, C.byref(ns), C.byref(ch), C.byref(gr))
    if n < 0:
        _check(-n)
    items = torch.zeros((max(n, 1), 4), dtype=torch.int32)
    splits = torch.zeros(B, dtype=torch.int32)
    n2 = lib.fa_decode_plan_host(C.cast(p, i32), B, max_pages, Hq, Hkv, num_splits, num_cus,
                                 C.cast(items.data_ptr(), i32), n, C.cast(splits.data_ptr(), i32),
                                 C.byref(ns), C.byref(ch), C.byref(gr))
    assert n2 == n
    return items[:n], splits, ns.value, ch.value, gr.value


class DecodePlan:
    """A decode plan plus the device workspace it lives in (torch-allocated)."""

    def __init__(self, handle, workspace, num_splits, B, Hq, Hkv, D, kv_dtype, seqlens_host):
        self.handle = handle
        self.workspace = workspace
        self.num_splits = num_splits
        self.B, self.Hq, self.Hkv, self.D, self.kv_dtype = B, Hq, Hkv, D, kv_dtype
        self.seqlens_host = seqlens_host

    def items(self):
        lib = load()
        n = lib.fa_decode_plan_items(self.handle, None, 0, None, None)
        items = torch.zeros((max(n, 1), 4), dtype=torch.int32)
        splits = torch.zeros(self.B, dtype=torch.int32)
        ch = C.c_int(0)
        i32 = C.POINTER(C.c_int32)
        lib.fa_decode_plan_items(self.handle, C.cast(items.data_ptr(), i32), n,
                                 C.cast(splits.data_ptr(), i32), C.byref(ch))
        return items[:n], splits, ch.value

    def __del__(self):
        if getattr(self, "handle", None) and _LIB is not None:
            _LIB.fa_decode_plan_destroy(self.handle)
            self.handle = None


def fa_decode_plan(seqlens, page_table, num_pages, Hq, Hkv, D=128, kv_dtype=BF16, num_splits=0,
                   num_cus=0, device=None, stream=None):
    """Plan a paged decode batch. ``seqlens`` / ``page_table`` may live on either side;
    their host copies are read (the page table only to validate its entries)."""
    lib = load()
    sl, sp = _i32_host(seqlens.cpu() if isinstance(seqlens, torch.Tensor) else seqlens)
    pt = page_table.cpu() if isinstance(page_table, torch.Tensor) else torch.as_tensor(page_table)
    pt, pp = _i32_host(pt)
    if pt.dim() != 2 or pt.shape[0] != sl.numel():
        raise FAError(1, "page_table must be [B, max_pages]")
    B, stride = pt.shape
    i32 = C.POINTER(C.c_int32)
    ws_bytes = lib.fa_decode_workspace_size(C.cast(sp, i32), B, Hq, Hkv, D, num_splits, num_cus)
    if ws_bytes == 0:
        raise FAError(1, "invalid decode shape: " + lib.fa_last_error().decode())
    device = device or torch.device("cuda", torch.cuda.current_device())
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
    handle = C.c_void_p()
    ns = C.c_int(0)
    _check(lib.fa_decode_plan(C.cast(sp, i32), C.cast(pp, i32), B, stride, num_pages, Hq, Hkv, D,
                              kv_dtype, num_splits, num_cus, _ptr(ws), ws_bytes, _stream(stream),
                              C.byref(handle), C.byref(ns)))
    return DecodePlan(handle, ws, ns.value, B, Hq, Hkv, D, kv_dtype, sl)


def fa_decode_run(plan, q, k_pages, v_pages, page_table, seqlens, num_splits, out, lse,
                  k_scale=None, v_scale=None, scale=0.0, stream=None):
    """Split-KV decode + LSE merge into caller-owned ``out`` [B,Hq,D] bf16, ``lse`` [B,Hq] fp32."""
    lib = load()
    _need(q, "q", torch.bfloat16)
    kvt = torch.bfloat16 if plan.kv_dtype == BF16 else torch.uint8
    _need(k_pages, "k_pages", kvt)
    _need(v_pages, "v_pages", kvt)
    _need(page_table, "page_table", torch.int32)
    _need(seqlens, "seqlens", torch.int32)
    _need(out, "out", torch.bfloat16)
    _need(lse, "lse", torch.float32)
    if plan.kv_dtype == FP8_E4M3FN:
        _need(k_scale, "k_scale", torch.float32)
        _need(v_scale, "v_scale", torch.float32)
    B, Hq, D = q.shape
    if (B, Hq, D) != (plan.B, plan.Hq, plan.D) or out.shape != q.shape or lse.shape != (B, Hq):
        raise FAError(1, "q/out/lse shapes do not match the plan")
    if k_pages.dim() != 4 or k_pages.shape[1:] != (plan.Hkv, 64, D) or v_pages.shape != k_pages.shape:
        raise FAError(1, "KV pools must be [P, Hkv, 64, D]")
    _check(lib.fa_decode_run(plan.handle, _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_scale),
                             _ptr(v_scale), _ptr(page_table), _ptr(seqlens), int(num_splits),
                             float(scale or 0.0), _ptr(out), _ptr(lse), _ptr(plan.workspace),
                             _stream(stream)))
    return out, lse


def decode(plan, q, k_pages, v_pages, page_table, seqlens, k_scale=None, v_scale=None, scale=None,
           stream=None):
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    return fa_decode_run(plan, q, k_pages, v_pages, page_table, seqlens, plan.num_splits, out, lse,
                         k_scale, v_scale, scale or 0.0, stream)


def fa_debug_gather_kv(pages, kv_dtype, page_table, num_pages, b, L, kv_head, stream=None):
    """[L, D] copy of request b's tokens for one KV head, gathered on the device."""
    lib = load()
    P, Hkv, _, D = pages.shape
    dst = torch.zeros((L, D), dtype=pages.dtype, device=pages.device)
    _check(lib.fa_debug_gather_kv(_ptr(pages), kv_dtype, _ptr(page_table), page_table.shape[1],
                                  num_pages, Hkv, D, b, L, kv_head, _ptr(dst), _stream(stream)))
    return dst


# ------------------------------------------------------------------ ragged paged prefill

def _host_i32(x):
    return _i32_host(x.cpu() if isinstance(x, torch.Tensor) else x)


def fa_kv_append(k_new, v_new, k_pages, v_pages, page_table, seqlens, cu_seqlens_q, stream=None):
    """Write the packed new tokens' K/V [T, Hkv, D] into their pages (in place)."""
    lib = load()
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (k_pages, "k_pages"), (v_pages, "v_pages")):
        _need(t, n, torch.bfloat16)
    for t, n in ((page_table, "page_table"), (seqlens, "seqlens"), (cu_seqlens_q, "cu_seqlens_q")):
        _need(t, n, torch.int32)
    T, Hkv, D = k_new.shape
    if v_new.shape != k_new.shape or k_pages.dim() != 4 or k_pages.shape[1:] != (Hkv, 64, D) \
            or v_pages.shape != k_pages.shape:
        raise FAError(1, "k_new/v_new must be [T, Hkv, D] and pools [P, Hkv, 64, D]")
    B = seqlens.numel()
    if cu_seqlens_q.numel() != B + 1 or page_table.dim() != 2 or page_table.shape[0] != B:
        raise FAError(1, "cu_seqlens_q must have B + 1 entries and page_table B rows")
    _check(lib.fa_kv_append(_ptr(k_new), _ptr(v_new), _ptr(k_pages), _ptr(v_pages), _ptr(page_table),
                            _ptr(seqlens), _ptr(cu_seqlens_q), B, T, page_table.shape[1],
                            k_pages.shape[0], Hkv, D, _stream(stream)))


def fa_prefill_paged_plan_host(seqlens, cu_seqlens_q):
    """Pure host planning: work items [n, 2] (request, query tile), heaviest first."""
    lib = load()
    sl, sp = _host_i32(seqlens)
    cu, cp = _host_i32(cu_seqlens_q)
    i32 = C.POINTER(C.c_int32)
    B = sl.numel()
    n = lib.fa_prefill_paged_plan_host(C.cast(sp, i32), C.cast(cp, i32), B, None, 0)
    if n < 0:
        _check(-n)
    items = torch.zeros((max(n, 1), 2), dtype=torch.int32)
    lib.fa_prefill_paged_plan_host(C.cast(sp, i32), C.cast(cp, i32), B, C.cast(items.data_ptr(), i32), n)
    return items[:n]


def fa_prefill_paged_workspace_size(seqlens, cu_seqlens_q):
    sl, sp = _host_i32(seqlens)
    cu, cp = _host_i32(cu_seqlens_q)
    i32 = C.POINTER(C.c_int32)
    n = load().fa_prefill_paged_workspace_size(C.cast(sp, i32), C.cast(cp, i32), sl.numel())
    if n == 0:
        raise FAError(1, "invalid lengths for the ragged prefill workspace")
    return n


class PrefillPlan:
    """A ragged prefill plan plus the device workspace holding its work list."""

    def __init__(self, handle, workspace, B, Hq, Hkv, D, n_items):
        self.handle = handle
        self.workspace = workspace
        self.B, self.Hq, self.Hkv, self.D, self.n_items = B, Hq, Hkv, D, n_items

    def __del__(self):
        if getattr(self, "handle", None) and _LIB is not None:
            _LIB.fa_prefill_paged_plan_destroy(self.handle)
            self.handle = None


def fa_prefill_paged_plan(seqlens, cu_seqlens_q, page_table, num_pages, Hq, Hkv, D=128, device=None,
                          stream=None):
    """Plan a ragged prefill batch from host copies of its lengths (and page table, validated)."""
    lib = load()
    sl, sp = _host_i32(seqlens)
    cu, cp = _host_i32(cu_seqlens_q)
    pt, pp = _host_i32(page_table)
    if pt.dim() != 2 or pt.shape[0] != sl.numel() or cu.numel() != sl.numel() + 1:
        raise FAError(1, "page_table must be [B, max_pages] and cu_seqlens_q [B + 1]")
    B, stride = pt.shape
    i32 = C.POINTER(C.c_int32)
    ws_bytes = lib.fa_prefill_paged_workspace_size(C.cast(sp, i32), C.cast(cp, i32), B)
    if ws_bytes == 0:
        raise FAError(1, "invalid ragged lengths")
    device = device or torch.device("cuda", torch.cuda.current_device())
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
    handle = C.c_void_p()
    _check(lib.fa_prefill_paged_plan(C.cast(sp, i32), C.cast(cp, i32), C.cast(pp, i32), B, stride,
                                     int(num_pages), Hq, Hkv, D, _ptr(ws), ws_bytes, _stream(stream),
                                     C.byref(handle)))
    n = lib.fa_prefill_paged_plan_host(C.cast(sp, i32), C.cast(cp, i32), B, None, 0)
    return PrefillPlan(handle, ws, B, Hq, Hkv, D, n)


def fa_prefill_paged_run(plan, q, k_pages, v_pages, page_table, seqlens, cu_seqlens_q, out, lse,
                         scale=0.0, stream=None):
    """Causal attention of the packed new tokens q [T, Hq, D] over their paged caches."""
    lib = load()
    for t, n in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages"), (out, "out")):
        _need(t, n, torch.bfloat16)
    _need(lse, "lse", torch.float32)
    for t, n in ((page_table, "page_table"), (seqlens, "seqlens"), (cu_seqlens_q, "cu_seqlens_q")):
        _need(t, n, torch.int32)
    T, Hq, D = q.shape
    if (Hq, D) != (plan.Hq, plan.D) or out.shape != q.shape or lse.shape != (T, Hq):
        raise FAError(1, "q/out/lse shapes do not match the plan")
    if k_pages.dim() != 4 or k_pages.shape[1:] != (plan.Hkv, 64, D) or v_pages.shape != k_pages.shape:
        raise FAError(1, "KV pools must be [P, Hkv, 64, D]")
    _check(lib.fa_prefill_paged_run(plan.handle, _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(page_table),
                                    _ptr(seqlens), _ptr(cu_seqlens_q), float(scale or 0.0), _ptr(out),
                                    _ptr(lse), _ptr(plan.workspace), _stream(stream)))
    return out, lse


def prefill_paged(plan, q, k_pages, v_pages, page_table, seqlens, cu_seqlens_q, scale=None,
                  stream=None):
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    return fa_prefill_paged_run(plan, q, k_pages, v_pages, page_table, seqlens, cu_seqlens_q, out, lse,
                                scale or 0.0, stream)


# ------------------------------------------------------------------ shared-prefix (cascade) decode

def _cascade_host_args(seqlens, prefix_group, prefix_pages):
    sl, sp = _host_i32(seqlens)
    gr, gp = _host_i32(prefix_group)
    pg, pp = _host_i32(prefix_pages if len(prefix_pages) else [0])
    if gr.numel() != sl.numel():
        raise FAError(1, "prefix_group needs one entry per request")
    i32 = C.POINTER(C.c_int32)
    return (sl, gr, pg), C.cast(sp, i32), C.cast(gp, i32), C.cast(pp, i32), len(prefix_pages)


def fa_decode_cascade_workspace_size(seqlens, max_pages, Hq, Hkv, prefix_group, prefix_pages, D=128,
                                     num_cus=0):
    keep, sp, gp, pp, ng = _cascade_host_args(seqlens, prefix_group, prefix_pages)
    n = load().fa_decode_cascade_workspace_size(sp, keep[0].numel(), max_pages, Hq, Hkv, D, gp, pp, ng, num_cus)
    if n == 0:
        raise FAError(1, "invalid cascade arguments: " + load().fa_last_error().decode())
    return n


def fa_decode_plan_cascade_host(seqlens, max_pages, Hq, Hkv, prefix_group, prefix_pages, num_cus=256):
    """Pure host cascade planning: (suffix items [n,4], prefix items [m,8], splits [B], num_splits)."""
    lib = load()
    keep, sp, gp, pp, ng = _cascade_host_args(seqlens, prefix_group, prefix_pages)
    B = keep[0].numel()
    npi, ns = C.c_int(0), C.c_int(0)
    i32 = C.POINTER(C.c_int32)
    n = lib.fa_decode_plan_cascade_host(sp, B, max_pages, Hq, Hkv, gp, pp, ng, num_cus, None, 0, None, 0, None,
                                        C.byref(npi), C.byref(ns))
    if n < 0:
        _check(-n)
    items = torch.zeros((max(n, 1), 4), dtype=torch.int32)
    pitems = torch.zeros((max(npi.value, 1), 8), dtype=torch.int32)
    splits = torch.zeros(B, dtype=torch.int32)
    lib.fa_decode_plan_cascade_host(sp, B, max_pages, Hq, Hkv, gp, pp, ng, num_cus,
                                    C.cast(items.data_ptr(), i32), n, C.cast(pitems.data_ptr(), i32), npi.value,
                                    C.cast(splits.data_ptr(), i32), C.byref(npi), C.byref(ns))
    return items[:n], pitems[:npi.value], splits, ns.value


def fa_decode_plan_cascade(seqlens, page_table, num_pages, Hq, Hkv, prefix_group, prefix_pages, D=128,
                           num_cus=0, device=None, stream=None):
    """Plan a shared-prefix decode batch (bf16 KV); run it with fa_decode_run / decode."""
    lib = load()
    keep, sp, gp, pp, ng = _cascade_host_args(seqlens, prefix_group, prefix_pages)
    pt, ptp = _host_i32(page_table)
    if pt.dim() != 2 or pt.shape[0] != keep[0].numel():
        raise FAError(1, "page_table must be [B, max_pages]")
    B, stride = pt.shape
    i32 = C.POINTER(C.c_int32)
    ws_bytes = lib.fa_decode_cascade_workspace_size(sp, B, stride, Hq, Hkv, D, gp, pp, ng, num_cus)
    if ws_bytes == 0:
        raise FAError(1, "invalid cascade arguments: " + lib.fa_last_error().decode())
    device = device or torch.device("cuda", torch.cuda.current_device())
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
    handle = C.c_void_p()
    ns = C.c_int(0)
    _check(lib.fa_decode_plan_cascade(sp, C.cast(ptp, i32), B, stride, int(num_pages), Hq, Hkv, D, gp, pp, ng,
                                      num_cus, _ptr(ws), ws_bytes, _stream(stream), C.byref(handle), C.byref(ns)))
    return DecodePlan(handle, ws, ns.value, B, Hq, Hkv, D, BF16, keep[0])


# ------------------------------------------------------------------ fp8 prefill

def fa_prefill_fp8_fwd(q8, k8, v8, q_scale, k_scale, v_scale, out, lse, causal=True, scale=0.0, stream=None):
    """fp8 (e4m3fn codes, uint8) prefill into caller-owned out [B,Hq,Sq,128] bf16, lse [B,Hq,Sq] fp32."""
    lib = load()
    for t, n in ((q8, "q"), (k8, "k"), (v8, "v")):
        _need(t, n, torch.uint8)
    for t, n in ((q_scale, "q_scale"), (k_scale, "k_scale"), (v_scale, "v_scale"), (lse, "lse")):
        _need(t, n, torch.float32)
    _need(out, "out", torch.bfloat16)
    B, Hq, Sq, D = q8.shape
    Hkv, Sk = k8.shape[1], k8.shape[2]
    if k8.shape != (B, Hkv, Sk, D) or v8.shape != k8.shape or out.shape != q8.shape or lse.shape != (B, Hq, Sq) \
            or q_scale.shape != (B, Hq) or k_scale.shape != (B, Hkv) or v_scale.shape != (B, Hkv):
        raise FAError(1, "inconsistent shapes")
    _check(lib.fa_prefill_fp8_fwd(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale),
                                  _ptr(out), _ptr(lse), B, Hq, Hkv, Sq, Sk, D, int(bool(causal)),
                                  float(scale or 0.0), _stream(stream)))
    return out, lse


def prefill_fp8(q8, k8, v8, q_scale, k_scale, v_scale, causal=True, scale=None, stream=None):
    out = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty(q8.shape[:3], dtype=torch.float32, device=q8.device)
    return fa_prefill_fp8_fwd(q8, k8, v8, q_scale, k_scale, v_scale, out, lse, causal, scale or 0.0, stream)


# ------------------------------------------------------------------ backward

def fa_prefill_bwd_workspace_size(B, Hq, Sq):
    return load().fa_prefill_bwd_workspace_size(B, Hq, Sq)


def fa_prefill_bwd(q, k, v, o, lse, dout, dq, dk, dv, causal=True, scale=0.0, workspace=None, stream=None):
    """Gradients into caller-owned dq [B,Hq,Sq,128], dk/dv [B,Hkv,Sk,128] (bf16)."""
    lib = load()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need(t, n, torch.bfloat16)
    _need(lse, "lse", torch.float32)
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    if k.shape != (B, Hkv, Sk, D) or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape \
            or dq.shape != q.shape or dk.shape != k.shape or dv.shape != k.shape or lse.shape != (B, Hq, Sq):
        raise FAError(1, "inconsistent shapes")
    need = lib.fa_prefill_bwd_workspace_size(B, Hq, Sq)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(lib.fa_prefill_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                              _ptr(dv), B, Hq, Hkv, Sq, Sk, D, int(bool(causal)), float(scale or 0.0),
                              _ptr(workspace), workspace.numel(), _stream(stream)))
    return dq, dk, dv


def fa_prefill_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, causal=True, scale=0.0, stream=None):
    """fa_prefill_bwd with the library's static device scratch in place of a workspace
    (for callers that cannot allocate); same outputs, written into dq, dk, dv."""
    lib = load()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need(t, n, torch.bfloat16)
    _need(lse, "lse", torch.float32)
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    if k.shape != (B, Hkv, Sk, D) or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape \
            or dq.shape != q.shape or dk.shape != k.shape or dv.shape != k.shape or lse.shape != (B, Hq, Sq):
        raise FAError(1, "inconsistent shapes")
    _check(lib.fa_prefill_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                      _ptr(dk), _ptr(dv), B, Hq, Hkv, Sq, Sk, D, int(bool(causal)),
                                      float(scale or 0.0), _stream(stream)))
    return dq, dk, dv


def prefill_bwd(q, k, v, o, lse, dout, causal=True, scale=None, stream=None):
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    return fa_prefill_bwd(q, k, v, o, lse, dout, dq, dk, dv, causal, scale or 0.0, None, stream)
