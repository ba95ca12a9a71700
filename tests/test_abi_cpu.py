"""The C-ABI library on the CPU: it loads, exports every declared symbol, rejects
invalid arguments before touching the device, and plans correctly.

No test here launches a kernel: argument checks run before any HIP call.
"""
import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

import exact_attention_20_amd as fa
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.lib_path()):
        pytest.skip("libfa.so not built")
    return fa.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("fa_prefill_fwd", "fa_decode_plan", "fa_decode_run", "fa_last_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", fa.lib_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (fa_\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    for n in declared_functions():
        assert hasattr(lib, n)
    assert lib.fa_abi_version() == 2


def _prefill(lib, **kw):
    a = dict(q=C.c_void_p(16), k=C.c_void_p(16), v=C.c_void_p(16), out=C.c_void_p(16),
             lse=C.c_void_p(16), B=1, Hq=2, Hkv=2, Sq=8, Sk=8, D=128, dtype=fa.BF16, causal=1,
             scale=0.0, map=None, stream=None)
    a.update(kw)
    return lib.fa_prefill_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                              a["Sq"], a["Sk"], a["D"], a["dtype"], a["causal"], a["scale"], a["map"],
                              a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), 1), (dict(Hq=0), 1), (dict(Sq=-1), 1), (dict(Sk=-2), 1),
    (dict(causal=2), 1), (dict(scale=float("nan")), 1), (dict(Hq=3, Hkv=2), 1),
    (dict(D=64), 2), (dict(dtype=fa.F32, D=96), 2), (dict(dtype=7), 2), (dict(dtype=fa.FP8_E4M3FN), 2),
    (dict(Hq=300, Hkv=300), 2), (dict(q=None), 1), (dict(k=None), 1), (dict(lse=None), 1),
    (dict(Sk=1 << 23), 2),  # bf16 K/V buffer resource is Sk * 256 bytes
])
def test_prefill_rejects(lib, kw, code):
    assert _prefill(lib, **kw) == code
    assert lib.fa_last_error().decode()


def test_prefill_bad_map(lib):
    bad = (C.c_int32 * 2)(0, 5)
    assert _prefill(lib, map=C.cast(bad, C.POINTER(C.c_int32))) == 1
    assert b"kv_head_map" in lib.fa_last_error()


def test_prefill_sq0_is_noop(lib):
    assert _prefill(lib, Sq=0, q=None, out=None, lse=None) == 0


def _plan(lib, seqlens, table=None, **kw):
    a = dict(B=len(seqlens), stride=8, P=100, Hq=8, Hkv=2, D=128, dt=fa.BF16, ns=0, cus=4,
             ws=C.c_void_p(256), wsb=1 << 30)
    a.update(kw)
    sl = (C.c_int32 * len(seqlens))(*seqlens)
    tb = None if table is None else C.cast((C.c_int32 * len(table))(*table), C.POINTER(C.c_int32))
    h, n = C.c_void_p(), C.c_int()
    st = lib.fa_decode_plan(C.cast(sl, C.POINTER(C.c_int32)), tb, a["B"], a["stride"], a["P"], a["Hq"],
                            a["Hkv"], a["D"], a["dt"], a["ns"], a["cus"], a["ws"], a["wsb"], None,
                            C.byref(h), C.byref(n))
    return st


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=6, Hkv=4), 1), (dict(Hq=24, Hkv=2), 2), (dict(D=64), 2), (dict(dt=fa.F32), 2),
    (dict(stride=1), 1), (dict(P=0), 1), (dict(ns=-1), 1), (dict(cus=-1), 1),
    (dict(ws=None), 3), (dict(wsb=16), 3), (dict(ws=C.c_void_p(264)), 1),  # misaligned workspace
])
def test_plan_rejects(lib, kw, code):
    assert _plan(lib, [100, 300], **kw) == code


def test_plan_rejects_negative_length(lib):
    assert _plan(lib, [100, -1]) == 1


def test_plan_checks_page_ids(lib):
    # request 0 has 2 pages, request 1 has 5; stride 8
    table = [0, 1] + [-1] * 6 + [2, 3, 4, 5, 100] + [-1] * 3
    assert _plan(lib, [100, 300], table) == 1
    assert b"page_table" in lib.fa_last_error()


def test_run_rejects_null_plan(lib):
    assert lib.fa_decode_run(None, None, None, None, None, None, None, None, 0, 0.0, None, None, None, None) == 1


def test_gather_rejects(lib):
    assert lib.fa_debug_gather_kv(C.c_void_p(16), 7, C.c_void_p(16), 4, 10, 2, 128, 0, 10, 0, C.c_void_p(16), None) == 2
    assert lib.fa_debug_gather_kv(C.c_void_p(16), fa.BF16, C.c_void_p(16), 1, 10, 2, 128, 0, 100, 0, C.c_void_p(16), None) == 1
    assert lib.fa_debug_gather_kv(C.c_void_p(16), fa.BF16, C.c_void_p(16), 4, 10, 2, 128, 0, 10, 2, C.c_void_p(16), None) == 1


# ------------------------------------------------------------------ plan properties

def _check_plan(seqlens, items, splits, num_splits, Hkv, forced=0, grid=None, chunk=None):
    """Exact coverage and split numbering of a decode plan; an equal-chunk plan
    (grid == item count) also has near-equal splits, longest items first; a
    window plan keeps every workgroup's items (w, w + grid, ...) within the
    cost bound (pages + 2 per item)."""
    L = np.asarray(seqlens)
    pages = (L + 63) // 64
    windows = grid is not None and grid != len(items)
    if windows:
        assert len(items) % grid == 0 and not forced
        for w in range(grid):
            own = [it for it in items[w::grid].tolist() if it[0] >= 0]
            assert own, "idle workgroup"
            assert sum(p1 - p0 + 2 for _, _, p0, p1 in own) <= chunk
        items = items[items[:, 0] >= 0]
    else:
        assert (items[:, 0] >= 0).all(), "padding outside a window plan"
    cover = {}
    for b, gs, p0, p1 in items.tolist():
        g, s = gs & 255, gs >> 8
        assert 0 <= g < Hkv and 0 <= s < splits[b] <= num_splits
        assert 0 <= p0 < p1 <= pages[b]
        for p in range(p0, p1):
            key = (b, g, p)
            assert key not in cover, "page covered twice"
            cover[key] = s
    for b in range(len(L)):
        for g in range(Hkv):
            for p in range(pages[b]):
                assert (b, g, p) in cover, "page not covered"
    # splits of a request are contiguous, in order, near-equal
    for b in range(len(L)):
        if pages[b] == 0:
            assert splits[b] == 0
            continue
        sizes = {}
        for (bb, g, p), s in cover.items():
            if bb == b and g == 0:
                sizes[s] = sizes.get(s, 0) + 1
        assert sorted(sizes) == list(range(splits[b]))
        first = {s: min(p for (bb, g, p), ss in cover.items() if bb == b and g == 0 and ss == s) for s in sizes}
        assert [first[s] for s in range(splits[b])] == sorted(first.values()), "splits out of page order"
        if not windows:
            assert max(sizes.values()) - min(sizes.values()) <= 1
        if forced:
            assert splits[b] == min(forced, pages[b])
    assert num_splits == max(splits.tolist() + [0])
    if not windows:
        lens = (items[:, 3] - items[:, 2]).tolist()
        assert lens == sorted(lens, reverse=True), "longest items first"


@pytest.mark.parametrize("wid", [4, 5])
def test_plan_workloads(lib, wid):
    w = workloads.WORKLOADS[wid]
    L = workloads.context_lengths(wid, w.B, w.lengths)
    stride = int(((L + 63) // 64).max())
    items, splits, ns, chunk, grid = fa.fa_decode_plan_host(L, stride, w.Hq, w.Hkv, 0, 256)
    _check_plan(L, items, splits, ns, w.Hkv, grid=grid, chunk=chunk)
    total = int(((L + 63) // 64).sum()) * w.Hkv
    # balance: every item holds at most one chunk; enough work to fill 256 CUs
    assert int((items[:, 3] - items[:, 2]).max()) <= chunk
    assert grid >= 256 or total < 256 * 4


@pytest.mark.parametrize("seqlens", [[1], [0, 5, 0], [64, 65, 4096, 1, 0], list(range(0, 2000, 97))])
@pytest.mark.parametrize("forced", [0, 1, 3, 64])
def test_plan_edge_lengths(lib, seqlens, forced):
    L = np.asarray(seqlens, dtype=np.int32)
    stride = max(1, int(((L + 63) // 64).max()))
    items, splits, ns, chunk, grid = fa.fa_decode_plan_host(L, stride, 8, 2, forced, 16)
    _check_plan(L, items, splits, ns, 2, forced, grid=grid, chunk=chunk)


@pytest.mark.parametrize("seqlens", [
    [3362, 320, 997, 1431, 3493, 237, 1691], [785, 1231, 211, 2060, 2061, 167, 676, 1710, 246],
    [932, 2912, 576, 2164, 699, 207, 1597], [548, 418, 3068, 883, 47, 1706, 1381],
])
def test_window_plans(lib, seqlens):
    """Batches whose equal-chunk plan fits one round get cost-balanced windows
    (some crossing two request boundaries): exact coverage, splits in page
    order, every workgroup within the bound, padding only in later rounds."""
    L = np.asarray(seqlens, dtype=np.int32)
    items, splits, ns, chunk, grid = fa.fa_decode_plan_host(L, int(((L + 63) // 64).max()), 8, 2, 0, 16)
    assert grid < len(items), "expected a window plan"
    _check_plan(L, items, splits, ns, 2, grid=grid, chunk=chunk)
    it = items.numpy()
    assert (it[:grid, 0] >= 0).all(), "the first round has no padding"
    assert max(sum(1 for b in it[w::grid, 0] if b >= 0) for w in range(grid)) == 3


def test_plan_is_deterministic(lib):
    L = workloads.context_lengths(4, 64, ("uniform", 512, 16384))
    a = fa.fa_decode_plan_host(L, 256, 32, 8, 0, 256)
    b = fa.fa_decode_plan_host(L, 256, 32, 8, 0, 256)
    assert np.array_equal(a[0].numpy(), b[0].numpy()) and a[2:] == b[2:]


def test_backward_workspace_size(lib):
    """The backward's first kernel leaves two fp32 values per query row for the second (the
    row term D and the LSE in log2 units), each array starting on a 256-byte boundary; the
    size covers both and rejects shapes the entry point rejects."""
    for B, Hq, Sq in ((1, 1, 1), (4, 32, 4096), (2, 3, 257), (1, 8, 0)):
        n = lib.fa_prefill_bwd_workspace_size(B, Hq, Sq)
        one = -(-4 * B * Hq * Sq // 256) * 256
        assert n >= 2 * one, (B, Hq, Sq, n)
    assert lib.fa_prefill_bwd_workspace_size(0, 1, 1) == 0
    assert lib.fa_prefill_bwd_workspace_size(1, 0, 1) == 0
    assert lib.fa_prefill_bwd_workspace_size(1, 1, -1) == 0


def test_backward_noalloc_rejects_before_the_device(lib):
    """The static-scratch backward checks its arguments and its 32 MiB limit on the host:
    bad shapes and calls whose per-row arrays would not fit return an error and launch
    nothing (no device is touched, so this runs on the CPU)."""
    p = C.c_void_p(256)
    args = lambda B, Hq, Hkv, Sq, Sk, D=128: (p, p, p, p, p, p, p, p, p, B, Hq, Hkv, Sq, Sk, D, 1, 0.0, None)  # noqa: E731
    assert lib.fa_prefill_bwd_noalloc(*args(0, 1, 1, 8, 8)) == 1
    assert lib.fa_prefill_bwd_noalloc(*args(1, 6, 4, 8, 8)) == 1
    assert lib.fa_prefill_bwd_noalloc(*args(1, 2, 2, 8, 8, D=64)) == 2
    assert lib.fa_prefill_bwd_noalloc(*args(1, 1, 1, 0, 0)) == 0      # nothing to do
    # 32 heads x 131072 rows = 4.19M rows need 2 x 16 MiB + 256 B: just over the limit
    assert lib.fa_prefill_bwd_noalloc(*args(1, 32, 8, 131072, 16)) == 3
    assert b"static" in lib.fa_last_error()
    assert lib.fa_prefill_bwd_workspace_size(1, 32, 131072) > 32 << 20
    assert lib.fa_prefill_bwd_workspace_size(1, 32, 131064) <= 32 << 20


def test_workspace_size(lib):
    L = [100, 300, 0]
    n = fa.fa_decode_workspace_size(L, 8, 2, 128, 0, 16)
    items, splits, ns, _, _ = fa.fa_decode_plan_host(L, 8, 8, 2, 0, 16)
    assert n >= len(items) * 16 + 3 * 4 + 3 * 8 * ns * 129 * 4


def test_device_status_rejects_null(lib):
    # Checked before any HIP call, so it runs without a GPU.
    assert lib.fa_device_status(None, 0) == 1
    assert b"flags_out" in lib.fa_last_error()


def test_host_calls_from_many_threads(lib):
    """The host side is safe to call from several threads at once (ctypes
    drops the GIL around each call): plans match the single-threaded ones,
    and each thread reads back its own last error."""
    import threading

    rng = np.random.default_rng(11)
    inputs = [rng.integers(1, 9000, size=int(rng.integers(200, 600))).astype(np.int32) for _ in range(8)]
    ref = [fa.fa_decode_plan_host(sl, 160, 32, 8) for sl in inputs]
    i32 = C.POINTER(C.c_int32)
    failures = []

    def worker(t):
        try:
            for _ in range(30):
                items, splits, ns, ch, grid = fa.fa_decode_plan_host(inputs[t], 160, 32, 8)
                r = ref[t]
                if not (np.array_equal(items.numpy(), r[0].numpy()) and np.array_equal(splits.numpy(), r[1].numpy())
                        and (ns, ch, grid) == r[2:]):
                    failures.append(f"thread {t}: plan differs")
                    return
                # An error of this thread's own: Hq not a multiple of Hkv, with values naming the thread.
                hq = 16 + 2 * t + 1
                sl = inputs[t]
                size = lib.fa_decode_workspace_size(C.cast(sl.ctypes.data, i32), len(sl), hq, 2, 128, 0, 256)
                msg = lib.fa_last_error().decode()
                if size != 0 or f"({hq}, 2)" not in msg:
                    failures.append(f"thread {t}: size {size}, last error {msg!r}")
                    return
        except Exception as e:  # noqa: BLE001 - reported below
            failures.append(f"thread {t}: {e!r}")

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not failures, failures
